// Internal definitions shared by the HIP translation units of libglowq (not installed).
//
// Device layout of one INT4-g128 module (n_out x k_in, G = k_in / 128 groups, NT = ceil(n_out/16)
// row tiles of 16 rows):
//   q  : G x NT blocks of 1024 bytes, block (rt, g) at byte (g * NT + rt) * 1024 (group-major: the
//        blocks of one input group are adjacent for all row tiles, so workgroups that stream their
//        tiles in step read one contiguous region of memory at a time).  Lane l (0..63)
//        of a wavefront owns the 16 bytes at l * 16: four 32-bit words, word j (0..3) holding the
//        eight inputs k = 128 g + 32 j + 8 (l / 16) + e, e = 0..7, of row 16 rt + (l % 16).  This
//        is exactly the A/B operand of v_mfma_f32_16x16x32_f16 (lane l: row l % 16, k-slice
//        8 (l / 16) .. +8) for the j-th 32-wide slice of the group, so one 128-bit load per lane
//        brings a whole group's operands for four matrix-core steps.  Inside a word, nibble slot
//        p (bits 4p..4p+3) holds e = 2p for p < 4 and e = 2(p - 4) + 1 for p >= 4, so that
//        masking with 0x000F000F / 0x00F000F0 (after a shift by 0 or 8) yields the fp16 pairs
//        (e0, e1), (e2, e3), (e4, e5), (e6, e7) with the 0x6400 exponent trick.
//   sz : G x NT blocks of 64 bytes, block (rt, g) at byte (g * NT + rt) * 64: sixteen (z, s) fp16
//        pairs, pair i for row 16 rt + i.
//   Rows >= n_out are zero (q = 0, z = 0, s = 0).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace glowq {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

constexpr int kGroup = 128;
constexpr int kMaxModules = 8;
constexpr int kMaxRank = 256;
constexpr size_t kWsHeader = 8192;  // workspace bytes reserved for synchronisation words
// Synchronisation words of the decode hand-off, int32 offsets into the workspace header, each on
// its own 64-byte line.  The projection R travels as (value, tag) pairs written with single 64-bit
// stores; a pair is current when its tag equals epoch + 1, where epoch is the header word read by
// every workgroup at start.  The last arrival of a call (slot counters, then a counter over the
// slots) advances the epoch, so no memset is ever needed and stale pairs never match:
// tags run 1 .. 2^32 - 1 (the epoch skips 2^32 - 1), and the calls with tags 1 and 2^32 - 1
// clear every pair outside their own range.  A pair that still held tag t when the tag comes
// round again would have outlived a whole wrap, so also the last of those two calls before it:
// that call either overwrote the pair with its own tag or cleared it.
// Arrivals: workgroup b adds to the counter of slot b % kArriveSlots; the slot's last arrival
// resets it and adds to the top counter, whose last arrival advances the epoch.  64 slots rather
// than one per XCD: same-address atomics serialise (a streaming launch of 832 workgroups with one
// arrival each takes 7.09 us on 8 counters, 6.55 us on 64, 6.37 us without).
constexpr int kArriveSlots = 64;
constexpr int kSyncEpoch = 0;     // epoch of the call in flight
constexpr int kSyncDone = 16;     // done[s] at word kSyncDone + 16 s: arrivals of slot s
constexpr int kSyncTop = kSyncDone + 16 * kArriveSlots;  // slots whose workgroups all arrived
constexpr int kSyncError = kSyncTop + 16;  // nonzero when a bounded wait expired (results invalid)
static_assert((kSyncError + 16) * 4 <= (int)kWsHeader, "synchronisation words fit the header");
constexpr int kSpinLimit = 1 << 20;
// The decode projection is written in kRReplicas copies, one per XCD (copy b % 8 is read by
// workgroup b), so that the consumers polling it spread over eight sets of cache lines.
constexpr int kRReplicas = 8;
// Token count above which the prefill (dequant-to-register MFMA GEMM) kernels are used.
constexpr int kDecodeMaxT = 64;
// Between kDecodeWideT and kDecodeMaxT tokens the activations no longer fit in LDS and the decode
// kernel re-reads them from L2 for every 16-row tile; a call with at least kPrefillMinRowTiles
// 128-row tiles (a wide group) then runs the prefill path instead, whose tiles share them.
constexpr int kDecodeWideT = 16;
constexpr int kPrefillMinRowTiles = 40;
// The correcting narrow calls of kDecodeWideT + 1 .. kDecodeMaxT tokens that stay on the decode
// path (fewer than kPrefillMinRowTiles 128-row tiles, so at most kNarrowMaxRows rows) with long
// rows (at least kNarrowMinGroups input groups) split K into kNarrowKs ranges over workgroups of
// kNarrowRt row tiles: the activations each CU reads from L2 shrink 4x at the same workgroup
// count; the first range carries the correction and a second launch adds the fp32 partial sums
// in range order (down_proj 4096 <- 14336 at T = 64: 67.6 -> 42.9 us; at d = 4096 the split is
// no faster, its ranges being two groups per wave).
constexpr int kNarrowKs = 4;
constexpr int kNarrowRt = 4;
constexpr int kNarrowMinGroups = 64;
constexpr int kNarrowMaxRows = kPrefillMinRowTiles * 128;
// The decode pairs live in a fixed area right after the header, sized for the largest decode
// call (T <= kDecodeMaxT, r <= kMaxRank, up to kMaxModules projections, kRReplicas copies), so
// that no other data (the prefill projection of an earlier call) ever lies where a later decode
// call polls for its tags.
constexpr size_t kDecodeAreaPairs = (size_t)kDecodeMaxT * kMaxRank * kMaxModules * kRReplicas;
constexpr int kMaxProducers = 64;
// Largest activation block ((T + 1) x d fp16 bytes) the decode kernel stages in LDS.
constexpr size_t kDecodeXLdsMax = 48 * 1024;
// Decode workgroup shape: 8 waves when a launch has at most kDecodeWide8Tiles 16-row tiles and
// long rows (at least kDecodeWide8Groups input groups); two row tiles per workgroup when it has
// more than kDecodeRt2Tiles (so that every workgroup is resident at once).
constexpr int kDecodeWide8Tiles = 512;
constexpr int kDecodeWide8Groups = 64;
constexpr int kDecodeRt2Tiles = 1024;
// Without the activations in LDS (6 to 16 tokens at d = 4096) every workgroup reads them from L2
// with its weights; two row tiles per workgroup then halve that traffic once a launch has this many
// 16-row tiles (QKV decode at T = 16: 25.8 -> 18.5 us).
constexpr int kDecodeRt2NoLdsTiles = 512;

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// --------------------------------------------------------------------- device helpers
__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

// Bit masks of the nibble unpacking, held in VGPRs so that each mask-and-or is one v_and_or_b32
// (a VALU instruction can read only one scalar constant on this architecture).
struct NibConsts {
    uint32_t lo, hi, magic;
};
__device__ __forceinline__ NibConsts nib_consts() {
    NibConsts n;
    asm volatile("v_mov_b32 %0, 0x000f000f" : "=v"(n.lo));
    asm volatile("v_mov_b32 %0, 0x00f000f0" : "=v"(n.hi));
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(n.magic));
    return n;
}

// Eight nibbles of one device-layout word -> the eight integer differences (q - z) as fp16,
// exact for integer z in [-1024, 1024]: 0x6400 | q is the fp16 value 1024 + q, 0x6400 | (q << 4)
// is 1024 + 16 q; subtracting 1024 + z (resp. scaling by 1/16 and subtracting 64 + z) is exact.
__device__ __forceinline__ h8 nib8_minus_z(uint32_t w, h2 zc1024, h2 zc64, const NibConsts& n) {
    const uint32_t lo = w, hi = w >> 8;
    const h2 p0 = as_h2((lo & n.lo) | n.magic);
    const h2 p1 = as_h2((lo & n.hi) | n.magic);
    const h2 p2 = as_h2((hi & n.lo) | n.magic);
    const h2 p3 = as_h2((hi & n.hi) | n.magic);
    const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2 d0 = p0 - zc1024;
    const h2 d1 = p1 * sixteenth - zc64;
    const h2 d2 = p2 - zc1024;
    const h2 d3 = p3 * sixteenth - zc64;
    h8 r;
    r[0] = d0[0]; r[1] = d0[1]; r[2] = d1[0]; r[3] = d1[1];
    r[4] = d2[0]; r[5] = d2[1]; r[6] = d3[0]; r[7] = d3[1];
    return r;
}

// (1024 + z, 1024 + z) and (64 + z, 64 + z) from the (z, s) pair word of a row.
__device__ __forceinline__ void zero_consts(uint32_t zs, h2& zc1024, h2& zc64) {
    const _Float16 z = as_h2(zs)[0];
    const _Float16 a = (_Float16)1024.0f + z;
    const _Float16 b = (_Float16)64.0f + z;
    zc1024 = h2{a, a};
    zc64 = h2{b, b};
}

// --------------------------------------------------------------------- MX weight formats
// Device layout of an MX module (elements of the OCP Microscaling v1.0 formats, one E8M0 scale per
// 32 inputs of a row), in the INT4 block geometry but with one MX block per lane:
//   q  : G x NT blocks of Fmt<F>::qblock bytes, block (rt, g) at (g NT + rt) qblock.  Lane l owns
//        the 32 codes of row 16 rt + l % 16 for the inputs 128 g + 32 (l / 16) + n, n = 0..31 -- the
//        whole MX block l / 16 of that row, so a lane needs one scale.  MXFP4: the 16 bytes at 16 l,
//        code n in bits 4n..4n+3 (the scaled fp4 conversion turns byte b of a word into the fp16
//        pair (2b, 2b + 1), low nibble first; the block-scaled matrix cores read the same 16 bytes as
//        their FP4 operand).  MXFP6: 24 bytes in two naturally aligned planes, 16 at 16 l and 8 at
//        1024 + 8 l, code n in bits 6n..6n+5 of their 192-bit concatenation (the order of the
//        32-value fp6 conversion).
//        For the fp16 matrix cores (16x16x32 steps) word j of a lane, codes 8j .. 8j + 7, is the
//        A operand of step j, so the activation operand of lane (t, q) at step j is the 8 inputs
//        128 g + 32 q + 8 j .. + 7 of token t ("block order", instead of INT4's 128 g + 32 j + 8 q).
//   sz : 64-byte blocks as for INT4; row i's word at 4 i holds in byte q the E8M0 scale S of the
//        inputs 128 g + 32 q .. + 31.  Rows >= n_out have codes 0 and scale bytes 127.
// The repack admits only scales for which every element times 2^(S - 127) is an fp16 value, so
// the dequantised operands are exact.
enum : int { kFmtInt4 = 0, kFmtMxfp4 = 1, kFmtMxfp6E2M3 = 2, kFmtMxfp6E3M2 = 3 };
template <int F>
struct Fmt {
    static constexpr bool mx = F != kFmtInt4;
    static constexpr bool six = F == kFmtMxfp6E2M3 || F == kFmtMxfp6E3M2;
    static constexpr int qblock = six ? 1536 : 1024;
    // activation operand of matrix-core step j for lane group q (offsets in inputs within a group)
    static __device__ __forceinline__ int xofs(int q) { return mx ? 32 * q : 8 * q; }
    static constexpr int xstep = mx ? 8 : 32;
};
typedef _Float16 h32 __attribute__((ext_vector_type(32)));
typedef uint32_t u6 __attribute__((ext_vector_type(6)));

// The fp32 power of two 2^(S - 127) of scale byte q of a row's scale word (S in 1..254).
__device__ __forceinline__ float mx_scale(uint32_t sw, int q) {
    return __builtin_bit_cast(float, ((sw >> (8 * q)) & 0xFFu) << 23);
}

// Eight FP4 codes (one word, code e in bits 4e..4e+3) -> fp16 element * scale.
__device__ __forceinline__ h8 mx4_h8(uint32_t w, float s) {
    const h2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, 0);
    const h2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, 1);
    const h2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, 2);
    const h2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, 3);
    return h8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// A lane's 32 FP6 codes (one MX block) -> fp16 element * scale (exact in the admitted range).
template <int F>
__device__ __forceinline__ h32 mx6_h32(u4 lo, u2 hi, float s) {
    const u6 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1]};
    if constexpr (F == kFmtMxfp6E3M2)
        return __builtin_amdgcn_cvt_scalef32_pk32_f16_bf6(w, s);
    else
        return __builtin_amdgcn_cvt_scalef32_pk32_f16_fp6(w, s);
}

// The same conversion, never merged with an identical one: kernels that hold many row tiles take
// one slice per conversion instead of keeping all 32 values live across their slice loop (the
// empty asm makes the input a fresh value; it emits no instruction).
template <int F>
__device__ __forceinline__ h32 mx6_h32_fresh(u4 lo, u2 hi, float s) {
    uint32_t w0 = lo[0];
    asm volatile("" : "+v"(w0));
    return mx6_h32<F>(u4{w0, lo[1], lo[2], lo[3]}, hi, s);
}

// Slice j (codes 8 j .. 8 j + 7) of a lane's 32 converted values.
__device__ __forceinline__ h8 mx6_slice(const h32& v, int j) {
    return h8{v[8 * j], v[8 * j + 1], v[8 * j + 2], v[8 * j + 3], v[8 * j + 4], v[8 * j + 5], v[8 * j + 6],
              v[8 * j + 7]};
}

__device__ __forceinline__ f4 mfma16(h8 a, h8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ h8 load_h8(const void* p) {
    return __builtin_bit_cast(h8, *reinterpret_cast<const u4*>(p));
}

// --------------------------------------------------------------------- launch arguments
struct ModuleArgs {
    const uint8_t* q;    // device layout
    const uint8_t* sz;   // device layout
    const _Float16* a;   // [n_out][r] (may be null when no correction)
    _Float16* y;         // [T][n_out]
    int32_t n_out;
    int32_t n_tiles16;   // ceil(n_out / 16)
    int32_t tile_begin;  // first work tile of this module in the launch's tile numbering
    int32_t proj;        // which projection R_p this module adds (0 for shared B)
    int32_t row_begin;   // first row of this module in the launch's concatenated rows
};

struct ForwardArgs {
    const _Float16* x;   // [T][d]
    int32_t T, d, G;     // G = d / 128
    int32_t fmt;         // weight format of every module (kFmt*)
    int32_t r;           // rank (0 = no correction)
    int32_t r_pad;       // r rounded up to 32 (prefill R row stride)
    int32_t n_mod;
    int32_t tile_begin[kMaxModules];  // first work tile of each module (contiguous: one scalar load)
    int32_t n_tiles;     // total work tiles of the launch
    int32_t m_tiles;     // token tiles (prefill)
    int32_t tile_tt;     // prefill tile shape: 16-token tiles per wave
    int32_t tile_rr;     // prefill tile shape: 16-row tiles per wave (4 waves side by side)
    int32_t tile_ks;     // prefill small grids: wave groups splitting the input groups (1, 2 or 4)
    void* R;             // projections: decode (fp32, tag) pairs [n_proj][T][r]; prefill fp16 [n_proj][T][r_pad]
    int32_t* sync;       // workspace header (decode)
    int32_t n_proj;      // projections (1 shared, m layerwise)
    int32_t n_prod;      // decode: producer workgroups forming R (0 without correction)
    int32_t prod_rows;   // decode: stacked projection rows per producer
    int32_t r_lds_off;   // decode: byte offset of the R copy in dynamic LDS (set by the launcher)
    int32_t dec_kw;      // decode: waves per workgroup (4 or 8)
    int32_t dec_rt;      // decode: 16-row tiles per workgroup (1, 2, or 4 with a K split)
    int32_t dec_ks;      // decode: K ranges per row block (1, or kNarrowKs for narrow calls)
    int32_t dec_gk;      // decode: input groups per K range
    int32_t dec_tiles;   // decode: row blocks (n_tiles = dec_tiles * dec_ks consumer workgroups)
    int32_t rows_total;  // decode: rows of all modules
    float* ypart;        // decode with a K split: fp32 partial sums [dec_ks][T][rows_total]
    const int8_t* xq;     // W4A8: token codes [T][d] in the matrix-core operand order
    const int32_t* xsum;  // W4A8: per (token, group) code sums [T][G]
    const float* xscale;  // W4A8: per-token scales [T]
    const uint8_t* x8;       // MXFP8 activations: E4M3 codes [T][d] in the block-scaled operand order
    const uint8_t* x8scale;  // MXFP8 activations: E8M0 block scales [T][d / 32]
    const _Float16* b[kMaxModules];  // [r][d] right factors, one per projection
    ModuleArgs mod[kMaxModules];
};

struct ProjArgs {
    const _Float16* x;   // [T][d]
    int32_t T, d, r, r_pad, n_proj;
    int32_t ks, k_per;   // K split: ks ranges of k_per inputs (a multiple of 128)
    int32_t tok_tiles;   // 16-token tiles per workgroup: 1, or 2 when r_pad <= 128
    float* part;         // fp32 partials [ks][n_proj][T][r_pad]
    const _Float16* b[kMaxModules];  // [r][d] per projection
    void* R;             // output
};

// Mixture of experts: stacked expert modules and device-side routing (one launch for all experts).
constexpr int kMoeMaxExperts = 256;
constexpr int kMoeMaxMod = 4;
constexpr int64_t kMoeMaxGrid = 2048;  // persistent workgroups of a grouped launch
struct MoeArgs {
    const _Float16* x;          // [T][d]; row j reads x[row_token[j]] (or x[j] without row_token)
    int32_t T, d, G;
    const int32_t* row_token;   // [n_rows] or nullptr
    const int32_t* offsets;     // [n_exp + 1]
    int32_t n_exp, n_rows, m;
    const uint8_t* q[kMoeMaxMod];
    const uint8_t* sz[kMoeMaxMod];
    int64_t qbytes[kMoeMaxMod], szbytes[kMoeMaxMod];  // one expert's module, bytes
    const _Float16* a[kMoeMaxMod];  // [n_exp][n_out][r]
    _Float16* y[kMoeMaxMod];        // [n_rows][n_out]
    int32_t n_out[kMoeMaxMod], n_tiles16[kMoeMaxMod];
    int32_t rb_begin[kMoeMaxMod + 1];  // prefix of the modules' row blocks (64 RR rows)
    int32_t n_rb;
    int32_t r, r_pad;
    const _Float16* R;          // fp16 projection rows [.][r_pad]
    int32_t r_by_token;         // 1: R row = the row's token (one B for all experts); 0: R row = j
    int32_t tile_tt;            // 16 TT routed rows per block (0: decode items of 16 rows x 16 routed rows)
    int32_t* err;               // workspace error word (bit 1: routing data out of range)
    const _Float16* b;          // per-expert right factors [n_exp][r][d] (projection launch)
    _Float16* Rout;             // projection output [n_rows][r_pad]
};
hipError_t launch_moe_proj(const MoeArgs& a, int64_t max_items, hipStream_t stream);
hipError_t launch_moe_gemm(const MoeArgs& a, int64_t max_items, hipStream_t stream);

// Module owning work tile `tile` (uniform across the workgroup): one contiguous scalar load of the
// tile_begin table, so the module's own arguments are fetched with a single dependent load.
__device__ __forceinline__ int module_of(const ForwardArgs& a, int tile) {
    int i = 0;
#pragma unroll
    for (int k = 1; k < kMaxModules; ++k) i += (k < a.n_mod && tile >= a.tile_begin[k]) ? 1 : 0;
    return __builtin_amdgcn_readfirstlane(i);
}

// --------------------------------------------------------------------- launchers
hipError_t launch_repack(const uint32_t* qc, const _Float16* s, const _Float16* z, int64_t n_out,
                         int64_t k_in, uint8_t* q_dev, uint8_t* sz_dev, int32_t* flag,
                         hipStream_t stream);
hipError_t launch_flag_clear(int32_t* flag, hipStream_t stream);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream);
hipError_t launch_dequant(int fmt, const uint8_t* q, const uint8_t* sz, int64_t n_out, int64_t k_in, void* out,
                          int dtype, hipStream_t stream);
hipError_t launch_repack_mx(int fmt, const uint8_t* codes, const uint8_t* scales, int64_t n_out, int64_t k_in,
                            uint8_t* q_dev, uint8_t* sz_dev, int32_t* flag, hipStream_t stream);
hipError_t launch_proj_prefill(const ProjArgs& p, hipStream_t stream);
hipError_t launch_decode(const ForwardArgs& a, hipStream_t stream);
// y = the a.dec_ks fp32 partial sums at a.ypart ([dec_ks][T][rows_total]) added in range order,
// rounded once to fp16 into the modules' outputs (the second launch of a K-split call)
hipError_t launch_part_reduce(const ForwardArgs& a, hipStream_t stream);
hipError_t launch_prefill(const ForwardArgs& a, hipStream_t stream);
hipError_t launch_quant_mx8(const _Float16* x, int T, int d, uint8_t* xq, uint8_t* xs, hipStream_t stream);
hipError_t launch_mx8(const ForwardArgs& a, hipStream_t stream);
hipError_t launch_quant_x(const _Float16* x, int T, int d, int8_t* xq, int32_t* xsum, float* xscale,
                          hipStream_t stream);
hipError_t launch_w4a8(const ForwardArgs& a, hipStream_t stream);
// W4A8: features of a call (the quantise kernel holds a token's row in registers)
constexpr int64_t kW4a8MaxD = 16384;

// Prefill projection launch: largest K split, and the workgroup count the split aims at (one per
// CU; 512 workgroups, also with 16 splits, measured slower).
constexpr int kProjMaxSplit = 8;
constexpr int64_t kProjWant = 256;

// Fewest tiles (128 tokens x 256 rows) for which the prefill launch uses the wide kernel.
constexpr int64_t kWideMinTiles = 256;

}  // namespace glowq
