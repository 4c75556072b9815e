// C ABI of libglowq: host-side validation (before any HIP call), planning and launches.
//
// The schedule follows the pages' inference form (GlowQ paper note, key design 4): per call the
// projection R = X B^T is formed once for the group (or once per module for the layerwise
// baseline), then one launch computes every module's quantised product and adds R A_i^T.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <algorithm>
#include <cstring>
#include <mutex>
#include <vector>

#include "glowq.h"
#include "glowq_internal.h"
#include "glowq_offline.h"
#include "mid.h"

using namespace glowq;

namespace {

constexpr int64_t kMaxT = 1 << 20;
constexpr int64_t kMaxD = 1 << 20;
constexpr int64_t kMaxRows = 1 << 24;
constexpr int64_t kMaxMomentD = 16384;              // features of a second-moment call
constexpr int64_t kMaxMomentElems = (int64_t)1 << 31;  // N d (int32 offsets stay in range)
// Forward calls: the kernels form activation byte offsets T d 2 in 32 bits and number their work
// tiles in int32; calls past these bounds are rejected before any HIP call.
constexpr int64_t kMaxActElems = (int64_t)1 << 30;     // T d
constexpr int64_t kMaxTiles = ((int64_t)1 << 31) - 1;  // 16-token tiles x 16-row tiles

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

inline int64_t r_pad_of(int32_t r) { return ceil_div(r, 32) * 32; }

// Workspace after the header: the fixed decode area (the projection as (fp32, tag) pairs in
// kRReplicas copies, sized for any decode call), then the prefill projection in fp16 with rows
// padded to 32 and its split-K partials.  No call ever writes anything but pairs into the decode
// area, so tags can never be confused with other data.
inline size_t round256(size_t n) { return (n + 255u) / 256u * 256u; }
constexpr size_t kDecodeAreaBytes = kDecodeAreaPairs * 8u;
inline size_t prefill_r_bytes(int64_t T, int32_t r, int32_t n_proj) {
    return round256((size_t)T * (size_t)r_pad_of(r) * 2u * (size_t)n_proj);
}
// fp32 partial outputs of a K-split call of 17 .. 64 tokens ([ranges][T][rows], ranges x rows at
// most kNarrowPartRows), after the projection's split-K partials
constexpr int64_t kNarrowPartRows = 28672;
static_assert(kNarrowPartRows >= (int64_t)kNarrowKs * kNarrowMaxRows, "narrow decode partials fit");
inline size_t narrow_part_bytes(int64_t T) { return round256((size_t)kNarrowPartRows * (size_t)T * 4u); }

inline size_t prefill_part_bytes(int64_t T, int32_t r, int32_t n_proj) {
    return round256((size_t)kProjMaxSplit * (size_t)T * (size_t)r_pad_of(r) * 4u * (size_t)n_proj);
}

// Everything needed to launch one group / solo / layerwise call.
struct Call {
    const void* x;
    int64_t T, d;
    int32_t m;
    const glowq_qweight* w;
    const void* const* b;  // n_proj pointers (1 for shared)
    const void* b_one;     // storage for the shared pointer
    int32_t n_proj;
    const void* const* a;
    int32_t r;
    bool correct;
    void* const* y;
    bool w4a8;  // 8-bit activations (glowq_group_forward_w4a8)
    bool mx8;   // MXFP4 weights x MXFP8 activations (glowq_group_forward_mx8)
};

int validate(const Call& c, void* workspace, size_t ws_bytes) {
    if (c.m < 1) return GLOWQ_ERR_SHAPE;
    if (c.m > GLOWQ_MAX_MODULES) return GLOWQ_ERR_UNSUPPORTED;
    if (c.T < 0 || c.d < kGroup || c.d % kGroup != 0) return GLOWQ_ERR_SHAPE;
    if (c.T > kMaxT || c.d > kMaxD) return GLOWQ_ERR_UNSUPPORTED;
    if (c.r < 0) return GLOWQ_ERR_SHAPE;
    if (c.r > GLOWQ_MAX_RANK || c.r % 8 != 0) return GLOWQ_ERR_UNSUPPORTED;
    if (c.T * c.d > kMaxActElems) return GLOWQ_ERR_UNSUPPORTED;
    if (c.w == nullptr || c.y == nullptr) return GLOWQ_ERR_INVALID_ARG;
    if (c.T > 0 && c.x == nullptr) return GLOWQ_ERR_INVALID_ARG;
    int64_t tiles16 = 0;
    for (int i = 0; i < c.m; ++i) {
        const glowq_qweight& w = c.w[i];
        if (w.q == nullptr || w.sz == nullptr) return GLOWQ_ERR_INVALID_ARG;
        if (w.format < GLOWQ_FMT_INT4_G128 || w.format > GLOWQ_FMT_MXFP6_E3M2 || w.reserved != 0)
            return GLOWQ_ERR_INVALID_ARG;
        if (w.format != c.w[0].format) return GLOWQ_ERR_UNSUPPORTED;  // one format per call
        if (c.T > 0 && c.y[i] == nullptr) return GLOWQ_ERR_INVALID_ARG;
        if (w.n_out < 1 || w.k_in != c.d) return GLOWQ_ERR_SHAPE;
        if (w.n_out > kMaxRows) return GLOWQ_ERR_UNSUPPORTED;
        if (!aligned(w.q, 16) || !aligned(w.sz, 16) || !aligned(c.y[i], 16)) return GLOWQ_ERR_ALIGN;
        tiles16 += ceil_div(w.n_out, 16);
    }
    // every launch has at most (16-token tiles) x (16-row tiles) work tiles
    if (ceil_div(c.T, 16) * tiles16 > kMaxTiles) return GLOWQ_ERR_UNSUPPORTED;
    if (c.x != nullptr && !aligned(c.x, 16)) return GLOWQ_ERR_ALIGN;
    if (c.w4a8 && (c.d > kW4a8MaxD || c.w[0].format != GLOWQ_FMT_INT4_G128)) return GLOWQ_ERR_UNSUPPORTED;
    if (c.mx8 && c.w[0].format == GLOWQ_FMT_INT4_G128) return GLOWQ_ERR_UNSUPPORTED;  // MX weights only
    if (c.correct) {
        if (c.a == nullptr || c.b == nullptr) return GLOWQ_ERR_INVALID_ARG;
        for (int i = 0; i < c.m; ++i)
            if (c.a[i] == nullptr) return GLOWQ_ERR_INVALID_ARG;
        for (int p = 0; p < c.n_proj; ++p)
            if (c.b[p] == nullptr) return GLOWQ_ERR_INVALID_ARG;
        for (int i = 0; i < c.m; ++i)
            if (!aligned(c.a[i], 16)) return GLOWQ_ERR_ALIGN;
        for (int p = 0; p < c.n_proj; ++p)
            if (!aligned(c.b[p], 16)) return GLOWQ_ERR_ALIGN;
    }
    if (c.T > 0) {
        // W4A8 calls always need their workspace (the activation codes); the others only to correct
        const size_t need = c.w4a8  ? glowq_w4a8_workspace_bytes(c.T, c.d, c.correct ? c.r : 0)
                            : c.mx8 ? glowq_mx8_workspace_bytes(c.T, c.d, c.correct ? c.r : 0)
                                    : (c.correct ? glowq_workspace_bytes(c.T, c.r, c.n_proj) : 0);
        if (need > 0) {
            if (workspace == nullptr || ws_bytes < need) return GLOWQ_ERR_WORKSPACE;
            if (!aligned(workspace, 256)) return GLOWQ_ERR_ALIGN;
        }
    }
    return GLOWQ_OK;
}

// Below this many 64 x 128 tiles the prefill launch takes 64 x 64 tiles (twice the workgroups,
// each wave one 16-row tile, always 4 wave groups), and below this many of those 32 x 64 tiles
// (the tile count stays under 256 either way).  LLaMA-3.1-8B QKV group at T = 64 (48 tiles of
// 64 x 128): 35.8 us per call, 29.6 us with 64 x 64 tiles, 24.3 us with 32 x 64.
constexpr int64_t kPrefillHalfRowTiles = 128;

// Prefill tiles of the call for a tile of 16 tt tokens x 64 rr rows.
int64_t prefill_tiles(const Call& c, int tt, int rr) {
    int64_t nb = 0;
    for (int i = 0; i < c.m; ++i) nb += ceil_div(ceil_div(c.w[i].n_out, 16), 4 * rr);
    return ceil_div(c.T, 16 * tt) * nb;
}

// Choose the prefill kernel: the wide tile (128 tokens x 256 rows) when it gives at least one
// workgroup per CU; otherwise 64 x 128 tiles with 4, 2 or 1 wave groups per workgroup splitting
// the input groups, so that about four wavefronts share every SIMD.  (Measured at T = 512 with the
// weights coming from HBM: gate/up, 344 wide tiles, 111 us wide vs 127 us with 64 x 256 tiles;
// QKV, 192 wide tiles, 75 us wide vs 68 us with 768 small tiles; o_proj and down_proj, 256 small
// tiles, 46 us on average with 4 wave groups vs 70 us with one.)
void choose_prefill_shape(const Call& c, int& tt, int& rr, int& ks) {
    if (prefill_tiles(c, 8, 4) >= kWideMinTiles) {
        // MXFP6 takes the wide tile with 64 tokens (the kernel's registers)
        tt = c.w[0].format == GLOWQ_FMT_MXFP6_E2M3 || c.w[0].format == GLOWQ_FMT_MXFP6_E3M2 ? 4 : 8;
        rr = 4, ks = 1;
        return;
    }
    tt = 4, rr = 2;
    int64_t n = prefill_tiles(c, 4, 2);
    if (n < kPrefillHalfRowTiles) {  // too few workgroups to stream the weights: 64 x 64 tiles
        rr = 1;
        n = prefill_tiles(c, 4, 1);
        if (n < kPrefillHalfRowTiles) {  // and still too few: 32 x 64 tiles
            tt = 2;
            n = prefill_tiles(c, 2, 1);
        }
    }
    ks = n <= 256 ? 4 : (n <= 512 ? 2 : 1);
}

// The projection R = X B_p^T into fp16 [n_proj][T][r_pad] at R (followed by its fp32 split-K
// partials): 32-token blocks (16 when that leaves the chip idle even at the largest split, or when
// r_pad > 128), then as many K ranges as make about kProjWant workgroups.
hipError_t launch_projection(const Call& c, void* R, hipStream_t stream) {
    const int32_t rp = (int32_t)r_pad_of(c.r);
    ProjArgs p;
    std::memset(&p, 0, sizeof(p));
    p.x = static_cast<const _Float16*>(c.x);
    p.T = (int32_t)c.T;
    p.d = (int32_t)c.d;
    p.r = c.r;
    p.r_pad = rp;
    p.n_proj = c.n_proj;
    for (int i = 0; i < c.n_proj; ++i) p.b[i] = static_cast<const _Float16*>(c.b[i]);
    p.R = R;
    const int64_t G = c.d / kGroup;
    p.tok_tiles = (rp <= 128 && ceil_div(c.T, 32) * c.n_proj * kProjMaxSplit >= kProjWant) ? 2 : 1;
    const int64_t blocks = ceil_div(c.T, 16 * p.tok_tiles) * c.n_proj;
    int64_t ks = ceil_div(kProjWant, blocks);
    ks = ks > kProjMaxSplit ? kProjMaxSplit : ks;
    ks = ks > G ? G : ks;
    p.k_per = (int32_t)(ceil_div(G, ks) * kGroup);
    p.ks = (int32_t)ceil_div(c.d, p.k_per);
    p.part = reinterpret_cast<float*>(static_cast<uint8_t*>(R) + prefill_r_bytes(c.T, c.r, c.n_proj));
    return launch_proj_prefill(p, stream);
}

// Correcting calls of 17 .. 64 tokens with INT4 weights and at least kMidMinBlocks workgroups of 8
// row tiles: the one-token-block tile (launch_mid), its projection formed in the same launch.
// Measured on LLaMA-3.1-8B shapes (r = 64, weights streamed from HBM): gate/up 30.8 us per call at
// T = 64 and 26.1 us at T = 32, against 33.9 and 31.4 us on the small prefill tiles.  QKV-sized
// calls (48 such workgroups) and calls without the correction were faster on the other tiles
// (QKV T = 64: 22.7 vs 16.3 us; gate/up without the correction: 28.2 vs 26.7 us).
constexpr int64_t kMidMinBlocks = 160;
// Fewer row blocks, long rows (at least kNarrowMinGroups input groups) and at least kMidSplitMinT
// tokens: the same tile over K ranges of at least kMidMinRangeGroups input groups, about
// kMidSplitWorkgroups workgroups in all (one per CU: the tile takes all of a CU's LDS), each range's
// fp32 sums in the workspace, added in range order by a second launch; the producers split the
// projection over the same ranges (partial tiles as tagged pairs after the copies of R).  Measured
// (r = 64, weights streamed from HBM): down_proj 4096 <- 14336 at T = 64 43.1 -> 32.8 us, 4096 <-
// 11008 39.1 -> 32.3 us against the K-split decode tile.  Where it lost it is not used: at T = 17
// and 32 (24.2 -> 27.3 and 26.3 -> 28.7 us: the 64-token tile's cost does not shrink with T while
// the decode tile's does) and at d = 4096 (LLaMA-3.1-8B QKV T = 64: 17.8 -> 28.8 us, ranges of 8
// groups being mostly the ring's fill).
constexpr int64_t kMidSplitWorkgroups = 256;
constexpr int64_t kMidMinRangeGroups = 8;
constexpr int64_t kMidSplitMinT = 48;

bool choose_mid_shape(const Call& c, int& tt, int& rb, int& ks, int& gk) {
    if (!c.correct || c.T <= kDecodeWideT || c.T > kDecodeMaxT || c.w[0].format != GLOWQ_FMT_INT4_G128)
        return false;
    tt = c.T <= 32 ? 2 : 4;
    rb = 8;
    int64_t n = 0, rows = 0;
    for (int i = 0; i < c.m; ++i) {
        n += ceil_div(ceil_div(c.w[i].n_out, 16), rb);
        rows += c.w[i].n_out;
    }
    const int64_t G = c.d / kGroup;
    ks = 1;
    gk = (int)G;
    if (n >= kMidMinBlocks) return true;
    if (c.T < kMidSplitMinT || G < kNarrowMinGroups) return false;
    // the decode area holds the kRReplicas copies of R and the partial tiles of ks - 1 ranges
    const int64_t copy = (int64_t)c.n_proj * c.T * c.r;
    const int64_t k_area = (int64_t)kDecodeAreaPairs / copy - kRReplicas + 1;
    const int64_t k = std::min(std::min(kMidSplitWorkgroups / n, G / kMidMinRangeGroups),
                               std::min(kNarrowPartRows / rows, k_area));
    if (k < 2 || n * k < kMidSplitWorkgroups / 2) return false;
    gk = (int)ceil_div(G, k);
    ks = (int)ceil_div(G, gk);
    return ks >= 2;
}

int run_mid(const Call& c, void* workspace, hipStream_t stream, int tt, int rb, int ks, int gk) {
    const int32_t rp = (int32_t)r_pad_of(c.r);
    ForwardArgs f;
    std::memset(&f, 0, sizeof(f));
    f.x = static_cast<const _Float16*>(c.x);
    f.T = (int32_t)c.T;
    f.d = (int32_t)c.d;
    f.G = (int32_t)(c.d / kGroup);
    f.fmt = c.w[0].format;
    f.r = c.correct ? c.r : 0;
    f.r_pad = c.correct ? rp : 0;
    f.n_mod = c.m;
    f.n_proj = c.n_proj;
    if (c.correct) {
        // the projection is formed in the launch: 16 x 16 tiles of R as tagged pairs in the decode area
        f.R = static_cast<uint8_t*>(workspace) + kWsHeader;
        f.sync = static_cast<int32_t*>(workspace);
        for (int i = 0; i < c.n_proj; ++i) f.b[i] = static_cast<const _Float16*>(c.b[i]);
        f.n_prod = (int32_t)(ceil_div(c.T, 16) * c.n_proj * (rp / 16) * ks);
    }
    f.tile_tt = tt;
    f.tile_rr = rb;
    f.tile_ks = 1;
    int64_t tiles = 0, rows = 0;
    for (int i = 0; i < c.m; ++i) {
        ModuleArgs& M = f.mod[i];
        M.q = static_cast<const uint8_t*>(c.w[i].q);
        M.sz = static_cast<const uint8_t*>(c.w[i].sz);
        M.a = c.correct ? static_cast<const _Float16*>(c.a[i]) : nullptr;
        M.y = static_cast<_Float16*>(c.y[i]);
        M.n_out = (int32_t)c.w[i].n_out;
        M.n_tiles16 = (int32_t)ceil_div(c.w[i].n_out, 16);
        M.tile_begin = (int32_t)tiles;
        f.tile_begin[i] = (int32_t)tiles;
        M.proj = c.n_proj > 1 ? i : 0;
        M.row_begin = (int32_t)rows;
        rows += c.w[i].n_out;
        tiles += ceil_div(M.n_tiles16, rb);
    }
    f.rows_total = (int32_t)rows;
    f.m_tiles = 1;
    f.dec_tiles = (int32_t)tiles;
    f.dec_ks = ks;
    f.dec_gk = gk;
    f.n_tiles = (int32_t)(tiles * ks);
    if (ks > 1)
        f.ypart = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + kWsHeader + kDecodeAreaBytes +
                                           prefill_r_bytes(c.T, c.r, c.n_proj) +
                                           prefill_part_bytes(c.T, c.r, c.n_proj));
    return launch_mid(f, stream) == hipSuccess ? GLOWQ_OK : GLOWQ_ERR_HIP;
}

int run(const Call& c, void* workspace, hipStream_t stream) {
    if (c.T == 0) return GLOWQ_OK;
    int mid_tt = 0, mid_rb = 0, mid_ks = 1, mid_gk = 1;
    if (choose_mid_shape(c, mid_tt, mid_rb, mid_ks, mid_gk))
        return run_mid(c, workspace, stream, mid_tt, mid_rb, mid_ks, mid_gk);
    int64_t row_tiles = 0;
    for (int i = 0; i < c.m; ++i) row_tiles += ceil_div(c.w[i].n_out, 128);
    const bool prefill = c.T > kDecodeMaxT || (c.T > kDecodeWideT && row_tiles >= kPrefillMinRowTiles);
    const int32_t rp = (int32_t)r_pad_of(c.r);
    int tt = 0, rr = 0, ks = 1;
    if (prefill) choose_prefill_shape(c, tt, rr, ks);
    // 17 .. 64 tokens on the small prefill tiles: the projection is formed inside the launch by
    // producer workgroups and handed over as tagged pairs (one launch instead of three)
    const bool fuse = c.correct && prefill && c.T <= kDecodeMaxT && rr != 4;  // rr == 4: the wide tile
    if (fuse && tt == 4 && rr == 2 && ks == 4) ks = 2;  // the fused 64 x 128 tile: two wave groups
    void* R = nullptr;
    if (c.correct) {
        uint8_t* base = static_cast<uint8_t*>(workspace) + kWsHeader;
        R = (prefill && !fuse) ? base + kDecodeAreaBytes : base;
    }

    if (c.correct && prefill && !fuse) {
        if (launch_projection(c, R, stream) != hipSuccess) return GLOWQ_ERR_HIP;
    }

    ForwardArgs f;
    std::memset(&f, 0, sizeof(f));
    f.x = static_cast<const _Float16*>(c.x);
    f.T = (int32_t)c.T;
    f.d = (int32_t)c.d;
    f.G = (int32_t)(c.d / kGroup);
    f.fmt = c.w[0].format;
    f.r = c.correct ? c.r : 0;
    f.r_pad = c.correct ? rp : 0;
    f.n_mod = c.m;
    f.R = R;
    f.sync = c.correct ? static_cast<int32_t*>(workspace) : nullptr;
    f.n_proj = c.n_proj;
    for (int i = 0; i < c.n_proj; ++i) f.b[i] = c.correct ? static_cast<const _Float16*>(c.b[i]) : nullptr;
    if (c.correct && !prefill) {
        const int64_t total = (int64_t)c.n_proj * c.r;
        f.prod_rows = (int32_t)ceil_div(total, kMaxProducers);
        // one producer per (row block, token tile); tiles of 1, 4 or 16 tokens as the kernel picks
        const int64_t ptt = c.T == 1 ? 1 : (c.T <= 4 ? 4 : 16);
        f.n_prod = (int32_t)(ceil_div(total, f.prod_rows) * ceil_div(c.T, ptt));
    }
    if (fuse) f.n_prod = (int32_t)(ceil_div(c.T, 16) * c.n_proj * (rp / 16));  // 16 x 16 tiles of R
    f.tile_tt = tt;
    f.tile_rr = rr;
    f.tile_ks = ks;
    int dec_rt = 1;
    if (!prefill) {
        int64_t total16 = 0;
        for (int i = 0; i < c.m; ++i) total16 += ceil_div(c.w[i].n_out, 16);
        const bool xlds = c.T <= 16 && (size_t)(c.T + 1) * (size_t)c.d * 2u <= kDecodeXLdsMax;
        f.dec_kw = (total16 <= kDecodeWide8Tiles && f.G >= kDecodeWide8Groups) ? 8 : 4;
        const bool rt2 = xlds ? total16 > kDecodeRt2Tiles : (c.T <= 16 && total16 >= kDecodeRt2NoLdsTiles);
        dec_rt = (f.dec_kw == 4 && rt2) ? 2 : 1;
        f.dec_ks = 1;
        f.dec_gk = f.G;
        if (c.T > kDecodeWideT && c.correct && f.G >= kNarrowMinGroups) {  // narrow, long rows: split K
            f.dec_kw = 4;
            dec_rt = kNarrowRt;
            f.dec_ks = (int32_t)(f.G < kNarrowKs ? f.G : kNarrowKs);
            f.dec_gk = (int32_t)ceil_div(f.G, f.dec_ks);
            f.dec_ks = (int32_t)ceil_div(f.G, f.dec_gk);
            uint8_t* base = static_cast<uint8_t*>(workspace) + kWsHeader + kDecodeAreaBytes +
                            prefill_r_bytes(c.T, c.r, c.n_proj) + prefill_part_bytes(c.T, c.r, c.n_proj);
            f.ypart = reinterpret_cast<float*>(base);
        }
        f.dec_rt = dec_rt;
    }
    int64_t tiles = 0, rows = 0;
    for (int i = 0; i < c.m; ++i) {
        ModuleArgs& M = f.mod[i];
        M.q = static_cast<const uint8_t*>(c.w[i].q);
        M.sz = static_cast<const uint8_t*>(c.w[i].sz);
        M.a = c.correct ? static_cast<const _Float16*>(c.a[i]) : nullptr;
        M.y = static_cast<_Float16*>(c.y[i]);
        M.n_out = (int32_t)c.w[i].n_out;
        M.n_tiles16 = (int32_t)ceil_div(c.w[i].n_out, 16);
        M.tile_begin = (int32_t)tiles;
        f.tile_begin[i] = (int32_t)tiles;
        M.proj = c.n_proj > 1 ? i : 0;
        M.row_begin = (int32_t)rows;
        rows += c.w[i].n_out;
        tiles += prefill ? ceil_div(M.n_tiles16, 4 * rr) : ceil_div(M.n_tiles16, dec_rt);
    }
    f.rows_total = (int32_t)rows;
    hipError_t e;
    if (prefill) {
        f.m_tiles = (int32_t)ceil_div(c.T, 16 * tt);
        f.n_tiles = (int32_t)(tiles * f.m_tiles);
        e = launch_prefill(f, stream);
    } else {
        f.m_tiles = 1;
        f.dec_tiles = (int32_t)tiles;
        f.n_tiles = (int32_t)(tiles * f.dec_ks);
        e = launch_decode(f, stream);
    }
    return e == hipSuccess ? GLOWQ_OK : GLOWQ_ERR_HIP;
}

Call make_group(const void* x, int64_t T, int64_t d, int32_t m, const glowq_qweight* w,
                const void* const* b, int32_t n_proj, const void* const* a, int32_t r, int32_t restore,
                void* const* y) {
    Call c;
    c.x = x;
    c.T = T;
    c.d = d;
    c.m = m;
    c.w = w;
    c.b = b;
    c.b_one = nullptr;
    c.n_proj = n_proj;
    c.a = a;
    c.r = r;
    c.correct = restore != 0 && r > 0;
    c.y = y;
    c.w4a8 = false;
    c.mx8 = false;
    return c;
}

// W4A8 tile: 16, 32 or 64 tokens (decode-sized calls take one token tile) x 128 rows, 64 rows when
// that leaves fewer than 128 tiles; wave groups splitting the input groups as in the prefill
// kernel, so that about four wavefronts share every SIMD on small grids.
void choose_w4a8_shape(const Call& c, int& tt, int& rr, int& ks) {
    if (c.mx8 && prefill_tiles(c, 8, 8) >= kWideMinTiles) {  // MXFP8: the 128 x 512 tile on large grids
        tt = 8, rr = 8, ks = 1;
        return;
    }
    tt = c.T <= 16 ? 1 : (c.T <= 32 ? 2 : 4);
    rr = 2;
    int64_t n = prefill_tiles(c, tt, rr);
    if (n < kPrefillHalfRowTiles) {
        rr = 1;
        n = prefill_tiles(c, tt, rr);
    }
    ks = n <= 256 ? 4 : (n <= 512 ? 2 : 1);
    if (tt == 4 && rr == 2 && ks == 4) ks = 2;  // 1024 threads would cap this tile at 128 VGPRs (spills)
}

// MXFP8 activation scales: one 512-byte record per (128-token block, input group).
size_t mx8_scale_bytes(int64_t T, int64_t d) { return (size_t)ceil_div(T, 128) * (size_t)(d / kGroup) * 512u; }

// W4A8 workspace: codes [T][d] int8 | code sums [T][G] int32 | scales [T] fp32 | for correcting
// calls the fp16 projection [T][r_pad] and its split-K partials.
// W4A8 and MXFP8 forms: quantise the activations into the workspace, form the projection from the
// fp16 activations, then one GEMM launch over the prefill-style tiles.
// W4A8 workspace: codes [T][d] int8 | code sums [T][G] int32 | scales [T] fp32 | projection;
// MXFP8 workspace: codes [T][d] (operand order) | block scales (512-byte records per 128 tokens and
// group) | projection.
int run_w4a8(const Call& c, void* workspace, hipStream_t stream) {
    if (c.T == 0) return GLOWQ_OK;
    uint8_t* base = static_cast<uint8_t*>(workspace);
    int8_t* xq = nullptr;
    int32_t* xsum = nullptr;
    float* xscale = nullptr;
    uint8_t *x8 = nullptr, *x8s = nullptr;
    if (c.mx8) {
        x8 = base;
        base += round256((size_t)c.T * c.d);
        x8s = base;
        base += mx8_scale_bytes(c.T, c.d);
    } else {
        xq = reinterpret_cast<int8_t*>(base);
        base += round256((size_t)c.T * c.d);
        xsum = reinterpret_cast<int32_t*>(base);
        base += round256((size_t)c.T * (c.d / kGroup) * 4u);
        xscale = reinterpret_cast<float*>(base);
        base += round256((size_t)c.T * 4u);
    }
    void* R = c.correct ? base : nullptr;
    const hipError_t eq = c.mx8 ? launch_quant_mx8(static_cast<const _Float16*>(c.x), (int)c.T, (int)c.d, x8, x8s, stream)
                                : launch_quant_x(static_cast<const _Float16*>(c.x), (int)c.T, (int)c.d, xq, xsum, xscale,
                                                 stream);
    if (eq != hipSuccess) return GLOWQ_ERR_HIP;
    if (c.correct && launch_projection(c, R, stream) != hipSuccess) return GLOWQ_ERR_HIP;
    ForwardArgs f;
    std::memset(&f, 0, sizeof(f));
    f.x = static_cast<const _Float16*>(c.x);
    f.T = (int32_t)c.T;
    f.d = (int32_t)c.d;
    f.G = (int32_t)(c.d / kGroup);
    f.r = c.correct ? c.r : 0;
    f.r_pad = c.correct ? (int32_t)r_pad_of(c.r) : 0;
    f.n_mod = c.m;
    f.R = R;
    f.n_proj = 1;
    f.b[0] = c.correct ? static_cast<const _Float16*>(c.b[0]) : nullptr;
    f.xq = xq;
    f.xsum = xsum;
    f.xscale = xscale;
    f.x8 = x8;
    f.x8scale = x8s;
    f.fmt = c.w[0].format;
    int tt = 1, rr = 1, ks = 1;
    choose_w4a8_shape(c, tt, rr, ks);
    f.tile_tt = tt;
    f.tile_rr = rr;
    f.tile_ks = ks;
    int64_t tiles = 0;
    for (int i = 0; i < c.m; ++i) {
        ModuleArgs& M = f.mod[i];
        M.q = static_cast<const uint8_t*>(c.w[i].q);
        M.sz = static_cast<const uint8_t*>(c.w[i].sz);
        M.a = c.correct ? static_cast<const _Float16*>(c.a[i]) : nullptr;
        M.y = static_cast<_Float16*>(c.y[i]);
        M.n_out = (int32_t)c.w[i].n_out;
        M.n_tiles16 = (int32_t)ceil_div(c.w[i].n_out, 16);
        M.tile_begin = (int32_t)tiles;
        f.tile_begin[i] = (int32_t)tiles;
        M.proj = 0;
        tiles += ceil_div(M.n_tiles16, 4 * rr);
    }
    f.m_tiles = (int32_t)ceil_div(c.T, 16 * tt);
    f.n_tiles = (int32_t)(tiles * f.m_tiles);
    return (c.mx8 ? launch_mx8(f, stream) : launch_w4a8(f, stream)) == hipSuccess ? GLOWQ_OK : GLOWQ_ERR_HIP;
}

}  // namespace

extern "C" {

const char* glowq_status_string(int status) {
    switch (status) {
        case GLOWQ_OK: return "GLOWQ_OK";
        case GLOWQ_ERR_INVALID_ARG: return "GLOWQ_ERR_INVALID_ARG: null pointer or bad enum value";
        case GLOWQ_ERR_SHAPE: return "GLOWQ_ERR_SHAPE: size out of range";
        case GLOWQ_ERR_ALIGN: return "GLOWQ_ERR_ALIGN: pointer misaligned";
        case GLOWQ_ERR_UNSUPPORTED: return "GLOWQ_ERR_UNSUPPORTED: configuration not supported";
        case GLOWQ_ERR_WORKSPACE: return "GLOWQ_ERR_WORKSPACE: workspace missing or too small";
        case GLOWQ_ERR_HIP: return "GLOWQ_ERR_HIP: HIP runtime or launch failure";
        case GLOWQ_ERR_RANGE: return "GLOWQ_ERR_RANGE: value out of range (zero point, scale, or a matrix that is not positive semidefinite)";
        case GLOWQ_ERR_HANDOFF: return "GLOWQ_ERR_HANDOFF: a bounded wait for the projection expired; outputs since the last check are invalid";
        default: return "GLOWQ_ERR_UNKNOWN";
    }
}

int glowq_version(void) { return 300; }

int glowq_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (workspace == nullptr) return GLOWQ_ERR_INVALID_ARG;
    if (!aligned(workspace, 256)) return GLOWQ_ERR_ALIGN;
    if (workspace_bytes < kWsHeader) return GLOWQ_ERR_WORKSPACE;
    return launch_fill_zero(workspace, workspace_bytes, stream) == hipSuccess ? GLOWQ_OK : GLOWQ_ERR_HIP;
}

int glowq_workspace_status(void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (workspace == nullptr) return GLOWQ_ERR_INVALID_ARG;
    if (!aligned(workspace, 256)) return GLOWQ_ERR_ALIGN;
    if (workspace_bytes < kWsHeader) return GLOWQ_ERR_WORKSPACE;
    int32_t* word = static_cast<int32_t*>(workspace) + kSyncError;
    int32_t h = 0;
    if (hipMemcpyAsync(&h, word, sizeof(h), hipMemcpyDeviceToHost, stream) != hipSuccess) return GLOWQ_ERR_HIP;
    if (hipStreamSynchronize(stream) != hipSuccess) return GLOWQ_ERR_HIP;
    if (h == 0) return GLOWQ_OK;
    if (launch_flag_clear(word, stream) != hipSuccess) return GLOWQ_ERR_HIP;
    if (hipStreamSynchronize(stream) != hipSuccess) return GLOWQ_ERR_HIP;
    return (h & 1) ? GLOWQ_ERR_HANDOFF : GLOWQ_ERR_ROUTING;
}

size_t glowq_moe_workspace_bytes(int64_t n_rows, int64_t T, int32_t r, int32_t share) {
    if (n_rows < 0 || T < 0 || r < 0 || r > GLOWQ_MAX_RANK || n_rows > kMaxT * 8 || T > kMaxT) return 0;
    if (share != GLOWQ_MOE_SHARE_EXPERT && share != GLOWQ_MOE_SHARE_ALL) return 0;
    size_t n = kWsHeader;
    if (r > 0 && n_rows > 0) {
        if (share == GLOWQ_MOE_SHARE_ALL) n += prefill_r_bytes(T, r, 1) + prefill_part_bytes(T, r, 1);
        else n += prefill_r_bytes(n_rows, r, 1);
    }
    return n;
}

int glowq_moe_forward(const void* x, int64_t T, int64_t d, int32_t n_exp, int32_t m, const glowq_moe_module* mods,
                      const void* b, int32_t share, int32_t r, int32_t restore, const int32_t* row_token_dev,
                      const int32_t* offsets_dev, int64_t n_rows, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
    if (n_exp < 1 || n_exp > GLOWQ_MOE_MAX_EXPERTS || m < 1 || m > GLOWQ_MOE_MAX_MODULES) return GLOWQ_ERR_UNSUPPORTED;
    if (share != GLOWQ_MOE_SHARE_EXPERT && share != GLOWQ_MOE_SHARE_ALL) return GLOWQ_ERR_INVALID_ARG;
    if (n_rows < 0 || T < 0 || d < kGroup || d % kGroup != 0) return GLOWQ_ERR_SHAPE;
    if (r < 0) return GLOWQ_ERR_SHAPE;
    if (r > GLOWQ_MAX_RANK || r % 8 != 0) return GLOWQ_ERR_UNSUPPORTED;
    if (n_rows > kMaxT * 8 || T > kMaxT || d > kMaxD || T * d > kMaxActElems) return GLOWQ_ERR_UNSUPPORTED;
    if (mods == nullptr) return GLOWQ_ERR_INVALID_ARG;
    if (n_rows == 0) return GLOWQ_OK;
    if (x == nullptr || offsets_dev == nullptr) return GLOWQ_ERR_INVALID_ARG;
    if (row_token_dev == nullptr && T != n_rows) return GLOWQ_ERR_SHAPE;
    if (T < 1) return GLOWQ_ERR_SHAPE;
    const bool correct = restore != 0 && r > 0;
    int64_t rb = 0;
    for (int i = 0; i < m; ++i) {
        const glowq_moe_module& M = mods[i];
        if (M.q == nullptr || M.sz == nullptr || M.y == nullptr) return GLOWQ_ERR_INVALID_ARG;
        if (M.n_out < 1 || M.k_in != d) return GLOWQ_ERR_SHAPE;
        if (M.n_out > kMaxRows) return GLOWQ_ERR_UNSUPPORTED;
        if (!aligned(M.q, 16) || !aligned(M.sz, 16) || !aligned(M.y, 16)) return GLOWQ_ERR_ALIGN;
        if (correct && (M.a == nullptr)) return GLOWQ_ERR_INVALID_ARG;
        if (correct && !aligned(M.a, 16)) return GLOWQ_ERR_ALIGN;
        rb += ceil_div(ceil_div(M.n_out, 16), 4 * 2);
    }
    if (correct && b == nullptr) return GLOWQ_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(offsets_dev, 4) || (row_token_dev && !aligned(row_token_dev, 4)) ||
        (correct && !aligned(b, 16)))
        return GLOWQ_ERR_ALIGN;
    if (workspace == nullptr || workspace_bytes < glowq_moe_workspace_bytes(n_rows, T, correct ? r : 0, share))
        return GLOWQ_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return GLOWQ_ERR_ALIGN;
    // items of the grouped launch: at most n_rb (n_rows / BM + n_exp)
    // the grouped tile (16 tt routed rows x 128 rows) unless it would have fewer than 512 items
    // (at most min(n_rows, n_exp) active experts x rb row blocks), as at single-token decode; then
    // 16-row items with the input groups split over the waves (T = 1, 60 experts, top-4: gate/up
    // 27.4 -> 20.6 us; at 16 and 64 tokens the grouped tile was faster: 45 vs 63, 58 vs 89 us)
    const int64_t avg = ceil_div(n_rows, n_exp);
    const int64_t max_active = n_rows < n_exp ? n_rows : n_exp;
    const int tt = (avg <= 16 && max_active * rb < 512) ? 0 : (avg <= 16 ? 1 : (avg <= 32 ? 2 : 4));
    const int rows_per_item = tt == 0 ? 16 : 16 * tt;
    if (rb * 8 * (ceil_div(n_rows, rows_per_item) + n_exp) > kMaxTiles) return GLOWQ_ERR_UNSUPPORTED;

    MoeArgs a;
    std::memset(&a, 0, sizeof(a));
    a.x = static_cast<const _Float16*>(x);
    a.T = (int32_t)T;
    a.d = (int32_t)d;
    a.G = (int32_t)(d / kGroup);
    a.row_token = row_token_dev;
    a.offsets = offsets_dev;
    a.n_exp = n_exp;
    a.n_rows = (int32_t)n_rows;
    a.m = m;
    int32_t rbs = 0;
    for (int i = 0; i < m; ++i) {
        const glowq_moe_module& M = mods[i];
        a.q[i] = static_cast<const uint8_t*>(M.q);
        a.sz[i] = static_cast<const uint8_t*>(M.sz);
        a.qbytes[i] = (int64_t)glowq_q_bytes(M.n_out, M.k_in);
        a.szbytes[i] = (int64_t)glowq_sz_bytes(M.n_out, M.k_in);
        a.a[i] = correct ? static_cast<const _Float16*>(M.a) : nullptr;
        a.y[i] = static_cast<_Float16*>(M.y);
        a.n_out[i] = (int32_t)M.n_out;
        a.n_tiles16[i] = (int32_t)ceil_div(M.n_out, 16);
        a.rb_begin[i] = rbs;
        rbs += (int32_t)(tt == 0 ? a.n_tiles16[i] : ceil_div(a.n_tiles16[i], 8));
    }
    a.rb_begin[m] = rbs;
    a.n_rb = rbs;
    a.r = correct ? r : 0;
    a.r_pad = correct ? (int32_t)r_pad_of(r) : 0;
    a.tile_tt = tt;
    a.err = static_cast<int32_t*>(workspace) + kSyncError;
    uint8_t* R = static_cast<uint8_t*>(workspace) + kWsHeader;
    // persistent grids: (expert, block) pairs number at most n_rows / rows per block plus the active
    // experts, and every active expert holds at least one routed row
    const int64_t active_max = std::min<int64_t>(n_exp, n_rows);
    if (correct) {
        a.R = reinterpret_cast<const _Float16*>(R);
        if (share == GLOWQ_MOE_SHARE_ALL) {
            a.r_by_token = 1;
            const void* bp[1] = {b};
            Call c = make_group(x, T, d, 1, nullptr, bp, 1, nullptr, r, 1, nullptr);
            if (launch_projection(c, R, stream) != hipSuccess) return GLOWQ_ERR_HIP;
        } else {
            a.r_by_token = 0;
            a.b = static_cast<const _Float16*>(b);
            a.Rout = reinterpret_cast<_Float16*>(R);
            if (launch_moe_proj(a, ceil_div(n_rows, 16) + active_max, stream) != hipSuccess) return GLOWQ_ERR_HIP;
        }
    }
    if (launch_moe_gemm(a, (int64_t)rbs * (ceil_div(n_rows, rows_per_item) + active_max), stream) != hipSuccess)
        return GLOWQ_ERR_HIP;
    return GLOWQ_OK;
}

size_t glowq_q_bytes(int64_t n_out, int64_t k_in) {
    if (n_out < 1 || k_in < kGroup || k_in % kGroup != 0 || n_out > kMaxRows || k_in > kMaxD) return 0;
    return (size_t)ceil_div(n_out, 16) * (size_t)(k_in / kGroup) * 1024u;
}

size_t glowq_sz_bytes(int64_t n_out, int64_t k_in) {
    if (n_out < 1 || k_in < kGroup || k_in % kGroup != 0 || n_out > kMaxRows || k_in > kMaxD) return 0;
    return (size_t)ceil_div(n_out, 16) * (size_t)(k_in / kGroup) * 64u;
}

size_t glowq_mx_q_bytes(int32_t format, int64_t n_out, int64_t k_in) {
    if (format != GLOWQ_FMT_MXFP4 && format != GLOWQ_FMT_MXFP6_E2M3 && format != GLOWQ_FMT_MXFP6_E3M2) return 0;
    const size_t q4 = glowq_q_bytes(n_out, k_in);
    return format == GLOWQ_FMT_MXFP4 ? q4 : q4 / 2u * 3u;
}

int glowq_repack_mx(int32_t format, const void* codes_dev, const void* scales_dev, int64_t n_out, int64_t k_in,
                    void* q_dev, void* sz_dev, int32_t* flag_dev, hipStream_t stream) {
    if (format != GLOWQ_FMT_MXFP4 && format != GLOWQ_FMT_MXFP6_E2M3 && format != GLOWQ_FMT_MXFP6_E3M2)
        return GLOWQ_ERR_INVALID_ARG;
    if (!codes_dev || !scales_dev || !q_dev || !sz_dev || !flag_dev) return GLOWQ_ERR_INVALID_ARG;
    if (n_out < 1 || k_in < kGroup || k_in % kGroup != 0) return GLOWQ_ERR_SHAPE;
    if (n_out > kMaxRows || k_in > kMaxD) return GLOWQ_ERR_UNSUPPORTED;
    if (!aligned(codes_dev, 16) || !aligned(scales_dev, 4) || !aligned(q_dev, 16) || !aligned(sz_dev, 16) ||
        !aligned(flag_dev, 4))
        return GLOWQ_ERR_ALIGN;
    if (launch_flag_clear(flag_dev, stream) != hipSuccess) return GLOWQ_ERR_HIP;
    if (launch_repack_mx(format, static_cast<const uint8_t*>(codes_dev), static_cast<const uint8_t*>(scales_dev),
                         n_out, k_in, static_cast<uint8_t*>(q_dev), static_cast<uint8_t*>(sz_dev), flag_dev,
                         stream) != hipSuccess)
        return GLOWQ_ERR_HIP;
    int32_t flag = 0;
    if (hipMemcpyAsync(&flag, flag_dev, sizeof(flag), hipMemcpyDeviceToHost, stream) != hipSuccess)
        return GLOWQ_ERR_HIP;
    if (hipStreamSynchronize(stream) != hipSuccess) return GLOWQ_ERR_HIP;
    return flag ? GLOWQ_ERR_RANGE : GLOWQ_OK;
}

size_t glowq_w4a8_workspace_bytes(int64_t T, int64_t d, int32_t r) {
    if (T <= 0 || d < kGroup || d % kGroup != 0 || d > kW4a8MaxD || r < 0 || r > GLOWQ_MAX_RANK) return 0;
    size_t n = round256((size_t)T * d) + round256((size_t)T * (d / kGroup) * 4u) + round256((size_t)T * 4u);
    if (r > 0) n += prefill_r_bytes(T, r, 1) + prefill_part_bytes(T, r, 1);
    return n;
}

size_t glowq_mx8_workspace_bytes(int64_t T, int64_t d, int32_t r) {
    if (T <= 0 || d < kGroup || d % kGroup != 0 || d > kMaxD || r < 0 || r > GLOWQ_MAX_RANK) return 0;
    size_t n = round256((size_t)T * d) + mx8_scale_bytes(T, d);
    if (r > 0) n += prefill_r_bytes(T, r, 1) + prefill_part_bytes(T, r, 1);
    return n;
}

int glowq_group_forward_mx8(const void* x, int64_t T, int64_t d, int32_t m, const glowq_qweight* w,
                            const void* b_shared, const void* const* a, int32_t r, int32_t restore,
                            void* workspace, size_t workspace_bytes, void* const* y, hipStream_t stream) {
    const void* bp[1] = {b_shared};
    Call c = make_group(x, T, d, m, w, bp, 1, a, r, restore, y);
    c.mx8 = true;
    const int v = validate(c, workspace, workspace_bytes);
    if (v != GLOWQ_OK) return v;
    return run_w4a8(c, workspace, stream);
}

int glowq_group_forward_w4a8(const void* x, int64_t T, int64_t d, int32_t m, const glowq_qweight* w,
                             const void* b_shared, const void* const* a, int32_t r, int32_t restore,
                             void* workspace, size_t workspace_bytes, void* const* y, hipStream_t stream) {
    const void* bp[1] = {b_shared};
    Call c = make_group(x, T, d, m, w, bp, 1, a, r, restore, y);
    c.w4a8 = true;
    const int v = validate(c, workspace, workspace_bytes);
    if (v != GLOWQ_OK) return v;
    return run_w4a8(c, workspace, stream);
}

size_t glowq_workspace_bytes(int64_t T, int32_t r, int32_t n_proj) {
    if (T <= 0 || r <= 0 || n_proj <= 0) return 0;
    if (T > kDecodeWideT) return kWsHeader + kDecodeAreaBytes + prefill_r_bytes(T, r, n_proj) +
                                 prefill_part_bytes(T, r, n_proj) + (T <= kDecodeMaxT ? narrow_part_bytes(T) : 0);
    return kWsHeader + kDecodeAreaBytes;
}

int glowq_repack(const void* q_canon_dev, const void* scales_dev, const void* zeros_dev, int64_t n_out,
                 int64_t k_in, void* q_dev, void* sz_dev, int32_t* flag_dev, hipStream_t stream) {
    if (!q_canon_dev || !scales_dev || !zeros_dev || !q_dev || !sz_dev || !flag_dev)
        return GLOWQ_ERR_INVALID_ARG;
    if (n_out < 1 || k_in < kGroup || k_in % kGroup != 0) return GLOWQ_ERR_SHAPE;
    if (n_out > kMaxRows || k_in > kMaxD) return GLOWQ_ERR_UNSUPPORTED;
    if (!aligned(q_canon_dev, 4) || !aligned(scales_dev, 2) || !aligned(zeros_dev, 2) ||
        !aligned(q_dev, 16) || !aligned(sz_dev, 16) || !aligned(flag_dev, 4))
        return GLOWQ_ERR_ALIGN;
    if (launch_flag_clear(flag_dev, stream) != hipSuccess) return GLOWQ_ERR_HIP;
    if (launch_repack(static_cast<const uint32_t*>(q_canon_dev), static_cast<const _Float16*>(scales_dev),
                      static_cast<const _Float16*>(zeros_dev), n_out, k_in, static_cast<uint8_t*>(q_dev),
                      static_cast<uint8_t*>(sz_dev), flag_dev, stream) != hipSuccess)
        return GLOWQ_ERR_HIP;
    int32_t flag = 0;
    if (hipMemcpyAsync(&flag, flag_dev, sizeof(flag), hipMemcpyDeviceToHost, stream) != hipSuccess)
        return GLOWQ_ERR_HIP;
    if (hipStreamSynchronize(stream) != hipSuccess) return GLOWQ_ERR_HIP;
    return flag ? GLOWQ_ERR_RANGE : GLOWQ_OK;
}

int glowq_dequant(const glowq_qweight* w, void* out_dev, int32_t out_dtype, hipStream_t stream) {
    if (!w || !out_dev || !w->q || !w->sz) return GLOWQ_ERR_INVALID_ARG;
    if (out_dtype != GLOWQ_DTYPE_F32 && out_dtype != GLOWQ_DTYPE_F16) return GLOWQ_ERR_INVALID_ARG;
    if (w->format < GLOWQ_FMT_INT4_G128 || w->format > GLOWQ_FMT_MXFP6_E3M2 || w->reserved != 0)
        return GLOWQ_ERR_INVALID_ARG;
    if (w->n_out < 1 || w->k_in < kGroup || w->k_in % kGroup != 0) return GLOWQ_ERR_SHAPE;
    if (w->n_out > kMaxRows || w->k_in > kMaxD) return GLOWQ_ERR_UNSUPPORTED;
    if (!aligned(w->q, 16) || !aligned(w->sz, 16) || !aligned(out_dev, 16)) return GLOWQ_ERR_ALIGN;
    const hipError_t e = launch_dequant(w->format, static_cast<const uint8_t*>(w->q), static_cast<const uint8_t*>(w->sz),
                                        w->n_out, w->k_in, out_dev, out_dtype == GLOWQ_DTYPE_F32 ? 0 : 1,
                                        stream);
    return e == hipSuccess ? GLOWQ_OK : GLOWQ_ERR_HIP;
}

size_t glowq_ner_workspace_bytes(int64_t n_out) {
    if (n_out < 1 || n_out > kMaxRows) return 0;
    return round256((size_t)ceil_div(n_out, 16) * 16u);
}

int glowq_ner_sums_batch(int32_t n, const void* const* w_devs, const glowq_qweight* wqs, void* workspace,
                         size_t workspace_bytes, double* sums_dev, hipStream_t stream) {
    if (n < 1 || !w_devs || !wqs || !sums_dev || !workspace) return GLOWQ_ERR_INVALID_ARG;
    size_t need = 0;
    for (int32_t i = 0; i < n; ++i) {
        const glowq_qweight& w = wqs[i];
        if (!w_devs[i] || !w.q || !w.sz) return GLOWQ_ERR_INVALID_ARG;
        if (w.format != GLOWQ_FMT_INT4_G128) return GLOWQ_ERR_UNSUPPORTED;  // INT4 weights only
        if (w.n_out < 1 || w.k_in < kGroup || w.k_in % kGroup != 0) return GLOWQ_ERR_SHAPE;
        if (w.n_out > kMaxRows || w.k_in > kMaxD) return GLOWQ_ERR_UNSUPPORTED;
        if (!aligned(w_devs[i], 16) || !aligned(w.q, 16) || !aligned(w.sz, 16)) return GLOWQ_ERR_ALIGN;
        need += glowq_ner_workspace_bytes(w.n_out);
    }
    if (!aligned(sums_dev, 16) || !aligned(workspace, 256)) return GLOWQ_ERR_ALIGN;
    if (workspace_bytes < need) return GLOWQ_ERR_WORKSPACE;
    // launches of up to kNerBatch modules; module i's tile partials at its own offset
    double* part = static_cast<double*>(workspace);
    for (int32_t c0 = 0; c0 < n; c0 += kNerBatch) {
        NerBatch a;
        std::memset(&a, 0, sizeof(a));
        a.n_mod = n - c0 < kNerBatch ? n - c0 : kNerBatch;
        int32_t tiles = 0;
        for (int k = 0; k < a.n_mod; ++k) {
            const glowq_qweight& w = wqs[c0 + k];
            a.tile_begin[k] = tiles;
            a.n_out[k] = (int32_t)w.n_out;
            a.k_in[k] = (int32_t)w.k_in;
            a.w[k] = static_cast<const _Float16*>(w_devs[c0 + k]);
            a.q[k] = static_cast<const uint8_t*>(w.q);
            a.sz[k] = static_cast<const uint8_t*>(w.sz);
            tiles += (int32_t)ceil_div(w.n_out, 16);
        }
        a.tile_begin[a.n_mod] = tiles;
        a.part = part;
        a.sums = sums_dev + 2 * (size_t)c0;
        if (launch_ner(a, stream) != hipSuccess) return GLOWQ_ERR_HIP;
        part += 2 * (size_t)tiles;
    }
    return GLOWQ_OK;
}

int glowq_ner_sums(const void* w_dev, const glowq_qweight* wq, void* workspace, size_t workspace_bytes,
                   double* sums_dev, hipStream_t stream) {
    if (!w_dev || !wq) return GLOWQ_ERR_INVALID_ARG;
    const void* w_devs[1] = {w_dev};
    return glowq_ner_sums_batch(1, w_devs, wq, workspace, workspace_bytes, sums_dev, stream);
}

}  // extern "C"

namespace {

// Token ranges of the second-moment launch: the count in 1..16 whose workgroup total comes
// closest to whole rounds of the resident workgroups, at least one round when the ranges allow
// (each range at least 32 tokens).
void moment_plan(int64_t N, int64_t d, int32_t& n_tiles, int32_t& S, int32_t& kc) {
    const int64_t nb = ceil_div(d, kMomentTile);  // the last block may be half empty (d % 256 == 128)
    n_tiles = (int32_t)(nb * (nb + 1) / 2);
    const int64_t steps = ceil_div(N, 32);
    double best = 1e30;
    int32_t best_s = 1;
    for (int32_t s = 1; s <= 16 && s <= steps; ++s) {
        const double units = (double)n_tiles * s;
        const double rounds = (double)ceil_div((int64_t)units, kMomentResident);
        const double waste = rounds / (units / kMomentResident) + (units < kMomentResident ? 1.0 : 0.0);
        if (waste < best - 1e-9) {
            best = waste;
            best_s = s;
        }
    }
    S = best_s;
    kc = (int32_t)(ceil_div(steps, S) * 32);
    S = (int32_t)ceil_div(N, kc);
}

}  // namespace

extern "C" {

size_t glowq_second_moment_workspace_bytes(int64_t N, int64_t d) {
    if (N < 1 || d < kGroup || d % kGroup != 0 || d > kMaxMomentD || N * d > kMaxMomentElems) return 0;
    int32_t n_tiles, S, kc;
    moment_plan(N, d, n_tiles, S, kc);
    return round256((size_t)S * n_tiles * kMomentTile * kMomentTile * 4u);
}

int glowq_second_moment(const void* x_dev, int64_t N, int64_t d, float* sigma_dev, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
    if (!x_dev || !sigma_dev || !workspace) return GLOWQ_ERR_INVALID_ARG;
    if (N < 1 || d < kGroup || d % kGroup != 0) return GLOWQ_ERR_SHAPE;
    if (d > kMaxMomentD || N * d > kMaxMomentElems) return GLOWQ_ERR_UNSUPPORTED;
    if (!aligned(x_dev, 16) || !aligned(sigma_dev, 16) || !aligned(workspace, 256)) return GLOWQ_ERR_ALIGN;
    if (workspace_bytes < glowq_second_moment_workspace_bytes(N, d)) return GLOWQ_ERR_WORKSPACE;
    MomentArgs a;
    std::memset(&a, 0, sizeof(a));
    a.x = static_cast<const _Float16*>(x_dev);
    a.N = (int32_t)N;
    a.d = (int32_t)d;
    moment_plan(N, d, a.n_tiles, a.S, a.kc);
    a.inv_n = (float)(1.0 / (double)N);
    a.part = static_cast<float*>(workspace);
    a.sigma = sigma_dev;
    return launch_moment(a, stream) == hipSuccess ? GLOWQ_OK : GLOWQ_ERR_HIP;
}

// split-K partial products of the solve's skinny GEMMs (a tall operand against k columns)
static size_t solve_part_doubles(int64_t m, int64_t d, int32_t k) {
    return (size_t)kSolveSplitMax * (size_t)(m > d ? m : d) * (size_t)k;
}

// pseudo-inverse lift: the original diagonal of Sigma_x, the dropped-pivot marks and their list,
// the null-space basis and its orthonormalisation scratch, B times that basis
static size_t solve_null_doubles(int64_t d) {
    return (size_t)d + ((size_t)d + 1u) / 2u + (size_t)kSolveMaxNull / 2u + 2u * (size_t)d * kSolveMaxNull +
           3u * (size_t)kSolveMaxNull * kSolveMaxNull;
}

size_t glowq_solve_workspace_bytes(int64_t m, int64_t d, int32_t k, int32_t r) {
    if (m < 1 || d < 1 || r < 1 || k < r || k > kSolveMaxK || k > d || m > kMaxRows || d > kMaxMomentD) return 0;
    const size_t n = (size_t)d * d + (size_t)m * k + 3u * (size_t)d * k + 2u * (size_t)k * k + (size_t)k +
                     (size_t)(m > d ? m : d) * k + (size_t)k * k + 2u + solve_part_doubles(m, d, k) +
                     solve_null_doubles(d);
    return round256(n * sizeof(double));
}

int glowq_solve_factors(const double* e_dev, int64_t m, int64_t d, const double* sigma_dev,
                        const double* omega_dev, int32_t r, int32_t k, int32_t q, double* a_dev, double* b_dev,
                        double* s_dev, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!e_dev || !sigma_dev || !omega_dev || !a_dev || !b_dev || !s_dev || !workspace) return GLOWQ_ERR_INVALID_ARG;
    if (m < 1 || d < 1 || r < 1 || k < r || q < 0 || q > 16) return GLOWQ_ERR_SHAPE;
    if (k > kSolveMaxK || k > d || m > kMaxRows || d > kMaxMomentD) return GLOWQ_ERR_UNSUPPORTED;
    const void* ptrs[] = {e_dev, sigma_dev, omega_dev, a_dev, b_dev, s_dev};
    for (const void* p : ptrs)
        if (!aligned(p, 16)) return GLOWQ_ERR_ALIGN;
    if (!aligned(workspace, 256)) return GLOWQ_ERR_ALIGN;
    if (workspace_bytes < glowq_solve_workspace_bytes(m, d, k, r)) return GLOWQ_ERR_WORKSPACE;
    const int M = (int)m, D = (int)d;
    double* L = static_cast<double*>(workspace);
    double* Y = L + (size_t)d * d;                  // range basis Q (m x k)
    double* Z = Y + (size_t)m * k;                  // co-range basis (d x k)
    double* W = Z + (size_t)d * k;                  // L times a d x k block
    double* P = W + (size_t)d * k;                  // E_cat^T Q (d x k)
    double* G = P + (size_t)d * k;
    double* V = G + (size_t)k * k;
    double* w = V + (size_t)k * k;
    double* T = w + k;                              // orthonormalisation scratch, then B_small^T
    double* Ri = T + (size_t)(m > d ? m : d) * k;
    double* part = Ri + (size_t)k * k;             // split-K partial products
    const int64_t part_cap = (int64_t)solve_part_doubles(m, d, k);
    int* flag = reinterpret_cast<int*>(part + part_cap);
    double* dg = part + part_cap + 2;                                       // diag(Sigma_x)
    int* drop = reinterpret_cast<int*>(dg + d);                             // dropped pivots [d]
    int* list = drop + 2 * (((size_t)d + 1u) / 2u);                         // their indices
    double* Nb = reinterpret_cast<double*>(list + kSolveMaxNull);           // null basis [d][n0]
    double* Nt = Nb + (size_t)d * kSolveMaxNull;                            // orth scratch [d][n0]
    double* Ng = Nt + (size_t)d * kSolveMaxNull;                            // [n0][n0]
    double* Nr = Ng + (size_t)kSolveMaxNull * kSolveMaxNull;                // [n0][n0]
    double* BN = Nr + (size_t)kSolveMaxNull * kSolveMaxNull;                // B N [r][n0]
    auto gemm = [&](int Mm, int Nn, int Kk, const double* A, int lda, int ta, const double* B, int ldb, int tb,
                    double* C, int ldc) {
        GemmArgs g{};
        g.M = Mm, g.N = Nn, g.K = Kk, g.A = A, g.lda = lda, g.ta = ta, g.B = B, g.ldb = ldb, g.tb = tb;
        g.C = C, g.ldc = ldc, g.alpha = 1.0, g.beta = 0.0, g.part = part, g.part_cap = part_cap;
        return launch_gemm(g, stream) == hipSuccess;
    };
    // The whitened error E~ = E_cat L is never formed: every product with it is taken as a product
    // with E_cat and one with L (a d x k block), E~ X = E_cat (L X), E~^T Y = L^T (E_cat^T Y).
    bool ok = hipMemcpyAsync(L, sigma_dev, (size_t)d * d * sizeof(double), hipMemcpyDeviceToDevice, stream) ==
              hipSuccess;
    ok = ok && launch_cholesky(L, D, flag, dg, drop, stream) == hipSuccess;  // Sigma_x = L L^T
    if (!ok) return GLOWQ_ERR_HIP;
    // not positive semidefinite: stop; numerically zero pivots: their columns of L are zero and the
    // lift below projects B onto the range of Sigma_x (pseudo-inverse)
    int h = 0;
    std::vector<int> dropped((size_t)d);
    if (hipMemcpyAsync(&h, flag, sizeof(int), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipMemcpyAsync(dropped.data(), drop, (size_t)d * sizeof(int), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return GLOWQ_ERR_HIP;
    if (h) return GLOWQ_ERR_RANGE;
    std::vector<int> nulls;
    for (int i = 0; i < D; ++i)
        if (dropped[(size_t)i]) nulls.push_back(i);
    const int n0 = (int)nulls.size();
    if (n0 > kSolveMaxNull) return GLOWQ_ERR_UNSUPPORTED;
    if (n0 > 0 && hipMemcpyAsync(list, nulls.data(), (size_t)n0 * sizeof(int), hipMemcpyHostToDevice, stream) != hipSuccess)
        return GLOWQ_ERR_HIP;
    ok = ok && gemm(D, k, D, L, D, 0, omega_dev, k, 0, W, k);               // L Omega
    ok = ok && gemm(M, k, D, e_dev, D, 0, W, k, 0, Y, k);                   // Y = E~ Omega
    ok = ok && launch_orth(Y, M, k, T, G, Ri, part, part_cap, stream) == hipSuccess;
    for (int it = 0; it < q && ok; ++it) {
        ok = ok && gemm(D, k, M, e_dev, D, 1, Y, k, 0, P, k);               // E_cat^T Q
        ok = ok && gemm(D, k, D, L, D, 1, P, k, 0, Z, k);                   // Z = orth(E~^T Q)
        ok = ok && launch_orth(Z, D, k, T, G, Ri, part, part_cap, stream) == hipSuccess;
        ok = ok && gemm(D, k, D, L, D, 0, Z, k, 0, W, k);                   // L Z
        ok = ok && gemm(M, k, D, e_dev, D, 0, W, k, 0, Y, k);               // Q = orth(E~ Z)
        ok = ok && launch_orth(Y, M, k, T, G, Ri, part, part_cap, stream) == hipSuccess;
    }
    ok = ok && gemm(D, k, M, e_dev, D, 1, Y, k, 0, P, k);                   // P = E_cat^T Q
    ok = ok && gemm(D, k, D, L, D, 1, P, k, 0, T, k);                       // B_small^T = (Q^T E~)^T = L^T P
    ok = ok && gemm(k, k, D, T, k, 1, T, k, 0, G, k);                       // B_small B_small^T = U S^2 U^T
    ok = ok && launch_jacobi(G, k, w, V, stream) == hipSuccess;
    ok = ok && launch_sqrt(w, s_dev, r, stream) == hipSuccess;
    ok = ok && gemm(M, r, k, Y, k, 0, V, k, 0, a_dev, r);                   // A = Q U_r S_r^{1/2}
    ok = ok && launch_colscale(a_dev, r, M, r, w, 0, 0, stream) == hipSuccess;
    // B = S_r^{1/2} V_r^T L^{-1} = S_r^{-1/2} U_r^T Q^T E~ L^{-1} = S_r^{-1/2} U_r^T (Q^T E_cat), since
    // E~ = E_cat L: the lift needs no triangular solve
    ok = ok && gemm(r, D, k, V, k, 1, P, k, 1, b_dev, D);                   // U_r^T P^T
    ok = ok && launch_colscale(b_dev, D, r, D, w, 1, 1, stream) == hipSuccess;  // rows times S_r^{-1/2}
    if (ok && n0 > 0) {
        // pseudo-inverse lift: B = S_r^{1/2} V_r^T L^+ = S_r^{-1/2} U_r^T Q^T E_cat (L L^+), and L L^+ is
        // the orthogonal projector onto range(Sigma_x) = I - N N^T for an orthonormal basis N of the
        // null space: B <- B - (B N) N^T
        ok = launch_null_vectors(L, D, drop, list, n0, Nb, stream) == hipSuccess;
        ok = ok && launch_orth(Nb, D, n0, Nt, Ng, Nr, part, part_cap, stream) == hipSuccess;
        if (ok) {
            GemmArgs g1{};  // B N
            g1.M = r, g1.N = n0, g1.K = D, g1.A = b_dev, g1.lda = D, g1.ta = 0, g1.B = Nb, g1.ldb = n0, g1.tb = 0;
            g1.C = BN, g1.ldc = n0, g1.alpha = 1.0, g1.beta = 0.0;
            ok = launch_gemm(g1, stream) == hipSuccess;
            GemmArgs g2{};  // B - (B N) N^T
            g2.M = r, g2.N = D, g2.K = n0, g2.A = BN, g2.lda = n0, g2.ta = 0, g2.B = Nb, g2.ldb = n0, g2.tb = 1;
            g2.C = b_dev, g2.ldc = D, g2.alpha = -1.0, g2.beta = 1.0;
            ok = ok && launch_gemm(g2, stream) == hipSuccess;
        }
    }
    if (!ok) return GLOWQ_ERR_HIP;
    return hipStreamSynchronize(stream) == hipSuccess ? GLOWQ_OK : GLOWQ_ERR_HIP;
}

size_t glowq_ec_score_workspace_bytes(int64_t m, int64_t d) {
    if (m < 1 || d < 1 || m > kMaxRows || d > kMaxMomentD) return 0;
    return round256(((size_t)d * d + (size_t)d) * sizeof(double));
}

int glowq_ec_score(const double* e_dev, int64_t m, int64_t d, const double* sigma_dev, const double* s_dev,
                   int32_t r, double* out_dev, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!e_dev || !sigma_dev || !out_dev || !workspace || (r > 0 && !s_dev)) return GLOWQ_ERR_INVALID_ARG;
    if (m < 1 || d < 1 || r < 0 || r > m || r > d) return GLOWQ_ERR_SHAPE;
    if (m > kMaxRows || d > kMaxMomentD) return GLOWQ_ERR_UNSUPPORTED;
    if (!aligned(e_dev, 16) || !aligned(sigma_dev, 16) || !aligned(out_dev, 16) || (s_dev && !aligned(s_dev, 16)) ||
        !aligned(workspace, 256))
        return GLOWQ_ERR_ALIGN;
    if (workspace_bytes < glowq_ec_score_workspace_bytes(m, d)) return GLOWQ_ERR_WORKSPACE;
    double* C = static_cast<double*>(workspace);
    double* part = C + (size_t)d * d;
    GemmArgs g{};  // C = E_cat^T E_cat, lower triangle
    g.M = (int32_t)d, g.N = (int32_t)d, g.K = (int32_t)m;
    g.A = e_dev, g.lda = (int32_t)d, g.ta = 1;
    g.B = e_dev, g.ldb = (int32_t)d, g.tb = 0;
    g.C = C, g.ldc = (int32_t)d, g.alpha = 1.0, g.beta = 0.0, g.c_lower = 1;
    if (launch_gemm(g, stream) != hipSuccess) return GLOWQ_ERR_HIP;
    return launch_ec(C, sigma_dev, (int)d, s_dev, r, part, out_dev, stream) == hipSuccess ? GLOWQ_OK : GLOWQ_ERR_HIP;
}

int glowq_restore_select(const double* sums_dev, int32_t n_units, int32_t n_per_unit, int32_t k, double rel_tol,
                         double* scores_dev, int32_t* mask_dev, hipStream_t stream) {
    if (!sums_dev || !scores_dev || !mask_dev) return GLOWQ_ERR_INVALID_ARG;
    if (!(rel_tol >= 0.0 && rel_tol <= 1.0)) return GLOWQ_ERR_INVALID_ARG;  // also rejects NaN
    if (n_units < 1 || n_units > kMaxScoreUnits || n_per_unit < 1 || n_per_unit > 1024 || k < 0 ||
        k > n_units)
        return GLOWQ_ERR_SHAPE;
    if (!aligned(sums_dev, 16) || !aligned(scores_dev, 16) || !aligned(mask_dev, 16)) return GLOWQ_ERR_ALIGN;
    const hipError_t e = launch_topk(sums_dev, n_units, n_per_unit, k, rel_tol, scores_dev, mask_dev, stream);
    return e == hipSuccess ? GLOWQ_OK : GLOWQ_ERR_HIP;
}

int glowq_restore_topk(const double* sums_dev, int32_t n_units, int32_t n_per_unit, int32_t k,
                       double* scores_dev, int32_t* mask_dev, hipStream_t stream) {
    return glowq_restore_select(sums_dev, n_units, n_per_unit, k, 0.0, scores_dev, mask_dev, stream);
}

int glowq_group_forward(const void* x, int64_t T, int64_t d, int32_t m, const glowq_qweight* w,
                        const void* b_shared, const void* const* a, int32_t r, int32_t restore,
                        void* workspace, size_t workspace_bytes, void* const* y, hipStream_t stream) {
    const void* bp[1] = {b_shared};
    const Call c = make_group(x, T, d, m, w, bp, 1, a, r, restore, y);
    const int v = validate(c, workspace, workspace_bytes);
    if (v != GLOWQ_OK) return v;
    return run(c, workspace, stream);
}

int glowq_solo_forward(const void* x, int64_t T, int64_t d, const glowq_qweight* w, const void* b,
                       const void* a, int32_t r, int32_t restore, void* workspace, size_t workspace_bytes,
                       void* y, hipStream_t stream) {
    const void* bp[1] = {b};
    const void* ap[1] = {a};
    void* yp[1] = {y};
    const Call c = make_group(x, T, d, 1, w, bp, 1, ap, r, restore, yp);
    const int v = validate(c, workspace, workspace_bytes);
    if (v != GLOWQ_OK) return v;
    return run(c, workspace, stream);
}

}  // extern "C"

// ------------------------------------------------------------------ allocation-free variant
// Scratch of glowq_group_forward_static: a file-scope device array of kStaticScratchBytes, one copy
// per GPU, held until the process ends.  Host code never passes the array's name to a kernel (on
// the host it only stands for the symbol): its device address is taken once per device with
// hipGetSymbolAddress and that pointer is used everywhere.
namespace {
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

static __device__ __attribute__((aligned(256))) uint8_t scratch[kStaticScratchBytes];

namespace {
// Device address of the current device's scratch; the first call on a device looks it up and
// zero-fills the array with a kernel on `stream` (stream-ordered before this call's kernels).
int static_scratch(hipStream_t stream, void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GLOWQ_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return GLOWQ_ERR_HIP;
        if (launch_fill_zero(p, kStaticScratchBytes, stream) != hipSuccess) return GLOWQ_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return GLOWQ_OK;
}
}  // namespace

extern "C" {

size_t glowq_static_scratch_bytes(void) { return kStaticScratchBytes; }

int glowq_group_forward_static(const void* x, int64_t T, int64_t d, int32_t m, const glowq_qweight* w,
                               const void* b_shared, const void* const* a, int32_t r, int32_t restore,
                               void* const* y, hipStream_t stream) {
    const void* bp[1] = {b_shared};
    const Call c = make_group(x, T, d, m, w, bp, 1, a, r, restore, y);
    // the scratch stands in for the workspace: validate against its size with a stand-in
    // address (aligned, never dereferenced), then substitute the device pointer
    void* const stand_in = reinterpret_cast<void*>((uintptr_t)256);
    const int v = validate(c, stand_in, kStaticScratchBytes);
    if (v != GLOWQ_OK) return v;
    if (T == 0) return GLOWQ_OK;
    void* ws = nullptr;
    if (c.correct) {
        const int s = static_scratch(stream, &ws);
        if (s != GLOWQ_OK) return s;
    }
    return run(c, ws, stream);
}

int glowq_layerwise_forward(const void* x, int64_t T, int64_t d, int32_t m, const glowq_qweight* w,
                            const void* const* b, const void* const* a, int32_t r, int32_t restore,
                            void* workspace, size_t workspace_bytes, void* const* y, hipStream_t stream) {
    if (m < 1) return GLOWQ_ERR_SHAPE;
    if (m > GLOWQ_MAX_MODULES) return GLOWQ_ERR_UNSUPPORTED;
    const Call c = make_group(x, T, d, m, w, b, m, a, r, restore, y);
    const int v = validate(c, workspace, workspace_bytes);
    if (v != GLOWQ_OK) return v;
    return run(c, workspace, stream);
}

int glowq_path_forward(const glowq_unit* units, int32_t n_units, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
    if (n_units < 0) return GLOWQ_ERR_SHAPE;
    if (n_units > 0 && units == nullptr) return GLOWQ_ERR_INVALID_ARG;
    // validate every unit first: a rejected schedule launches nothing
    for (int32_t u = 0; u < n_units; ++u) {
        const glowq_unit& U = units[u];
        if (U.kind != GLOWQ_UNIT_GROUP && U.kind != GLOWQ_UNIT_SOLO) return GLOWQ_ERR_INVALID_ARG;
        if (U.kind == GLOWQ_UNIT_SOLO && U.m != 1) return GLOWQ_ERR_SHAPE;
        const void* bp[1] = {U.b};
        const Call c = make_group(U.x, U.T, U.d, U.m, U.w, bp, 1, U.a, U.r, U.restore, U.y);
        const int v = validate(c, workspace, workspace_bytes);
        if (v != GLOWQ_OK) return v;
    }
    for (int32_t u = 0; u < n_units; ++u) {
        const glowq_unit& U = units[u];
        const void* bp[1] = {U.b};
        const Call c = make_group(U.x, U.T, U.d, U.m, U.w, bp, 1, U.a, U.r, U.restore, U.y);
        const int v = run(c, workspace, stream);
        if (v != GLOWQ_OK) return v;
    }
    return GLOWQ_OK;
}

}  // extern "C"
