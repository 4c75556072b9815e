// MX weights (MXFP4, MXFP6 E2M3 / E3M2) against MXFP8 activations on the gfx950 block-scaled matrix
// cores (v_mfma_scale_f32_16x16x128_f8f6f4): the 8-bit-activation form of the method (GlowQ arXiv
// page, Tables 14 and 15) with weights and activations both in the microscaling family of Table 13.
//
//   x8[t, k], S[t, b] = MXFP8 quantisation of X (OCP MX v1.0): per token and 32-input block b the
//                       shared exponent floor(log2 max|x|) - 8, each element the nearest E4M3 value
//                       (ties to even, saturating at 448)
//   y_i[t, o]        = sum_b 2^(S_w[o, b] + S[t, b] - 254) sum_{k in b} w[o, k] x8[t, k]
//                      + R[t] . A_i[o],   R = X B^T from the fp16 X, formed once per call
// (w the weight element values).  The matrix cores apply both block scales themselves: one
// 16x16x128 step covers a 128-input group of 16 rows and 16 tokens, four scale groups of 32
// products each.
//
// Operand pairing of the step (measured with in-bounds probes on the device): lane l of the weight
// operand holds row l % 16 and the 32 elements of scale group l / 16 (the weight layout's one MX
// block per lane; its scale is the lane's E8M0 byte); the FP8 operand's lane l holds column (token)
// l % 16 and 32 bytes, byte p of lane group h pairing with weight element n = 16 (h % 2) + p % 16 of
// scale group g = 2 (p / 16) + h / 2, whose activation scale the lane l % 16 + 16 g supplies.  So the
// activation codes of a 128-input group are stored in that order: input 32 g + n of the group at
// byte 32 (2 (g % 2) + n / 16) + 16 (g / 2) + n % 16, and a lane reads its 32 operand bytes at 32 h.
// The activation scales are stored so that a lane finds all the scales it needs for one group in one
// 8-byte word: per 128-token block tb and group G a 512-byte record at (tb G_count + G) 512, the scale
// of token t and block g of the group at byte 8 (16 g + t % 16) + (t % 128) / 16 -- lane l of the
// step (column l % 16, scale group l / 16) reads the word at 8 l, byte j holding the scale of its
// token in the block's 16-token tile j.
#include <type_traits>

#include "glowq_internal.h"

namespace glowq {

typedef int32_t i8v __attribute__((ext_vector_type(8)));

// E4M3 code of u (exact fp32 input, |u| < 512): nearest value, ties to the even mantissa, saturating
// at 448; subnormals below 2^-6 in steps of 2^-9.  Branch-free and exact: in the normal range the
// code is the fp32 bit pattern rounded to 3 mantissa bits (round half to even on the 20 dropped
// bits; a mantissa carry moves into the exponent as it should) with the exponent rebased from 127
// to 7; below 2^-6 it is the nearest multiple of 2^-9 (8 of them being the smallest normal, 0x08).
__device__ __forceinline__ uint32_t e4m3_code(float u) {
    const float a = fminf(fabsf(u), 448.0f);
    const uint32_t b = __builtin_bit_cast(uint32_t, a);
    const uint32_t normal = ((b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20) - ((127u - 7u) << 3);
    const uint32_t sub = (uint32_t)__builtin_rintf(a * 512.0f);
    const uint32_t code = a < 0.015625f ? sub : normal;
    return (u < 0.0f && code != 0) ? (code | 0x80u) : code;
}

// One thread per (token, 32-input block) over a flat grid: the block's largest magnitude, its
// scale byte, the codes stored in the operand order above (two 16-byte stores per block).
constexpr int kMx8QuantThreads = 256;

// Weight format of the block-scaled step: the A operand's element code (cbsz) and the lane's operand
// words: MXFP4 16 bytes (32 nibbles), MXFP6 24 bytes (the 16-byte plane and the 8-byte plane of the
// device layout, element n at bits 6 n of their concatenation -- the operand order of the step, probed
// like the FP4 one: element n of lane l pairs with the same FP8 byte as FP4 element n).
template <int F>
struct Mx8W {
    static_assert(F == kFmtMxfp4 || F == kFmtMxfp6E2M3 || F == kFmtMxfp6E3M2, "MX weight format");
    static constexpr bool six = F != kFmtMxfp4;
    static constexpr int cbsz = F == kFmtMxfp4 ? 4 : (F == kFmtMxfp6E2M3 ? 2 : 3);
    static constexpr int qblock = six ? 1536 : 1024;
    static __device__ __forceinline__ i8v operand(const u4& lo, const u2& hi) {
        if constexpr (six)
            return i8v{(int32_t)lo[0], (int32_t)lo[1], (int32_t)lo[2], (int32_t)lo[3], (int32_t)hi[0], (int32_t)hi[1], 0, 0};
        else
            return i8v{(int32_t)lo[0], (int32_t)lo[1], (int32_t)lo[2], (int32_t)lo[3], 0, 0, 0, 0};
    }
};

// Byte offset of the 512-byte scale record of token t's 128-token block and group G, plus the
// token's position (t % 128) / 16 in each 8-byte word.
__device__ __forceinline__ size_t mx8_scale_offset(int t, int G, int n_groups) {
    return ((size_t)(t >> 7) * n_groups + G) * 512 + ((t & 127) >> 4);
}

__global__ __launch_bounds__(kMx8QuantThreads) void quant_mx8_kernel(const _Float16* __restrict__ x, int T, int d,
                                                                   uint8_t* __restrict__ xq,
                                                                   uint8_t* __restrict__ xs) {
    const int nb = d / 32;
    const int64_t i = (int64_t)blockIdx.x * kMx8QuantThreads + threadIdx.x;
    if (i < (int64_t)T * nb) {
        const int t = (int)(i / nb), b = (int)(i - (int64_t)t * nb);
        const _Float16* row = x + (size_t)t * d;
        h8 v[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = load_h8(row + 32 * b + 8 * c);
        float amax = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)v[c][e]));
        int X = -127;  // a block of zeros: the smallest scale, zero codes
        if (amax > 0.f) X = (int)((__builtin_bit_cast(uint32_t, amax) >> 23) & 0xFFu) - 127 - 8;
        // 2^-X as an fp32 power of two (X in -32 .. 7 for fp16 inputs)
        const float inv = __builtin_bit_cast(float, (uint32_t)(127 - (amax > 0.f ? X : 0)) << 23);
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t word = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = 4 * i + j;
                word |= e4m3_code((float)v[n >> 3][n & 7] * inv) << (8 * j);
            }
            w[i] = word;
        }
        const int G = b >> 2, g = b & 3;
        uint8_t* base = xq + (size_t)t * d + (size_t)G * kGroup + 16 * (g >> 1);
        *reinterpret_cast<u4*>(base + 32 * (2 * (g & 1))) = u4{w[0], w[1], w[2], w[3]};      // n = 0 .. 15
        *reinterpret_cast<u4*>(base + 32 * (2 * (g & 1) + 1)) = u4{w[4], w[5], w[6], w[7]};  // n = 16 .. 31
        xs[mx8_scale_offset(t, G, d / kGroup) + 8 * (16 * g + (t & 15))] = (uint8_t)(X + 127);
    }
}

// GEMM tile: 16 TT tokens x 64 RR rows, four waves side by side in N (wave w owns RR row tiles of
// 16 rows, all tokens), KS groups of four waves splitting the input groups (added through LDS in
// wave-group order, deterministic).  Per group: the token codes (BM x 128 bytes) staged in LDS,
// double-buffered, with each token tile's activation scales; weights (16 bytes per lane for MXFP4,
// 16 + 8 for MXFP6: the operand as stored) and their scale words straight from HBM, one group ahead
// in registers; one
// block-scaled matrix-core step per (row tile, token tile).  After the K loop r_pad / 32 fp16
// matrix-core steps add R A_i^T, one rounding to fp16.
template <int F, int TT, int RR, int KS>
__global__ __launch_bounds__(256 * KS, (KS == 1 ? 2 : 1)) void mx8_kernel(const ForwardArgs args) {
    using WF = Mx8W<F>;
    constexpr bool SIX = WF::six;
    constexpr int QB = WF::qblock;
    constexpr int BM = 16 * TT;
    constexpr int LSB = 144;             // LDS row stride in bytes (128 + 16 padding)
    constexpr int NCH = BM * 8 / 256;    // 16-byte code chunks per thread per group (BM rows x 8)
    constexpr int NCHP = NCH > 0 ? NCH : 1;
    constexpr int kTileBytes = KS * 2 * BM * LSB;
    constexpr int kRedBytes = (KS - 1) * TT * RR * 256 * 16;
    __shared__ __attribute__((aligned(16))) uint8_t smem[kTileBytes > kRedBytes ? kTileBytes : kRedBytes];
    uint8_t (*xsm)[2][BM * LSB] = reinterpret_cast<uint8_t (*)[2][BM * LSB]>(smem);

    const int mb = blockIdx.x % args.m_tiles, nbl = blockIdx.x / args.m_tiles;
    const ModuleArgs M = args.mod[module_of(args, nbl)];
    const int nb = nbl - M.tile_begin;
    const int m0 = mb * BM;
    const int tid = threadIdx.x & 255, lane = tid & 63;
    const int kg = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 8);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int T = args.T, d = args.d, G = args.G;
    const int rt0 = nb * 4 * RR + wave * RR;
    const size_t qstride = (size_t)M.n_tiles16 * QB, szstride = (size_t)M.n_tiles16 * 64;
    const int sgrp = lane >> 4;  // the lane's scale group in a 128-input group
    const int q6ofs = 1024 + 8 * lane - 16 * lane;  // MXFP6: the lane's 8-byte plane, from its 16 bytes

    const uint8_t* qp[RR];
    const uint8_t* zp[RR];
    bool w_ok[RR];
#pragma unroll
    for (int rr = 0; rr < RR; ++rr) {
        const int rt = rt0 + rr;
        w_ok[rr] = rt < M.n_tiles16;
        qp[rr] = M.q + (size_t)(w_ok[rr] ? rt : 0) * QB + lane * 16;
        zp[rr] = M.sz + (size_t)(w_ok[rr] ? rt : 0) * 64 + (lane & 15) * 4;
    }
    // code staging: BM rows x 8 chunks of 16 bytes per group; thread tid copies chunks tid + 256 c
    const uint8_t* xsrc[NCHP];
    bool x_ok[NCHP];
    int xdst[NCHP];
#pragma unroll
    for (int c = 0; c < NCHP; ++c) {
        const int idx = c * 256 + tid;
        const int row = idx >> 3, col = (idx & 7) * 16;
        const int t = m0 + row;
        x_ok[c] = idx < BM * 8 && t < T;
        xsrc[c] = args.x8 + (size_t)(x_ok[c] ? t : 0) * d + col;
        xdst[c] = (idx < BM * 8 ? row : 0) * LSB + col;
    }
    // this lane's tokens (one per token tile) and their activation scales (tile m0 / 16 + tt of the
    // scale records; a tile past T reads scales never written, feeding only outputs never stored)
    int tok[TT];
    bool t_ok[TT];
    const uint8_t* srow[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        tok[tt] = m0 + 16 * tt + (lane & 15);
        t_ok[tt] = tok[tt] < T;
        srow[tt] = args.x8scale + mx8_scale_offset(m0 + 16 * tt, 0, G) + 8 * lane;
    }
    const u4 zero4 = {0u, 0u, 0u, 0u};
    const int n_it = (G + KS - 1) / KS;
    const bool act0 = kg < G;
    const bool copier = BM * 8 >= 256 || tid < BM * 8;  // TT = 1: 128 of 256 threads copy

    const u2 zero2 = {0u, 0u};
    u4 st[NCHP];
    u4 qv[RR];
    u2 q6[RR];
    uint32_t zw[RR];
    uint32_t sb[TT];
#pragma unroll
    for (int c = 0; c < NCHP; ++c)
        st[c] = (act0 && x_ok[c]) ? *reinterpret_cast<const u4*>(xsrc[c] + (size_t)kg * kGroup) : zero4;
#pragma unroll
    for (int rr = 0; rr < RR; ++rr) {
        qv[rr] = (act0 && w_ok[rr]) ? *reinterpret_cast<const u4*>(qp[rr] + (size_t)kg * qstride) : zero4;
        q6[rr] = (SIX && act0 && w_ok[rr]) ? *reinterpret_cast<const u2*>(qp[rr] + (size_t)kg * qstride + q6ofs) : zero2;
        zw[rr] = (act0 && w_ok[rr]) ? *reinterpret_cast<const uint32_t*>(zp[rr] + (size_t)kg * szstride) : 0u;
    }
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) sb[tt] = act0 ? srow[tt][(size_t)kg * 512] : 0u;
    if (copier) {
#pragma unroll
        for (int c = 0; c < NCHP; ++c)
            if (c * 256 + tid < BM * 8) *reinterpret_cast<u4*>(&xsm[kg][0][xdst[c]]) = st[c];
    }
    __syncthreads();

    f4 acc[TT][RR];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int rr = 0; rr < RR; ++rr) acc[tt][rr] = f4{0.f, 0.f, 0.f, 0.f};

    for (int it = 0; it < n_it; ++it) {
        const int g = it * KS + kg;
        const int buf = it & 1;
        const bool act = g < G, more = g + KS < G;
        u4 qn[RR];
        u2 q6n[RR];
        uint32_t zn[RR], sbn[TT];
        if (more) {
#pragma unroll
            for (int c = 0; c < NCHP; ++c)
                st[c] = x_ok[c] ? *reinterpret_cast<const u4*>(xsrc[c] + (size_t)(g + KS) * kGroup) : zero4;
#pragma unroll
            for (int rr = 0; rr < RR; ++rr) {
                qn[rr] = w_ok[rr] ? *reinterpret_cast<const u4*>(qp[rr] + (size_t)(g + KS) * qstride) : zero4;
                q6n[rr] = (SIX && w_ok[rr]) ? *reinterpret_cast<const u2*>(qp[rr] + (size_t)(g + KS) * qstride + q6ofs)
                                            : zero2;
                zn[rr] = w_ok[rr] ? *reinterpret_cast<const uint32_t*>(zp[rr] + (size_t)(g + KS) * szstride) : 0u;
            }
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) sbn[tt] = srow[tt][(size_t)(g + KS) * 512];
        }
        if (act) {
            const uint8_t* xb = &xsm[kg][buf][(lane & 15) * LSB + 32 * sgrp];
            i8v a[RR];
            int32_t sa[RR];
#pragma unroll
            for (int rr = 0; rr < RR; ++rr) {
                a[rr] = WF::operand(qv[rr], q6[rr]);
                sa[rr] = (int32_t)((zw[rr] >> (8 * sgrp)) & 0xFFu);
            }
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                const u4 b0 = *reinterpret_cast<const u4*>(xb + tt * 16 * LSB);
                const u4 b1 = *reinterpret_cast<const u4*>(xb + tt * 16 * LSB + 16);
                const i8v b = {(int32_t)b0[0], (int32_t)b0[1], (int32_t)b0[2], (int32_t)b0[3],
                               (int32_t)b1[0], (int32_t)b1[1], (int32_t)b1[2], (int32_t)b1[3]};
#pragma unroll
                for (int rr = 0; rr < RR; ++rr)
                    acc[tt][rr] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[rr], b, acc[tt][rr], WF::cbsz, 0, 0,
                                                                                  sa[rr], 0, (int32_t)sb[tt]);
            }
        }
        if (more) {
            if (copier) {
#pragma unroll
                for (int c = 0; c < NCHP; ++c)
                    if (c * 256 + tid < BM * 8) *reinterpret_cast<u4*>(&xsm[kg][buf ^ 1][xdst[c]]) = st[c];
            }
#pragma unroll
            for (int rr = 0; rr < RR; ++rr) {
                qv[rr] = qn[rr];
                q6[rr] = q6n[rr];
                zw[rr] = zn[rr];
            }
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) sb[tt] = sbn[tt];
        }
        __syncthreads();
    }

    if (KS > 1) {
        f4* red = reinterpret_cast<f4*>(smem);
        if (kg > 0) {
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                for (int rr = 0; rr < RR; ++rr) red[(((kg - 1) * TT + tt) * RR + rr) * 256 + tid] = acc[tt][rr];
        }
        __syncthreads();
        if (kg > 0) return;
#pragma unroll
        for (int k = 1; k < KS; ++k)
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                for (int rr = 0; rr < RR; ++rr) acc[tt][rr] += red[(((k - 1) * TT + tt) * RR + rr) * 256 + tid];
    }

    // the correction on the fp16 projection
    const int kofs = 8 * (lane >> 4);
    if (args.r > 0 && M.a != nullptr) {
        const int r = args.r, rp = args.r_pad;
        const _Float16* R = reinterpret_cast<const _Float16*>(args.R) + (size_t)M.proj * T * rp;
        const h8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int kb = 0; kb < rp / 32; ++kb) {
            const int col = 32 * kb + kofs;
            h8 a[RR];
#pragma unroll
            for (int rr = 0; rr < RR; ++rr) {
                const int row = (rt0 + rr) * 16 + (lane & 15);
                a[rr] = (row < M.n_out && col < r) ? load_h8(M.a + (size_t)row * r + col) : zero8;
            }
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                const h8 b = (t_ok[tt] && col < rp) ? load_h8(R + (size_t)tok[tt] * rp + col) : zero8;
#pragma unroll
                for (int rr = 0; rr < RR; ++rr) acc[tt][rr] = mfma16(a[rr], b, acc[tt][rr]);
            }
        }
    }

    const bool vec = (M.n_out & 3) == 0;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        if (!t_ok[tt]) continue;
        _Float16* yrow = M.y + (size_t)tok[tt] * M.n_out;
#pragma unroll
        for (int rr = 0; rr < RR; ++rr) {
            if (rt0 + rr >= M.n_tiles16) continue;
            const int row0 = (rt0 + rr) * 16 + 4 * (lane >> 4);
            const f4 v = acc[tt][rr];
            if (vec && row0 + 3 < M.n_out) {
                const h2 lo = {(_Float16)v[0], (_Float16)v[1]}, hi = {(_Float16)v[2], (_Float16)v[3]};
                *reinterpret_cast<u2*>(yrow + row0) = u2{as_u32(lo), as_u32(hi)};
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (row0 + i < M.n_out) yrow[row0 + i] = (_Float16)v[i];
            }
        }
    }
}

// Wide tile for large grids: 128 tokens (one scale block) x 512 rows, eight waves (two per SIMD)
// each owning 4 row tiles and all 8 token tiles, so that every FP8 operand read from LDS feeds 4
// block-scaled steps and every weight operand 8 (32 steps per wave and group).  Nothing in flight
// sits in registers: per group the codes (128 rows x 128 bytes, read by every wave), each wave's
// weight blocks (4 x 1 KB for MXFP4, 4 x 1.5 KB for MXFP6: the operands as stored) and their scale
// words, and the token block's activation-scale record are copied HBM/L2 -> LDS by the load unit
// (global_load_lds) into a ring of stages (three, two groups ahead, for MXFP4; two, one group ahead,
// for the larger MXFP6 blocks, so that the ring fits the 160 KB of LDS), so that the loop carries no
// register loads (whose waits the compiler would place conservatively at the loop head) and every
// wait is the explicit one before each group's barrier.  In a stage, code row r keeps its 16-byte chunk c at position
// c ^ f(r), f(r) = (r % 8) ^ ((r / 8) % 2), so that the operand reads of 16 consecutive rows fall
// in distinct bank groups; a wave's scale words sit as [row][row tile], so that a lane reads its
// four with one 16-byte read.  Tokens past T read token T - 1 and row tiles past the module its
// last tile; neither is stored.
template <int I>
using ic = std::integral_constant<int, I>;
typedef __attribute__((address_space(3))) void lds_void8;

constexpr int kMx8WideWaves = 8;
constexpr int kMx8CodeBytes = 128 * 128;                          // codes of one group
constexpr int kMx8ZBytes = kMx8WideWaves * 256;                   // weight scale words
constexpr int kMx8SBytes = kMx8WideWaves * 256;                   // activation scales (two copies per half)

template <int F>
__global__ __launch_bounds__(512, 1) void mx8_wide_kernel(const ForwardArgs args) {
    using WF = Mx8W<F>;
    constexpr bool SIX = WF::six;
    constexpr int QB = WF::qblock;
    constexpr int TT = 8, RR = 4, BM = 128, NW = kMx8WideWaves;
    constexpr int NST = SIX ? 2 : 3;                   // stages of the ring
    constexpr int WW = RR * QB;                        // one wave's weight blocks per group
    constexpr int NWI = WW / 1024;                     // their 1 KB copies
    constexpr int PER = 2 + NWI + 2;                   // copies per wave and group
    static_assert(PER < 16, "vmcnt immediate");
    constexpr int W_AT = kMx8CodeBytes, Z_AT = W_AT + NW * WW, S_AT = Z_AT + kMx8ZBytes;
    constexpr int SB = S_AT + kMx8SBytes;              // bytes per stage
    static_assert(NST * SB <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(16))) uint8_t st0[SB];
    __shared__ __attribute__((aligned(16))) uint8_t st1[SB];
    __shared__ __attribute__((aligned(16))) uint8_t st2[NST == 3 ? SB : 16];

    int mb, nbl;
    if ((args.m_tiles & 3) == 0) {
        // XCD x = 4 q + p (workgroups b with b % 8 == x) owns token blocks [p m / 4, (p + 1) m / 4)
        // and the row blocks of parity q: four token blocks share every weight block in its L2
        const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3, mp = args.m_tiles >> 2;
        const int p = xcd & 3, q = xcd >> 2;
        const int nl = local / mp;
        nbl = 2 * nl + q;
        mb = p * mp + (local - nl * mp);
        if (nbl >= args.n_tiles / args.m_tiles) return;
    } else {
        mb = (int)blockIdx.x % args.m_tiles;
        nbl = (int)blockIdx.x / args.m_tiles;
    }
    const ModuleArgs M = args.mod[module_of(args, nbl)];
    const int nb = nbl - M.tile_begin;
    const int m0 = mb * BM;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int T = args.T, d = args.d, G = args.G;
    const int NT = M.n_tiles16;
    const int rt0 = nb * NW * RR + wave * RR;
    const int sgrp = lane >> 4;

    int rtc[RR];
#pragma unroll
    for (int rr = 0; rr < RR; ++rr) rtc[rr] = min(rt0 + rr, NT - 1);
    // code copy: instruction i of wave w fills code rows 16 w + 8 i .. + 7 (1 KB); lane l lands at
    // row 16 w + 8 i + l / 8, position l % 8, holding the row's chunk (l % 8) ^ f(row)
    uint32_t xoff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = 16 * wave + 8 * i + (lane >> 3);
        const int f = (row & 7) ^ ((row >> 3) & 1);
        xoff[i] = (uint32_t)(min(m0 + row, T - 1) * d + 16 * ((lane & 7) ^ f));
    }
    // scale-word copy: lane l fetches the word of row l / 4 of row tile l % 4
    const uint32_t zsrc = (uint32_t)(min(rt0 + (lane & 3), NT - 1) * 64 + (lane >> 2) * 4);
    const int fr = (lane & 7) ^ ((lane >> 3) & 1);  // f of this lane's operand rows (16 tt + lane % 16)
    const int rofs0 = (lane & 15) * 128 + 16 * ((2 * sgrp) ^ fr);
    const int rofs1 = (lane & 15) * 128 + 16 * ((2 * sgrp + 1) ^ fr);

    const uint32_t slane = (wave & 1) * 256 + lane * 4;
    // weight copy i of a wave covers bytes 1024 i .. + 1023 of its RR blocks (lane l: 16 bytes at
    // 1024 i + 16 l, in block (1024 i + 16 l) / QB), each lane's source block clamped on its own
    uint32_t woff[NWI];
#pragma unroll
    for (int i = 0; i < NWI; ++i) {
        const int b = 1024 * i + 16 * lane, rr = b / QB;
        int rt = rtc[0];
#pragma unroll
        for (int k = 1; k < RR; ++k)
            if (rr == k) rt = rtc[k];
        woff[i] = (uint32_t)((rt - rtc[0]) * QB + (b - rr * QB));
    }
    auto copy = [&](int g, uint8_t* stg) {
        const int gg = min(g, G - 1);
        const uint8_t* xb = args.x8 + (size_t)gg * kGroup;
#pragma unroll
        for (int i = 0; i < 2; ++i)
            __builtin_amdgcn_global_load_lds((const void*)(xb + xoff[i]), (lds_void8*)(stg + (16 * wave + 8 * i) * 128),
                                             16, 0, 0);
        const uint8_t* qb = M.q + ((size_t)gg * NT + rtc[0]) * QB;
#pragma unroll
        for (int i = 0; i < NWI; ++i)
            __builtin_amdgcn_global_load_lds((const void*)(qb + woff[i]), (lds_void8*)(stg + W_AT + wave * WW + i * 1024), 16,
                                             0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(M.sz + (size_t)gg * NT * 64 + zsrc),
                                         (lds_void8*)(stg + Z_AT + wave * 256), 4, 0, 0);
        // the activation-scale record (512 bytes): wave w copies half w % 2 (every wave issues the
        // same copies)
        __builtin_amdgcn_global_load_lds((const void*)(args.x8scale + ((size_t)mb * G + gg) * 512 + slane),
                                         (lds_void8*)(stg + S_AT + wave * 256), 4, 0, 0);
    };

    f4 acc[TT][RR];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int rr = 0; rr < RR; ++rr) acc[tt][rr] = f4{0.f, 0.f, 0.f, 0.f};

    // every group issues the same PER copies per wave, so that with three stages the copies of g + 1
    // have landed at the end of group g once at most PER copies (those of g + 2) are in flight
    // (s_waitcnt immediate: vmcnt in bits 3:0, expcnt and lgkmcnt left at their maxima)
    copy(0, st0);
    if constexpr (NST == 3) {
        copy(1, st1);
        __builtin_amdgcn_s_waitcnt(0x0F70 | PER);
    } else {
        __builtin_amdgcn_s_waitcnt(0x0F70);
    }
    __builtin_amdgcn_s_barrier();

    // group g, S = g % NST: its data in stage S (published by the previous barrier).  The copies of
    // g + NST - 1 go to stage S + NST - 1, which every wave finished reading in group g - 1 (its
    // operands fed steps issued before that group's barrier).
    auto step = [&](int g, auto Sc) {
        constexpr int S = decltype(Sc)::value;
        constexpr int SN = (S + NST - 1) % NST;
        uint8_t* cur = S == 0 ? st0 : (S == 1 ? st1 : st2);
        uint8_t* nxt = SN == 0 ? st0 : (SN == 1 ? st1 : st2);
        copy(g + NST - 1, nxt);
        __builtin_amdgcn_sched_barrier(0);
        auto bread = [&](int tt) {
            const u4 b0 = *reinterpret_cast<const u4*>(cur + tt * 16 * 128 + rofs0);
            const u4 b1 = *reinterpret_cast<const u4*>(cur + tt * 16 * 128 + rofs1);
            return i8v{(int32_t)b0[0], (int32_t)b0[1], (int32_t)b0[2], (int32_t)b0[3],
                       (int32_t)b1[0], (int32_t)b1[1], (int32_t)b1[2], (int32_t)b1[3]};
        };
        const u4 zq = *reinterpret_cast<const u4*>(cur + Z_AT + wave * 256 + (lane & 15) * 16);
        const u2 sw = *reinterpret_cast<const u2*>(cur + S_AT + (lane >> 5) * 256 + (lane & 31) * 8);
        i8v a[RR];
        int32_t sa[RR];
#pragma unroll
        for (int rr = 0; rr < RR; ++rr) {
            const uint8_t* wb = cur + W_AT + wave * WW + rr * QB;
            const u4 q = *reinterpret_cast<const u4*>(wb + lane * 16);
            const u2 q6 = SIX ? *reinterpret_cast<const u2*>(wb + 1024 + lane * 8) : u2{0u, 0u};
            a[rr] = WF::operand(q, q6);
            sa[rr] = (int32_t)((zq[rr] >> (8 * sgrp)) & 0xFFu);
        }
        i8v bq[2];
        bq[0] = bread(0);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            if (tt + 1 < TT) bq[(tt + 1) & 1] = bread(tt + 1);
            const int32_t sb = (int32_t)((sw[tt >> 2] >> (8 * (tt & 3))) & 0xFFu);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int rr = 0; rr < RR; ++rr)
                acc[tt][rr] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[rr], bq[tt & 1], acc[tt][rr], WF::cbsz, 0,
                                                                              0, sa[rr], 0, sb);
            __builtin_amdgcn_sched_barrier(0);
        }
        // the copies of g + 1 have landed (three stages: those of g + 2 may stay in flight)
        __builtin_amdgcn_s_waitcnt(NST == 3 ? (0x0F70 | PER) : 0x0F70);
        __builtin_amdgcn_s_barrier();
    };
    int g0 = 0;
    if constexpr (NST == 3) {
        for (; g0 + 3 <= G; g0 += 3) {
            step(g0, ic<0>{});
            step(g0 + 1, ic<1>{});
            step(g0 + 2, ic<2>{});
        }
        if (g0 < G) step(g0, ic<0>{});
        if (g0 + 1 < G) step(g0 + 1, ic<1>{});
    } else {
        for (; g0 + 2 <= G; g0 += 2) {
            step(g0, ic<0>{});
            step(g0 + 1, ic<1>{});
        }
        if (g0 < G) step(g0, ic<0>{});
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no copy may land in LDS after the workgroup ends

    // the correction on the fp16 projection: r_pad / 32 fp16 steps
    if (args.r > 0 && M.a != nullptr) {
        const int r = args.r, rp = args.r_pad;
        const _Float16* R = reinterpret_cast<const _Float16*>(args.R) + (size_t)M.proj * T * rp;
        const h8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
        const int kofs = 8 * (lane >> 4);
        for (int kb = 0; kb < rp / 32; ++kb) {
            const int col = 32 * kb + kofs;
            h8 av[RR];
#pragma unroll
            for (int rr = 0; rr < RR; ++rr) {
                const int row = (rt0 + rr) * 16 + (lane & 15);
                av[rr] = (row < M.n_out && col < r) ? load_h8(M.a + (size_t)row * r + col) : zero8;
            }
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                const int t = m0 + 16 * tt + (lane & 15);
                const h8 bv = t < T ? load_h8(R + (size_t)t * rp + col) : zero8;
#pragma unroll
                for (int rr = 0; rr < RR; ++rr) acc[tt][rr] = mfma16(av[rr], bv, acc[tt][rr]);
            }
        }
    }

    const bool vec = (M.n_out & 3) == 0;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const int t = m0 + 16 * tt + (lane & 15);
        if (t >= T) continue;
        _Float16* yrow = M.y + (size_t)t * M.n_out;
#pragma unroll
        for (int rr = 0; rr < RR; ++rr) {
            if (rt0 + rr >= NT) continue;
            const int row0 = (rt0 + rr) * 16 + 4 * (lane >> 4);
            const f4 v = acc[tt][rr];
            if (vec && row0 + 3 < M.n_out) {
                const h2 lo = {(_Float16)v[0], (_Float16)v[1]}, hi = {(_Float16)v[2], (_Float16)v[3]};
                *reinterpret_cast<u2*>(yrow + row0) = u2{as_u32(lo), as_u32(hi)};
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (row0 + i < M.n_out) yrow[row0 + i] = (_Float16)v[i];
            }
        }
    }
}

hipError_t launch_quant_mx8(const _Float16* x, int T, int d, uint8_t* xq, uint8_t* xs, hipStream_t stream) {
    if (d % kGroup != 0) return hipErrorInvalidValue;
    const int64_t blocks = ((int64_t)T * (d / 32) + kMx8QuantThreads - 1) / kMx8QuantThreads;
    hipLaunchKernelGGL(quant_mx8_kernel, dim3((unsigned)blocks), dim3(kMx8QuantThreads), 0, stream, x, T, d, xq, xs);
    return hipGetLastError();
}

template <int F, int TT, int RR>
static hipError_t launch_mx8_rr(const ForwardArgs& a, hipStream_t stream) {
    const dim3 grid(a.n_tiles);
    switch (a.tile_ks) {
        case 4:
            if constexpr (TT * RR >= 8) return hipErrorInvalidValue;  // not built: register budget
            else hipLaunchKernelGGL((mx8_kernel<F, TT, RR, 4>), grid, dim3(1024), 0, stream, a);
            break;
        case 2: hipLaunchKernelGGL((mx8_kernel<F, TT, RR, 2>), grid, dim3(512), 0, stream, a); break;
        case 1: hipLaunchKernelGGL((mx8_kernel<F, TT, RR, 1>), grid, dim3(256), 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int F, int TT>
static hipError_t launch_mx8_tt(const ForwardArgs& a, hipStream_t stream) {
    if (a.tile_rr == 2) return launch_mx8_rr<F, TT, 2>(a, stream);
    if (a.tile_rr == 1) return launch_mx8_rr<F, TT, 1>(a, stream);
    return hipErrorInvalidValue;
}

template <int F>
static hipError_t launch_mx8_fmt(const ForwardArgs& a, hipStream_t stream) {
    if (a.tile_rr == 8) {  // the wide tile: 128 tokens x 512 rows
        if (a.tile_tt != 8 || a.tile_ks != 1) return hipErrorInvalidValue;
        // token-block quarters x row-block parities over the eight XCDs: 8 x (m / 4) x ceil(n / 2)
        // workgroups, those past the last row block return at once
        const int n = a.n_tiles / a.m_tiles;
        const unsigned grid = (a.m_tiles % 4 == 0) ? 8u * (unsigned)(a.m_tiles / 4) * (unsigned)((n + 1) / 2)
                                                   : (unsigned)a.n_tiles;
        hipLaunchKernelGGL((mx8_wide_kernel<F>), dim3(grid), dim3(64 * kMx8WideWaves), 0, stream, a);
        return hipGetLastError();
    }
    switch (a.tile_tt) {
        case 1: return launch_mx8_tt<F, 1>(a, stream);
        case 2: return launch_mx8_tt<F, 2>(a, stream);
        case 4: return launch_mx8_tt<F, 4>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_mx8(const ForwardArgs& a, hipStream_t stream) {
    switch (a.fmt) {
        case kFmtMxfp4: return launch_mx8_fmt<kFmtMxfp4>(a, stream);
        case kFmtMxfp6E2M3: return launch_mx8_fmt<kFmtMxfp6E2M3>(a, stream);
        case kFmtMxfp6E3M2: return launch_mx8_fmt<kFmtMxfp6E3M2>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace glowq
