// Prefill path (T > 64 tokens): the group's quantised product is a dense contraction, run on the
// gfx950 matrix cores with the INT4 weights dequantised in registers, and the low-rank correction
// appended as a short extra K range: y_i = [X | R] [W_hat_i | A_i]^T (GlowQ paper note, key design
// 4: R is materialised once per group and consumed by every module).
//
// Workgroup tile: BM = 16 TT tokens x BN = 64 RR rows, four wavefronts side by side in N (wave w
// owns RR row tiles of 16 rows and all BM tokens).  Per 128-input group:
//   * the X tile (BM x 128 fp16) is staged in LDS (double-buffered, one barrier per group; the
//     next group's global loads are in flight while the current one is multiplied);
//   * each wave loads its RR weight blocks straight from HBM in operand order (one 16-byte load
//     per lane per row tile), turns nibbles into exact fp16 (q - z) and scales them by the
//     row's fp16 scale (one round-to-nearest), and feeds v_mfma_f32_16x16x32_f16 with the X
//     operand read from LDS; every dequantised operand is reused across TT token tiles.
// After the d loop, r_pad / 32 more matrix-core steps multiply A_i (fp16, from HBM) by the
// group's R (fp16, from the workspace).  fp32 accumulation throughout; one rounding to fp16.
//
// Workgroups are numbered XCD-aware: consecutive logical tiles (same weight block, successive
// token blocks) land on the same XCD and share its L2.
#include "glowq_internal.h"

namespace glowq {

// Physical workgroup id -> logical tile id such that XCD x (workgroups b with b % 8 == x)
// receives a contiguous range of logical tiles.
__device__ __forceinline__ int xcd_remap(int b, int n) {
    const int xcd = b & 7, local = b >> 3;
    const int per = n >> 3, rem = n & 7;
    return xcd * per + (xcd < rem ? xcd : rem) + local;
}

template <int TT, int RR>
__global__ __launch_bounds__(256, 2) void prefill_kernel(const ForwardArgs args) {
    constexpr int BM = 16 * TT;
    constexpr int LS = 136;              // LDS row stride in halves (128 + 8 padding)
    constexpr int NCH = BM * 16 / 256;   // 16-byte X chunks per thread per group
    __shared__ __attribute__((aligned(16))) _Float16 xs[2][BM * LS];

    const int L = xcd_remap(blockIdx.x, args.n_tiles);
    const int mb = L % args.m_tiles, nbl = L / args.m_tiles;
    const ModuleArgs M = args.mod[module_of(args, nbl)];
    const int nb = nbl - M.tile_begin;
    const int m0 = mb * BM;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int T = args.T, d = args.d, G = args.G;
    const NibConsts nc = nib_consts();
    const int kofs = 8 * (lane >> 4);
    const int rt0 = nb * 4 * RR + wave * RR;
    const size_t qstride = (size_t)M.n_tiles16 * 1024, szstride = (size_t)M.n_tiles16 * 64;  // per group

    const uint8_t* qp[RR];
    const uint8_t* zp[RR];
    bool w_ok[RR];
#pragma unroll
    for (int rr = 0; rr < RR; ++rr) {
        const int rt = rt0 + rr;
        w_ok[rr] = rt < M.n_tiles16;
        qp[rr] = M.q + (size_t)(w_ok[rr] ? rt : 0) * 1024 + lane * 16;
        zp[rr] = M.sz + (size_t)(w_ok[rr] ? rt : 0) * 64 + (lane & 15) * 4;
    }
    const _Float16* xsrc[NCH];
    bool x_ok[NCH];
    int xdst[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int idx = c * 256 + tid;
        const int row = idx >> 4, col = (idx & 15) * 8;
        const int t = m0 + row;
        x_ok[c] = t < T;
        xsrc[c] = args.x + (size_t)(x_ok[c] ? t : 0) * d + col;
        xdst[c] = row * LS + col;
    }
    const u4 zero4 = {0u, 0u, 0u, 0u};

    u4 st[NCH];
    u4 qv[RR];
    uint32_t zs[RR];
#pragma unroll
    for (int c = 0; c < NCH; ++c) st[c] = x_ok[c] ? *reinterpret_cast<const u4*>(xsrc[c]) : zero4;
#pragma unroll
    for (int rr = 0; rr < RR; ++rr) {
        qv[rr] = w_ok[rr] ? *reinterpret_cast<const u4*>(qp[rr]) : zero4;
        zs[rr] = w_ok[rr] ? *reinterpret_cast<const uint32_t*>(zp[rr]) : 0u;
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c) *reinterpret_cast<u4*>(&xs[0][xdst[c]]) = st[c];
    __syncthreads();

    f4 acc[TT][RR];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int rr = 0; rr < RR; ++rr) acc[tt][rr] = f4{0.f, 0.f, 0.f, 0.f};

    for (int g = 0; g < G; ++g) {
        const int buf = g & 1;
        const bool more = g + 1 < G;
        u4 qn[RR];
        uint32_t zn[RR];
        if (more) {
#pragma unroll
            for (int c = 0; c < NCH; ++c)
                st[c] = x_ok[c] ? *reinterpret_cast<const u4*>(xsrc[c] + (size_t)(g + 1) * kGroup) : zero4;
#pragma unroll
            for (int rr = 0; rr < RR; ++rr) {
                qn[rr] = w_ok[rr] ? *reinterpret_cast<const u4*>(qp[rr] + (size_t)(g + 1) * qstride) : zero4;
                zn[rr] = w_ok[rr] ? *reinterpret_cast<const uint32_t*>(zp[rr] + (size_t)(g + 1) * szstride) : 0u;
            }
        }
        h2 c1024[RR], c64[RR];
        h8 s8[RR];
#pragma unroll
        for (int rr = 0; rr < RR; ++rr) {
            zero_consts(zs[rr], c1024[rr], c64[rr]);
            const _Float16 s = as_h2(zs[rr])[1];
            s8[rr] = h8{s, s, s, s, s, s, s, s};
        }
        const _Float16* xb = &xs[buf][(lane & 15) * LS + kofs];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            h8 a[RR];
#pragma unroll
            for (int rr = 0; rr < RR; ++rr) a[rr] = nib8_minus_z(qv[rr][j], c1024[rr], c64[rr], nc) * s8[rr];
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                const h8 b = *reinterpret_cast<const h8*>(xb + tt * 16 * LS + 32 * j);
#pragma unroll
                for (int rr = 0; rr < RR; ++rr) acc[tt][rr] = mfma16(a[rr], b, acc[tt][rr]);
            }
        }
        if (more) {
#pragma unroll
            for (int c = 0; c < NCH; ++c) *reinterpret_cast<u4*>(&xs[buf ^ 1][xdst[c]]) = st[c];
#pragma unroll
            for (int rr = 0; rr < RR; ++rr) {
                qv[rr] = qn[rr];
                zs[rr] = zn[rr];
            }
        }
        __syncthreads();
    }

    // correction: r_pad / 32 more K steps, A-operand A_i rows, B-operand R tokens
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
                const int t = m0 + 16 * tt + (lane & 15);
                const h8 b = t < T ? load_h8(R + (size_t)t * rp + col) : zero8;
#pragma unroll
                for (int rr = 0; rr < RR; ++rr) acc[tt][rr] = mfma16(a[rr], b, acc[tt][rr]);
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

hipError_t launch_prefill(const ForwardArgs& a, hipStream_t stream) {
    const dim3 grid(a.n_tiles), block(256);
    if (a.tile_tt == 4 && a.tile_rr == 4)
        hipLaunchKernelGGL((prefill_kernel<4, 4>), grid, block, 0, stream, a);
    else if (a.tile_tt == 8 && a.tile_rr == 2)
        hipLaunchKernelGGL((prefill_kernel<8, 2>), grid, block, 0, stream, a);
    else if (a.tile_tt == 4 && a.tile_rr == 2)
        hipLaunchKernelGGL((prefill_kernel<4, 2>), grid, block, 0, stream, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace glowq
