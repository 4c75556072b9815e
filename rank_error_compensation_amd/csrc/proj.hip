// The right projection R_p = X B_p^T of the low-rank correction, formed once per call for the
// whole input-sharing group (p = 0, the anchor's B_shared) or once per module for the
// layerwise baseline (GlowQ paper note, key design 4: the anchor materialises R_l = X B^T once
// and the consumers reuse it; motivation: the layerwise form recomputes B_l X per module).
//
// This file holds the prefill form (the decode kernel forms R itself, in its producer
// workgroups): a matrix-core GEMM, tokens as M and rank as N, fp32 accumulation, rounded once to fp16
//   for the correction step of the prefill GEMM.  Output fp16 [n_proj][T][r_pad], columns
//   r .. r_pad-1 written as zeros.
#include "glowq_internal.h"

namespace glowq {

__device__ __forceinline__ const _Float16* pick_b(const ProjArgs& p, int i) {
    const _Float16* b = p.b[0];
#pragma unroll
    for (int k = 1; k < kMaxModules; ++k)
        if (k == i) b = p.b[k];
    return b;
}

// prefill: workgroup = 4 waves, 64 tokens x 64 rank columns; wave w owns tokens 16w..16w+15.
__global__ __launch_bounds__(256) void proj_prefill_kernel(const ProjArgs p) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int pi = blockIdx.z;
    const int T = p.T, d = p.d, r = p.r;
    const int t_lane = blockIdx.x * 64 + wave * 16 + (lane & 15);  // A-operand row
    const int j0 = blockIdx.y * 64;
    const int kofs = 8 * (lane >> 4);
    const _Float16* B = pick_b(p, pi);
    const bool t_ok = t_lane < T;
    const _Float16* xr = p.x + (size_t)(t_ok ? t_lane : 0) * d + kofs;
    const _Float16* br[4];
    bool j_ok[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
        const int j = j0 + 16 * jt + (lane & 15);
        j_ok[jt] = j < r;
        br[jt] = B + (size_t)(j_ok[jt] ? j : 0) * d + kofs;
    }
    f4 acc[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) acc[jt] = f4{0.f, 0.f, 0.f, 0.f};
    const h8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int k = 0; k < d; k += 32) {
        const h8 a = t_ok ? load_h8(xr + k) : zero8;
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            const h8 b = j_ok[jt] ? load_h8(br[jt] + k) : zero8;
            acc[jt] = mfma16(a, b, acc[jt]);
        }
    }
    _Float16* R = reinterpret_cast<_Float16*>(p.R) + (size_t)pi * T * p.r_pad;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
        const int j = j0 + 16 * jt + (lane & 15);
        if (j >= p.r_pad) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = blockIdx.x * 64 + wave * 16 + 4 * (lane >> 4) + i;
            if (t < T) R[(size_t)t * p.r_pad + j] = (_Float16)acc[jt][i];
        }
    }
}

hipError_t launch_proj_prefill(const ProjArgs& p, hipStream_t stream) {
    const dim3 grid((unsigned)ceil_div(p.T, 64), (unsigned)ceil_div(p.r_pad, 64), p.n_proj);
    hipLaunchKernelGGL(proj_prefill_kernel, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace glowq
