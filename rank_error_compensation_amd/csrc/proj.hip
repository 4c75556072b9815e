// The right projection R_p = X B_p^T of the low-rank correction, formed once per call for the
// whole input-sharing group (p = 0, the anchor's B_shared) or once per module for the
// layerwise baseline (GlowQ paper note, key design 4: the anchor materialises R_l = X B^T once
// and the consumers reuse it; motivation: the layerwise form recomputes B_l X per module).
//
// This file holds the prefill form (the decode kernel forms R itself, in its producer
// workgroups): a matrix-core GEMM, tokens as M and rank as N, split over K into ks fp32 partials
// (enough workgroups to fill the chip), then a fixed-order sum rounded once to fp16 for the
// correction step of the prefill GEMM.  Output fp16 [n_proj][T][r_pad], columns r .. r_pad-1
// written as zeros.
#include "glowq_internal.h"

namespace glowq {

__device__ __forceinline__ const _Float16* pick_b(const ProjArgs& p, int i) {
    const _Float16* b = p.b[0];
#pragma unroll
    for (int k = 1; k < kMaxModules; ++k)
        if (k == i) b = p.b[k];
    return b;
}

// Split-K partial projection: workgroup (token block of 64, K split ks, projection p) with 4 waves,
// wave w owning tokens 16w..16w+15 of the block and all r_pad rank columns (NJ tiles of 16).  Four
// K steps of 32 are loaded before they are multiplied.  Output: fp32 partials
// [ks][n_proj][T][r_pad].
template <int NJ>
__global__ __launch_bounds__(256) void proj_partial_kernel(const ProjArgs p) {
    constexpr int S = 4;  // K steps in flight
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int ks = blockIdx.y, pi = blockIdx.z;
    const int T = p.T, d = p.d, r = p.r;
    const int t_lane = blockIdx.x * 64 + wave * 16 + (lane & 15);  // A-operand row
    const int kofs = 8 * (lane >> 4);
    const _Float16* B = pick_b(p, pi);
    const bool t_ok = t_lane < T;
    const _Float16* xr = p.x + (size_t)(t_ok ? t_lane : 0) * d + kofs;
    const _Float16* br[NJ];
    bool j_ok[NJ];
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) {
        const int j = 16 * jt + (lane & 15);
        j_ok[jt] = j < r;
        br[jt] = B + (size_t)(j_ok[jt] ? j : 0) * d + kofs;
    }
    f4 acc[NJ];
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) acc[jt] = f4{0.f, 0.f, 0.f, 0.f};
    const h8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
    const int k0 = ks * p.k_per, k1 = min(k0 + p.k_per, d);
    for (int k = k0; k < k1; k += 32 * S) {
        h8 a[S], b[S][NJ];
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int kk = min(k + 32 * s, k1 - 32);  // steps past the range reload the last (unused)
            a[s] = t_ok ? load_h8(xr + kk) : zero8;
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt) b[s][jt] = j_ok[jt] ? load_h8(br[jt] + kk) : zero8;
        }
#pragma unroll
        for (int s = 0; s < S; ++s) {
            if (k + 32 * s < k1) {
#pragma unroll
                for (int jt = 0; jt < NJ; ++jt) acc[jt] = mfma16(a[s], b[s][jt], acc[jt]);
            }
        }
    }
    float* P = p.part + ((size_t)ks * p.n_proj + pi) * T * p.r_pad;
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) {
        const int j = 16 * jt + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = blockIdx.x * 64 + wave * 16 + 4 * (lane >> 4) + i;
            if (t < T) P[(size_t)t * p.r_pad + j] = acc[jt][i];
        }
    }
}

// Sum of the ks partials in a fixed order (deterministic), rounded once to fp16:
// R [n_proj][T][r_pad].
__global__ __launch_bounds__(256) void proj_reduce_kernel(const ProjArgs p) {
    const size_t n = (size_t)p.n_proj * p.T * p.r_pad / 4;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= n) return;
    const size_t plane = (size_t)p.n_proj * p.T * p.r_pad / 4;
    const f4* P = reinterpret_cast<const f4*>(p.part);
    f4 s = P[idx];
    for (int k = 1; k < p.ks; ++k) s += P[(size_t)k * plane + idx];
    const h2 lo = {(_Float16)s[0], (_Float16)s[1]}, hi = {(_Float16)s[2], (_Float16)s[3]};
    reinterpret_cast<u2*>(p.R)[idx] = u2{as_u32(lo), as_u32(hi)};
}

hipError_t launch_proj_prefill(const ProjArgs& p, hipStream_t stream) {
    const dim3 grid((unsigned)ceil_div(p.T, 64), (unsigned)p.ks, (unsigned)p.n_proj);
    switch (p.r_pad / 16) {
        case 2: hipLaunchKernelGGL((proj_partial_kernel<2>), grid, dim3(256), 0, stream, p); break;
        case 4: hipLaunchKernelGGL((proj_partial_kernel<4>), grid, dim3(256), 0, stream, p); break;
        case 6: hipLaunchKernelGGL((proj_partial_kernel<6>), grid, dim3(256), 0, stream, p); break;
        case 8: hipLaunchKernelGGL((proj_partial_kernel<8>), grid, dim3(256), 0, stream, p); break;
        case 10: hipLaunchKernelGGL((proj_partial_kernel<10>), grid, dim3(256), 0, stream, p); break;
        case 12: hipLaunchKernelGGL((proj_partial_kernel<12>), grid, dim3(256), 0, stream, p); break;
        case 14: hipLaunchKernelGGL((proj_partial_kernel<14>), grid, dim3(256), 0, stream, p); break;
        case 16: hipLaunchKernelGGL((proj_partial_kernel<16>), grid, dim3(256), 0, stream, p); break;
        default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t n = (size_t)p.n_proj * p.T * p.r_pad / 4;
    hipLaunchKernelGGL(proj_reduce_kernel, dim3((unsigned)ceil_div((int64_t)n, 256)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace glowq
