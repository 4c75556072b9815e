// The right projection R_p = X B_p^T of the low-rank correction, formed once per call for the
// whole input-sharing group (p = 0, the anchor's B_shared) or once per module for the
// layerwise baseline (GlowQ paper note, key design 4: the anchor materialises R_l = X B^T once
// and the consumers reuse it; motivation: the layerwise form recomputes B_l X per module).
//
// decode (T <= 64): one workgroup per (row j of B, projection p); every thread dots 8-input
//   slices of B_p[j] with the tokens in fp32 (products of fp16 are exact in fp32), then a
//   fixed-order block reduction.  Output fp32 [n_proj][T][r].
// prefill: matrix-core GEMM, tokens as M and rank as N, fp32 accumulation, rounded once to fp16
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

__global__ __launch_bounds__(256) void proj_decode_kernel(const ProjArgs p) {
    __shared__ float part[4][16];
    const int j = blockIdx.x, pi = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int T = p.T, d = p.d;
    const _Float16* brow = pick_b(p, pi) + (size_t)j * d;
    float* R = reinterpret_cast<float*>(p.R) + (size_t)pi * T * p.r;
    for (int t0 = 0; t0 < T; t0 += 16) {
        float acc[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) acc[t] = 0.f;
        for (int c = threadIdx.x; c < d / 8; c += 256) {
            const h8 bv = load_h8(brow + 8 * c);
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                if (t0 + t < T) {
                    const h8 xv = load_h8(p.x + (size_t)(t0 + t) * d + 8 * c);
                    float s = acc[t];
#pragma unroll
                    for (int e = 0; e < 8; ++e) s = fmaf((float)bv[e], (float)xv[e], s);
                    acc[t] = s;
                }
            }
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            float v = acc[t];
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
            acc[t] = v;
        }
        if (lane == 0) {
#pragma unroll
            for (int t = 0; t < 16; ++t) part[wave][t] = acc[t];
        }
        __syncthreads();
        if (threadIdx.x < 16 && t0 + (int)threadIdx.x < T) {
            const int t = threadIdx.x;
            R[(size_t)(t0 + t) * p.r + j] = ((part[0][t] + part[1][t]) + part[2][t]) + part[3][t];
        }
        __syncthreads();
    }
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

hipError_t launch_proj_decode(const ProjArgs& p, hipStream_t stream) {
    hipLaunchKernelGGL(proj_decode_kernel, dim3(p.r, p.n_proj), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_proj_prefill(const ProjArgs& p, hipStream_t stream) {
    const dim3 grid((unsigned)ceil_div(p.T, 64), (unsigned)ceil_div(p.r_pad, 64), p.n_proj);
    hipLaunchKernelGGL(proj_prefill_kernel, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace glowq
