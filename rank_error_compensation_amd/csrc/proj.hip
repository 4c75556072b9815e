// The right projection R_p = X B_p^T of the low-rank correction, formed once per call for the
// whole input-sharing group (p = 0, the anchor's B_shared) or once per module for the
// layerwise baseline (GlowQ paper note, key design 4: the anchor materialises R_l = X B^T once
// and the consumers reuse it; motivation: the layerwise form recomputes B_l X per module).
//
// This file holds the prefill form (the decode kernel forms R itself, in its producer
// workgroups): a matrix-core GEMM, tokens as M and rank as N, split over K into ks ranges when
// the token blocks alone would leave the chip idle (fp32 partials, then a fixed-order sum), and
// rounded once to fp16 for the correction step of the prefill GEMM.  Output fp16
// [n_proj][T][r_pad], columns r .. r_pad-1 written as zeros.
#include "glowq_internal.h"

namespace glowq {

__device__ __forceinline__ const _Float16* pick_b(const ProjArgs& p, int i) {
    const _Float16* b = p.b[0];
#pragma unroll
    for (int k = 1; k < kMaxModules; ++k)
        if (k == i) b = p.b[k];
    return b;
}

// Projection of one block of 16 TT tokens over one K range (split ks of the launch) for
// projection p: the four waves take interleaved 32-input steps of the range (wave w: steps
// w, w + 4, ...), each holding all r_pad rank columns (NJ tiles of 16) for the block's TT token
// tiles, four steps of loads in flight; the four partial sums are added through LDS in wave
// order.  With one K range the block's R rows are rounded to fp16 here; otherwise they go to the
// fp32 partials [ks][n_proj][T][r_pad] for proj_reduce_kernel.
template <int NJ, int TT>
__global__ __launch_bounds__(256) void proj_kernel(const ProjArgs p) {
    constexpr int S = 4;
    __shared__ f4 red[3][TT * NJ][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ks = blockIdx.y, pi = blockIdx.z;
    const int T = p.T, d = p.d, r = p.r;
    const int kofs = 8 * (lane >> 4);
    const int t0 = blockIdx.x * 16 * TT;
    const _Float16* B = pick_b(p, pi);
    const _Float16* xr[TT];
    bool t_ok[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const int t = t0 + 16 * tt + (lane & 15);
        t_ok[tt] = t < T;
        xr[tt] = p.x + (size_t)(t_ok[tt] ? t : 0) * d + kofs;
    }
    const _Float16* br[NJ];
    bool j_ok[NJ];
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) {
        const int j = 16 * jt + (lane & 15);
        j_ok[jt] = j < r;
        br[jt] = B + (size_t)(j_ok[jt] ? j : 0) * d + kofs;
    }
    f4 acc[TT][NJ];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) acc[tt][jt] = f4{0.f, 0.f, 0.f, 0.f};
    const h8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
    const int kb = ks * p.k_per;
    const int n = (min(kb + p.k_per, d) - kb) / 128;  // steps of this wave (k_per, d multiples of 128)
    const int k0 = kb + 32 * wave;
    for (int c = 0; c < n; c += S) {
        h8 a[S][TT], b[S][NJ];
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int kk = k0 + 128 * min(c + s, n - 1);  // steps past the range reload the last (unused)
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) a[s][tt] = t_ok[tt] ? load_h8(xr[tt] + kk) : zero8;
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt) b[s][jt] = j_ok[jt] ? load_h8(br[jt] + kk) : zero8;
        }
#pragma unroll
        for (int s = 0; s < S; ++s) {
            if (c + s < n) {
#pragma unroll
                for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                    for (int jt = 0; jt < NJ; ++jt) acc[tt][jt] = mfma16(a[s][tt], b[s][jt], acc[tt][jt]);
            }
        }
    }
    if (wave > 0) {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt) red[wave - 1][tt * NJ + jt][lane] = acc[tt][jt];
    }
    __syncthreads();
    if (wave != 0) return;
    const bool direct = p.ks == 1;
    _Float16* Rh = static_cast<_Float16*>(p.R) + (size_t)pi * T * p.r_pad;
    float* P = p.part + ((size_t)ks * p.n_proj + pi) * T * p.r_pad;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) {
            f4 v = acc[tt][jt];
#pragma unroll
            for (int w = 0; w < 3; ++w) v += red[w][tt * NJ + jt][lane];
            const int j = 16 * jt + (lane & 15);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = t0 + 16 * tt + 4 * (lane >> 4) + i;
                if (t >= T) continue;
                if (direct)
                    Rh[(size_t)t * p.r_pad + j] = (_Float16)v[i];
                else
                    P[(size_t)t * p.r_pad + j] = v[i];
            }
        }
    }
}

// Sum of the ks partials in a fixed order (deterministic), rounded once to fp16:
// R [n_proj][T][r_pad].  All ks loads are issued before the adds.
__global__ __launch_bounds__(256) void proj_reduce_kernel(const ProjArgs p) {
    const size_t n = (size_t)p.n_proj * p.T * p.r_pad / 4;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= n) return;
    const f4* P = reinterpret_cast<const f4*>(p.part);
    f4 v[kProjMaxSplit];
#pragma unroll
    for (int k = 0; k < kProjMaxSplit; ++k) v[k] = k < p.ks ? P[(size_t)k * n + idx] : f4{0.f, 0.f, 0.f, 0.f};
    f4 s = v[0];
#pragma unroll
    for (int k = 1; k < kProjMaxSplit; ++k)
        if (k < p.ks) s += v[k];
    const h2 lo = {(_Float16)s[0], (_Float16)s[1]}, hi = {(_Float16)s[2], (_Float16)s[3]};
    reinterpret_cast<u2*>(p.R)[idx] = u2{as_u32(lo), as_u32(hi)};
}

template <int NJ>
void launch_proj_nj(const ProjArgs& p, dim3 grid, hipStream_t stream) {
    if (p.tok_tiles == 2)
        hipLaunchKernelGGL((proj_kernel<NJ, NJ <= 8 ? 2 : 1>), grid, dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL((proj_kernel<NJ, 1>), grid, dim3(256), 0, stream, p);
}

hipError_t launch_proj_prefill(const ProjArgs& p, hipStream_t stream) {
    // two token tiles per workgroup only where the kernel is built with them
    if (p.tok_tiles != 1 && !(p.tok_tiles == 2 && p.r_pad <= 128)) return hipErrorInvalidValue;
    if (p.ks < 1 || p.ks > kProjMaxSplit) return hipErrorInvalidValue;
    const dim3 grid((unsigned)ceil_div(p.T, 16 * p.tok_tiles), (unsigned)p.ks, (unsigned)p.n_proj);
    switch (p.r_pad / 16) {
        case 2: launch_proj_nj<2>(p, grid, stream); break;
        case 4: launch_proj_nj<4>(p, grid, stream); break;
        case 6: launch_proj_nj<6>(p, grid, stream); break;
        case 8: launch_proj_nj<8>(p, grid, stream); break;
        case 10: launch_proj_nj<10>(p, grid, stream); break;
        case 12: launch_proj_nj<12>(p, grid, stream); break;
        case 14: launch_proj_nj<14>(p, grid, stream); break;
        case 16: launch_proj_nj<16>(p, grid, stream); break;
        default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.ks == 1) return e;
    const size_t n = (size_t)p.n_proj * p.T * p.r_pad / 4;
    hipLaunchKernelGGL(proj_reduce_kernel, dim3((unsigned)ceil_div((int64_t)n, 256)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace glowq
