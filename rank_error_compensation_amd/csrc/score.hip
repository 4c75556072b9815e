// GlowQ-S restore selection on the GPU (GlowQ paper note, key design 4: units are ranked by an
// importance score and only the top k are restored; one of the two scores is the normalised error
// ratio g_ner(u) = ||E_u||_F^2 / ||W_u||_F^2 with E = W - W_hat; the arXiv page, Figure 12, sorts
// restorable groups by this ratio among other metrics).
//
//   * ner_partial_kernel: one launch for a batch of up to kNerBatch modules, one workgroup per
//     16-row tile of each module (module found from a prefix table); the four waves take the
//     input groups g = w, w + 4, ... (four groups of loads in flight per wave), read the fp16
//     weight W and the packed INT4 weight in its device layout, rebuild W_hat = (q - z) s exactly
//     (the same in-register unpacking as the forward kernels, then one exact fp32 product) and
//     accumulate (W - W_hat)^2 and W^2 in fp64 -- the difference of an fp16 and a 22-bit value is
//     exact in fp64, and so is its square (at most 2 x 25 significant bits); the lanes and waves
//     are summed in a fixed order.
//   * ner_finish_kernel: one workgroup per module adds its per-tile partial sums in a fixed order.
//   * topk_kernel: one workgroup forms each unit's score sum_m err / sum_m w over its modules
//     (0 when sum_m w is 0) and restores the k best units, equal scores going to the lower unit
//     index (the order in which the pages fall back to layer order).
// Everything HBM-bound: per weight element 2 bytes of W, half a byte of q, 4/128 of (z, s).
#include "glowq_offline.h"

namespace glowq {

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Module of work tile `tile` in a batch (uniform across the workgroup).
__device__ __forceinline__ int ner_module_of(const NerBatch& a, int tile) {
    int i = 0;
#pragma unroll
    for (int k = 1; k < kNerBatch; ++k) i += (k < a.n_mod && tile >= a.tile_begin[k]) ? 1 : 0;
    return __builtin_amdgcn_readfirstlane(i);
}

__global__ __launch_bounds__(256) void ner_partial_kernel(const NerBatch a) {
    constexpr int U = 4;  // groups of loads in flight per wave
    __shared__ double red[4][2];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tile = blockIdx.x;
    const int mi = ner_module_of(a, tile);
    const int rt = tile - a.tile_begin[mi];
    const int n_out = a.n_out[mi], k_in = a.k_in[mi], G = k_in / kGroup, NT = (n_out + 15) / 16;
    const uint8_t* q = a.q[mi];
    const uint8_t* sz = a.sz[mi];
    const int row = rt * 16 + (lane & 15);
    const bool ok = row < n_out;
    const NibConsts nc = nib_consts();
    const _Float16* wr = a.w[mi] + (size_t)(ok ? row : 0) * k_in + 8 * (lane >> 4);
    const u4 zero4 = {0u, 0u, 0u, 0u};
    const h8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
    double e2 = 0.0, w2 = 0.0;
    for (int g0 = wave; g0 < G; g0 += 4 * U) {
        u4 qv[U];
        uint32_t zs[U];
        h8 wv[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int g = g0 + 4 * u;
            const bool live = g < G;
            const size_t blk = (size_t)(live ? g : 0) * NT + rt;
            qv[u] = live ? *reinterpret_cast<const u4*>(q + blk * 1024 + lane * 16) : zero4;
            zs[u] = live ? *reinterpret_cast<const uint32_t*>(sz + blk * 64 + (lane & 15) * 4) : 0u;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                wv[u][j] = (live && ok) ? load_h8(wr + (size_t)g * kGroup + 32 * j) : zero8;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (!(g0 + 4 * u < G) || !ok) continue;
            h2 c1024, c64;
            zero_consts(zs[u], c1024, c64);
            const float sc = (float)as_h2(zs[u])[1];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const h8 qz = nib8_minus_z(qv[u][j], c1024, c64, nc);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const double wd = (double)(float)wv[u][j][e];
                    const double de = wd - (double)((float)qz[e] * sc);
                    e2 = fma(de, de, e2);
                    w2 = fma(wd, wd, w2);
                }
            }
        }
    }
    e2 = wave_sum(e2);
    w2 = wave_sum(w2);
    if (lane == 0) {
        red[wave][0] = e2;
        red[wave][1] = w2;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        a.part[2 * tile] = ((red[0][0] + red[1][0]) + red[2][0]) + red[3][0];
        a.part[2 * tile + 1] = ((red[0][1] + red[1][1]) + red[2][1]) + red[3][1];
    }
}

// Workgroup m: the partial sums of module m's tiles, in a fixed order.
__global__ __launch_bounds__(256) void ner_finish_kernel(const NerBatch a) {
    __shared__ double red[2][256];
    const int m = blockIdx.x;
    double e2 = 0.0, w2 = 0.0;
    for (int i = a.tile_begin[m] + threadIdx.x; i < a.tile_begin[m + 1]; i += 256) {
        e2 += a.part[2 * i];
        w2 += a.part[2 * i + 1];
    }
    red[0][threadIdx.x] = e2;
    red[1][threadIdx.x] = w2;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h) {
            red[0][threadIdx.x] += red[0][threadIdx.x + h];
            red[1][threadIdx.x] += red[1][threadIdx.x + h];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        a.sums[2 * m] = red[0][0];
        a.sums[2 * m + 1] = red[1][0];
    }
}

struct TopkArgs {
    const double* sums;  // [n_units][n_per][2]
    int32_t n_units, n_per, k;
    double rel_tol;      // 0: exact ranking; > 0: steps of rel_tol times the best score
    double* scores;      // [n_units]
    int32_t* mask;       // [n_units]
};

// With rel_tol > 0 a unit's key is floor((max - score) / (rel_tol max)), fp64, and units with equal
// keys go in layer order (the fallback of key design 4 when the signal is weak: all scores within
// one step of the best restore the first k units).
__global__ __launch_bounds__(256) void topk_kernel(const TopkArgs a) {
    __shared__ double sc[kMaxScoreUnits];
    __shared__ double red[256];
    for (int u = threadIdx.x; u < a.n_units; u += 256) {
        double e2 = 0.0, w2 = 0.0;
        for (int m = 0; m < a.n_per; ++m) {
            e2 += a.sums[((size_t)u * a.n_per + m) * 2];
            w2 += a.sums[((size_t)u * a.n_per + m) * 2 + 1];
        }
        const double s = w2 > 0.0 ? e2 / w2 : 0.0;
        sc[u] = s;
        a.scores[u] = s;
    }
    __syncthreads();
    if (a.rel_tol > 0.0) {
        double m = 0.0;
        for (int u = threadIdx.x; u < a.n_units; u += 256) m = fmax(m, sc[u]);
        red[threadIdx.x] = m;
        __syncthreads();
        if (threadIdx.x == 0) {
            double mx = red[0];
            for (int t = 1; t < 256; ++t) mx = fmax(mx, red[t]);
            red[0] = mx;
        }
        __syncthreads();
        const double mx = red[0];
        __syncthreads();
        if (mx > 0.0) {
            const double step = a.rel_tol * mx;
            for (int u = threadIdx.x; u < a.n_units; u += 256) sc[u] = -floor((mx - sc[u]) / step);  // higher is better
            __syncthreads();
        }
    }
    for (int u = threadIdx.x; u < a.n_units; u += 256) {
        const double su = sc[u];
        int rank = 0;
        for (int v = 0; v < a.n_units; ++v) rank += (sc[v] > su || (sc[v] == su && v < u)) ? 1 : 0;
        a.mask[u] = rank < a.k ? 1 : 0;
    }
}

// The other score, g_ec(u): the share of a unit's whitened error energy that its best rank r
// captures, sum_{j <= r} sigma_j^2 / ||E_cat L||_F^2 (GlowQ paper note, key design 4; the
// singular values are those of the whitened error, e.g. from the factor solve).  With
// C = E_cat^T E_cat (lower triangle, from the fp64 GEMM) the energy is
// ||E_cat L||_F^2 = trace(E_cat Sigma_x E_cat^T) = sum_ij Sigma_ij C_ij, whichever square root L
// of Sigma_x whitens.
//   * ec_rows_kernel: workgroup i adds Sigma_ij C_ij over j < i, doubles it (the mirror terms)
//     and adds the diagonal term, lanes and waves in a fixed order.
//   * ec_finish_kernel: one workgroup adds the rows in a fixed order, then the r squared singular
//     values in order, and forms the ratio (0 for a zero error).
__global__ __launch_bounds__(256) void ec_rows_kernel(const double* C, const double* sigma, int d, double* part) {
    __shared__ double red[256];
    const int i = blockIdx.x;
    const double* c = C + (size_t)i * d;
    const double* sg = sigma + (size_t)i * d;
    double v = 0.0;
    for (int j = threadIdx.x; j < i; j += 256) v = fma(sg[j], c[j], v);
    red[threadIdx.x] = v;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
        __syncthreads();
    }
    if (threadIdx.x == 0) part[i] = 2.0 * red[0] + sg[i] * c[i];
}

__global__ __launch_bounds__(256) void ec_finish_kernel(const double* part, int d, const double* sv, int r,
                                                        double* out) {
    __shared__ double red[256];
    double v = 0.0;
    for (int i = threadIdx.x; i < d; i += 256) v += part[i];
    red[threadIdx.x] = v;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        const double energy = red[0];
        double cap = 0.0;
        for (int j = 0; j < r; ++j) cap = fma(sv[j], sv[j], cap);
        out[0] = energy;
        out[1] = cap;
        out[2] = energy > 0.0 ? cap / energy : 0.0;
    }
}

hipError_t launch_ec(const double* C, const double* sigma, int d, const double* sv, int r, double* part,
                     double* out, hipStream_t stream) {
    hipLaunchKernelGGL(ec_rows_kernel, dim3((unsigned)d), dim3(256), 0, stream, C, sigma, d, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(ec_finish_kernel, dim3(1), dim3(256), 0, stream, part, d, sv, r, out);
    return hipGetLastError();
}

hipError_t launch_ner(const NerBatch& a, hipStream_t stream) {
    hipLaunchKernelGGL(ner_partial_kernel, dim3((unsigned)a.tile_begin[a.n_mod]), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(ner_finish_kernel, dim3((unsigned)a.n_mod), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_topk(const double* sums, int32_t n_units, int32_t n_per, int32_t k, double rel_tol, double* scores,
                       int32_t* mask, hipStream_t stream) {
    TopkArgs a;
    a.sums = sums;
    a.n_units = n_units;
    a.n_per = n_per;
    a.k = k;
    a.rel_tol = rel_tol;
    a.scores = scores;
    a.mask = mask;
    hipLaunchKernelGGL(topk_kernel, dim3(1), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace glowq
