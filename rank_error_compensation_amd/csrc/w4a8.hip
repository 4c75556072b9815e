// W4A8 form of the group forward: INT4-g128 weights against per-token 8-bit activations on the
// gfx950 int8 matrix cores, with the low-rank correction kept on the fp16 activations (the
// W4A8 rows of the GlowQ arXiv page, Tables 14 and 15; the paper note's results bullets).
//
//   codes, scale_t = per-token symmetric int8 quantisation of X (round half to even, -127..127,
//                    scale = max_k |x[t, k]| / 127, fp32)
//   y_i[t, o]      = scale_t sum_g s[o, g] (sum_{k in g} q[o, k] code[t, k] - z[o, g] csum[t, g])
//                    + R[t] . A_i[o],   R = X B^T from the fp16 X, formed once per call
// with csum[t, g] the sum of token t's codes over group g: sum_k (q - z) code splits into the
// nibble product, which fits the signed 8-bit operands (q <= 15), and one integer correction per
// (row, group, token).  Every group's integer sum is exact in int32; it is scaled in fp32.
//
// Activation code layout (internal, in the workspace): per token and 128-input group, position
// 16 (4 m + g) + 8 h + b holds the code of input 64 m + 32 h + 8 g + p[b], p = {0, 4, 1, 5, 2, 6,
// 3, 7}.  That is byte b of lane group g of the int8 operand of matrix-core step m (of two per
// group) exactly where the weight operand has the same input: the device weight layout keeps
// inputs 32 j + 8 g + e of a lane in word j with nibble slot p holding e = 2 p (p < 4) or
// 2 (p - 4) + 1, so (w & 0x0F0F0F0F) yields the inputs e = 0, 4, 1, 5 as bytes and
// ((w >> 4) & 0x0F0F0F0F) the inputs 2, 6, 3, 7; words 2 m and 2 m + 1 make the 16 operand bytes
// of step m.  One 16-byte read per lane then feeds each step.
#include "glowq_internal.h"

namespace glowq {

typedef int32_t i4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i4v mfma_i8(i4v a, i4v b, i4v c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// One workgroup per token: the row's largest magnitude, the scale, the codes in the layout above
// (one 8-byte chunk of positions per thread and step), and the per-group code sums.
constexpr int kQuantThreads = 256;
constexpr int kQuantChunks = 8;  // 8-input chunks per thread: d <= 8 * 8 * 256 = 16384

__global__ __launch_bounds__(kQuantThreads) void quant_x_kernel(const _Float16* __restrict__ x, int d,
                                                              int8_t* __restrict__ xq, int32_t* __restrict__ xsum,
                                                              float* __restrict__ xscale) {
    __shared__ float red[kQuantThreads / 64];
    const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n8 = d / 8;  // chunks of the row
    const _Float16* row = x + (size_t)t * d;
    h8 v[kQuantChunks];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < kQuantChunks; ++i) {
        const int c = tid + kQuantThreads * i;  // position chunk: m = c / 8 in its group ...
        if (c < n8) {
            const int grp = c >> 4, cc = c & 15;
            const int m = cc >> 3, g = (cc >> 1) & 3, h = cc & 1;
            const int k0 = grp * kGroup + 64 * m + 32 * h + 8 * g;  // natural inputs k0 .. k0 + 7
            v[i] = load_h8(row + k0);
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)v[i][e]));
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    if (lane == 0) red[wave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float scale = amax / 127.0f;  // IEEE division (correctly rounded)
    if (tid == 0) xscale[t] = scale;
    constexpr int perm[8] = {0, 4, 1, 5, 2, 6, 3, 7};
#pragma unroll
    for (int i = 0; i < kQuantChunks; ++i) {
        const int c = tid + kQuantThreads * i;
        int sum = 0;
        if (c < n8) {
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                int code = 0;
                if (scale > 0.f) {
                    const float rq = __builtin_rintf((float)v[i][perm[b]] / scale);
                    code = (int)fminf(127.f, fmaxf(-127.f, rq));
                }
                sum += code;
                const uint32_t byte = (uint32_t)(code & 0xFF);
                if (b < 4) lo |= byte << (8 * b);
                else hi |= byte << (8 * (b - 4));
            }
            *reinterpret_cast<u2*>(xq + (size_t)t * d + 8 * (size_t)c) = u2{lo, hi};
        }
        // the 16 chunks of one group are 16 consecutive threads (n8 is a multiple of 16)
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
        if (c < n8 && (c & 15) == 0) xsum[(size_t)t * (d / kGroup) + (c >> 4)] = sum;
    }
}

// GEMM tile: 16 TT tokens x 64 RR rows, four waves side by side in N (wave w owns RR row tiles of
// 16 rows, all tokens), KS groups of four waves splitting the input groups (added through LDS in
// wave-group order, deterministic).  Per group: the token codes (BM x 128 bytes) staged in LDS,
// double-buffered; weights straight from HBM in operand order, one group ahead in registers; two
// int8 matrix-core steps per (row tile, token tile) give the exact nibble products, then
// acc += s (sum - z csum) in fp32.  After the K loop: times the token scale, then r_pad / 32 fp16
// matrix-core steps add R A_i^T, one rounding to fp16.
template <int TT, int RR, int KS>
__global__ __launch_bounds__(256 * KS, (KS == 1 ? 2 : 1)) void w4a8_kernel(const ForwardArgs args) {
    constexpr int BM = 16 * TT;
    constexpr int LSB = 144;             // LDS row stride in bytes (128 + 16 padding)
    constexpr int NCH = BM * 8 / 256;    // 16-byte code chunks per thread per group (BM rows x 8)
    constexpr int NCHP = NCH > 0 ? NCH : 1;
    // the code tiles, reused after the K loop for the wave groups' sums
    constexpr int kTileBytes = KS * 2 * BM * LSB;
    constexpr int kRedBytes = (KS - 1) * TT * RR * 256 * 16;
    __shared__ __attribute__((aligned(16))) int8_t smem[kTileBytes > kRedBytes ? kTileBytes : kRedBytes];
    int8_t (*xs)[2][BM * LSB] = reinterpret_cast<int8_t (*)[2][BM * LSB]>(smem);

    const int mb = blockIdx.x % args.m_tiles, nbl = blockIdx.x / args.m_tiles;
    const ModuleArgs M = args.mod[module_of(args, nbl)];
    const int nb = nbl - M.tile_begin;
    const int m0 = mb * BM;
    const int tid = threadIdx.x & 255, lane = tid & 63;
    const int kg = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 8);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int T = args.T, d = args.d, G = args.G;
    const int rt0 = nb * 4 * RR + wave * RR;
    const size_t qstride = (size_t)M.n_tiles16 * 1024, szstride = (size_t)M.n_tiles16 * 64;

    const uint8_t* qp[RR];
    const uint8_t* zp[RR];
    bool w_ok[RR];
#pragma unroll
    for (int rr = 0; rr < RR; ++rr) {
        const int rt = rt0 + rr;
        w_ok[rr] = rt < M.n_tiles16;
        qp[rr] = M.q + (size_t)(w_ok[rr] ? rt : 0) * 1024 + lane * 16;
        zp[rr] = M.sz + (size_t)(w_ok[rr] ? rt : 0) * 64 + (lane >> 4) * 16;
    }
    // code staging: BM rows x 8 chunks of 16 bytes per group; thread tid copies chunks tid + 256 c
    const int8_t* xsrc[NCHP];
    bool x_ok[NCHP];
    int xdst[NCHP];
#pragma unroll
    for (int c = 0; c < NCHP; ++c) {
        const int idx = c * 256 + tid;
        const int row = idx >> 3, col = (idx & 7) * 16;
        const int t = m0 + row;
        x_ok[c] = idx < BM * 8 && t < T;
        xsrc[c] = args.xq + (size_t)(x_ok[c] ? t : 0) * d + col;
        xdst[c] = (idx < BM * 8 ? row : 0) * LSB + col;
    }
    // this lane's tokens (one per token tile) for the code sums and the scale
    int tok[TT];
    bool t_ok[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        tok[tt] = m0 + 16 * tt + (lane & 15);
        t_ok[tt] = tok[tt] < T;
    }
    const u4 zero4 = {0u, 0u, 0u, 0u};
    const int n_it = (G + KS - 1) / KS;
    const bool act0 = kg < G;
    const bool copier = BM * 8 >= 256 || tid < BM * 8;  // TT = 1: 128 of 256 threads copy

    u4 st[NCHP];
    u4 qv[RR], zv[RR];
    int32_t cs[TT];
#pragma unroll
    for (int c = 0; c < NCHP; ++c)
        st[c] = (act0 && x_ok[c]) ? *reinterpret_cast<const u4*>(xsrc[c] + (size_t)kg * kGroup) : zero4;
#pragma unroll
    for (int rr = 0; rr < RR; ++rr) {
        qv[rr] = (act0 && w_ok[rr]) ? *reinterpret_cast<const u4*>(qp[rr] + (size_t)kg * qstride) : zero4;
        zv[rr] = (act0 && w_ok[rr]) ? *reinterpret_cast<const u4*>(zp[rr] + (size_t)kg * szstride) : zero4;
    }
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) cs[tt] = (act0 && t_ok[tt]) ? args.xsum[(size_t)tok[tt] * G + kg] : 0;
    if (copier) {
#pragma unroll
        for (int c = 0; c < NCHP; ++c)
            if (c * 256 + tid < BM * 8) *reinterpret_cast<u4*>(&xs[kg][0][xdst[c]]) = st[c];
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
        u4 qn[RR], zn[RR];
        int32_t csn[TT];
        if (more) {
#pragma unroll
            for (int c = 0; c < NCHP; ++c)
                st[c] = x_ok[c] ? *reinterpret_cast<const u4*>(xsrc[c] + (size_t)(g + KS) * kGroup) : zero4;
#pragma unroll
            for (int rr = 0; rr < RR; ++rr) {
                qn[rr] = w_ok[rr] ? *reinterpret_cast<const u4*>(qp[rr] + (size_t)(g + KS) * qstride) : zero4;
                zn[rr] = w_ok[rr] ? *reinterpret_cast<const u4*>(zp[rr] + (size_t)(g + KS) * szstride) : zero4;
            }
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) csn[tt] = t_ok[tt] ? args.xsum[(size_t)tok[tt] * G + g + KS] : 0;
        }
        if (act) {
            i4v part[TT][RR];
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                for (int rr = 0; rr < RR; ++rr) part[tt][rr] = i4v{0, 0, 0, 0};
            const int8_t* xb = &xs[kg][buf][(lane & 15) * LSB + 16 * (lane >> 4)];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                i4v a[RR];
#pragma unroll
                for (int rr = 0; rr < RR; ++rr) {
                    const uint32_t w0 = qv[rr][2 * m], w1 = qv[rr][2 * m + 1];
                    a[rr] = i4v{(int32_t)(w0 & 0x0F0F0F0Fu), (int32_t)((w0 >> 4) & 0x0F0F0F0Fu),
                                (int32_t)(w1 & 0x0F0F0F0Fu), (int32_t)((w1 >> 4) & 0x0F0F0F0Fu)};
                }
#pragma unroll
                for (int tt = 0; tt < TT; ++tt) {
                    const i4v b = *reinterpret_cast<const i4v*>(xb + tt * 16 * LSB + 64 * m);
#pragma unroll
                    for (int rr = 0; rr < RR; ++rr) part[tt][rr] = mfma_i8(a[rr], b, part[tt][rr]);
                }
            }
            // acc += s (sum - z csum): lane holds rows 4 (lane / 16) + i of each row tile
#pragma unroll
            for (int rr = 0; rr < RR; ++rr) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const h2 zs = as_h2(zv[rr][i]);
                    const int32_t z = (int32_t)(float)zs[0];
                    const float s = (float)zs[1];
#pragma unroll
                    for (int tt = 0; tt < TT; ++tt)
                        acc[tt][rr][i] = fmaf(s, (float)(part[tt][rr][i] - z * cs[tt]), acc[tt][rr][i]);
                }
            }
        }
        if (more) {
            if (copier) {
#pragma unroll
                for (int c = 0; c < NCHP; ++c)
                    if (c * 256 + tid < BM * 8) *reinterpret_cast<u4*>(&xs[kg][buf ^ 1][xdst[c]]) = st[c];
            }
#pragma unroll
            for (int rr = 0; rr < RR; ++rr) {
                qv[rr] = qn[rr];
                zv[rr] = zn[rr];
            }
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) cs[tt] = csn[tt];
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

    // token scales, then the correction on the fp16 projection (not scaled)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const float sc = t_ok[tt] ? args.xscale[tok[tt]] : 0.f;
#pragma unroll
        for (int rr = 0; rr < RR; ++rr) acc[tt][rr] *= sc;
    }
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

hipError_t launch_quant_x(const _Float16* x, int T, int d, int8_t* xq, int32_t* xsum, float* xscale,
                          hipStream_t stream) {
    if (d % kGroup != 0 || d > kQuantChunks * 8 * kQuantThreads) return hipErrorInvalidValue;
    hipLaunchKernelGGL(quant_x_kernel, dim3((unsigned)T), dim3(kQuantThreads), 0, stream, x, d, xq, xsum, xscale);
    return hipGetLastError();
}

template <int TT, int RR>
static hipError_t launch_w4a8_rr(const ForwardArgs& a, hipStream_t stream) {
    const dim3 grid(a.n_tiles);
    switch (a.tile_ks) {
        case 4:
            if constexpr (TT * RR >= 8) return hipErrorInvalidValue;  // not built: would spill
            else hipLaunchKernelGGL((w4a8_kernel<TT, RR, 4>), grid, dim3(1024), 0, stream, a);
            break;
        case 2: hipLaunchKernelGGL((w4a8_kernel<TT, RR, 2>), grid, dim3(512), 0, stream, a); break;
        case 1: hipLaunchKernelGGL((w4a8_kernel<TT, RR, 1>), grid, dim3(256), 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int TT>
static hipError_t launch_w4a8_tt(const ForwardArgs& a, hipStream_t stream) {
    if (a.tile_rr == 2) return launch_w4a8_rr<TT, 2>(a, stream);
    if (a.tile_rr == 1) return launch_w4a8_rr<TT, 1>(a, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_w4a8(const ForwardArgs& a, hipStream_t stream) {
    switch (a.tile_tt) {
        case 1: return launch_w4a8_tt<1>(a, stream);
        case 2: return launch_w4a8_tt<2>(a, stream);
        case 4: return launch_w4a8_tt<4>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace glowq
