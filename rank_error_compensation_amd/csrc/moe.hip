// Mixture-of-experts form of the group forward (the GlowQ arXiv page, Figures 7-9: the
// covariance-aligned shared basis of the MLP gate/up projections holds per expert and across all
// experts of Qwen1.5-MoE-A2.7B).  Every routed row (a token sent to one expert) is multiplied by
// that expert's modules: one launch covers every expert, its work items (expert, block of 64 RR
// rows of one module, block of 16 TT routed rows) enumerated on the device from the routing
// offsets, so the host never needs the per-expert counts.
//
//   rows offsets[e] .. offsets[e + 1] - 1 belong to expert e; row j reads X[row_token[j]] (or X[j])
//   y_i[j] = X[tok j] W_hat_{e,i}^T + R[.] A_{e,i}^T
// with R the expert's own projection of its rows (R_e = X_e B_e^T, one per expert, formed once for
// all its modules) or one projection per token shared by every expert (R = X B^T).
//
// Expert weights are stacked: module i of expert e is the device-layout module at byte
// e * (its size) of the module's buffers, its A at e * n_out * r elements.
#include <algorithm>

#include "glowq_internal.h"

namespace glowq {

// Block-wide exclusive prefix of v over 256 threads (every thread gets its prefix; *total the sum).
__device__ __forceinline__ int block_exclusive_scan256(int v, int* sh, int* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int n = __shfl_up(incl, off, 64);
        if (lane >= off) incl += n;
    }
    if (lane == 63) sh[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += sh[w];
    *total = sh[0] + sh[1] + sh[2] + sh[3];
    __syncthreads();
    return base + incl - v;
}

// Routing of one launch, shared by its workgroups through LDS: clamped offsets and the prefix of
// the per-expert block counts.  Out-of-range routing data (offsets not non-decreasing within
// 0 .. n_rows, a token index outside 0 .. T - 1) is clamped, never read out of bounds, and raises
// bit 1 of the error word.
struct MoeShared {
    int off[kMoeMaxExperts + 1];
    int end[kMoeMaxExperts];
    int pre[kMoeMaxExperts + 1];  // prefix of ceil(count / rows per block)
    int scan[4];
    int total;
};

__device__ void moe_routing(const MoeArgs& a, int rows_per_block, MoeShared& s) {
    const int e = threadIdx.x;  // 256 threads, kMoeMaxExperts = 256
    int lo = 0, hi = 0;
    bool bad = false;
    if (e < a.n_exp) {
        const int o0 = a.offsets[e], o1 = a.offsets[e + 1];
        bad = o0 < 0 || o1 > a.n_rows || o1 < o0 || (e == 0 && o0 != 0) || (e == a.n_exp - 1 && o1 != a.n_rows);
        lo = min(max(o0, 0), a.n_rows);
        hi = min(max(o1, lo), a.n_rows);
    }
    if (bad && blockIdx.x == 0) __hip_atomic_fetch_or(a.err, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int nb = (hi - lo + rows_per_block - 1) / rows_per_block;
    int tot = 0;
    const int p = block_exclusive_scan256(nb, s.scan, &tot);
    if (e < a.n_exp) {
        s.off[e] = lo;
        s.end[e] = hi;
        s.pre[e] = p;
    }
    if (e == 0) {
        s.pre[a.n_exp] = tot;
        s.total = tot;
    }
    __syncthreads();
}

// Expert of block index bi (0 <= bi < pre[n_exp]): the last e with pre[e] <= bi.
__device__ __forceinline__ int moe_expert_of(const MoeShared& s, int n_exp, int bi) {
    int lo = 0, hi = n_exp - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s.pre[mid] <= bi) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

__device__ __forceinline__ int moe_token(const MoeArgs& a, int j) {
    if (a.row_token == nullptr) return j;
    const int t = a.row_token[j];
    if (t < 0 || t >= a.T) {
        __hip_atomic_fetch_or(a.err, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return t < 0 ? 0 : a.T - 1;
    }
    return t;
}

// Per-expert projection: items (expert e, block of 16 of its rows) -> R[j][0 .. r_pad) =
// X[tok j] . B_e, fp16 (columns r .. r_pad - 1 zero).  The four waves take interleaved 32-input
// steps (four steps of loads in flight) and add their sums through LDS in wave order.
template <int NJ>
__global__ __launch_bounds__(256) void moe_proj_kernel(const MoeArgs a) {
    __shared__ MoeShared s;
    __shared__ f4 red[3][NJ][64];
    moe_routing(a, 16, s);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int d = a.d, r = a.r, rp = a.r_pad;
    const int kofs = 8 * (lane >> 4);
    const h8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int item = blockIdx.x; item < s.total; item += gridDim.x) {
        const int e = moe_expert_of(s, a.n_exp, item);
        const int j0 = s.off[e] + (item - s.pre[e]) * 16;
        const int j1 = s.end[e];
        const int jl = j0 + (lane & 15);
        const bool ok = jl < j1 && jl < a.n_rows;
        const _Float16* xr = a.x + (size_t)moe_token(a, ok ? jl : j0) * d + kofs;
        const _Float16* B = a.b + (size_t)e * r * d;
        const _Float16* br[NJ];
        bool j_ok[NJ];
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) {
            const int jj = 16 * jt + (lane & 15);
            j_ok[jt] = jj < r;
            br[jt] = B + (size_t)(j_ok[jt] ? jj : 0) * d + kofs;
        }
        f4 acc[NJ];
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) acc[jt] = f4{0.f, 0.f, 0.f, 0.f};
        const int n = d / 128;  // steps of this wave: 32 inputs at 128 i + 32 wave
        const int k0 = 32 * wave;
        for (int c = 0; c < n; c += 4) {
            h8 xa[4], bb[4][NJ];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int kk = k0 + 128 * min(c + u, n - 1);
                xa[u] = ok ? load_h8(xr + kk) : zero8;
#pragma unroll
                for (int jt = 0; jt < NJ; ++jt) bb[u][jt] = j_ok[jt] ? load_h8(br[jt] + kk) : zero8;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (c + u < n) {
#pragma unroll
                    for (int jt = 0; jt < NJ; ++jt) acc[jt] = mfma16(xa[u], bb[u][jt], acc[jt]);
                }
        }
        if (wave > 0) {
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt) red[wave - 1][jt][lane] = acc[jt];
        }
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt) {
                f4 v = acc[jt];
#pragma unroll
                for (int w = 0; w < 3; ++w) v += red[w][jt][lane];
                const int col = 16 * jt + (lane & 15);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int j = j0 + 4 * (lane >> 4) + i;  // output rows: tokens of the block
                    if (j < j1 && j < a.n_rows && col < rp) a.Rout[(size_t)j * rp + col] = (_Float16)v[i];
                }
            }
        }
        __syncthreads();
    }
}

// Per-expert projection for few routed rows per expert (decode-sized calls): items (expert e,
// block of 16 of its rows, 16-column tile jt of R), so that the expert's B is read by NJ workgroups
// at once rather than streamed by one; the four waves take interleaved 32-input steps with up to
// 16 steps of loads in flight (d <= 8192: one memory round trip per item) and add their sums through
// LDS in wave order.
template <int NJ>
__global__ __launch_bounds__(256) void moe_proj_cols_kernel(const MoeArgs a) {
    constexpr int U = 16;
    __shared__ MoeShared s;
    __shared__ f4 red[3][64];
    moe_routing(a, 16, s);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int d = a.d, r = a.r, rp = a.r_pad;
    const int kofs = 8 * (lane >> 4);
    const h8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int item = blockIdx.x; item < s.total * NJ; item += gridDim.x) {
        const int bi = item / NJ, jt = item - bi * NJ;
        const int e = moe_expert_of(s, a.n_exp, bi);
        const int j0 = s.off[e] + (bi - s.pre[e]) * 16;
        const int j1 = s.end[e];
        const int jl = j0 + (lane & 15);
        const bool ok = jl < j1 && jl < a.n_rows;
        const _Float16* xr = a.x + (size_t)moe_token(a, ok ? jl : j0) * d + kofs;
        const int jj = 16 * jt + (lane & 15);
        const bool j_ok = jj < r;
        const _Float16* br = a.b + (size_t)e * r * d + (size_t)(j_ok ? jj : 0) * d + kofs;
        f4 acc = {0.f, 0.f, 0.f, 0.f};
        const int n = d / 128;  // steps of this wave: 32 inputs at 128 i + 32 wave
        const int k0 = 32 * wave;
        for (int c = 0; c < n; c += U) {
            h8 xa[U], bb[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int kk = k0 + 128 * min(c + u, n - 1);
                xa[u] = ok ? load_h8(xr + kk) : zero8;
                bb[u] = j_ok ? load_h8(br + kk) : zero8;
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (c + u < n) acc = mfma16(xa[u], bb[u], acc);
        }
        if (wave > 0) red[wave - 1][lane] = acc;
        __syncthreads();
        if (wave == 0) {
            f4 v = acc;
#pragma unroll
            for (int w = 0; w < 3; ++w) v += red[w][lane];
            const int col = 16 * jt + (lane & 15);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int jrow = j0 + 4 * (lane >> 4) + i;  // output rows: tokens of the block
                if (jrow < j1 && jrow < a.n_rows && col < rp) a.Rout[(size_t)jrow * rp + col] = (_Float16)v[i];
            }
        }
        __syncthreads();
    }
}

// Grouped GEMM: items (expert e, row block rb of 64 RR rows of one module, block tb of 16 TT of
// e's routed rows), in that order, so that consecutive items share the expert's weight block.
// Per item the prefill tile: 4 waves side by side in N, the gathered activation rows staged in
// LDS per 128-input group (double-buffered), weights dequantised in registers, fp32 accumulation
// on v_mfma_f32_16x16x32_f16, then r_pad / 32 correction steps with R, one fp16 rounding.
template <int TT, int RR>
__global__ __launch_bounds__(256, 2) void moe_gemm_kernel(const MoeArgs a) {
    constexpr int BM = 16 * TT;
    constexpr int LS = 136;
    constexpr int NCH = BM * 16 / 256;
    constexpr int NCHP = NCH > 0 ? NCH : 1;
    __shared__ MoeShared s;
    __shared__ __attribute__((aligned(16))) _Float16 xs[2][BM * LS];
    moe_routing(a, BM, s);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int d = a.d, G = a.G;
    const NibConsts nc = nib_consts();
    const int kofs = 8 * (lane >> 4);
    const u4 zero4 = {0u, 0u, 0u, 0u};
    const h8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
    const int total = s.total * a.n_rb;
    for (int item = blockIdx.x; item < total; item += gridDim.x) {
        // items run (e, rb, tb): the expert from the block prefix scaled by n_rb
        int e = 0;
        {
            int lo = 0, hi = a.n_exp - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (s.pre[mid] * a.n_rb <= item) lo = mid;
                else hi = mid - 1;
            }
            e = lo;
        }
        const int nbe = s.pre[e + 1] - s.pre[e];  // token blocks of expert e (>= 1 here)
        const int local = item - s.pre[e] * a.n_rb;
        const int rb = local / nbe, tb = local - rb * nbe;
        int mi = 0;
#pragma unroll
        for (int k = 1; k < kMoeMaxMod; ++k) mi += (k < a.m && rb >= a.rb_begin[k]) ? 1 : 0;
        mi = __builtin_amdgcn_readfirstlane(mi);
        const int n_out = a.n_out[mi], nt16 = a.n_tiles16[mi];
        const uint8_t* Mq = a.q[mi] + (size_t)e * a.qbytes[mi];
        const uint8_t* Msz = a.sz[mi] + (size_t)e * a.szbytes[mi];
        const _Float16* Ma = a.a[mi] != nullptr ? a.a[mi] + (size_t)e * n_out * a.r : nullptr;
        _Float16* My = a.y[mi];
        const int rt0 = (rb - a.rb_begin[mi]) * 4 * RR + wave * RR;
        const int j0 = s.off[e] + tb * BM;
        const int j1 = s.end[e];
        const size_t qstride = (size_t)nt16 * 1024, szstride = (size_t)nt16 * 64;

        const uint8_t* qp[RR];
        const uint8_t* zp[RR];
        bool w_ok[RR];
#pragma unroll
        for (int rr = 0; rr < RR; ++rr) {
            const int rt = rt0 + rr;
            w_ok[rr] = rt < nt16;
            qp[rr] = Mq + (size_t)(w_ok[rr] ? rt : 0) * 1024 + lane * 16;
            zp[rr] = Msz + (size_t)(w_ok[rr] ? rt : 0) * 64 + (lane & 15) * 4;
        }
        const _Float16* xsrc[NCHP];
        bool x_ok[NCHP];
        int xdst[NCHP];
#pragma unroll
        for (int c = 0; c < NCHP; ++c) {
            const int idx = c * 256 + tid;
            const int row = idx >> 4, col = (idx & 15) * 8;
            const int j = j0 + row;
            x_ok[c] = idx < BM * 16 && j < j1;
            xsrc[c] = a.x + (size_t)moe_token(a, x_ok[c] ? j : j0) * d + col;
            xdst[c] = (idx < BM * 16 ? row : 0) * LS + col;
        }
        const bool copier = BM * 16 >= 256 || tid < BM * 16;
        u4 st[NCHP];
        u4 qv[RR];
        uint32_t zs[RR];
#pragma unroll
        for (int c = 0; c < NCHP; ++c) st[c] = x_ok[c] ? *reinterpret_cast<const u4*>(xsrc[c]) : zero4;
#pragma unroll
        for (int rr = 0; rr < RR; ++rr) {
            qv[rr] = w_ok[rr] ? *reinterpret_cast<const u4*>(qp[rr]) : zero4;
            zs[rr] = w_ok[rr] ? *reinterpret_cast<const uint32_t*>(zp[rr]) : 0u;
        }
        if (copier) {
#pragma unroll
            for (int c = 0; c < NCHP; ++c)
                if (c * 256 + tid < BM * 16) *reinterpret_cast<u4*>(&xs[0][xdst[c]]) = st[c];
        }
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
                for (int c = 0; c < NCHP; ++c)
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
                const _Float16 sc = as_h2(zs[rr])[1];
                s8[rr] = h8{sc, sc, sc, sc, sc, sc, sc, sc};
            }
            const _Float16* xb = &xs[buf][(lane & 15) * LS + kofs];
#pragma unroll
            for (int jw = 0; jw < 4; ++jw) {
                h8 av[RR];
#pragma unroll
                for (int rr = 0; rr < RR; ++rr) av[rr] = nib8_minus_z(qv[rr][jw], c1024[rr], c64[rr], nc) * s8[rr];
#pragma unroll
                for (int tt = 0; tt < TT; ++tt) {
                    const h8 b = *reinterpret_cast<const h8*>(xb + tt * 16 * LS + 32 * jw);
#pragma unroll
                    for (int rr = 0; rr < RR; ++rr) acc[tt][rr] = mfma16(av[rr], b, acc[tt][rr]);
                }
            }
            if (more) {
                if (copier) {
#pragma unroll
                    for (int c = 0; c < NCHP; ++c)
                        if (c * 256 + tid < BM * 16) *reinterpret_cast<u4*>(&xs[buf ^ 1][xdst[c]]) = st[c];
                }
#pragma unroll
                for (int rr = 0; rr < RR; ++rr) {
                    qv[rr] = qn[rr];
                    zs[rr] = zn[rr];
                }
            }
            __syncthreads();
        }
        // correction: R rows of this block (by routed row, or by token when shared by all experts)
        if (a.r > 0 && Ma != nullptr) {
            const int r = a.r, rp = a.r_pad;
            for (int kb = 0; kb < rp / 32; ++kb) {
                const int col = 32 * kb + kofs;
                h8 av[RR];
#pragma unroll
                for (int rr = 0; rr < RR; ++rr) {
                    const int row = (rt0 + rr) * 16 + (lane & 15);
                    av[rr] = (row < n_out && col < r) ? load_h8(Ma + (size_t)row * r + col) : zero8;
                }
#pragma unroll
                for (int tt = 0; tt < TT; ++tt) {
                    const int j = j0 + 16 * tt + (lane & 15);
                    h8 b = zero8;
                    if (j < j1) {
                        const int ri = a.r_by_token ? moe_token(a, j) : j;
                        b = load_h8(a.R + (size_t)ri * rp + col);
                    }
#pragma unroll
                    for (int rr = 0; rr < RR; ++rr) acc[tt][rr] = mfma16(av[rr], b, acc[tt][rr]);
                }
            }
        }
        const bool vec = (n_out & 3) == 0;
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            const int j = j0 + 16 * tt + (lane & 15);
            if (j >= j1) continue;
            _Float16* yrow = My + (size_t)j * n_out;
#pragma unroll
            for (int rr = 0; rr < RR; ++rr) {
                if (rt0 + rr >= nt16) continue;
                const int row0 = (rt0 + rr) * 16 + 4 * (lane >> 4);
                const f4 v = acc[tt][rr];
                if (vec && row0 + 3 < n_out) {
                    const h2 lo = {(_Float16)v[0], (_Float16)v[1]}, hi = {(_Float16)v[2], (_Float16)v[3]};
                    *reinterpret_cast<u2*>(yrow + row0) = u2{as_u32(lo), as_u32(hi)};
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (row0 + i < n_out) yrow[row0 + i] = (_Float16)v[i];
                }
            }
        }
    }
}

// Decode-sized calls (at most 16 routed rows per expert on average): items (expert e, one 16-row
// tile of one module, block of 16 of e's routed rows).  The four waves split the input groups
// (group g to wave g % 4), each keeping a ring of four groups of weight loads in flight; the routed
// rows' activations are read from L2 with each group (they are few); weights are turned into exact
// fp16 (q - z) and each group's sums scaled in fp32; every wave adds its share of the correction
// steps (rank columns 32 kb, kb = wave, wave + 4, ...), and the four partial tiles are added in LDS
// in wave order before the one fp16 rounding.
__global__ __launch_bounds__(256) void moe_decode_kernel(const MoeArgs a) {
    __shared__ MoeShared s;
    __shared__ f4 red[4][64];
    moe_routing(a, 16, s);
    constexpr int U = 4;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int d = a.d, G = a.G;
    const NibConsts nc = nib_consts();
    const int kofs = 8 * (lane >> 4);
    const h8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
    const int total = s.total * a.n_rb;
    for (int item = blockIdx.x; item < total; item += gridDim.x) {
        int e = 0;
        {
            int lo = 0, hi = a.n_exp - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (s.pre[mid] * a.n_rb <= item) lo = mid;
                else hi = mid - 1;
            }
            e = lo;
        }
        const int nbe = s.pre[e + 1] - s.pre[e];
        const int local = item - s.pre[e] * a.n_rb;
        const int rb = local / nbe, tb = local - rb * nbe;
        int mi = 0;
#pragma unroll
        for (int k = 1; k < kMoeMaxMod; ++k) mi += (k < a.m && rb >= a.rb_begin[k]) ? 1 : 0;
        mi = __builtin_amdgcn_readfirstlane(mi);
        const int n_out = a.n_out[mi], nt16 = a.n_tiles16[mi];
        const int rt = rb - a.rb_begin[mi];  // this item's 16-row tile
        const uint8_t* qb = a.q[mi] + (size_t)e * a.qbytes[mi] + (size_t)rt * 1024 + lane * 16;
        const uint8_t* zb = a.sz[mi] + (size_t)e * a.szbytes[mi] + (size_t)rt * 64;
        const size_t qstride = (size_t)nt16 * 1024, szstride = (size_t)nt16 * 64;
        const _Float16* Ma = a.a[mi] != nullptr ? a.a[mi] + (size_t)e * n_out * a.r : nullptr;
        const int j0 = s.off[e] + tb * 16, j1 = s.end[e];
        const int jl = j0 + (lane & 15);
        const bool row_ok = jl < j1;
        const int tok = moe_token(a, row_ok ? jl : j0);
        const _Float16* xr = a.x + (size_t)tok * d + kofs;
        const int n_my = G > wave ? (G - wave + 3) / 4 : 0;  // groups g = wave + 4 i

        u4 qv[U];
        uint32_t zso[U];
        u4 zs4[U];
        auto issue = [&](int u, int i) {
            const int g = wave + 4 * min(i, max(n_my - 1, 0));
            qv[u] = __builtin_nontemporal_load(reinterpret_cast<const u4*>(qb + (size_t)g * qstride));
            zso[u] = *reinterpret_cast<const uint32_t*>(zb + (size_t)g * szstride + (lane & 15) * 4);
            zs4[u] = *reinterpret_cast<const u4*>(zb + (size_t)g * szstride + (lane >> 4) * 16);
        };
        f4 acc = {0.f, 0.f, 0.f, 0.f};
        auto compute = [&](int u, int i) {
            // the routed rows' activations of this group come from L2 here: prefetching them with the
            // weights (16 more registers per slot) measured slower at every size
            const int g = wave + 4 * i;
            h8 bx[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) bx[j] = row_ok ? load_h8(xr + (size_t)g * kGroup + 32 * j) : zero8;
            h2 c1024, c64;
            zero_consts(zso[u], c1024, c64);
            f4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j) part = mfma16(nib8_minus_z(qv[u][j], c1024, c64, nc), bx[j], part);
#pragma unroll
            for (int k = 0; k < 4; ++k) acc[k] += (float)as_h2(zs4[u][k])[1] * part[k];
        };
        if (n_my > 0) {
#pragma unroll
            for (int u = 0; u < U; ++u) issue(u, u);
            int i0 = 0;
            for (; i0 + U < n_my; i0 += U) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    compute(u, i0 + u);
                    issue(u, i0 + U + u);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (i0 + u < n_my) compute(u, i0 + u);
        }
        // this wave's share of the correction: A rows of the tile x R rows of the routed block
        if (a.r > 0 && Ma != nullptr) {
            const int r = a.r, rp = a.r_pad;
            for (int kb = wave; kb * 32 < r; kb += 4) {
                const int col = 32 * kb + kofs;
                const int row = rt * 16 + (lane & 15);
                const h8 av = (row < n_out && col < r) ? load_h8(Ma + (size_t)row * r + col) : zero8;
                h8 bv = zero8;
                if (row_ok && col < r) {
                    const int ri = a.r_by_token ? tok : jl;
                    bv = load_h8(a.R + (size_t)ri * rp + col);
                }
                acc = mfma16(av, bv, acc);
            }
        }
        red[wave][lane] = acc;
        __syncthreads();
        if (wave == 0) {
            f4 v = red[0][lane];
#pragma unroll
            for (int w = 1; w < 4; ++w) v += red[w][lane];  // fixed order: deterministic
            const int row0 = rt * 16 + 4 * (lane >> 4);
            if (row_ok) {
                _Float16* yrow = a.y[mi] + (size_t)jl * n_out;
                if ((n_out & 3) == 0 && row0 + 3 < n_out) {
                    const h2 lo = {(_Float16)v[0], (_Float16)v[1]}, hi = {(_Float16)v[2], (_Float16)v[3]};
                    *reinterpret_cast<u2*>(yrow + row0) = u2{as_u32(lo), as_u32(hi)};
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (row0 + i < n_out) yrow[row0 + i] = (_Float16)v[i];
                }
            }
        }
        __syncthreads();
    }
}

template <int NJ>
static void launch_moe_proj_nj(const MoeArgs& a, unsigned grid, hipStream_t stream) {
    // fewer than 32 routed rows per expert on average: items per 16-column tile of R as well
    if ((int64_t)a.n_rows < 32 * (int64_t)a.n_exp) {
        const unsigned g2 = (unsigned)std::min<int64_t>((int64_t)grid * NJ, kMoeMaxGrid);
        hipLaunchKernelGGL((moe_proj_cols_kernel<NJ>), dim3(g2), dim3(256), 0, stream, a);
    } else {
        hipLaunchKernelGGL((moe_proj_kernel<NJ>), dim3(grid), dim3(256), 0, stream, a);
    }
}

hipError_t launch_moe_proj(const MoeArgs& a, int64_t max_items, hipStream_t stream) {
    const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>(max_items, kMoeMaxGrid));
    switch (a.r_pad / 16) {
        case 2: launch_moe_proj_nj<2>(a, grid, stream); break;
        case 4: launch_moe_proj_nj<4>(a, grid, stream); break;
        case 6: launch_moe_proj_nj<6>(a, grid, stream); break;
        case 8: launch_moe_proj_nj<8>(a, grid, stream); break;
        case 10: launch_moe_proj_nj<10>(a, grid, stream); break;
        case 12: launch_moe_proj_nj<12>(a, grid, stream); break;
        case 14: launch_moe_proj_nj<14>(a, grid, stream); break;
        case 16: launch_moe_proj_nj<16>(a, grid, stream); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_moe_gemm(const MoeArgs& a, int64_t max_items, hipStream_t stream) {
    const dim3 grid((unsigned)std::max<int64_t>(1, std::min<int64_t>(max_items, kMoeMaxGrid)));
    if (a.tile_tt == 0) hipLaunchKernelGGL(moe_decode_kernel, grid, dim3(256), 0, stream, a);
    else if (a.tile_tt == 1) hipLaunchKernelGGL((moe_gemm_kernel<1, 2>), grid, dim3(256), 0, stream, a);
    else if (a.tile_tt == 2) hipLaunchKernelGGL((moe_gemm_kernel<2, 2>), grid, dim3(256), 0, stream, a);
    else if (a.tile_tt == 4) hipLaunchKernelGGL((moe_gemm_kernel<4, 2>), grid, dim3(256), 0, stream, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace glowq
