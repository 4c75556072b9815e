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
#include "handoff.h"
#include "mid.h"

namespace glowq {

// Physical workgroup id -> logical tile id such that XCD x (workgroups b with b % 8 == x)
// receives a contiguous range of logical tiles.
__device__ __forceinline__ int xcd_remap(int b, int n) {
    const int xcd = b & 7, local = b >> 3;
    const int per = n >> 3, rem = n & 7;
    return xcd * per + (xcd < rem ? xcd : rem) + local;
}

// Producer of a fused launch (17 .. 64 tokens): workgroup p < n_prod forms one 16-token x 16-rank
// tile of the stacked projections R_p = X B_p^T over all of d with all its waves (32-input steps
// interleaved over the waves, eight steps of loads in flight per wave, sums added through LDS in
// wave order), and writes it as tagged pairs in every per-XCD copy, as the decode producers do.
// Tokens past T and ranks past r are never stored.
constexpr int kProdMaxWaves = 16;

// The producer's LDS: red (the waves' partial tiles) and the tag, given by the caller.
__device__ void produce_tile_in(const ForwardArgs& a, int p, f4 (*red)[64], uint32_t& ptag) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nw = (int)(blockDim.x >> 6);
    uint32_t epoch0 = 0;
    if (tid == 0) epoch0 = load_epoch(a);
    const int T = a.T, d = a.d, r = a.r, rp = a.r_pad;
    const int n_rt = a.n_proj * (rp / 16);  // rank tiles over the stacked projections
    // a K-split call splits the projection over the same input ranges: producer p forms the partial
    // tile of range kr; the producer of the last range adds the other ranges' partials to its own
    const int pk = a.dec_ks > 1 ? a.dec_ks : 1;
    const int n_tile = ((T + 15) >> 4) * n_rt;
    const int kr = p / n_tile;
    const int q = p - kr * n_tile;
    const int tt = q / n_rt, jt = q - tt * n_rt;
    const int pi = (jt * 16) / rp, j0 = (jt * 16) - pi * rp;
    const int t0 = 16 * tt;
    const int t = t0 + (lane & 15), j = j0 + (lane & 15);
    const bool t_ok = t < T, j_ok = j < r;
    const int kofs = 8 * (lane >> 4);
    const _Float16* xr = a.x + (size_t)(t_ok ? t : 0) * d + kofs;
    const _Float16* br = pick_bp(a, pi) + (size_t)(j_ok ? j : 0) * d + kofs;
    const h8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    constexpr int S = 8;
    const int n = d / 32;  // 32-input steps (four per input group); wave w takes s0 + w, s0 + w + nw, ...
    const int s0 = pk > 1 ? 4 * kr * a.dec_gk : 0, s1 = pk > 1 ? min(n, 4 * (kr + 1) * a.dec_gk) : n;
    for (int c = s0 + wave; c < s1; c += S * nw) {
        h8 xa[S], bb[S];
#pragma unroll
        for (int u = 0; u < S; ++u) {
            const int st = c + u * nw;
            const int kk = 32 * (st < s1 ? st : c);  // steps past the range reload the first (unused)
            xa[u] = t_ok ? load_h8(xr + kk) : zero8;
            bb[u] = j_ok ? load_h8(br + kk) : zero8;
        }
#pragma unroll
        for (int u = 0; u < S; ++u)
            if (c + u * nw < s1) acc = mfma16(xa[u], bb[u], acc);
    }
    if (wave > 0) red[wave - 1][lane] = acc;
    if (tid == 0) {
        ptag = epoch0 + 1u;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the epoch read completes before the arrival
    }
    __syncthreads();
    int arrived = 0;
    if (tid == 0) arrived = arrive(a);
    const uint32_t tag = ptag;
    u64* R = reinterpret_cast<u64*>(a.R);
    // pairs of this call: the kRReplicas copies of R, then the partial tiles of ranges 0 .. pk - 2
    const size_t copy = (size_t)a.n_proj * T * r;
    if (tag == 1u || tag == 0xFFFFFFFFu) {
        // first and last tag of a wrap: clear every pair of the decode area outside this call's range
        const size_t from = (size_t)(kRReplicas + pk - 1) * copy;
        for (size_t k = from + (size_t)p * blockDim.x + tid; k < kDecodeAreaPairs; k += (size_t)a.n_prod * blockDim.x)
            R[k] = 0ull;
    }
    if (wave == 0) {
        f4 v = acc;
        for (int w = 1; w < nw; ++w) v += red[w - 1][lane];  // fixed order: deterministic
        const int jj = j0 + (lane & 15);
        u64* part = R + (size_t)kRReplicas * copy;  // partial tile of range k at part + k copy
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ti = t0 + 4 * (lane >> 4) + i;  // output rows: tokens
            if (ti < T && jj < r) {
                const size_t off = ((size_t)pi * T + ti) * r + jj;
                if (kr < pk - 1) {
                    store_pair(part + (size_t)kr * copy + off, v[i], tag);
                } else {
                    // ranges in order, this producer's own (the last) added last: deterministic
                    float s = 0.f;
                    for (int k = 0; k < pk - 1; ++k) s += load_pair(a, part + (size_t)k * copy + off, tag);
                    const float tot = pk > 1 ? s + v[i] : v[i];
#pragma unroll
                    for (int c = 0; c < kRReplicas; ++c) store_pair(R + c * copy + off, tot, tag);
                }
            }
        }
    }
    if (tid == 0) finish(a, arrive_slot(a, arrived), epoch0);
}

__device__ void produce_tile(const ForwardArgs& a, int p) {
    __shared__ f4 red[kProdMaxWaves - 1][64];
    __shared__ uint32_t ptag;
    produce_tile_in(a, p, red, ptag);
}

// Small grids: KS groups of four wavefronts per workgroup (256 KS threads) share one output tile
// and split the input groups between them (group g goes to wave group g % KS), each with its own
// double-buffered activation tile in LDS; at the end the wave groups' sums are added through LDS
// in wave-group order (deterministic) and wave group 0 applies the correction and stores.  With
// KS = 4 a launch of one workgroup per CU keeps four wavefronts on every SIMD.
// FUSE (17 .. 64 tokens, correcting calls): the first n_prod workgroups are producers of the
// projection (produce_tile) and the tiles read R as tagged pairs at their correction step, so the
// whole call is one launch.
template <int F, int TT, int RR, int KS, bool FUSE>
__global__ __launch_bounds__(256 * KS, (KS == 1 ? 2 : 1)) void prefill_kernel(const ForwardArgs args) {
    constexpr bool MX = Fmt<F>::mx, SIX = Fmt<F>::six;
    constexpr int QB = Fmt<F>::qblock;
    constexpr int BM = 16 * TT;
    constexpr int LS = 136;              // LDS row stride in halves (128 + 8 padding)
    constexpr int NCH = BM * 16 / 256;   // 16-byte X chunks per thread per group
    __shared__ __attribute__((aligned(16))) _Float16 xs[KS][2][BM * LS];
    // hand-off state of thread 0 kept in LDS, not registers (the 1024-thread tiles have none spare)
    __shared__ uint32_t tag_lds;
    __shared__ int arrived_lds;

    if (FUSE && (int)blockIdx.x < args.n_prod) {
        produce_tile(args, blockIdx.x);
        return;
    }
    if (FUSE && threadIdx.x == 0) tag_lds = load_epoch(args) + 1u;
    const int L = xcd_remap(blockIdx.x - (FUSE ? args.n_prod : 0), args.n_tiles);
    const int mb = L % args.m_tiles, nbl = L / args.m_tiles;
    const ModuleArgs M = args.mod[module_of(args, nbl)];
    const int nb = nbl - M.tile_begin;
    const int m0 = mb * BM;
    const int tid = threadIdx.x & 255, lane = tid & 63;
    const int kg = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 8);  // wave group
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int T = args.T, d = args.d, G = args.G;
    const NibConsts nc = nib_consts();
    const int kofs = 8 * (lane >> 4);
    const int rt0 = nb * 4 * RR + wave * RR;
    const size_t qstride = (size_t)M.n_tiles16 * QB, szstride = (size_t)M.n_tiles16 * 64;  // per group
    const int q6ofs = 1024 + 8 * lane - 16 * lane;  // MXFP6: second plane of the lane's codes

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

    // this wave group's groups: kg, kg + KS, ... (G >= 1, so every wave group of KS = 1 has one;
    // with KS = 2 and G = 1 wave group 1 has none and only contributes zeros)
    const int n_it = (G + KS - 1) / KS;
    u4 st[NCH];
    u4 qv[RR];
    u2 q6[SIX ? RR : 1];
    uint32_t zs[RR];  // INT4: (z, s) of the row; MX: the row's four block scales
    const bool act0 = kg < G;
    const u2 zero2 = {0u, 0u};
#pragma unroll
    for (int c = 0; c < NCH; ++c)
        st[c] = (act0 && x_ok[c]) ? *reinterpret_cast<const u4*>(xsrc[c] + (size_t)kg * kGroup) : zero4;
#pragma unroll
    for (int rr = 0; rr < RR; ++rr) {
        qv[rr] = (act0 && w_ok[rr]) ? *reinterpret_cast<const u4*>(qp[rr] + (size_t)kg * qstride) : zero4;
        if constexpr (SIX)
            q6[SIX ? rr : 0] = (act0 && w_ok[rr]) ? *reinterpret_cast<const u2*>(qp[rr] + (size_t)kg * qstride + q6ofs) : zero2;
        zs[rr] = (act0 && w_ok[rr]) ? *reinterpret_cast<const uint32_t*>(zp[rr] + (size_t)kg * szstride) : 0u;
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c) *reinterpret_cast<u4*>(&xs[kg][0][xdst[c]]) = st[c];
    __syncthreads();  // tag_lds written (the epoch read complete) before the arrival
    if (FUSE && threadIdx.x == 0) arrived_lds = arrive(args);
    const uint32_t tag = FUSE ? tag_lds : 0u;

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
        u2 q6n[SIX ? RR : 1];
        uint32_t zn[RR];
        if (more) {
#pragma unroll
            for (int c = 0; c < NCH; ++c)
                st[c] = x_ok[c] ? *reinterpret_cast<const u4*>(xsrc[c] + (size_t)(g + KS) * kGroup) : zero4;
#pragma unroll
            for (int rr = 0; rr < RR; ++rr) {
                qn[rr] = w_ok[rr] ? *reinterpret_cast<const u4*>(qp[rr] + (size_t)(g + KS) * qstride) : zero4;
                if constexpr (SIX)
                    q6n[SIX ? rr : 0] =
                        w_ok[rr] ? *reinterpret_cast<const u2*>(qp[rr] + (size_t)(g + KS) * qstride + q6ofs) : zero2;
                zn[rr] = w_ok[rr] ? *reinterpret_cast<const uint32_t*>(zp[rr] + (size_t)(g + KS) * szstride) : 0u;
            }
        }
        if (act && MX) {
            // MX operands carry their block scales (exact fp16); a lane holds one MX block, so its
            // activation operands are the block's inputs in order (block order)
            const _Float16* xb = &xs[kg][buf][(lane & 15) * LS + Fmt<F>::xofs(lane >> 4)];
            float sc[RR];
#pragma unroll
            for (int rr = 0; rr < RR; ++rr) sc[rr] = mx_scale(zs[rr], lane >> 4);
            // MXFP6: one 32-value conversion per row tile, or per (row tile, slice) when the
            // 1024-thread tile of two row tiles could not hold both conversions' values
            constexpr bool kFresh = RR * KS >= 8;
            if constexpr (SIX && kFresh) {
                // row tile by row tile: one conversion live at a time (the activation operands are
                // read once per row tile)
#pragma unroll
                for (int rr = 0; rr < RR; ++rr) {
                    const h32 e = mx6_h32_fresh<F>(qv[rr], q6[rr], sc[rr]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const h8 a = mx6_slice(e, j);
#pragma unroll
                        for (int tt = 0; tt < TT; ++tt) {
                            const h8 b = *reinterpret_cast<const h8*>(xb + tt * 16 * LS + Fmt<F>::xstep * j);
                            acc[tt][rr] = mfma16(a, b, acc[tt][rr]);
                        }
                    }
                }
            }
            h32 e6[SIX && !kFresh ? RR : 1];
            if constexpr (SIX && !kFresh) {
#pragma unroll
                for (int rr = 0; rr < RR; ++rr) e6[rr] = mx6_h32<F>(qv[rr], q6[rr], sc[rr]);
            }
#pragma unroll
            for (int j = 0; j < 4 && !(SIX && kFresh); ++j) {
                h8 a[RR];
#pragma unroll
                for (int rr = 0; rr < RR; ++rr) {
                    if constexpr (SIX)
                        a[rr] = mx6_slice(e6[SIX && !kFresh ? rr : 0], j);
                    else
                        a[rr] = mx4_h8(qv[rr][j], sc[rr]);
                }
#pragma unroll
                for (int tt = 0; tt < TT; ++tt) {
                    const h8 b = *reinterpret_cast<const h8*>(xb + tt * 16 * LS + Fmt<F>::xstep * j);
#pragma unroll
                    for (int rr = 0; rr < RR; ++rr) acc[tt][rr] = mfma16(a[rr], b, acc[tt][rr]);
                }
            }
        } else if (act) {
            h2 c1024[RR], c64[RR];
            h8 s8[RR];
#pragma unroll
            for (int rr = 0; rr < RR; ++rr) {
                zero_consts(zs[rr], c1024[rr], c64[rr]);
                const _Float16 sc = as_h2(zs[rr])[1];
                s8[rr] = h8{sc, sc, sc, sc, sc, sc, sc, sc};
            }
            const _Float16* xb = &xs[kg][buf][(lane & 15) * LS + kofs];
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
        }
        if (more) {
#pragma unroll
            for (int c = 0; c < NCH; ++c) *reinterpret_cast<u4*>(&xs[kg][buf ^ 1][xdst[c]]) = st[c];
#pragma unroll
            for (int rr = 0; rr < RR; ++rr) {
                qv[rr] = qn[rr];
                if constexpr (SIX) q6[SIX ? rr : 0] = q6n[SIX ? rr : 0];
                zs[rr] = zn[rr];
            }
        }
        __syncthreads();
    }

    // fused launch: the tile's projection rows, waited for as tagged pairs by all threads at once
    // and kept in LDS as fp16 (after the wave groups' reduction area; the activation buffers are
    // free after the loop's last barrier)
    constexpr int kRedBytes = (KS - 1) * TT * RR * 256 * 16;
    _Float16* rl = reinterpret_cast<_Float16*>(reinterpret_cast<uint8_t*>(&xs[0][0][0]) + kRedBytes);
    if (FUSE && args.r > 0 && M.a != nullptr) {
        static_assert(sizeof(xs) >= kRedBytes + BM * kMaxRank * 2, "projection rows fit");
        const int r = args.r, rp = args.r_pad;
        const u64* Rp = reinterpret_cast<const u64*>(args.R) +
                        (size_t)(blockIdx.x & (kRReplicas - 1)) * args.n_proj * T * r + (size_t)M.proj * T * r;
        for (int k = threadIdx.x; k < BM * rp; k += 256 * KS) {
            const int tl = k / rp, col = k - tl * rp, t = m0 + tl;
            const float v = (t < T && col < r) ? load_pair(args, Rp + (size_t)t * r + col, tag) : 0.f;
            rl[k] = (_Float16)v;
        }
        __syncthreads();
    }

    if (KS > 1) {
        // wave groups 1 .. KS-1 hand their sums to wave group 0 through LDS (the activation
        // buffers are free after the loop's last barrier)
        f4* red = reinterpret_cast<f4*>(&xs[0][0][0]);
        static_assert(sizeof(xs) >= kRedBytes, "reduction space");
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

    // correction: r_pad / 32 more K steps, A-operand A_i rows, B-operand R tokens (fp16 from the
    // projection launch, or the producers' fp32 pairs of this launch rounded to fp16)
    if (FUSE && threadIdx.x == 0) arrived_lds = arrive_slot(args, arrived_lds);  // now the slot result
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
                h8 b = zero8;
                if (FUSE)
                    b = *reinterpret_cast<const h8*>(rl + (16 * tt + (lane & 15)) * rp + col);  // zero past T
                else
                    b = t < T ? load_h8(R + (size_t)t * rp + col) : zero8;
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
    if (FUSE && threadIdx.x == 0) finish(args, arrived_lds, tag_lds - 1u);
}

// Wide tile for large grids: BM = 128 tokens (64 for MXFP6) x BN = 256 rows, wave w owning 4 row
// tiles of 16 rows and all TT token tiles, so every activation operand read from LDS feeds 4
// matrix-core steps and every dequantised weight operand TT.  The activation tile of a 128-input group is
// copied HBM/L2 -> LDS by the load unit itself (16-byte global_load_lds, no registers), whole
// 256-byte rows per four lanes; in LDS row r keeps its 16-byte chunk c at position c ^ (r % 16),
// so that the operand reads (16 rows, one chunk each) hit 16 different bank groups.  Two LDS
// buffers (2 x 32 KiB): the copy of group g + 1 and the next weight blocks (registers) are in
// flight while group g is multiplied.  Inside a group the 32 (slice, token tile) steps are issued
// in a fixed order: operand reads two steps ahead, the next slice's unpacking spread between the
// matrix-core steps.  Tokens past T read row T - 1 and row tiles past the module read its last
// tile; neither is stored.
typedef __attribute__((address_space(3))) void lds_void;

template <int F, int TT>
__global__ __launch_bounds__(256, 2) void prefill_wide_kernel(const ForwardArgs args) {
    constexpr int RR = 4, BM = 16 * TT;
    constexpr bool MX = Fmt<F>::mx, SIX = Fmt<F>::six;
    constexpr int QB = Fmt<F>::qblock;
    extern __shared__ __attribute__((aligned(16))) u4 xw[];  // [2][TT * 4][64]
    static_assert(TT == 8 || TT == 4, "128 or 64 tokens per tile");

    int mb, nbl;
    if ((args.m_tiles & 7) == 0) {
        // XCD x (workgroups b with b % 8 == x) owns the token blocks [x m / 8, (x + 1) m / 8) for
        // every row block: its slice of the activations stays in its L2 while the weights stream
        // through (the row blocks in order, each used by the XCD's token blocks one after another)
        const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3, mp = args.m_tiles >> 3;
        nbl = local / mp;
        mb = xcd * mp + (local - nbl * mp);
    } else {
        const int L = xcd_remap(blockIdx.x, args.n_tiles);
        mb = L % args.m_tiles;
        nbl = L / args.m_tiles;
    }
    const ModuleArgs M = args.mod[module_of(args, nbl)];
    const int nb = nbl - M.tile_begin;
    const int m0 = mb * BM;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int T = args.T, d = args.d, G = args.G;
    const NibConsts nc = nib_consts();
    const int rt0 = nb * 4 * RR + wave * RR;
    const int NT = M.n_tiles16;

    // weight blocks: uniform byte offsets of this wave's row tiles (clamped to the module's last
    // tile) plus one per-lane 32-bit offset; activations: per-lane 32-bit byte offsets of the two
    // token rows this lane copies (the launcher keeps T d 2 below 2^31)
    uint32_t rtc[RR];
#pragma unroll
    for (int rr = 0; rr < RR; ++rr) rtc[rr] = (uint32_t)min(rt0 + rr, NT - 1);
    const uint32_t qlane = lane * 16, zlane = (lane & 15) * 4, q6lane = 1024 + 8 * lane;
    auto qaddr = [&](int g, int rr) {
        return reinterpret_cast<const u4*>(M.q + ((size_t)g * NT + rtc[rr]) * QB + qlane);
    };
    auto q6addr = [&](int g, int rr) {  // MXFP6: second plane of the lane's codes
        return reinterpret_cast<const u2*>(M.q + ((size_t)g * NT + rtc[rr]) * QB + q6lane);
    };
    auto zaddr = [&](int g, int rr) {
        return reinterpret_cast<const uint32_t*>(M.sz + ((size_t)g * NT + rtc[rr]) * 64 + zlane);
    };
    // activation copy: instruction i of wave w fills tile rows 4 TT w + 4 i .. + 3 (256 bytes each,
    // whole cache lines); lane l lands at LDS slot 16 l, i.e. row 4 TT w + 4 i + l / 16, 16-byte
    // position l % 16, which holds input chunk (l % 16) ^ (row % 16) of that row (XOR swizzle)
    uint32_t xoff[TT];
#pragma unroll
    for (int i = 0; i < TT; ++i) {
        const int row = 4 * TT * wave + 4 * i + (lane >> 4);
        const int t = min(m0 + row, T - 1);
        xoff[i] = (uint32_t)(t * d + 8 * ((lane & 15) ^ (row & 15))) * 2u;
    }
    const char* xbase = reinterpret_cast<const char*>(args.x);
    auto copy_x = [&](int g, int buf) {
#pragma unroll
        for (int i = 0; i < TT; ++i)
            __builtin_amdgcn_global_load_lds((const void*)(xbase + (size_t)g * kGroup * 2 + xoff[i]),
                                             (lds_void*)(xw + ((size_t)buf * BM + 4 * TT * wave + 4 * i) * 16), 16, 0, 0);
    };
    // operand read of slice j: lane l takes row 16 tt + l % 16, chunk 4 j + l / 16 (MX: 4 (l / 16) + j),
    // swizzled
    uint32_t bofs[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int chunk = MX ? 4 * (lane >> 4) + j : 4 * j + (lane >> 4);  // MX: block order
        bofs[j] = (uint32_t)((lane & 15) * 16 + (chunk ^ (lane & 15)));
    }

    u4 qv[RR];
    u2 q6[SIX ? RR : 1];
    uint32_t zs[RR];  // INT4: (z, s) of the row; MX: the row's four block scales
    copy_x(0, 0);
#pragma unroll
    for (int rr = 0; rr < RR; ++rr) {
        qv[rr] = *qaddr(0, rr);
        if constexpr (SIX) q6[SIX ? rr : 0] = *q6addr(0, rr);
        zs[rr] = *zaddr(0, rr);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
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
        u2 q6n[SIX ? RR : 1];
        uint32_t zn[RR];
        if (more) {
            copy_x(g + 1, buf ^ 1);
#pragma unroll
            for (int rr = 0; rr < RR; ++rr) {
                qn[rr] = *qaddr(g + 1, rr);
                if constexpr (SIX) q6n[SIX ? rr : 0] = *q6addr(g + 1, rr);
                zn[rr] = *zaddr(g + 1, rr);
            }
        }
        h2 c1024[RR], c64[RR];
        h8 s8[RR];
        if constexpr (!MX) {
#pragma unroll
            for (int rr = 0; rr < RR; ++rr) {
                zero_consts(zs[rr], c1024[rr], c64[rr]);
                const _Float16 s = as_h2(zs[rr])[1];
                s8[rr] = h8{s, s, s, s, s, s, s, s};
            }
        }
        // operand j of row tile rr: INT4 (q - z) s; MX element times its block scale (exact)
        // MXFP6 (64-token tile): each row tile's 32 values converted once per group, with the
        // lane's block scale
        h32 e6[SIX ? RR : 1];
        if constexpr (SIX) {
#pragma unroll
            for (int rr = 0; rr < RR; ++rr) e6[rr] = mx6_h32<F>(qv[rr], q6[rr], mx_scale(zs[rr], lane >> 4));
        }
        auto unpack = [&](int j, int rr) -> h8 {
            if constexpr (SIX)
                return mx6_slice(e6[SIX ? rr : 0], j);
            else if constexpr (MX)
                return mx4_h8(qv[rr][j], mx_scale(zs[rr], lane >> 4));
            else
                return nib8_minus_z(qv[rr][j], c1024[rr], c64[rr], nc) * s8[rr];
        };
        const u4* xb = xw + (size_t)buf * BM * 16;
        {
            // 32 steps (slice j, token tile tt): the activation operand of step st is read two
            // steps ahead, and the weight operands of slice j + 1 are unpacked during slice j, one
            // row tile every other step, so that the unpacking issues while the matrix cores run
            constexpr int NS = 4 * TT;
            h8 bq[3];
            auto bread = [&](int st) { return __builtin_bit_cast(h8, xb[(st % TT) * 256 + bofs[st / TT]]); };
            bq[0] = bread(0);
            bq[1] = bread(1);
            h8 aj[4][RR];
#pragma unroll
            for (int rr = 0; rr < RR; ++rr) aj[0][rr] = unpack(0, rr);
#pragma unroll
            for (int st = 0; st < NS; ++st) {
                const int j = st / TT, tt = st % TT;
                if (st + 2 < NS) bq[(st + 2) % 3] = bread(st + 2);
                constexpr int kEvery = TT / RR;  // steps per row tile's unpacking (2, or 1 at 64 tokens)
                if (j < 3 && tt % kEvery == 0) {
                    const int rr = tt / kEvery;
                    aj[j + 1][rr] = unpack(j + 1, rr);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int rr = 0; rr < RR; ++rr) acc[tt][rr] = mfma16(aj[j][rr], bq[st % 3], acc[tt][rr]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (more) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
            for (int rr = 0; rr < RR; ++rr) {
                qv[rr] = qn[rr];
                if constexpr (SIX) q6[SIX ? rr : 0] = q6n[SIX ? rr : 0];
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
        const int kofs = 8 * (lane >> 4);
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
            if (rt0 + rr >= NT) continue;
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

// 17 .. 64 tokens, INT4 weights: one token block (16 TT tokens, TT = 2 or 4), so every weight byte
// is read once, and 4 RR row tiles of 16 rows per workgroup of eight wavefronts.  Wave w owns RR row
// tiles (row part w % 4) and all TT token tiles for half of every input group (K slices 2 (w / 4)
// and 2 (w / 4) + 1 of 32 inputs), so every dequantised weight operand feeds TT matrix-core steps
// (the unpacking is the costly part at this size), every activation operand read from LDS feeds RR,
// and two wavefronts share each SIMD; the halves are added through LDS at the end, in a fixed order.
// Per 128-input group a stage holds the activation tile (16 TT rows x 256 bytes, XOR-swizzled as in
// the wide tile), the 4 RR weight blocks (1 KB each, operand order) and their (z, s) words, all
// three copied HBM/L2 -> LDS by the load unit (global_load_lds, no registers); NST stages form a
// ring, so the copies of the next NST - 1 groups are in flight while one group is multiplied, and
// every wave issues the same PER copies per group (duplicates where fewer are needed), which lets
// one s_waitcnt count decide when the next stage has landed.  The dequantised operands are those
// of the other tiles (exact (q - z), one rounding by the fp16 scale).  Correcting calls only: the
// first n_prod workgroups form R as 16 x 16 tiles (produce_tile_in) and every tile reads its rows
// as tagged pairs for the correction, as the fused small tiles do.
constexpr int kMidWaves = 8;
constexpr int kMidStageMax = 160 * 1024 - 512;  // stage ring bytes (the only LDS of the kernel)

template <int TT, int RR>
struct MidShape {
    static constexpr int RB = 4 * RR;            // row tiles per workgroup
    static constexpr int W_AT = TT * 4096;       // activation tile: 16 TT rows x 256 bytes
    static constexpr int Z_AT = W_AT + RB * 1024;
    static constexpr int SB = Z_AT + 4 * 256;    // (z, s) words: 256 bytes per row part
    static constexpr int NST = kMidStageMax / SB < 8 ? kMidStageMax / SB : 8;
    static constexpr int XI = TT / 2;            // activation copies per wave and group
    static constexpr int PER = XI + 2;           // copies per wave and group (one weight block, one (z, s))
    static constexpr int WAIT = (NST - 2) * PER; // copies allowed in flight once the next stage landed
    static_assert(RR == 2 && NST >= TT && NST >= 3 && WAIT < 64, "mid tile shape");
    static_assert(SB - 16 >= 16 * kMaxRank * 2 && SB >= (kMidWaves - 1) * 64 * 16, "stage reuse");
    static_assert(NST * SB >= 4 * TT * RR * 1024, "the halves' reduction fits the ring");
};

// s_waitcnt immediate: vmcnt n (bits 3:0 and 15:14), expcnt and lgkmcnt at their maxima
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
// the same with lgkmcnt 0 (bits 11:8): also every LDS read of the wave completed
constexpr int vm_lgkm0_imm(int n) { return 0x0070 | (n & 15) | ((n >> 4) << 14); }

template <int TT, int RR>
__global__ __launch_bounds__(64 * kMidWaves, 1) void mid_kernel(const ForwardArgs args) {
    using S = MidShape<TT, RR>;
    constexpr int RB = S::RB, NST = S::NST, SB = S::SB, W_AT = S::W_AT, Z_AT = S::Z_AT, XI = S::XI;
    // the stage ring is the kernel's only LDS object: the compiler then leaves the ordering of the
    // copies and the operand reads to the explicit waits below (with several objects it waits for
    // every copy in flight before each read).  After the loop the ring holds the halves' sums, the
    // projection rows (token tile tt in stage tt) and the tag (end of stage 0); producers keep their
    // partial tiles in stage 0 and their tag in stage 1.
    __shared__ __attribute__((aligned(16))) uint8_t stg[NST * SB];
    auto sp = [&](int k) -> uint8_t* { return stg + k * SB; };
    if ((int)blockIdx.x < args.n_prod) {
        produce_tile_in(args, blockIdx.x, reinterpret_cast<f4(*)[64]>(stg), *reinterpret_cast<uint32_t*>(stg + SB));
        return;
    }
    // thread 0's epoch read (the tag of this launch), before any arrival of this workgroup
    uint32_t epoch0 = 0;
    if (threadIdx.x == 0) epoch0 = load_epoch(args);
    // row block nbl, K range ks_idx (groups g0 .. g1 - 1; one range unless the call splits K)
    const int nbl_all = (int)blockIdx.x - args.n_prod;
    const int ks_idx = nbl_all / args.dec_tiles;
    const int nbl = nbl_all - ks_idx * args.dec_tiles;
    const ModuleArgs M = args.mod[module_of(args, nbl)];
    const int nb = nbl - M.tile_begin;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rw = wave & 3, kh = wave >> 2;  // row part, K half
    const int T = args.T, d = args.d, G = args.G;
    const int g0 = ks_idx * args.dec_gk, g1 = min(G, g0 + args.dec_gk);
    const bool split = args.dec_ks > 1;
    const int NT = M.n_tiles16;
    const NibConsts nc = nib_consts();
    const int rt0 = nb * RB + rw * RR;  // the wave's first row tile

    // activation copy: instruction i of wave w fills tile rows 4 XI w + 4 i .. + 3; lane l lands at
    // row + l / 16, 16-byte position l % 16, holding chunk (l % 16) ^ (row % 16)
    uint32_t xoff[XI];
#pragma unroll
    for (int i = 0; i < XI; ++i) {
        const int row = 4 * XI * wave + 4 * i + (lane >> 4);
        xoff[i] = (uint32_t)(min(row, T - 1) * d + 8 * ((lane & 15) ^ (row & 15))) * 2u;
    }
    // weight copy: wave w copies block w % RB of the workgroup (waves past RB repeat a block: same
    // bytes, same place); (z, s) copy: wave w the words of row part w % 4, lane l the word of row
    // l % 16 of the part's row tile l / 16 (past RR: the last)
    const int kw = wave % RB;
    const uint32_t wsrc = (uint32_t)(min(nb * RB + kw, NT - 1) * 1024 + lane * 16);
    const uint32_t zsrc = (uint32_t)(min(rt0 + min(lane >> 4, RR - 1), NT - 1) * 64 + (lane & 15) * 4);
    const char* xbase = reinterpret_cast<const char*>(args.x);
    auto copy = [&](int g, uint8_t* st) {
        const int gg = min(g, g1 - 1);  // past the range: a valid group into a stage no one reads
#pragma unroll
        for (int i = 0; i < XI; ++i)
            __builtin_amdgcn_global_load_lds((const void*)(xbase + (size_t)gg * kGroup * 2 + xoff[i]),
                                             (lds_void*)(st + (4 * XI * wave + 4 * i) * 256), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(M.q + (size_t)gg * NT * 1024 + wsrc),
                                         (lds_void*)(st + W_AT + kw * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(M.sz + (size_t)gg * NT * 64 + zsrc),
                                         (lds_void*)(st + Z_AT + rw * 256), 4, 0, 0);
    };
    // operand read of slice j, token tile tt: row 16 tt + l % 16, chunk 4 j + l / 16 (swizzled)
    uint32_t bofs[2];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
        const int j = 2 * kh + jj;
        bofs[jj] = (uint32_t)((lane & 15) * 256 + 16 * ((4 * j + (lane >> 4)) ^ (lane & 15)));
    }

    f4 acc[TT][RR];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int rr = 0; rr < RR; ++rr) acc[tt][rr] = f4{0.f, 0.f, 0.f, 0.f};

    for (int k = 0; k < NST - 1; ++k) copy(g0 + k, sp(k));
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(S::WAIT));
    __builtin_amdgcn_s_barrier();
    // the epoch read was thread 0's first load, so it has landed: use it now (a register load still
    // in flight across the loop would make the compiler drain the copies at every group)
    asm volatile("" : "+v"(epoch0));  // consumed here, so the compiler cannot sink the use past the loop
    const uint32_t tag0 = epoch0 + 1u;

    // a group's operands in registers: its weight words, (z, s) words and activation operands
    struct Ops {
        u2 q[RR];
        uint32_t zs[RR];
        h8 b[2][TT];
    };
    auto read_ops = [&](const uint8_t* st, Ops& o) {
#pragma unroll
        for (int rr = 0; rr < RR; ++rr) {
            o.q[rr] = *reinterpret_cast<const u2*>(st + W_AT + (RR * rw + rr) * 1024 + lane * 16 + 8 * kh);
            o.zs[rr] = *reinterpret_cast<const uint32_t*>(st + Z_AT + rw * 256 + rr * 64 + (lane & 15) * 4);
        }
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) o.b[jj][tt] = *reinterpret_cast<const h8*>(st + tt * 4096 + bofs[jj]);
    };
    auto multiply = [&](const Ops& o) {
#pragma unroll
        for (int rr = 0; rr < RR; ++rr) {
            h2 c1024, c64;
            zero_consts(o.zs[rr], c1024, c64);
            const _Float16 sc = as_h2(o.zs[rr])[1];
            const h8 s8 = h8{sc, sc, sc, sc, sc, sc, sc, sc};
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const h8 a = nib8_minus_z(o.q[rr][jj], c1024, c64, nc) * s8;
#pragma unroll
                for (int tt = 0; tt < TT; ++tt) acc[tt][rr] = mfma16(a, o.b[jj][tt], acc[tt][rr]);
            }
        }
    };
    int k = 0;  // stage of group g
    if constexpr (TT == 2) {
        // 32-token tile: the operands are read one group ahead, right after the barrier that shows
        // their stage has landed, so that the reads overlap the previous group's unpacking and
        // matrix-core steps (2-4 % faster per call; with 64 tokens, whose reads take as long as the
        // matrix-core steps, it was 3-5 % slower).  One group: issue the copies of g + NST - 1 (into
        // the stage of group g - 1, whose reads every wave completed before the last barrier), wait
        // until the copies of g + 1 have landed (at most those of g + 2 .. g + NST - 1 in flight) and
        // this wave's LDS reads are complete, read g + 1's operands into `nxt`, multiply g's `cur`.
        auto step = [&](int g, const Ops& cur, Ops& nxt) {
            copy(g + NST - 1, sp(k == 0 ? NST - 1 : k - 1));
            const int kn = k == NST - 1 ? 0 : k + 1;
            __builtin_amdgcn_s_waitcnt(vm_lgkm0_imm(S::WAIT));
            __builtin_amdgcn_s_barrier();
            read_ops(sp(kn), nxt);  // after the last group: the stage's clamped copy, never used
            __builtin_amdgcn_sched_barrier(0);  // the reads stay ahead of this group's work
            multiply(cur);
            k = kn;
        };
        // two register sets in turn (no copies between them)
        Ops opa, opb;
        read_ops(sp(0), opa);
        int g = g0;
        for (; g + 1 < g1; g += 2) {
            step(g, opa, opb);
            step(g + 1, opb, opa);
        }
        if (g < g1) step(g, opa, opb);
    } else {
        for (int g = g0; g < g1; ++g) {
            // the copies of g + NST - 1 go to the stage read in group g - 1 (done: the barrier below)
            copy(g + NST - 1, sp(k == 0 ? NST - 1 : k - 1));
            Ops cur;
            read_ops(sp(k), cur);
            multiply(cur);
            // the copies of g + 1 have landed once at most those of g + 2 .. g + NST - 1 are in flight
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(S::WAIT));
            __builtin_amdgcn_s_barrier();
            k = k == NST - 1 ? 0 : k + 1;
        }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no copy may land in LDS after this point
    __syncthreads();

    // the second K half hands its sums to the first through LDS; the first adds them (fixed order)
    f4* red = reinterpret_cast<f4*>(stg);
    if (kh == 1) {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
            for (int rr = 0; rr < RR; ++rr) red[((rw * TT + tt) * RR + rr) * 64 + lane] = acc[tt][rr];
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
            for (int rr = 0; rr < RR; ++rr) acc[tt][rr] += red[((rw * TT + tt) * RR + rr) * 64 + lane];
    }
    __syncthreads();  // the sums are read before the ring is reused

    // thread 0 arrives (after its epoch read: the value was used before the loop) and counts its
    // slot, and hands the tag to the workgroup through LDS
    int arrived = 0;
    if (threadIdx.x == 0) {
        *reinterpret_cast<uint32_t*>(stg + SB - 4) = tag0;
        arrived = arrive_slot(args, arrive(args));
    }
    {
        __syncthreads();
        const uint32_t tag = *reinterpret_cast<const uint32_t*>(stg + SB - 4);
        if (M.a != nullptr && ks_idx == 0) {
            // the tile's projection rows in LDS as fp16 (the producers' pairs, waited for by all
            // threads at once; token tile tt in stage tt), then r_pad / 32 more matrix-core steps
            // by the first K half
            const int r = args.r, rp = args.r_pad;
            const u64* Rp = reinterpret_cast<const u64*>(args.R) +
                            (size_t)(blockIdx.x & (kRReplicas - 1)) * args.n_proj * T * r + (size_t)M.proj * T * r;
            for (int e = tid; e < 16 * TT * rp; e += 64 * kMidWaves) {
                const int t = e / rp, col = e - t * rp;
                _Float16* rl = reinterpret_cast<_Float16*>(sp(t >> 4));
                rl[(t & 15) * rp + col] = (_Float16)((t < T && col < r) ? load_pair(args, Rp + (size_t)t * r + col, tag) : 0.f);
            }
            __syncthreads();
            if (kh == 0) {
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
                        const _Float16* rl = reinterpret_cast<const _Float16*>(sp(tt));
                        const h8 bv = *reinterpret_cast<const h8*>(rl + (lane & 15) * rp + col);
#pragma unroll
                        for (int rr = 0; rr < RR; ++rr) acc[tt][rr] = mfma16(av[rr], bv, acc[tt][rr]);
                    }
                }
            }
        }
    }

    if (kh == 0) {
        const bool vec = (M.n_out & 3) == 0;
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            const int t = 16 * tt + (lane & 15);
            if (t >= T) continue;
            _Float16* yrow = M.y + (size_t)t * M.n_out;
#pragma unroll
            for (int rr = 0; rr < RR; ++rr) {
                if (rt0 + rr >= NT) continue;
                const int row0 = (rt0 + rr) * 16 + 4 * (lane >> 4);
                const f4 v = acc[tt][rr];
                if (split) {  // the range's fp32 partial sums; the reduce launch adds them in order
                    float* pp = args.ypart + ((size_t)ks_idx * T + t) * args.rows_total + M.row_begin + row0;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (row0 + e < M.n_out) pp[e] = v[e];
                } else if (vec && row0 + 3 < M.n_out) {
                    const h2 lo = {(_Float16)v[0], (_Float16)v[1]}, hi = {(_Float16)v[2], (_Float16)v[3]};
                    *reinterpret_cast<u2*>(yrow + row0) = u2{as_u32(lo), as_u32(hi)};
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (row0 + e < M.n_out) yrow[row0 + e] = (_Float16)v[e];
                }
            }
        }
    }
    if (threadIdx.x == 0) finish(args, arrived, tag0 - 1u);
}

hipError_t launch_mid(const ForwardArgs& a, hipStream_t stream) {
    // correcting calls only: the projection comes from the producers of the same launch
    if (a.fmt != kFmtInt4 || a.m_tiles != 1 || a.T > 16 * a.tile_tt || a.tile_rr != 8) return hipErrorInvalidValue;
    if (a.r <= 0 || a.n_prod <= 0) return hipErrorInvalidValue;
    if (a.dec_ks < 1 || a.dec_gk < 1 || a.n_tiles != a.dec_tiles * a.dec_ks || (a.dec_ks - 1) * a.dec_gk >= a.G ||
        (int64_t)a.dec_ks * a.dec_gk < a.G || (a.dec_ks > 1 && a.ypart == nullptr))
        return hipErrorInvalidValue;
    const dim3 grid(a.n_tiles + a.n_prod), block(64 * kMidWaves);
    if (a.tile_tt == 4)
        hipLaunchKernelGGL((mid_kernel<4, 2>), grid, block, 0, stream, a);
    else if (a.tile_tt == 2)
        hipLaunchKernelGGL((mid_kernel<2, 2>), grid, block, 0, stream, a);
    else
        return hipErrorInvalidValue;
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    return a.dec_ks > 1 ? launch_part_reduce(a, stream) : hipSuccess;
}

template <int F, bool FUSE>
static hipError_t launch_prefill_small(const ForwardArgs& a, hipStream_t stream) {
    const dim3 grid(a.n_tiles + (FUSE ? a.n_prod : 0));
    if (a.tile_rr == 1) {  // small grids: 64 or 32 tokens x 64 rows, 4 wave groups
        if (a.tile_ks != 4 || (a.tile_tt != 4 && a.tile_tt != 2)) return hipErrorInvalidValue;
        if (a.tile_tt == 4)
            hipLaunchKernelGGL((prefill_kernel<F, 4, 1, 4, FUSE>), grid, dim3(1024), 0, stream, a);
        else
            hipLaunchKernelGGL((prefill_kernel<F, 2, 1, 4, FUSE>), grid, dim3(1024), 0, stream, a);
        return hipGetLastError();
    }
    if (a.tile_tt != 4 || a.tile_rr != 2) return hipErrorInvalidValue;
    if (a.tile_ks == 4) {
        // the fused form of this tile would need more than the 128 registers of a 1024-thread
        // workgroup; the launcher gives fused calls two wave groups instead
        if constexpr (FUSE) return hipErrorInvalidValue;
        else hipLaunchKernelGGL((prefill_kernel<F, 4, 2, 4, FUSE>), grid, dim3(1024), 0, stream, a);
    }
    else if (a.tile_ks == 2)
        hipLaunchKernelGGL((prefill_kernel<F, 4, 2, 2, FUSE>), grid, dim3(512), 0, stream, a);
    else if (a.tile_ks == 1)
        hipLaunchKernelGGL((prefill_kernel<F, 4, 2, 1, FUSE>), grid, dim3(256), 0, stream, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

template <int F>
static hipError_t launch_prefill_fmt(const ForwardArgs& a, hipStream_t stream) {
    if (a.tile_rr == 4) {
        // the wide tile takes R from a projection launch; MXFP6 runs it with 64 tokens (its 32-value
        // conversions would not fit beside 128 tokens' sums)
        if (a.n_prod > 0 || a.tile_tt != (Fmt<F>::six ? 4 : 8)) return hipErrorInvalidValue;
        constexpr int TT = Fmt<F>::six ? 4 : 8;
        hipLaunchKernelGGL((prefill_wide_kernel<F, TT>), dim3(a.n_tiles), dim3(256), 2 * TT * 4 * 64 * sizeof(u4), stream, a);
        return hipGetLastError();
    }
    return a.n_prod > 0 ? launch_prefill_small<F, true>(a, stream) : launch_prefill_small<F, false>(a, stream);
}

hipError_t launch_prefill(const ForwardArgs& a, hipStream_t stream) {
    switch (a.fmt) {
        case kFmtInt4: return launch_prefill_fmt<kFmtInt4>(a, stream);
        case kFmtMxfp4: return launch_prefill_fmt<kFmtMxfp4>(a, stream);
        case kFmtMxfp6E2M3: return launch_prefill_fmt<kFmtMxfp6E2M3>(a, stream);
        case kFmtMxfp6E3M2: return launch_prefill_fmt<kFmtMxfp6E3M2>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace glowq
