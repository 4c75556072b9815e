// Decode path (T <= 64 tokens): one launch per group call, fusing the shared projection, the
// dequant-in-register INT4 product on the matrix cores and the correction epilogue.
//
// For an input-sharing group every module's rows are one launch; module i's output is
//   y_i = X W_hat_i^T + R_p A_i^T,   R_p = X B_p^T  (p = 0 for the shared factor)
// (GlowQ paper note, key design 4 and the flowchart's last node: the anchor forms R once, every
// module consumes it).  In this launch the anchor's role is played by the first n_prod
// workgroups ("producers"): they compute R in fp32 and write it to the workspace as (value, tag)
// pairs, each pair one 64-bit store, the tag being the call's epoch + 1.  The other workgroups
// ("consumers") each own one 16-row tile of the concatenated modules: they stream their INT4
// weights first and read R only for the epilogue, polling the pairs themselves until every tag is
// current -- one coherent read both waits for and fetches R, and producers need no fence or
// counter.  Producers have the lowest workgroup ids and never wait, so they are dispatched before
// any consumer and always finish; every wait is bounded and raises a flag in the workspace header
// if it expires.
// Epoch: every workgroup reads it as its first load and then "arrives" (64 slot counters, then one
// counter over the slots); the last arrival of the launch resets the counters and advances the
// epoch, so stale pairs never match and no memset is ever needed.  Consumers arrive right after
// their first loads are issued and producers when their first sums are ready, so the counting
// overlaps the weight stream instead of lengthening the launch's tail.

// Main loop: the K dimension (input groups of 128) is split across the 4 wavefronts of a tile
// (group g goes to wave g % 4).  Each wave keeps a ring of U groups in flight (4 per row tile;
// deeper rings measured slower: the registers they take cost more than the extra loads gain):
// one 16-byte load per lane brings a whole group (16 rows x 128 inputs) in matrix-core operand
// order; after a group is consumed its slot is refilled with the group U ahead.  Nibbles become exact fp16
// (q - z) values in registers; four v_mfma_f32_16x16x32_f16 accumulate the group's partial sums
// against the tokens (padded to 16 per tile); the per-(row, group) scale is applied once per group
// in fp32.  The correction A_i R is r_pad / 32 more matrix-core steps shared out over the waves
// (R rounded once to fp16 for them, as in the prefill path; each wave's first A operand is loaded
// with the weight ring, 9 % faster per restored launch than loading A and adding in fp32 after the
// main loop).  The four waves' partial sums, each carrying its share of the correction terms, are
// reduced in LDS in a fixed order (deterministic) and rounded once to fp16.
#include "handoff.h"

namespace glowq {

// Producer workgroup p: rows [pr prod_rows, (pr + 1) prod_rows) of the stacked projections (row
// jj = projection jj / r, rank index jj % r) for the TT-token tile tt of the call's tokens, with
// p = pr n_tt + tt; fp32 accumulation of exact fp16 products, fixed-order block reduction, each
// value stored as a tagged pair.  Per 8-input chunk a thread reads the B chunk and the tile's TT
// token chunks (rows past T re-read the last token and are never stored) before any product, so
// a chunk costs one memory round trip, not one per token.
template <int KW, int TT>
__device__ void produce(const ForwardArgs& a, int p) {
    constexpr int NTH = 64 * KW;
    __shared__ float part[KW][16];
    __shared__ uint32_t ptag;
    // the epoch is thread 0's first load; the workgroup arrives (once) when its first partial sums
    // are ready, by which time the read has long completed
    uint32_t epoch0 = 0;
    if (threadIdx.x == 0) epoch0 = load_epoch(a);
    int arrived = 0;
    bool first = true, scrub = true;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int T = a.T, d = a.d, r = a.r;
    u64* R = reinterpret_cast<u64*>(a.R);
    const int total = a.n_proj * r;
    const int n_tt = (T + TT - 1) / TT;
    const int pr = p / n_tt, t0 = (p - pr * n_tt) * TT;
    const int nt = min(TT, T - t0);
    const int j0 = pr * a.prod_rows;
    const int j1 = min(j0 + a.prod_rows, total);
    const int n8 = d / 8;
    for (int jj = j0; jj < j1; ++jj) {
        const int pi = jj / r, j = jj - pi * r;
        const _Float16* brow = pick_bp(a, pi) + (size_t)j * d;
        float acc[TT];
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[t] = 0.f;
        for (int c = threadIdx.x; c < n8; c += NTH) {
            const h8 bv = load_h8(brow + 8 * c);
            h8 xv[TT];
#pragma unroll
            for (int t = 0; t < TT; ++t) xv[t] = load_h8(a.x + (size_t)(t0 + min(t, nt - 1)) * d + 8 * c);
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                float s = acc[t];
#pragma unroll
                for (int e = 0; e < 8; ++e) s = fmaf((float)bv[e], (float)xv[t][e], s);
                acc[t] = s;
            }
        }
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            float v = acc[t];
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
            acc[t] = v;
        }
        if (lane == 0) {
#pragma unroll
            for (int t = 0; t < TT; ++t) part[wave][t] = acc[t];
        }
        if (first) {
            if (threadIdx.x == 0) {
                ptag = epoch0 + 1u;
                // the epoch read must be complete before this workgroup's arrival can count: a
                // relaxed load and a relaxed atomic to another address are not ordered, so wait
                // for the load here (the compiler may not move memory operations across this)
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                arrived = arrive(a);
            }
            first = false;
        }
        __syncthreads();
        const uint32_t tag = ptag;
        if (scrub && (tag == 1u || tag == 0xFFFFFFFFu)) {
            // first and last tag of a wrap: clear every pair of the decode area outside this
            // call's range (no one reads them in this call)
            const size_t from = (size_t)kRReplicas * a.n_proj * T * r;
            for (size_t k = from + (size_t)p * NTH + threadIdx.x; k < kDecodeAreaPairs; k += (size_t)a.n_prod * NTH)
                R[k] = 0ull;
        }
        scrub = false;
        if ((int)threadIdx.x < nt) {
            const int t = threadIdx.x;
            float v = part[0][t];
#pragma unroll
            for (int w = 1; w < KW; ++w) v += part[w][t];
            const size_t off = ((size_t)pi * T + t0 + t) * r + j, copy = (size_t)a.n_proj * T * r;
#pragma unroll
            for (int c = 0; c < kRReplicas; ++c) store_pair(R + c * copy + off, v, tag);
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) finish(a, arrive_slot(a, arrived), epoch0);
}

// NTT: 16-token tiles.  RT: 16-row tiles per workgroup, multiplied side by side against the same
// activation operand (one workgroup per RT tiles of one module).  KW: waves per workgroup; K (the
// 128-input groups) is split across them, group g going to wave g % KW.
// XC > 0: the tokens' activations (T x d fp16, at most kDecodeXLdsMax bytes) are staged once in
// LDS with XC 16-byte loads per thread, issued before the weight loads so that waiting for them
// does not wait for the weights; lanes of padding tokens read an all-zero LDS row, so the B operand
// needs no masking.  XC == 0: each group's B operand is loaded from global memory together with
// the group's weights.
template <int F, int NTT, int XC, int KW, int RT>
__global__ __launch_bounds__(64 * KW) __attribute__((amdgpu_waves_per_eu((XC > 0 && KW == 4) ? (RT == 2 ? 3 : 4) : 1))) void decode_kernel(const ForwardArgs args) {
    constexpr bool XLDS = XC > 0;
    constexpr bool MX = Fmt<F>::mx, SIX = Fmt<F>::six;
    constexpr int QB = Fmt<F>::qblock;
    constexpr int NTH = 64 * KW;
    constexpr int U = NTT == 1 ? 4 / RT : 1;  // ring of groups per wave
    static_assert(U >= 1, "ring");
    __shared__ f4 red[KW][RT][NTT][64];
    extern __shared__ __attribute__((aligned(16))) _Float16 xs[];

    if ((int)blockIdx.x < args.n_prod) {
        // token tile of a producer: one token, up to 4, or 16 (the launcher sizes n_prod to match)
        if (args.T == 1)
            produce<KW, 1>(args, blockIdx.x);
        else if (args.T <= 4)
            produce<KW, 4>(args, blockIdx.x);
        else
            produce<KW, 16>(args, blockIdx.x);
        return;
    }
    // consumer workgroup: row block `tile`, K range `ks_idx` (one range unless the launch splits K)
    const int tile_all = blockIdx.x - args.n_prod;
    const int ks_idx = tile_all / args.dec_tiles;
    const int tile = tile_all - ks_idx * args.dec_tiles;
    const ModuleArgs M = args.mod[module_of(args, tile)];
    const int rt0 = (tile - M.tile_begin) * RT;  // first 16-row tile of this workgroup
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar branches
    const int G = args.G, T = args.T, d = args.d;
    const uint8_t* qbase[RT];
    const uint8_t* szbase[RT];
#pragma unroll
    for (int rr = 0; rr < RT; ++rr) {
        const int rt = min(rt0 + rr, M.n_tiles16 - 1);  // a tile past the module end rereads the last
        qbase[rr] = M.q + (size_t)rt * QB + lane * 16;
        szbase[rr] = M.sz + (size_t)rt * 64;
    }
    const size_t qstride = (size_t)M.n_tiles16 * QB, szstride = (size_t)M.n_tiles16 * 64;  // per group
    // MXFP6: the second plane of a lane's codes (8 bytes at 1024 + 8 lane of the block)
    const int q6ofs = 1024 + 8 * lane - 16 * lane;
    const int kofs = Fmt<F>::xofs(lane >> 4);  // the lane's activation operand within a group
    constexpr int XS = Fmt<F>::xstep;          // and its step per matrix-core slice
    const h8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
    const NibConsts nc = nib_consts();
    const int g0 = ks_idx * args.dec_gk, g1 = min(G, g0 + args.dec_gk);  // this workgroup's groups
    const int n_my = g1 - g0 > wave ? (g1 - g0 - wave + KW - 1) / KW : 0;  // g = g0 + wave + KW i
    const bool hand = args.n_prod > 0;  // correcting launch: R hand-off and epoch protocol
    // with a K split the partial sums go to the workspace (the first K range carrying the
    // correction) and a second launch adds them
    const bool split = args.dec_ks > 1;
    const bool correct = hand && M.a != nullptr && ks_idx == 0;
    const int r = args.r;
    // the epoch: one read per workgroup, the first load of thread 0 (so that waiting for it never
    // waits for weights), handed to the other waves through LDS
    __shared__ uint32_t tag_lds;
    uint32_t epoch0 = 0;
    if (hand && threadIdx.x == 0)
        epoch0 = (uint32_t)__hip_atomic_load(args.sync + kSyncEpoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    const _Float16* xrow[NTT];
    bool tok_ok[NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
        const int t = 16 * tt + (lane & 15);
        tok_ok[tt] = t < T;
        if (XLDS)
            xrow[tt] = xs + (size_t)(tok_ok[tt] ? t : T) * d + kofs;  // row T is all zeros
        else
            xrow[tt] = args.x + (size_t)(tok_ok[tt] ? t : 0) * d + kofs;
    }

    // activations first: slot c * NTH + tid of the (T + 1) x d LDS block, clamped to the last slot
    // (the tail rewrites a slot with its own value); slots past T x d are the zero row.
    const int n8x = T * d / 8, n8 = (T + 1) * d / 8;
    u4 xst[XLDS ? XC : 1];
    if (XLDS) {
#pragma unroll
        for (int c = 0; c < XC; ++c) {
            const int idx = min(c * NTH + (int)threadIdx.x, n8 - 1);
            const u4 v = reinterpret_cast<const u4*>(args.x)[min(idx, n8x - 1)];
            xst[c] = idx < n8x ? v : u4{0u, 0u, 0u, 0u};
        }
    }

    u4 qv[U][RT];
    u2 qv6[SIX ? U : 1][RT];
    uint32_t zso[U][RT];  // INT4: the row's (z, s) pair; MX: the row's four block scales
    u4 zs4[MX ? 1 : U][RT];
    h8 bx[XLDS ? 1 : U][NTT][4];
    auto issue = [&](int u, int i) {
        const int g = min(g0 + wave + KW * i, g1 - 1);  // always a valid group of this workgroup
        if (!XLDS) {
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const h8 v = load_h8(xrow[tt] + (size_t)g * kGroup + XS * j);
                    bx[XLDS ? 0 : u][tt][j] = tok_ok[tt] ? v : zero8;
                }
        }
#pragma unroll
        for (int rr = 0; rr < RT; ++rr) {
            qv[u][rr] = __builtin_nontemporal_load(reinterpret_cast<const u4*>(qbase[rr] + (size_t)g * qstride));
            if constexpr (SIX)
                qv6[SIX ? u : 0][rr] = __builtin_nontemporal_load(
                    reinterpret_cast<const u2*>(qbase[rr] + (size_t)g * qstride + q6ofs));
            zso[u][rr] = *reinterpret_cast<const uint32_t*>(szbase[rr] + (size_t)g * szstride + (lane & 15) * 4);
            if constexpr (!MX)
                zs4[MX ? 0 : u][rr] = *reinterpret_cast<const u4*>(szbase[rr] + (size_t)g * szstride + (lane >> 4) * 16);
        }
    };

    f4 acc[RT][NTT];
#pragma unroll
    for (int rr = 0; rr < RT; ++rr)
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) acc[rr][tt] = f4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int u, int i) {
        const int g = g0 + wave + KW * i;
        // activation operands first: the LDS reads complete while the weights are unpacked
        h8 bl[XLDS ? NTT : 1][4];
        if (XLDS) {
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    bl[XLDS ? tt : 0][j] = *reinterpret_cast<const h8*>(xrow[tt] + (size_t)g * kGroup + XS * j);
            __builtin_amdgcn_sched_barrier(0);
        }
        h8 aop[RT][4];
        if constexpr (MX) {
            // MX: the operands carry their block scales (exact fp16), so the matrix cores
            // accumulate straight into the running sums
#pragma unroll
            for (int rr = 0; rr < RT; ++rr) {
                const float sc = mx_scale(zso[u][rr], lane >> 4);  // the lane's MX block
                if constexpr (SIX) {
                    const h32 e = mx6_h32<F>(qv[u][rr], qv6[SIX ? u : 0][rr], sc);
#pragma unroll
                    for (int j = 0; j < 4; ++j) aop[rr][j] = mx6_slice(e, j);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) aop[rr][j] = mx4_h8(qv[u][rr][j], sc);
                }
            }
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const h8 b = XLDS ? bl[XLDS ? tt : 0][j] : bx[XLDS ? 0 : u][tt][j];
#pragma unroll
                    for (int rr = 0; rr < RT; ++rr) acc[rr][tt] = mfma16(aop[rr][j], b, acc[rr][tt]);
                }
            return;
        }
#pragma unroll
        for (int rr = 0; rr < RT; ++rr) {
            h2 c1024, c64;
            zero_consts(zso[u][rr], c1024, c64);
#pragma unroll
            for (int j = 0; j < 4; ++j) aop[rr][j] = nib8_minus_z(qv[u][rr][j], c1024, c64, nc);
        }
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
            f4 part[RT];
#pragma unroll
            for (int rr = 0; rr < RT; ++rr) part[rr] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const h8 b = XLDS ? bl[XLDS ? tt : 0][j] : bx[XLDS ? 0 : u][tt][j];
#pragma unroll
                for (int rr = 0; rr < RT; ++rr) part[rr] = mfma16(aop[rr][j], b, part[rr]);
            }
#pragma unroll
            for (int rr = 0; rr < RT; ++rr)
#pragma unroll
                for (int k = 0; k < 4; ++k) acc[rr][tt][k] += (float)as_h2(zs4[MX ? 0 : u][rr][k])[1] * part[rr][k];
        }
    };

    // prologue: fill the ring (indices past the wave's last group reload that group)
#pragma unroll
    for (int u = 0; u < U; ++u) issue(u, min(u, max(n_my - 1, 0)));
    // with the ring: the A operand of this wave's first correction step (rank columns
    // 32 wave .. 32 wave + 31), so that its latency is hidden by the weight stream
    h8 apre[RT];
#pragma unroll
    for (int rr = 0; rr < RT; ++rr) {
        const int row = (rt0 + rr) * 16 + (lane & 15);
        const int col = 32 * wave + 8 * (lane >> 4);
        apre[rr] = (correct && row < M.n_out && col < r) ? load_h8(M.a + (size_t)row * r + col) : zero8;
    }
    if (XLDS) {
#pragma unroll
        for (int c = 0; c < XC; ++c) {
            const int idx = min(c * NTH + (int)threadIdx.x, n8 - 1);
            reinterpret_cast<u4*>(xs)[idx] = xst[c];
        }
    }
    // the workgroup arrives once thread 0 holds the epoch (every wave reads it after the barrier)
    int arrived = 0, top_prev = -1;
    if (hand) {
        if (threadIdx.x == 0) tag_lds = epoch0 + 1u;  // needs the epoch load's value
        __syncthreads();  // a fence: the arrival below is not moved above the epoch's use
        if (threadIdx.x == 0) arrived = arrive(args);
    } else if (XLDS) {
        __syncthreads();
    }
    const uint32_t tag = hand ? tag_lds : 0u;

    if (n_my > 0) {
        int i0 = 0;
        // steady state: consume slot u, refill it with the group U ahead (clamped)
        for (; i0 + U < n_my; i0 += U) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                compute(u, i0 + u);
                issue(u, min(i0 + U + u, n_my - 1));
            }
        }
        // the arrival's count has returned by now: the slot's last arrival counts the slot before
        // the drain rather than at the tail
        if (hand && threadIdx.x == 0) top_prev = arrive_slot(args, arrived);
        // drain
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (i0 + u < n_my) compute(u, i0 + u);
    } else if (hand && threadIdx.x == 0) {
        top_prev = arrive_slot(args, arrived);
    }

    // correction epilogue on the matrix cores: acc += A_i[rows][32 kb .. +32) R[tokens][32 kb .. +32)^T
    // for the K steps kb = wave, wave + KW, ... (A operand: 16 rows x 32 rank columns straight
    // from A_i; B operand: R rounded once to fp16, as in the prefill path).  With one token tile R
    // is copied once into LDS (coherent 8-byte pair reads of this workgroup's copy, which also
    // wait for the producers) and read from there; otherwise each element is read as a pair.
    if (correct) {
        const u64* Rp = reinterpret_cast<const u64*>(args.R) +
                        (size_t)(blockIdx.x & (kRReplicas - 1)) * args.n_proj * T * r + (size_t)M.proj * T * r;
        float* rl = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(xs) + args.r_lds_off);
        if (NTT == 1) {
            for (int k = threadIdx.x; k < T * r; k += NTH) rl[k] = load_pair(args, Rp + k, tag);
            __syncthreads();
        }
        for (int kb = wave; kb * 32 < r; kb += KW) {
            const int col = 32 * kb + 8 * (lane >> 4);  // r % 8 == 0: col < r covers col .. col + 7
            h8 aop[RT];
#pragma unroll
            for (int rr = 0; rr < RT; ++rr) {
                const int row = (rt0 + rr) * 16 + (lane & 15);
                aop[rr] = kb == wave ? apre[rr]
                                     : ((row < M.n_out && col < r) ? load_h8(M.a + (size_t)row * r + col) : zero8);
            }
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
                const int t = 16 * tt + (lane & 15);
                h8 bop = zero8;
                if (t < T && col < r) {
                    if (NTT == 1) {
                        const f4* rp = reinterpret_cast<const f4*>(rl + (size_t)t * r + col);
                        const f4 r0 = rp[0], r1 = rp[1];
                        bop = h8{(_Float16)r0[0], (_Float16)r0[1], (_Float16)r0[2], (_Float16)r0[3],
                                 (_Float16)r1[0], (_Float16)r1[1], (_Float16)r1[2], (_Float16)r1[3]};
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) bop[e] = (_Float16)load_pair(args, Rp + (size_t)t * r + col + e, tag);
                    }
                }
#pragma unroll
                for (int rr = 0; rr < RT; ++rr) acc[rr][tt] = mfma16(aop[rr], bop, acc[rr][tt]);
            }
        }
    }

#pragma unroll
    for (int rr = 0; rr < RT; ++rr)
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) red[wave][rr][tt][lane] = acc[rr][tt];
    __syncthreads();
    // wave w stores (row tile, token tile) pairs w, w + KW, ...
    for (int job = wave; job < RT * NTT; job += KW) {
        const int rr = job / NTT, tt = job % NTT;
        f4 v = red[0][rr][tt][lane];
#pragma unroll
        for (int w = 1; w < KW; ++w) v += red[w][rr][tt][lane];  // fixed order: deterministic
        const int t = 16 * tt + (lane & 15);
        const int row0 = (rt0 + rr) * 16 + 4 * (lane >> 4);
        if (split && t < T && rt0 + rr < M.n_tiles16) {
            float* pp = args.ypart + ((size_t)ks_idx * T + t) * args.rows_total + M.row_begin + row0;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (row0 + i < M.n_out) pp[i] = v[i];
        } else if (t < T && rt0 + rr < M.n_tiles16) {
            _Float16 o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = (_Float16)v[i];
            _Float16* yp = M.y + (size_t)t * M.n_out + row0;
            if ((M.n_out & 3) == 0 && row0 + 3 < M.n_out) {
                h2 lo = {o[0], o[1]}, hi = {o[2], o[3]};
                *reinterpret_cast<u2*>(yp) = u2{as_u32(lo), as_u32(hi)};
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (row0 + i < M.n_out) yp[i] = o[i];
            }
        }
    }
    if (hand && threadIdx.x == 0) finish(args, top_prev, epoch0);
}

// Narrow calls with a K split: y = the K ranges' fp32 partial sums (the first range's carrying the
// correction) added in range order, rounded once to fp16.  One thread per (token, row): rows are
// consecutive across a wave, so every read and write is coalesced.
__global__ __launch_bounds__(256) void decode_reduce_kernel(const ForwardArgs a) {
    const size_t n = (size_t)a.T * a.rows_total;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= n) return;
    const int t = (int)(idx / a.rows_total), row = (int)(idx - (size_t)t * a.rows_total);
    // the module holding this row: field by field selection (no indexed load of the records)
    _Float16* y = a.mod[0].y;
    int n_out = a.mod[0].n_out, row_begin = 0;
#pragma unroll
    for (int k = 1; k < kMaxModules; ++k) {
        const bool in = k < a.n_mod && row >= a.mod[k].row_begin;
        y = in ? a.mod[k].y : y;
        n_out = in ? a.mod[k].n_out : n_out;
        row_begin = in ? a.mod[k].row_begin : row_begin;
    }
    float v = 0.f;
    for (int s = 0; s < a.dec_ks; ++s) v += a.ypart[((size_t)s * a.T + t) * a.rows_total + row];
    y[(size_t)t * n_out + (row - row_begin)] = (_Float16)v;
}

hipError_t launch_part_reduce(const ForwardArgs& a, hipStream_t stream) {
    const size_t n = (size_t)a.T * a.rows_total;
    if (n == 0 || a.ypart == nullptr || a.dec_ks < 2) return hipErrorInvalidValue;
    hipLaunchKernelGGL(decode_reduce_kernel, dim3((unsigned)ceil_div((int64_t)n, 256)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int F, int KW, int RT>
static hipError_t launch_decode_kw(const ForwardArgs& a, hipStream_t stream) {
    constexpr int NTH = 64 * KW;
    const int ntt = (int)ceil_div(a.T, 16);
    const dim3 grid(a.n_prod + a.n_tiles), block(NTH);
    const size_t xbytes = (size_t)(a.T + 1) * a.d * 2;  // tokens + one zero row
    const bool xlds = RT != kNarrowRt && ntt == 1 && xbytes <= kDecodeXLdsMax;
    const size_t xarea = xlds ? (xbytes + 15) / 16 * 16 : 0;
    const size_t rarea = (ntt == 1 && a.r > 0) ? (size_t)a.T * a.r * 4 : 0;
    ForwardArgs b = a;
    b.r_lds_off = (int32_t)xarea;
    const size_t shmem = xarea + rarea;
    if constexpr (RT != kNarrowRt) if (xlds) {
        const int chunks = (int)ceil_div((int64_t)xbytes / 16, NTH);
        if (chunks <= 2)
            hipLaunchKernelGGL((decode_kernel<F, 1, 2, KW, RT>), grid, block, shmem, stream, b);
        else if (chunks <= 4)
            hipLaunchKernelGGL((decode_kernel<F, 1, 4, KW, RT>), grid, block, shmem, stream, b);
        else if (chunks <= 8)
            hipLaunchKernelGGL((decode_kernel<F, 1, 8, KW, RT>), grid, block, shmem, stream, b);
        else
            hipLaunchKernelGGL((decode_kernel<F, 1, (int)(kDecodeXLdsMax / 16 / NTH), KW, RT>), grid, block, shmem,
                               stream, b);
        return hipGetLastError();
    }
    if constexpr (RT == kNarrowRt) {  // K-split narrow calls: 17 .. 64 tokens
        switch (ntt) {
            case 2: hipLaunchKernelGGL((decode_kernel<F, 2, 0, KW, RT>), grid, block, shmem, stream, b); break;
            case 3: hipLaunchKernelGGL((decode_kernel<F, 3, 0, KW, RT>), grid, block, shmem, stream, b); break;
            case 4: hipLaunchKernelGGL((decode_kernel<F, 4, 0, KW, RT>), grid, block, shmem, stream, b); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    if (RT != 1) {  // two row tiles share each activation operand read from L2 (one token tile)
        if (ntt != 1) return hipErrorInvalidValue;
        hipLaunchKernelGGL((decode_kernel<F, 1, 0, KW, RT>), grid, block, shmem, stream, b);
        return hipGetLastError();
    }
    switch (ntt) {
        case 1: hipLaunchKernelGGL((decode_kernel<F, 1, 0, KW, 1>), grid, block, shmem, stream, b); break;
        case 2: hipLaunchKernelGGL((decode_kernel<F, 2, 0, KW, 1>), grid, block, shmem, stream, b); break;
        case 3: hipLaunchKernelGGL((decode_kernel<F, 3, 0, KW, 1>), grid, block, shmem, stream, b); break;
        case 4: hipLaunchKernelGGL((decode_kernel<F, 4, 0, KW, 1>), grid, block, shmem, stream, b); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int F>
static hipError_t launch_decode_fmt(const ForwardArgs& a, hipStream_t stream) {
    if (a.dec_ks > 1) {  // narrow call with a K split: 4 waves, kNarrowRt row tiles, then the sums
        if (a.dec_kw != 4 || a.dec_rt != kNarrowRt) return hipErrorInvalidValue;
        hipError_t e = launch_decode_kw<F, 4, kNarrowRt>(a, stream);
        if (e != hipSuccess) return e;
        return launch_part_reduce(a, stream);
    }
    if (a.dec_kw == 8) return launch_decode_kw<F, 8, 1>(a, stream);
    return a.dec_rt == 2 ? launch_decode_kw<F, 4, 2>(a, stream) : launch_decode_kw<F, 4, 1>(a, stream);
}

hipError_t launch_decode(const ForwardArgs& a, hipStream_t stream) {
    switch (a.fmt) {
        case kFmtInt4: return launch_decode_fmt<kFmtInt4>(a, stream);
        case kFmtMxfp4: return launch_decode_fmt<kFmtMxfp4>(a, stream);
        case kFmtMxfp6E2M3: return launch_decode_fmt<kFmtMxfp6E2M3>(a, stream);
        case kFmtMxfp6E3M2: return launch_decode_fmt<kFmtMxfp6E3M2>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace glowq
