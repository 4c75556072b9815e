// Decode path (T <= 64 tokens): one launch per group call, fusing the shared projection, the
// dequant-in-register INT4 product on the matrix cores and the correction epilogue.
//
// For an input-sharing group every module's rows are one launch; module i's output is
//   y_i = X W_hat_i^T + R_p A_i^T,   R_p = X B_p^T  (p = 0 for the shared factor)
// (GlowQ paper note, key design 4 and the flowchart's last node: the anchor forms R once, every
// module consumes it).  In this launch the anchor's role is played by the first n_prod
// workgroups ("producers"): they compute R in fp32 into the workspace and publish it with an
// agent-scope release.  The other workgroups ("consumers") each own one 16-row tile of the
// concatenated modules: they stream their INT4 weights first and look at R only for the
// epilogue, so the projection overlaps the weight stream.  Producers have the lowest workgroup
// ids and never wait, so they are dispatched before any consumer and always finish; every wait is
// bounded and raises a flag in the workspace header if it expires.  The hand-off counters are
// replicated per XCD (consumer b uses copy b % 8) so that polls and arrivals spread over eight
// addresses; the last consumer of each copy resets it, leaving the workspace ready for the next
// call without a memset.
//
// Main loop: the K dimension (input groups of 128) is split across the 4 wavefronts of a tile
// (group g goes to wave g % 4).  Each wave keeps a ring of U groups in flight: one 16-byte load
// per lane brings a whole group (16 rows x 128 inputs) in matrix-core operand order; after a
// group is consumed its slot is refilled with the group U ahead.  Nibbles become exact fp16
// (q - z) values in registers; four v_mfma_f32_16x16x32_f16 accumulate the group's partial sums
// against the tokens (padded to 16 per tile); the per-(row, group) scale is applied once per group
// in fp32.  The four waves' partial sums, each carrying its share of the correction terms, are
// reduced in LDS in a fixed order (deterministic) and rounded once to fp16.
#include "glowq_internal.h"

namespace glowq {

__device__ __forceinline__ void pick_module(const ForwardArgs& a, int tile, ModuleArgs& m) {
    m = a.mod[0];
#pragma unroll
    for (int i = 1; i < kMaxModules; ++i)
        if (i < a.n_mod && tile >= a.mod[i].tile_begin) m = a.mod[i];
}

__device__ __forceinline__ const _Float16* pick_bp(const ForwardArgs& a, int i) {
    const _Float16* b = a.b[0];
#pragma unroll
    for (int k = 1; k < kMaxModules; ++k)
        if (k == i) b = a.b[k];
    return b;
}

// Number of workgroup ids b in [lo, hi) with b % 8 == x.
__device__ __forceinline__ int count_mod8(int lo, int hi, int x) {
    const int first = lo + (((x - (lo & 7)) % 8) + 8) % 8;
    return first < hi ? (hi - 1 - first) / 8 + 1 : 0;
}

// Producer workgroup: rows [p * prod_rows, (p+1) * prod_rows) of the stacked projections
// (row jj = projection jj / r, rank index jj % r), all tokens; fp32 accumulation of exact fp16
// products, fixed-order block reduction.  Only wave 0 stores R (threads 0..15), so only wave 0
// issues the agent-scope release before the counters are bumped.
__device__ void produce(const ForwardArgs& a, int p) {
    constexpr int C = 4;  // 8-input chunks per thread in flight
    __shared__ float part[4][16];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int T = a.T, d = a.d, r = a.r;
    float* R = reinterpret_cast<float*>(a.R);
    const int total = a.n_proj * r;
    const int j0 = p * a.prod_rows;
    const int j1 = min(j0 + a.prod_rows, total);
    const int n8 = d / 8;
    for (int jj = j0; jj < j1; ++jj) {
        const int pi = jj / r, j = jj - pi * r;
        const _Float16* brow = pick_bp(a, pi) + (size_t)j * d;
        for (int t0 = 0; t0 < T; t0 += 16) {
            const int nt = min(16, T - t0);
            float acc[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) acc[t] = 0.f;
            for (int c0 = threadIdx.x; c0 < n8; c0 += 256 * C) {
                h8 bv[C];
#pragma unroll
                for (int k = 0; k < C; ++k) {
                    const int c = min(c0 + 256 * k, n8 - 1);
                    bv[k] = load_h8(brow + 8 * c);
                }
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    if (t < nt) {
                        h8 xv[C];
#pragma unroll
                        for (int k = 0; k < C; ++k) {
                            const int c = min(c0 + 256 * k, n8 - 1);
                            xv[k] = load_h8(a.x + (size_t)(t0 + t) * d + 8 * c);
                        }
                        float s = acc[t];
#pragma unroll
                        for (int k = 0; k < C; ++k) {
                            if (c0 + 256 * k < n8) {
#pragma unroll
                                for (int e = 0; e < 8; ++e) s = fmaf((float)bv[k][e], (float)xv[k][e], s);
                            }
                        }
                        acc[t] = s;
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                if (t < nt) {
                    float v = acc[t];
#pragma unroll
                    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
                    acc[t] = v;
                }
            }
            if (lane == 0) {
#pragma unroll
                for (int t = 0; t < 16; ++t) part[wave][t] = acc[t];
            }
            __syncthreads();
            if (threadIdx.x < 16 && (int)threadIdx.x < nt) {
                const int t = threadIdx.x;
                R[((size_t)pi * T + t0 + t) * r + j] = ((part[0][t] + part[1][t]) + part[2][t]) + part[3][t];
            }
            __syncthreads();
        }
    }
    if (wave == 0) {
        // R stores of this wave become visible at agent scope before the counters move
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        if (lane == 0) {
            const int lo = a.n_prod, hi = a.n_prod + a.n_tiles;
#pragma unroll
            for (int x = 0; x < kXcds; ++x)
                if (count_mod8(lo, hi, x) > 0)
                    __hip_atomic_fetch_add(a.sync + kSyncReady + 16 * x, 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Consumer side of the hand-off.  Thread 0 polls its XCD's counter with agent-scope relaxed loads
// (coherent loads, no cache maintenance per poll); R is then read with agent-scope relaxed atomic
// loads, which are served from the coherence point, so no workgroup invalidates its caches.  The
// R loads are issued only after the counter value has come back (control dependence; a wavefront
// issues its memory operations in order), and every producer made its R stores visible at agent
// scope before incrementing the counters.
__device__ __forceinline__ void wait_ready(const ForwardArgs& a) {
    if (threadIdx.x == 0) {
        const int* ready = a.sync + kSyncReady + 16 * (blockIdx.x & 7);
        int spins = 0;
        while (__hip_atomic_load(ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < a.n_prod) {
            __builtin_amdgcn_s_sleep(1);
            if (++spins > kSpinLimit) {
                __hip_atomic_fetch_or(a.sync + kSyncError, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
    }
    __syncthreads();
}

__device__ __forceinline__ float load_r(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void signal_done(const ForwardArgs& a) {
    __syncthreads();
    if (threadIdx.x == 0) {
        const int x = blockIdx.x & 7;
        const int n = count_mod8(a.n_prod, a.n_prod + a.n_tiles, x);
        const int prev = __hip_atomic_fetch_add(a.sync + kSyncDone + 16 * x, 1, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
        if (prev == n - 1) {  // last consumer of this copy: every wait on it is over
            __hip_atomic_store(a.sync + kSyncReady + 16 * x, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.sync + kSyncDone + 16 * x, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// NTT: 16-token tiles.  XC > 0: the tokens' activations (T x d fp16, at most kDecodeXLdsMax bytes)
// are staged once in LDS with XC 16-byte loads per thread, issued before the weight loads so that
// waiting for them does not wait for the weights; lanes of padding tokens read an all-zero LDS row,
// so the B operand needs no masking.  XC == 0: each group's B operand is loaded from global memory
// together with the group's weights.
template <int NTT, int XC>
__global__ __launch_bounds__(256) void decode_kernel(const ForwardArgs args) {
    constexpr bool XLDS = XC > 0;
    constexpr int U = XLDS ? 8 : (NTT == 1 ? 4 : (NTT == 2 ? 2 : 1));  // ring of groups per wave
    __shared__ f4 red[4][NTT][64];
    extern __shared__ __attribute__((aligned(16))) _Float16 xs[];

    if ((int)blockIdx.x < args.n_prod) {
        produce(args, blockIdx.x);
        return;
    }
    const int tile = blockIdx.x - args.n_prod;
    ModuleArgs M;
    pick_module(args, tile, M);
    const int rt = tile - M.tile_begin;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar branches
    const int G = args.G, T = args.T, d = args.d;
    const uint8_t* qbase = M.q + (size_t)rt * G * 1024 + lane * 16;
    const uint8_t* szbase = M.sz + (size_t)rt * G * 64;
    const int kofs = 8 * (lane >> 4);
    const h8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
    const NibConsts nc = nib_consts();
    const int n_my = G > wave ? (G - wave + 3) / 4 : 0;  // groups of this wave: g = wave + 4 i

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

    // activations first: slot c * 256 + tid of the (T + 1) x d LDS block, clamped to the last slot
    // (the tail rewrites a slot with its own value); slots past T x d are the zero row.
    const int n8x = T * d / 8, n8 = (T + 1) * d / 8;
    u4 xst[XLDS ? XC : 1];
    if (XLDS) {
#pragma unroll
        for (int c = 0; c < XC; ++c) {
            const int idx = min(c * 256 + (int)threadIdx.x, n8 - 1);
            const u4 v = reinterpret_cast<const u4*>(args.x)[min(idx, n8x - 1)];
            xst[c] = idx < n8x ? v : u4{0u, 0u, 0u, 0u};
        }
    }

    u4 qv[U];
    uint32_t zso[U];
    u4 zs4[U];
    h8 bx[XLDS ? 1 : U][NTT][4];
    auto issue = [&](int u, int i) {
        const int g = min(wave + 4 * i, G - 1);  // always a valid group of this row tile
        if (!XLDS) {
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const h8 v = load_h8(xrow[tt] + (size_t)g * kGroup + 32 * j);
                    bx[XLDS ? 0 : u][tt][j] = tok_ok[tt] ? v : zero8;
                }
        }
        qv[u] = __builtin_nontemporal_load(reinterpret_cast<const u4*>(qbase + (size_t)g * 1024));
        zso[u] = *reinterpret_cast<const uint32_t*>(szbase + (size_t)g * 64 + (lane & 15) * 4);
        zs4[u] = *reinterpret_cast<const u4*>(szbase + (size_t)g * 64 + (lane >> 4) * 16);
    };

    f4 acc[NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) acc[tt] = f4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int u, int i) {
        const int g = wave + 4 * i;
        h2 c1024, c64;
        zero_consts(zso[u], c1024, c64);
        h8 aop[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) aop[j] = nib8_minus_z(qv[u][j], c1024, c64, nc);
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
            f4 part = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const h8 b = XLDS ? *reinterpret_cast<const h8*>(xrow[tt] + (size_t)g * kGroup + 32 * j)
                                  : bx[XLDS ? 0 : u][tt][j];
                part = mfma16(aop[j], b, part);
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) acc[tt][k] += (float)as_h2(zs4[u][k])[1] * part[k];
        }
    };

    // prologue: fill the ring (indices past the wave's last group reload that group)
#pragma unroll
    for (int u = 0; u < U; ++u) issue(u, min(u, max(n_my - 1, 0)));
    if (XLDS) {
#pragma unroll
        for (int c = 0; c < XC; ++c) {
            const int idx = min(c * 256 + (int)threadIdx.x, n8 - 1);
            reinterpret_cast<u4*>(xs)[idx] = xst[c];
        }
        __syncthreads();
    }
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
        // drain
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (i0 + u < n_my) compute(u, i0 + u);
    }

    // correction epilogue: this wave adds R[t][8c..8c+8) . A[row][8c..8c+8) for chunks c = wave mod 4.
    // The first A chunks are loaded before waiting for R; with one token tile R is copied once into
    // LDS (one coherent 4-byte load per thread) and read from there.
    const bool correct = args.r > 0 && M.a != nullptr;
    if (correct) {
        const int r = args.r;
        const int row0 = rt * 16 + 4 * (lane >> 4);
        const int nc8 = r / 8;
        constexpr int PF = 2;  // A chunks prefetched per wave
        h8 apf[PF][4];
#pragma unroll
        for (int k = 0; k < PF; ++k) {
            const int c = wave + 4 * k;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = row0 + i;
                apf[k][i] = (c < nc8 && row < M.n_out) ? load_h8(M.a + (size_t)row * r + 8 * c) : zero8;
            }
        }
        wait_ready(args);
        const float* R = reinterpret_cast<const float*>(args.R) + (size_t)M.proj * T * r;
        float* rl = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(xs) + args.r_lds_off);
        if (NTT == 1) {
            for (int k = threadIdx.x; k < T * r; k += 256) rl[k] = load_r(R + k);
            __syncthreads();
        }
        for (int c = wave, k = 0; c < nc8; c += 4, ++k) {
            h8 a8[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (k < PF) {
#pragma unroll
                    for (int kk = 0; kk < PF; ++kk)
                        if (kk == k) a8[i] = apf[kk][i];
                } else {
                    const int row = row0 + i;
                    a8[i] = row < M.n_out ? load_h8(M.a + (size_t)row * r + 8 * c) : zero8;
                }
            }
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
                const int t = 16 * tt + (lane & 15);
                if (t < T) {
                    float rv[8];
                    if (NTT == 1) {
                        const f4* rp = reinterpret_cast<const f4*>(rl + (size_t)t * r + 8 * c);
                        const f4 r0 = rp[0], r1 = rp[1];
                        rv[0] = r0[0]; rv[1] = r0[1]; rv[2] = r0[2]; rv[3] = r0[3];
                        rv[4] = r1[0]; rv[5] = r1[1]; rv[6] = r1[2]; rv[7] = r1[3];
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) rv[e] = load_r(R + (size_t)t * r + 8 * c + e);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float s = acc[tt][i];
#pragma unroll
                        for (int e = 0; e < 8; ++e) s = fmaf((float)a8[i][e], rv[e], s);
                        acc[tt][i] = s;
                    }
                }
            }
        }
    }

#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) red[wave][tt][lane] = acc[tt];
    __syncthreads();
    if (wave < NTT) {  // wave w stores token tile w
        const int tt = wave;
        const f4 v0 = red[0][tt][lane], v1 = red[1][tt][lane], v2 = red[2][tt][lane], v3 = red[3][tt][lane];
        const int t = 16 * tt + (lane & 15);
        const int row0 = rt * 16 + 4 * (lane >> 4);
        if (t < T) {
            _Float16 o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = (_Float16)(((v0[i] + v1[i]) + v2[i]) + v3[i]);
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
    if (correct) signal_done(args);
}

hipError_t launch_decode(const ForwardArgs& a_in, hipStream_t stream) {
    ForwardArgs a = a_in;
    const int ntt = (int)ceil_div(a.T, 16);
    const dim3 grid(a.n_prod + a.n_tiles), block(256);
    const size_t xbytes = (size_t)(a.T + 1) * a.d * 2;  // tokens + one zero row
    const bool xlds = ntt == 1 && xbytes <= kDecodeXLdsMax;
    const size_t xarea = xlds ? (xbytes + 15) / 16 * 16 : 0;
    const size_t rarea = (ntt == 1 && a.r > 0) ? (size_t)a.T * a.r * 4 : 0;
    a.r_lds_off = (int32_t)xarea;
    const size_t shmem = xarea + rarea;
    if (xlds) {
        const int chunks = (int)ceil_div((int64_t)xbytes / 16, 256);
        if (chunks <= 2)
            hipLaunchKernelGGL((decode_kernel<1, 2>), grid, block, shmem, stream, a);
        else if (chunks <= 4)
            hipLaunchKernelGGL((decode_kernel<1, 4>), grid, block, shmem, stream, a);
        else
            hipLaunchKernelGGL((decode_kernel<1, kDecodeXChunks>), grid, block, shmem, stream, a);
        return hipGetLastError();
    }
    switch (ntt) {
        case 1: hipLaunchKernelGGL((decode_kernel<1, 0>), grid, block, shmem, stream, a); break;
        case 2: hipLaunchKernelGGL((decode_kernel<2, 0>), grid, block, shmem, stream, a); break;
        case 3: hipLaunchKernelGGL((decode_kernel<3, 0>), grid, block, shmem, stream, a); break;
        case 4: hipLaunchKernelGGL((decode_kernel<4, 0>), grid, block, shmem, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace glowq
