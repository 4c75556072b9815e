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
#include "glowq_internal.h"

namespace glowq {

// Physical workgroup id -> logical tile id such that XCD x (workgroups b with b % 8 == x)
// receives a contiguous range of logical tiles.
__device__ __forceinline__ int xcd_remap(int b, int n) {
    const int xcd = b & 7, local = b >> 3;
    const int per = n >> 3, rem = n & 7;
    return xcd * per + (xcd < rem ? xcd : rem) + local;
}

// Small grids: KS groups of four wavefronts per workgroup (256 KS threads) share one output tile
// and split the input groups between them (group g goes to wave group g % KS), each with its own
// double-buffered activation tile in LDS; at the end the wave groups' sums are added through LDS
// in wave-group order (deterministic) and wave group 0 applies the correction and stores.  With
// KS = 4 a launch of one workgroup per CU keeps four wavefronts on every SIMD.
template <int TT, int RR, int KS>
__global__ __launch_bounds__(256 * KS, (KS == 1 ? 2 : 1)) void prefill_kernel(const ForwardArgs args) {
    constexpr int BM = 16 * TT;
    constexpr int LS = 136;              // LDS row stride in halves (128 + 8 padding)
    constexpr int NCH = BM * 16 / 256;   // 16-byte X chunks per thread per group
    __shared__ __attribute__((aligned(16))) _Float16 xs[KS][2][BM * LS];

    const int L = xcd_remap(blockIdx.x, args.n_tiles);
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
    const size_t qstride = (size_t)M.n_tiles16 * 1024, szstride = (size_t)M.n_tiles16 * 64;  // per group

    const uint8_t* qp[RR];
    const uint8_t* zp[RR];
    bool w_ok[RR];
#pragma unroll
    for (int rr = 0; rr < RR; ++rr) {
        const int rt = rt0 + rr;
        w_ok[rr] = rt < M.n_tiles16;
        qp[rr] = M.q + (size_t)(w_ok[rr] ? rt : 0) * 1024 + lane * 16;
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
    uint32_t zs[RR];
    const bool act0 = kg < G;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
        st[c] = (act0 && x_ok[c]) ? *reinterpret_cast<const u4*>(xsrc[c] + (size_t)kg * kGroup) : zero4;
#pragma unroll
    for (int rr = 0; rr < RR; ++rr) {
        qv[rr] = (act0 && w_ok[rr]) ? *reinterpret_cast<const u4*>(qp[rr] + (size_t)kg * qstride) : zero4;
        zs[rr] = (act0 && w_ok[rr]) ? *reinterpret_cast<const uint32_t*>(zp[rr] + (size_t)kg * szstride) : 0u;
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c) *reinterpret_cast<u4*>(&xs[kg][0][xdst[c]]) = st[c];
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
        u4 qn[RR];
        uint32_t zn[RR];
        if (more) {
#pragma unroll
            for (int c = 0; c < NCH; ++c)
                st[c] = x_ok[c] ? *reinterpret_cast<const u4*>(xsrc[c] + (size_t)(g + KS) * kGroup) : zero4;
#pragma unroll
            for (int rr = 0; rr < RR; ++rr) {
                qn[rr] = w_ok[rr] ? *reinterpret_cast<const u4*>(qp[rr] + (size_t)(g + KS) * qstride) : zero4;
                zn[rr] = w_ok[rr] ? *reinterpret_cast<const uint32_t*>(zp[rr] + (size_t)(g + KS) * szstride) : 0u;
            }
        }
        if (act) {
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
                zs[rr] = zn[rr];
            }
        }
        __syncthreads();
    }

    if (KS > 1) {
        // wave groups 1 .. KS-1 hand their sums to wave group 0 through LDS (the activation
        // buffers are free after the loop's last barrier)
        f4* red = reinterpret_cast<f4*>(&xs[0][0][0]);
        static_assert(sizeof(xs) >= (KS - 1) * TT * RR * 256 * sizeof(f4), "reduction space");
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

    // correction: r_pad / 32 more K steps, A-operand A_i rows, B-operand R tokens
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

// Wide tile for large grids: BM = 128 tokens x BN = 256 rows, wave w owning 4 row tiles of 16
// rows and all 8 token tiles, so every activation operand read from LDS feeds 4 matrix-core
// steps and every dequantised weight operand 8.  The activation tile of a 128-input group is
// copied HBM/L2 -> LDS by the load unit itself (16-byte global_load_lds, no registers), whole
// 256-byte rows per four lanes; in LDS row r keeps its 16-byte chunk c at position c ^ (r % 16),
// so that the operand reads (16 rows, one chunk each) hit 16 different bank groups.  Two LDS
// buffers (2 x 32 KiB): the copy of group g + 1 and the next weight blocks (registers) are in
// flight while group g is multiplied.  Inside a group the 32 (slice, token tile) steps are issued
// in a fixed order: operand reads two steps ahead, the next slice's unpacking spread between the
// matrix-core steps.  Tokens past T read row T - 1 and row tiles past the module read its last
// tile; neither is stored.
typedef __attribute__((address_space(3))) void lds_void;

__global__ __launch_bounds__(256, 2) void prefill_wide_kernel(const ForwardArgs args) {
    constexpr int TT = 8, RR = 4, BM = 128;
    extern __shared__ __attribute__((aligned(16))) u4 xw[];  // [2][TT * 4][64]

    const int L = xcd_remap(blockIdx.x, args.n_tiles);
    const int mb = L % args.m_tiles, nbl = L / args.m_tiles;
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
    const uint32_t qlane = lane * 16, zlane = (lane & 15) * 4;
    auto qaddr = [&](int g, int rr) {
        return reinterpret_cast<const u4*>(M.q + ((size_t)g * NT + rtc[rr]) * 1024 + qlane);
    };
    auto zaddr = [&](int g, int rr) {
        return reinterpret_cast<const uint32_t*>(M.sz + ((size_t)g * NT + rtc[rr]) * 64 + zlane);
    };
    // activation copy: instruction i of wave w fills tile rows 32 w + 4 i .. + 3 (256 bytes each,
    // whole cache lines); lane l lands at LDS slot 16 l, i.e. row 32 w + 4 i + l / 16, 16-byte
    // position l % 16, which holds input chunk (l % 16) ^ (row % 16) of that row (XOR swizzle)
    uint32_t xoff[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = 32 * wave + 4 * i + (lane >> 4);
        const int t = min(m0 + row, T - 1);
        xoff[i] = (uint32_t)(t * d + 8 * ((lane & 15) ^ (row & 15))) * 2u;
    }
    const char* xbase = reinterpret_cast<const char*>(args.x);
    auto copy_x = [&](int g, int buf) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            __builtin_amdgcn_global_load_lds((const void*)(xbase + (size_t)g * kGroup * 2 + xoff[i]),
                                             (lds_void*)(xw + ((size_t)buf * BM + 32 * wave + 4 * i) * 16), 16, 0, 0);
    };
    // operand read of slice j: lane l takes row 16 tt + l % 16, chunk 4 j + l / 16, swizzled
    uint32_t bofs[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bofs[j] = (uint32_t)((lane & 15) * 16 + ((4 * j + (lane >> 4)) ^ (lane & 15)));

    u4 qv[RR];
    uint32_t zs[RR];
    copy_x(0, 0);
#pragma unroll
    for (int rr = 0; rr < RR; ++rr) {
        qv[rr] = *qaddr(0, rr);
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
        uint32_t zn[RR];
        if (more) {
            copy_x(g + 1, buf ^ 1);
#pragma unroll
            for (int rr = 0; rr < RR; ++rr) {
                qn[rr] = *qaddr(g + 1, rr);
                zn[rr] = *zaddr(g + 1, rr);
            }
        }
        h2 c1024[RR], c64[RR];
        h8 s8[RR];
#pragma unroll
        for (int rr = 0; rr < RR; ++rr) {
            zero_consts(zs[rr], c1024[rr], c64[rr]);
            const _Float16 s = as_h2(zs[rr])[1];
            s8[rr] = h8{s, s, s, s, s, s, s, s};
        }
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
            for (int rr = 0; rr < RR; ++rr) aj[0][rr] = nib8_minus_z(qv[rr][0], c1024[rr], c64[rr], nc) * s8[rr];
#pragma unroll
            for (int st = 0; st < NS; ++st) {
                const int j = st / TT, tt = st % TT;
                if (st + 2 < NS) bq[(st + 2) % 3] = bread(st + 2);
                if (j < 3 && (tt & 1) == 0) {
                    const int rr = tt >> 1;
                    aj[j + 1][rr] = nib8_minus_z(qv[rr][j + 1], c1024[rr], c64[rr], nc) * s8[rr];
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

hipError_t launch_prefill(const ForwardArgs& a, hipStream_t stream) {
    const dim3 grid(a.n_tiles), block(256);
    if (a.tile_tt == 8 && a.tile_rr == 4) {
        hipLaunchKernelGGL(prefill_wide_kernel, grid, block, 2 * 8 * 4 * 64 * sizeof(u4), stream, a);
        return hipGetLastError();
    }
    if (a.tile_rr == 1) {  // small grids: 64 or 32 tokens x 64 rows, 4 wave groups
        if (a.tile_ks != 4 || (a.tile_tt != 4 && a.tile_tt != 2)) return hipErrorInvalidValue;
        if (a.tile_tt == 4)
            hipLaunchKernelGGL((prefill_kernel<4, 1, 4>), grid, dim3(1024), 0, stream, a);
        else
            hipLaunchKernelGGL((prefill_kernel<2, 1, 4>), grid, dim3(1024), 0, stream, a);
        return hipGetLastError();
    }
    if (a.tile_tt != 4 || a.tile_rr != 2) return hipErrorInvalidValue;
    if (a.tile_ks == 4)
        hipLaunchKernelGGL((prefill_kernel<4, 2, 4>), grid, dim3(1024), 0, stream, a);
    else if (a.tile_ks == 2)
        hipLaunchKernelGGL((prefill_kernel<4, 2, 2>), grid, dim3(512), 0, stream, a);
    else if (a.tile_ks == 1)
        hipLaunchKernelGGL((prefill_kernel<4, 2, 1>), grid, block, 0, stream, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace glowq
