// Input second moment of the calibration activations, Sigma_x = X^T X / N (GlowQ paper note, key
// design 2: the usage-weighted risk E||M x||^2 = ||M Sigma_x^{1/2}||_F^2 is built on it; the arXiv
// page, Figure 2, streams calibration samples and takes the empirical input covariance).  This is
// the first step of the offline factor solve and its largest contraction: 2 N d^2 flops.
//
// moment_kernel: one workgroup per (lower-triangle 256 x 256 tile of Sigma, range of tokens), one
// workgroup per CU.  Per step of 32 tokens the two 32 x 256 activation slices (the tile's row and
// column features) are copied HBM -> LDS by the load unit (global_load_lds, 16 bytes per lane,
// token-major as they lie in memory; 16-byte chunk c of token row r sits at position c ^ 4 (r % 4),
// so that the four rows a transposing read touches fall on different banks), in a ring of four
// steps (three in flight).  The matrix-core operands need the tokens (the contraction index)
// along each lane, i.e. the slices transposed: every operand is two ds_read_b64_tr_b16, which
// hand lane 4a + b of each 16-lane group element b of the 8-byte chunks addressed by lanes a,
// a + 4, a + 8, a + 12 -- with lane q addressing token t + q / 4, features f + 4 (q % 4), lane i
// receives feature f + i of tokens t .. t + 3.  Each wave owns a 128 x 128 quarter of the tile
// (4 x 4 v_mfma_f32_32x32x16_f16 blocks, fp32 accumulation: 8 operands per 16 matrix-core steps)
// and writes it as an fp32 partial.
// moment_reduce_kernel: adds the partials of the token ranges in range order (deterministic),
// scales by 1 / N and writes Sigma and its mirror image (only i >= j inside diagonal tiles, so that
// every element has one writer).
#include "glowq_offline.h"

namespace glowq {

typedef __fp16 fp16x4 __attribute__((vector_size(8)));
typedef float f16x __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_m;

__device__ __forceinline__ void tile_of(int t, int& bi, int& bj) {
    int i = (int)((sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
    while (i * (i + 1) / 2 > t) --i;
    while ((i + 1) * (i + 2) / 2 <= t) ++i;
    bi = i;
    bj = t - i * (i + 1) / 2;
}

// two transposing reads: features f0 + (lane % 16) of tokens k0 .. k0 + 7 for this lane's group
__device__ __forceinline__ h8 tr_operand(const _Float16* slice, int row0, int fchunk_half, int lane) {
    // provider role: lane q of the group addresses token row row0 + q / 4 (and + 4), features
    // fchunk_half + 4 (q % 4), i.e. 16-byte chunk (fchunk_half / 8) + (q % 4) / 2, 8-byte half (q % 2)
    const int q = lane & 15;
    h8 out;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int row = row0 + 4 * h + (q >> 2);
        const int feat = fchunk_half + 4 * (q & 3);
        const int chunk = (feat >> 3) ^ (4 * (row & 3));
        const _Float16* p = slice + row * kMomentTile + chunk * 8 + (feat & 7);
        const fp16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
            (__attribute__((address_space(3))) fp16x4*)((__attribute__((address_space(3))) _Float16*)p));
        const h4x w = __builtin_bit_cast(h4x, v);
#pragma unroll
        for (int e = 0; e < 4; ++e) out[4 * h + e] = w[e];
    }
    return out;
}

__global__ __launch_bounds__(256, 1) void moment_kernel(const MomentArgs a) {
    constexpr int R = kMomentStages;  // ring of 32-token steps in LDS
    constexpr int TB = kMomentTile;   // tile edge (features)
    static_assert(R == 4, "the step loop below is unrolled for four stages");
    // one array per stage: every copy and every read names its stage statically, so that waiting
    // for one stage's copy never waits for the copies of the others
    __shared__ __attribute__((aligned(16))) _Float16 xs0[2][32 * TB];
    __shared__ __attribute__((aligned(16))) _Float16 xs1[2][32 * TB];
    __shared__ __attribute__((aligned(16))) _Float16 xs2[2][32 * TB];
    __shared__ __attribute__((aligned(16))) _Float16 xs3[2][32 * TB];
    const int u = blockIdx.x;
    const int tile = u % a.n_tiles, s = u / a.n_tiles;
    int bi, bj;
    tile_of(tile, bi, bj);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int wi = wave >> 1, wj = wave & 1;  // this wave's 128 x 128 quarter
    const int t_begin = s * a.kc;
    const int t_end = min(t_begin + a.kc, a.N);
    const int steps = (t_end - t_begin + 31) / 32;
    const char* xb = reinterpret_cast<const char*>(a.x);
    const size_t dbytes = (size_t)a.d * 2;

    // copy of one 32-token step (2 slices x 32 rows x 512 bytes): instruction i of wave w fills
    // 1 KB block 8 w + i, i.e. slice blk / 16, token rows 2 (blk % 16) + lane / 32, 16-byte
    // position lane % 32, which holds feature chunk (lane % 32) ^ 4 (row % 4)
    auto copy = [&](int step, _Float16 (*xs)[32 * TB]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int blk = 8 * wave + i;
            const int sl = blk >> 4;
            const int row = ((blk & 15) << 1) + (lane >> 5);
            const int chunk = (lane & 31) ^ (4 * (row & 3));
            const int t = min(t_begin + 32 * step + row, a.N - 1);  // rows past the range: masked later
            // features past d (a half-empty last block) read a valid chunk of the row instead;
            // the tile elements they feed are never written
            const int f = min((sl == 0 ? bi : bj) * TB + 8 * chunk, a.d - 8);
            __builtin_amdgcn_global_load_lds((const void*)(xb + (size_t)t * dbytes + (size_t)f * 2),
                                             (lds_void_m*)(&xs[sl][0] + (blk & 15) * 512), 16, 0, 0);
        }
    };

    f16x acc[4][4];
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y)
#pragma unroll
            for (int k = 0; k < 16; ++k) acc[x][y][k] = 0.f;

    // R - 1 steps in flight: at step st this wave waits only for its own copy of step st (the
    // copies of the two later steps, 8 instructions each, may stay outstanding), then the barrier
    // makes every wave's copy visible; the copy of step st + R - 1 goes to the stage step st - 1
    // used, which every wave has finished reading (its operands fed matrix-core steps issued
    // before the barrier).  The barrier is the bare s_barrier: a fenced one would wait for every
    // copy in flight.  (The compiler still adds a full wait before the reads of two of the four
    // stages -- it cannot tell their copies apart from the younger ones -- so every other step
    // drains the ring: 3.06 ms at the calibration shape, against 3.30 ms with a fenced barrier.)
    auto step = [&](int st, _Float16 (*cur)[32 * TB], _Float16 (*nxt)[32 * TB]) {
        // every step issues the copy of step st + R - 1 (past the range: a clamped, unused copy),
        // so exactly 2 steps x 8 copies are younger than this step's: vmcnt(16) (gfx9 s_waitcnt
        // immediate: vmcnt bits 3:0 and 15:14, expcnt and lgkmcnt left at their maxima), as a
        // builtin so that the compiler's own wait insertion accounts for it
        __builtin_amdgcn_s_waitcnt(0x4F70);
        __builtin_amdgcn_s_barrier();
        copy(st + R - 1, nxt);
        const int valid = t_end - (t_begin + 32 * st);  // tokens of this step (>= 32 except the last)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            // k rows of this lane: 16 kk + 8 (lane / 32) .. + 7
            const int row0 = 16 * kk + 8 * (lane >> 5);
            h8 A[4], B[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                A[x] = tr_operand(&cur[0][0], row0, 128 * wi + 32 * x + 16 * ((lane >> 4) & 1), lane);
                B[x] = tr_operand(&cur[1][0], row0, 128 * wj + 32 * x + 16 * ((lane >> 4) & 1), lane);
            }
            if (valid < 32) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if (row0 + e >= valid) {
#pragma unroll
                        for (int x = 0; x < 4; ++x) {
                            A[x][e] = (_Float16)0.f;
                            B[x][e] = (_Float16)0.f;
                        }
                    }
                }
            }
#pragma unroll
            for (int x = 0; x < 4; ++x)
#pragma unroll
                for (int y = 0; y < 4; ++y) acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[x], B[y], acc[x][y], 0, 0, 0);
        }
    };
    copy(0, xs0);
    copy(1, xs1);
    copy(2, xs2);
    for (int st = 0; st < steps; st += R) {
        step(st, xs0, xs3);
        if (st + 1 < steps) step(st + 1, xs1, xs0);
        if (st + 2 < steps) step(st + 2, xs2, xs1);
        if (st + 3 < steps) step(st + 3, xs3, xs2);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no copy may land in LDS after the workgroup ends

    // partial tile: element (i, j) of the TB x TB tile at part[(s n_tiles + tile) TB^2 + TB i + j]
    float* P = a.part + ((size_t)s * a.n_tiles + tile) * TB * TB;
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y)
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const int i = 128 * wi + 32 * x + 8 * (k >> 2) + 4 * (lane >> 5) + (k & 3);
                const int j = 128 * wj + 32 * y + (lane & 31);
                P[i * TB + j] = acc[x][y][k];
            }
}

__global__ __launch_bounds__(256) void moment_reduce_kernel(const MomentArgs a) {
    constexpr int TB = kMomentTile;
    const int tile = blockIdx.y;
    int bi, bj;
    tile_of(tile, bi, bj);
    const int e = blockIdx.x * 256 + threadIdx.x;  // 0 .. TB^2 - 1
    const int i = e / TB, j = e % TB;
    if (bi == bj && i < j) return;
    float v = 0.f;
    for (int s = 0; s < a.S; ++s) v += a.part[((size_t)s * a.n_tiles + tile) * TB * TB + e];
    v *= a.inv_n;
    const size_t gi = (size_t)bi * TB + i, gj = (size_t)bj * TB + j;
    if (gi >= (size_t)a.d || gj >= (size_t)a.d) return;
    a.sigma[gi * a.d + gj] = v;
    a.sigma[gj * a.d + gi] = v;
}

hipError_t launch_moment(const MomentArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(moment_kernel, dim3((unsigned)(a.n_tiles * a.S)), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(moment_reduce_kernel, dim3(kMomentTile * kMomentTile / 256, (unsigned)a.n_tiles), dim3(256), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace glowq
