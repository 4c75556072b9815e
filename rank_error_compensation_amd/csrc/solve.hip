// Offline factor solve of one input-sharing group on the GPU, in fp64 (GlowQ paper note, key designs
// 1-3: stack the group's quantisation errors, whiten them by the input covariance, extract the
// dominant right subspace with a randomized SVD (p oversampling columns, q power iterations, Halko,
// Martinsson and Tropp), return balanced factors A = U_r S_r^{1/2}, B = S_r^{1/2} V_r^T lifted back
// to the original variables).
//
// Whitening uses the Cholesky factor L of Sigma_x (Sigma_x = L L^T) as the square root: the lifted
// product A B does not depend on which square root is used.  The lift B = S_r^{1/2} V_r^T L^{-1}
// needs no triangular solve: with V_r^T = S_r^{-1} U_r^T Q^T E~ and E~ = E_cat L it is
// S_r^{-1/2} U_r^T (Q^T E_cat), two more products on the matrix cores.  The range finder
// runs on the whitened stacked error E~ = E_cat L itself rather than on the QR-reduced core
// M = R_e L: with E~ = Q_e M and the same test matrix, every step (the ranges, their orthonormal
// bases, the small projected matrix and its SVD) is the same up to the left factor Q_e, which the
// final A = Q U_b S^{1/2} carries directly -- so A and B are those of the QR-reduced solve, without
// the extra thin QR.  E~ itself is never formed: E~ X = E_cat (L X) and E~^T Y = L^T (E_cat^T Y),
// so every product with it is one with E_cat and one with the triangle L against k columns.
//
// Kernels (all fp64):
//   gemm_kernel        C = alpha op(A) op(B) + beta C on the fp64 matrix cores, 128 x 128 tiles
//   chol_diag_kernel   one workgroup factors a 64 x 64 diagonal block in LDS (right-looking, one
//                      barrier per column)
//   chol_panel_kernel  rows below the block: x L_kk^T = a by forward substitution, a row per thread
//   chol_inv_small_kernel  orthonormal bases by Cholesky-QR, twice: G = X^T X, one workgroup
//                      factors G = R^T R (dropping columns already in the span) and inverts R,
//                      X <- X R^{-1}
//   jacobi_kernel      one workgroup: eigenvalues / eigenvectors of a symmetric k x k matrix in LDS
//                      (parallel cyclic Jacobi: disjoint rotations of a round-robin round applied
//                      together), sorted descending
#include "glowq_offline.h"

namespace glowq {

// --------------------------------------------------------------------------- GEMM
// 128 x 128 tile per workgroup, four waves of 64 x 64, each 4 x 4 v_mfma_f64_16x16x4_f64 tiles
// (A operand lane l: row l % 16, k l / 16; B operand lane l: k l / 16, column l % 16; result element
// e of lane l: row l / 16 + 4 e, column l % 16 -- measured with an in-bounds probe).  K in steps of 16 through LDS, the next step's global
// loads held in registers while the current one is multiplied.  c_lower: only tiles touching the
// lower triangle of C are computed.
typedef double d4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void gemm_kernel(const GemmArgs g) {
    __shared__ double As[16][128 + 2];
    __shared__ double Bs[16][128 + 2];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int wi = wave >> 1, wj = wave & 1;
    // tile of this workgroup: consecutive workgroup ids go to different XCDs, so the linear id is
    // remapped to give each XCD a contiguous range of tiles (row-major over the tile grid): the
    // workgroups resident on one XCD share A's row panel in its L2
    int ty, tx;
    {
        const int n = (int)(gridDim.x * gridDim.y), b = (int)(blockIdx.y * gridDim.x + blockIdx.x);
        const int xcd = b & 7, local = b >> 3, per = n >> 3, rem = n & 7;
        const int L = xcd * per + (xcd < rem ? xcd : rem) + local;
        ty = L / (int)gridDim.x;
        tx = L - ty * (int)gridDim.x;
    }
    const int i0 = ty * 128, j0 = tx * 128;
    if (g.c_lower && j0 > i0 + 127) return;
    // K range: all of K, or range z of a split launch (never combined with c_lower)
    const bool split = g.splits > 1;
    const int kbeg = split ? (int)blockIdx.z * g.kc : 0;
    const int kend = split ? min(g.K, kbeg + g.kc) : g.K;
    d4 acc[4][4];
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = d4{0.0, 0.0, 0.0, 0.0};

    double ra[8], rb[8];
    auto load = [&](int k0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int idx = threadIdx.x + 256 * e;  // 0 .. 2047; consecutive threads walk the
                                                    // contiguous index of each operand as stored
            {
                const int ii = g.ta ? (idx & 127) : (idx >> 4), kk = g.ta ? (idx >> 7) : (idx & 15);
                const int i = i0 + ii, k = k0 + kk;
                ra[e] = (i < g.M && k < kend) ? (g.ta ? g.A[(size_t)k * g.lda + i] : g.A[(size_t)i * g.lda + k]) : 0.0;
            }
            {
                const int jj = g.tb ? (idx >> 4) : (idx & 127), kk = g.tb ? (idx & 15) : (idx >> 7);
                const int j = j0 + jj, k = k0 + kk;
                rb[e] = (j < g.N && k < kend) ? (g.tb ? g.B[(size_t)j * g.ldb + k] : g.B[(size_t)k * g.ldb + j]) : 0.0;
            }
        }
    };
    auto store = [&]() {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int idx = threadIdx.x + 256 * e;
            {
                const int ii = g.ta ? (idx & 127) : (idx >> 4), kk = g.ta ? (idx >> 7) : (idx & 15);
                As[kk][ii] = ra[e];
            }
            {
                const int jj = g.tb ? (idx >> 4) : (idx & 127), kk = g.tb ? (idx & 15) : (idx >> 7);
                Bs[kk][jj] = rb[e];
            }
        }
    };
    if (kbeg < kend) load(kbeg);
    for (int k0 = kbeg; k0 < kend; k0 += 16) {
        store();
        __syncthreads();
        if (k0 + 16 < kend) load(k0 + 16);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int kr = 4 * ks + (lane >> 4);
            double a[4], b[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                a[x] = As[kr][64 * wi + 16 * x + (lane & 15)];
                b[x] = Bs[kr][64 * wj + 16 * x + (lane & 15)];
            }
#pragma unroll
            for (int x = 0; x < 4; ++x)
#pragma unroll
                for (int y = 0; y < 4; ++y) acc[x][y] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[x], b[y], acc[x][y], 0, 0, 0);
        }
        __syncthreads();
    }
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = i0 + 64 * wi + 16 * x + (lane >> 4) + 4 * e;
                const int j = j0 + 64 * wj + 16 * y + (lane & 15);
                if (i < g.M && j < g.N) {
                    if (split) {
                        g.part[((size_t)blockIdx.z * g.M + i) * g.N + j] = acc[x][y][e];
                    } else {
                        double* c = g.C + (size_t)i * g.ldc + j;
                        *c = g.alpha * acc[x][y][e] + (g.beta != 0.0 ? g.beta * *c : 0.0);
                    }
                }
            }
}

// C = alpha (sum of the split partial products, in range order) + beta C
__global__ __launch_bounds__(256) void gemm_reduce_kernel(const GemmArgs g) {
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t mn = (size_t)g.M * g.N;
    if (idx >= mn) return;
    double s = 0.0;
    for (int z = 0; z < g.splits; ++z) s += g.part[(size_t)z * mn + idx];
    const int i = (int)(idx / g.N), j = (int)(idx % g.N);
    double* c = g.C + (size_t)i * g.ldc + j;
    *c = g.alpha * s + (g.beta != 0.0 ? g.beta * *c : 0.0);
}

hipError_t launch_gemm(const GemmArgs& g0, hipStream_t stream) {
    if (g0.M <= 0 || g0.N <= 0) return hipSuccess;
    GemmArgs g = g0;
    const int64_t tiles = ceil_div(g.N, 128) * ceil_div(g.M, 128);
    const int64_t mn = (int64_t)g.M * g.N;
    int64_t s = 1;
    if (g.part != nullptr && !g.c_lower && tiles < kGemmWant) {
        s = ceil_div(kGemmWant, tiles);
        s = std::min<int64_t>(s, g.K / kGemmMinK);
        s = std::min<int64_t>(s, g.part_cap / mn);
        s = std::max<int64_t>(s, 1);
    }
    // K ranges of a multiple of 16 (the kernel's step), and no empty range
    const int64_t kc = g.K > 0 ? ceil_div(ceil_div(g.K, s), 16) * 16 : 16;
    s = g.K > 0 ? ceil_div(g.K, kc) : 1;
    g.splits = (int32_t)s;
    g.kc = (int32_t)kc;
    const dim3 grid((unsigned)ceil_div(g.N, 128), (unsigned)ceil_div(g.M, 128), (unsigned)s);
    hipLaunchKernelGGL(gemm_kernel, grid, dim3(256), 0, stream, g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || s == 1) return e;
    hipLaunchKernelGGL(gemm_reduce_kernel, dim3((unsigned)ceil_div(mn, 256)), dim3(256), 0, stream, g);
    return hipGetLastError();
}

// --------------------------------------------------------------------------- Cholesky
constexpr int kSmallThreads = 1024;  // one-workgroup factorisations: threads per workgroup

// Semidefinite Cholesky: a pivot at or below kPsdTol times the original diagonal entry dg[j] of
// its column is numerically zero.  For a positive semidefinite matrix the rest of such a column is
// then zero as well (|S_ij|^2 <= S_ii S_jj): the column of L is set to zero and the index marked
// dropped, so that L L^T = S still holds and L's nonzero columns span the range of S.  A pivot
// below -kPsdTol dg[j] (or a negative diagonal entry) means S is not positive semidefinite and
// sets *flag.
constexpr double kPsdTol = 1e-10;

__global__ __launch_bounds__(256) void diag_kernel(const double* S, int d, double* dg) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < d) dg[i] = S[(size_t)i * d + i];
}

// Factor the nb x nb diagonal block at (n0, n0) of the lower triangle of S (row stride ld) in
// place, dropping numerically zero pivots (drop[n0 + j] = 1, column zero); a negative one sets
// *flag.
__global__ __launch_bounds__(kSmallThreads) void chol_diag_kernel(double* S, int ld, int n0, int nb, int* flag,
                                                                  const double* dg, int* drop) {
    __shared__ double a[64][65];
    if (n0 == 0 && threadIdx.x == 0) *flag = 0;  // the first block clears the flag before any pivot
    for (int idx = threadIdx.x; idx < nb * nb; idx += kSmallThreads) {
        const int i = idx / nb, j = idx % nb;
        a[i][j] = S[(size_t)(n0 + i) * ld + n0 + j];
    }
    __syncthreads();
    // thread t updates column c = t % 64 on rows t / 64 + RS q.  Step j (one barrier): with the
    // pivot v = a[j][j], the trailing lower triangle loses a[i][j] a[c][j] / v (j < c <= i), which
    // only reads column j; then column j itself is finished (L_jj = sqrt v, L_ij = a[i][j] / L_jj)
    // while the next step reads only columns past j.
    constexpr int RS = kSmallThreads / 64;
    const int c = threadIdx.x & 63, i0 = threadIdx.x >> 6;
    for (int j = 0; j < nb; ++j) {
        const double v = a[j][j];
        const double dj = dg[n0 + j];
        const bool ok = v > kPsdTol * dj;                      // a live column
        const bool bad = dj < 0.0 || v < -kPsdTol * dj;        // not positive semidefinite
        if (ok && c > j && c < nb) {
            const double acj = a[c][j] / v;
            for (int i = c + ((i0 - c) & (RS - 1)); i < nb; i += RS) a[i][c] -= a[i][j] * acj;  // rows i >= c
        }
        __syncthreads();
        const double piv = ok ? sqrt(v) : 0.0;
        if (threadIdx.x == 0) {
            if (bad) atomicOr(flag, 1);
            a[j][j] = piv;
            drop[n0 + j] = ok ? 0 : 1;
        }
        for (int i = j + 1 + (int)threadIdx.x; i < nb; i += kSmallThreads) a[i][j] = ok ? a[i][j] / piv : 0.0;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < nb * nb; idx += kSmallThreads) {
        const int i = idx / nb, j = idx % nb;
        S[(size_t)(n0 + i) * ld + n0 + j] = j <= i ? a[i][j] : 0.0;
    }
}

// Rows n0 + nb .. n - 1: L[i][n0 .. n0 + nb) = S[i][n0 .. n0 + nb) L_kk^{-T}, i.e. x L_kk^T = s
// for each such row s: x_l = s_l / L_ll (times the reciprocal), then s_j -= x_l L_jl for j > l.  A row per thread, kept
// in registers; L_kk is held transposed in LDS (lt[l][j] = L_jl, so that each step reads a
// contiguous run), every element a broadcast read.
__global__ __launch_bounds__(128) void chol_panel_kernel(double* S, int ld, int n, int n0) {
    constexpr int nb = 64;  // only a full block has rows below it
    __shared__ double lt[64][64];
    __shared__ double rd[64];  // 1 / L_ll
    for (int idx = threadIdx.x; idx < 64 * 64; idx += 128) {
        const int i = idx >> 6, j = idx & 63;  // L element (i, j) -> lt[j][i]
        lt[j][i] = j <= i ? S[(size_t)(n0 + i) * ld + n0 + j] : 0.0;
    }
    __syncthreads();
    // a dropped column (zero pivot) gives a zero column of L below it
    if (threadIdx.x < 64) rd[threadIdx.x] = lt[threadIdx.x][threadIdx.x] > 0.0 ? 1.0 / lt[threadIdx.x][threadIdx.x] : 0.0;
    __syncthreads();
    const int row = n0 + nb + blockIdx.x * 128 + threadIdx.x;
    if (row >= n) return;
    double* srow = S + (size_t)row * ld + n0;
    double x[64];
#pragma unroll
    for (int j = 0; j < 64; ++j) x[j] = srow[j];
#pragma unroll
    for (int l = 0; l < 64; ++l) {
        x[l] *= rd[l];
#pragma unroll
        for (int j = l + 1; j < 64; ++j) x[j] -= x[l] * lt[l][j];
    }
#pragma unroll
    for (int j = 0; j < 64; ++j) srow[j] = x[j];
}

__global__ __launch_bounds__(256) void zero_upper_kernel(double* S, int ld, int n) {
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)n * n) return;
    const int i = (int)(idx / n), j = (int)(idx % n);
    if (j > i) S[(size_t)i * ld + j] = 0.0;
}

// Null space of a semidefinite Cholesky factor: for each dropped index j = list[b] the vector v with
// L^T v = 0, v_j = 1 and v_i = 0 for i > j, by back substitution on the upper triangle L^T:
// v_i = -(sum_{i < l <= j} L_li v_l) / L_ii for a live i, 0 for a dropped i.  Column-oriented: once
// v_l is known, every i < l gains L_li v_l (row l of L, contiguous), and the owner of index l - 1
// finishes v_{l-1}; one barrier per step.  The vectors are linearly independent (each ends at its
// own j) and span the null space of L^T, i.e. of S = L L^T.  Output column b of N [d][n0].
constexpr int kNullThreads = 1024;
constexpr int kNullPer = kMaxSolveD / kNullThreads;  // indices per thread

__global__ __launch_bounds__(kNullThreads) void null_vec_kernel(const double* L, int d, const int* drop,
                                                               const int* list, int n0, double* N) {
    __shared__ double vsh[2];
    const int b = blockIdx.x, j = list[b];
    const int t = threadIdx.x;
    double acc[kNullPer];
#pragma unroll
    for (int q = 0; q < kNullPer; ++q) acc[q] = 0.0;
    for (int i = t; i < d; i += kNullThreads)
        if (i >= j) N[(size_t)i * n0 + b] = i == j ? 1.0 : 0.0;
    double v = 1.0;
    for (int l = j; l >= 1; --l) {
        if (v != 0.0) {
            const double* row = L + (size_t)l * d;
#pragma unroll
            for (int q = 0; q < kNullPer; ++q) {
                const int i = t + kNullThreads * q;
                if (i < l) acc[q] += row[i] * v;
            }
        }
        const int o = l - 1;
        if (t == o % kNullThreads) {
            double a = 0.0;
#pragma unroll
            for (int q = 0; q < kNullPer; ++q)
                if (q == o / kNullThreads) a = acc[q];
            const double vn = drop[o] ? 0.0 : -a / L[(size_t)o * d + o];
            vsh[l & 1] = vn;
            N[(size_t)o * n0 + b] = vn;
        }
        __syncthreads();
        v = vsh[l & 1];
    }
}

// --------------------------------------------------------------------------- small dense steps
__device__ __forceinline__ double block_sum(double v, double* red) {
    // 1024 threads: wave sums, then the 16 wave results in order
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    double s = 0.0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) s += red[w];
    return s;
}

// Cholesky factor with dropped columns and its inverse, for an orthonormal basis of the columns of
// X from their Gram G = X^T X (k x k): G = R^T R (R upper triangular); a column whose remaining
// pivot falls to 1e-24 of its diagonal entry (or is 0) lies in the span of the earlier ones and
// is dropped (row and column of R zero, Rinv column zero), so X Rinv has orthonormal columns
// where X has new directions and zero columns elsewhere.  One workgroup, R and Rinv in LDS.
__global__ __launch_bounds__(kSmallThreads) void chol_inv_small_kernel(const double* G, int k, double* Rinv_out) {
    __shared__ double R[kSolveMaxK][kSolveMaxK + 1];
    __shared__ double Ri[kSolveMaxK][kSolveMaxK + 1];
    __shared__ int live[kSolveMaxK];
    for (int idx = threadIdx.x; idx < k * k; idx += kSmallThreads) {
        const int i = idx / k, j = idx % k;
        R[i][j] = G[idx];
        Ri[i][j] = i == j ? 1.0 : 0.0;
    }
    __syncthreads();
    // thread t works on column c = t % 128 (c < k), rows t / 128 + RS q.
    constexpr int RS = kSmallThreads / 128;
    const int c = threadIdx.x & 127, a0 = threadIdx.x >> 7;
    // Right-looking, one barrier per step: with the pivot v = R[j][j] of a live column j, the
    // trailing upper triangle loses R[j][a] R[j][c] / v (j < a <= c), which only reads row j; then
    // row j itself is finished (R_jj = sqrt v, R_jc = R[j][c] / R_jj; a dropped column's row is
    // zero) while the next step reads only rows past j.
    for (int j = 0; j < k; ++j) {
        const double v = R[j][j];
        const bool ok = v > 1e-24 * G[(size_t)j * k + j] && v > 0.0;
        if (ok && c > j && c < k) {
            const double rjc = R[j][c] / v;
            for (int a = j + 1 + ((a0 - j - 1) & (RS - 1)); a <= c; a += RS) R[a][c] -= R[j][a] * rjc;  // j < a <= c
        }
        __syncthreads();
        if (threadIdx.x == 0) live[j] = ok ? 1 : 0;
        const double p = ok ? sqrt(v) : 0.0;
        for (int cc = (int)threadIdx.x; cc < k; cc += kSmallThreads) {
            if (cc < j) R[j][cc] = 0.0;
            else if (cc > j) R[j][cc] = ok ? R[j][cc] / p : 0.0;
        }
        if (threadIdx.x == 0) R[j][j] = p;
    }
    __syncthreads();
    // Rinv = R^{-1} on the live columns by back substitution for all columns at once: for i from
    // the last row, row i of Rinv is divided by R_ii (zero for a dropped i), then every row l < i
    // loses R[l][i] times it.  Dropped columns of Rinv are zero.
    for (int i = k - 1; i >= 0; --i) {
        const bool li = live[i] != 0;
        const double rii = R[i][i];
        if (a0 == 0 && c < k) Ri[i][c] = li ? Ri[i][c] / rii : 0.0;
        __syncthreads();
        if (li && c < k) {
            const double x = Ri[i][c];
            for (int l = a0; l < i; l += RS) Ri[l][c] -= R[l][i] * x;
        }
        __syncthreads();
    }
    for (int idx = threadIdx.x; idx < k * k; idx += kSmallThreads) {
        const int i = idx / k, cc = idx % k;
        Rinv_out[idx] = live[cc] ? Ri[i][cc] : 0.0;
    }
}

constexpr int kJacobiThreads = 1024;

// Symmetric k x k G (row-major) -> eigenvalues w (descending) and eigenvectors as the columns of
// V (k x k, row-major).  Parallel cyclic Jacobi: each sweep is n - 1 rounds of a round-robin
// tournament over the n = k (rounded up to even) indices; a round's n / 2 pairs are disjoint, so
// their rotations (each zeroing one off-diagonal pair) are computed from the same matrix and
// applied together.  Sweeps repeat until the off-diagonal Frobenius mass is below 1e-30 of the
// total (or 40 sweeps).
__global__ __launch_bounds__(kJacobiThreads) void jacobi_kernel(const double* G, int k, double* w, double* V) {
    __shared__ double a[kSolveMaxK][kSolveMaxK + 1];
    __shared__ double v[kSolveMaxK][kSolveMaxK + 1];
    __shared__ double cs[kSolveMaxK / 2][2];
    __shared__ int pr[kSolveMaxK / 2][2];
    __shared__ double red[kJacobiThreads / 64];
    __shared__ int order[kSolveMaxK];
    const int n = k + (k & 1);  // index k (when k is odd) is a dummy: its pairs are skipped
    for (int idx = threadIdx.x; idx < k * k; idx += kJacobiThreads) {
        const int i = idx / k, j = idx % k;
        a[i][j] = G[idx];
        v[i][j] = i == j ? 1.0 : 0.0;
    }
    __syncthreads();
    // round-robin tournament: index 0 stays, positions 1 .. n - 1 rotate by one per round, so in
    // round rd position i holds 1 + ((i - 1 - rd) mod (n - 1)); pair t is positions t, n - 1 - t
    auto pos = [&](int i, int rd) { return i == 0 ? 0 : 1 + ((i - 1 - rd) % (n - 1) + (n - 1)) % (n - 1); };
    // thread t updates column (or row) e = t % 128 of the pairs t / 128 + JS i
    constexpr int JS = kJacobiThreads / 128;
    const int e = threadIdx.x & 127, t0 = threadIdx.x >> 7;
    for (int sweep = 0; sweep < 40; ++sweep) {
        double off = 0.0, tot = 0.0;
        for (int idx = threadIdx.x; idx < k * k; idx += kJacobiThreads) {
            const int i = idx / k, j = idx % k;
            const double x = a[i][j] * a[i][j];
            tot += x;
            if (i != j) off += x;
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            off += __shfl_xor(off, o, 64);
            tot += __shfl_xor(tot, o, 64);
        }
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = off;
        __syncthreads();
        double off_all = 0.0;
        for (int wv = 0; wv < kJacobiThreads / 64; ++wv) off_all += red[wv];
        __syncthreads();
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = tot;
        __syncthreads();
        double tot_all = 0.0;
        for (int wv = 0; wv < kJacobiThreads / 64; ++wv) tot_all += red[wv];
        __syncthreads();
        if (!(off_all > 1e-30 * tot_all)) break;
        for (int round = 0; round < n - 1; ++round) {
            // pairs of this round and their rotations, all from the current matrix
            for (int t = threadIdx.x; t < n / 2; t += kJacobiThreads) {
                int p = pos(t, round), q = pos(n - 1 - t, round);
                if (p > q) {
                    const int x = p;
                    p = q;
                    q = x;
                }
                double c = 1.0, sn = 0.0;
                if (q < k) {
                    const double apq = a[p][q];
                    if (apq != 0.0) {
                        const double tau = (a[q][q] - a[p][p]) / (2.0 * apq);
                        const double tt = (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
                        c = 1.0 / sqrt(1.0 + tt * tt);
                        sn = tt * c;
                    }
                }
                pr[t][0] = p;
                pr[t][1] = q;
                cs[t][0] = c;
                cs[t][1] = sn;
            }
            __syncthreads();
            // columns: A <- A J and V <- V J (pair t touches columns p, q only); row i = e
            if (e < k) {
                for (int t = t0; t < n / 2; t += JS) {
                    const int p = pr[t][0], q = pr[t][1];
                    const double c = cs[t][0], sn = cs[t][1];
                    if (q >= k || sn == 0.0) continue;
                    const double aip = a[e][p], aiq = a[e][q];
                    a[e][p] = c * aip - sn * aiq;
                    a[e][q] = sn * aip + c * aiq;
                    const double vip = v[e][p], viq = v[e][q];
                    v[e][p] = c * vip - sn * viq;
                    v[e][q] = sn * vip + c * viq;
                }
            }
            __syncthreads();
            // rows: A <- J^T A (pair t touches rows p, q only); column j = e
            if (e < k) {
                for (int t = t0; t < n / 2; t += JS) {
                    const int p = pr[t][0], q = pr[t][1];
                    const double c = cs[t][0], sn = cs[t][1];
                    if (q >= k || sn == 0.0) continue;
                    const double apj = a[p][e], aqj = a[q][e];
                    a[p][e] = c * apj - sn * aqj;
                    a[q][e] = sn * apj + c * aqj;
                }
            }
            __syncthreads();
        }
    }
    // sort descending (selection by rank, ties to the lower index)
    for (int i = threadIdx.x; i < k; i += kJacobiThreads) {
        int rank = 0;
        for (int j = 0; j < k; ++j) rank += (a[j][j] > a[i][i] || (a[j][j] == a[i][i] && j < i)) ? 1 : 0;
        order[rank] = i;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < k * k; idx += kJacobiThreads) {
        const int i = idx / k, c = idx % k;
        V[idx] = v[i][order[c]];
    }
    for (int c = threadIdx.x; c < k; c += kJacobiThreads) w[c] = a[order[c]][order[c]];
}

// Scale by the eigenvalues w of the Gram (w = S^2): element (i, c) of X (n x r) times f(w[c])
// (by_row = 0) or f(w[i]) (by_row = 1), f = S^{1/2} (mode 0) or 1 / S^{1/2} (mode 1); a
// non-positive w gives 0.
__global__ __launch_bounds__(256) void colscale_kernel(double* X, int ld, int n, int r, const double* w, int mode,
                                                       int by_row) {
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)n * r) return;
    const int i = (int)(idx / r), c = (int)(idx % r);
    const double s2 = w[by_row ? i : c];
    double f = 0.0;
    if (s2 > 0.0) {
        const double sh = sqrt(sqrt(s2));
        f = mode == 0 ? sh : 1.0 / sh;
    }
    X[(size_t)i * ld + c] *= f;
}

__global__ __launch_bounds__(256) void sqrt_kernel(const double* w, double* s, int r) {
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c < r) s[c] = w[c] > 0.0 ? sqrt(w[c]) : 0.0;
}

// --------------------------------------------------------------------------- launchers
// S -= L L^T over rows / columns [c0, d) with L the columns [l0, l0 + kw) of the rows [c0, d)
// (only tiles touching the lower triangle), or, with ncols > 0, only the columns [c0, c0 + ncols)
// of those rows.
static hipError_t chol_update(double* S, int d, int c0, int l0, int kw, int ncols, hipStream_t stream) {
    GemmArgs g{};
    g.M = d - c0, g.N = ncols > 0 ? ncols : d - c0, g.K = kw;
    g.A = S + (size_t)c0 * d + l0, g.lda = d, g.ta = 0;
    g.B = S + (size_t)c0 * d + l0, g.ldb = d, g.tb = 1;
    g.C = S + (size_t)c0 * d + c0, g.ldc = d;
    g.alpha = -1.0, g.beta = 1.0, g.c_lower = 1;
    return launch_gemm(g, stream);
}

// Blocked right-looking Cholesky with 128-column blocks, each factored as two 64-column halves:
// the first half's diagonal block and the rows below it, the second half's columns updated by the
// first half, the second half's diagonal block and rows below, then one trailing update with both
// halves (K = 128: half the passes over the trailing matrix of a 64-column blocking).
hipError_t launch_cholesky(double* S, int d, int* flag, double* dg, int* drop, hipStream_t stream) {
    hipLaunchKernelGGL(diag_kernel, dim3((unsigned)ceil_div(d, 256)), dim3(256), 0, stream, S, d, dg);
    hipError_t e = hipGetLastError();
    for (int n0 = 0; n0 < d && e == hipSuccess; n0 += 128) {
        const int nb2 = min(128, d - n0);
        for (int h = 0; h < nb2 && e == hipSuccess; h += 64) {
            const int c0 = n0 + h, nb = min(64, nb2 - h);
            if (h > 0) {
                e = chol_update(S, d, c0, n0, 64, nb, stream);  // second half's columns, first half's L
                if (e != hipSuccess) break;
            }
            hipLaunchKernelGGL(chol_diag_kernel, dim3(1), dim3(kSmallThreads), 0, stream, S, d, c0, nb, flag, dg,
                               drop);
            const int rest = d - c0 - nb;
            if (rest > 0)  // a full 64-wide block has rows below it
                hipLaunchKernelGGL(chol_panel_kernel, dim3((unsigned)ceil_div(rest, 128)), dim3(128), 0, stream, S, d,
                                   d, c0);
            e = hipGetLastError();
        }
        if (e == hipSuccess && n0 + nb2 < d) e = chol_update(S, d, n0 + nb2, n0, nb2, 0, stream);
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(zero_upper_kernel, dim3((unsigned)ceil_div((int64_t)d * d, 256)), dim3(256), 0, stream, S, d, d);
    return hipGetLastError();
}

// Orthonormal basis of the columns of X (n x k, contiguous rows) in place, by two Cholesky-QR
// passes (the second restores orthogonality lost to the conditioning of the first): G = X^T X,
// Rinv from chol_inv_small_kernel, X <- X Rinv.  T (n x k) and G, Rinv (k x k) are scratch.
hipError_t launch_orth(double* X, int n, int k, double* T, double* G, double* Rinv, double* part, int64_t part_cap,
                       hipStream_t stream) {
    for (int pass = 0; pass < 2; ++pass) {
        double* src = pass == 0 ? X : T;
        double* dst = pass == 0 ? T : X;
        GemmArgs g{};
        g.M = k, g.N = k, g.K = n, g.A = src, g.lda = k, g.ta = 1, g.B = src, g.ldb = k, g.tb = 0;
        g.C = G, g.ldc = k, g.alpha = 1.0, g.beta = 0.0, g.part = part, g.part_cap = part_cap;
        hipError_t e = launch_gemm(g, stream);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(chol_inv_small_kernel, dim3(1), dim3(kSmallThreads), 0, stream, G, k, Rinv);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        GemmArgs h{};
        h.M = n, h.N = k, h.K = k, h.A = src, h.lda = k, h.ta = 0, h.B = Rinv, h.ldb = k, h.tb = 0;
        h.C = dst, h.ldc = k, h.alpha = 1.0, h.beta = 0.0;
        e = launch_gemm(h, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_null_vectors(const double* L, int d, const int* drop, const int* list, int n0, double* N,
                               hipStream_t stream) {
    if (d > kMaxSolveD) return hipErrorInvalidValue;
    hipLaunchKernelGGL(null_vec_kernel, dim3((unsigned)n0), dim3(kNullThreads), 0, stream, L, d, drop, list, n0, N);
    return hipGetLastError();
}

hipError_t launch_jacobi(const double* G, int k, double* w, double* V, hipStream_t stream) {
    hipLaunchKernelGGL(jacobi_kernel, dim3(1), dim3(kJacobiThreads), 0, stream, G, k, w, V);
    return hipGetLastError();
}

hipError_t launch_colscale(double* X, int ld, int n, int r, const double* w, int mode, int by_row,
                           hipStream_t stream) {
    hipLaunchKernelGGL(colscale_kernel, dim3((unsigned)ceil_div((int64_t)n * r, 256)), dim3(256), 0, stream, X, ld, n,
                       r, w, mode, by_row);
    return hipGetLastError();
}

hipError_t launch_sqrt(const double* w, double* s, int r, hipStream_t stream) {
    hipLaunchKernelGGL(sqrt_kernel, dim3((unsigned)ceil_div(r, 256)), dim3(256), 0, stream, w, s, r);
    return hipGetLastError();
}

}  // namespace glowq
