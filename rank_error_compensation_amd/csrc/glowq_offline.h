// Offline steps around the inference path (restore selection, factor solve): kernel argument
// blocks and launchers shared by score.hip / moment.hip and the C ABI.
#ifndef GLOWQ_OFFLINE_H
#define GLOWQ_OFFLINE_H

#include "glowq_internal.h"

namespace glowq {

// Modules of one restore-score launch (their descriptors travel in the kernel arguments).
constexpr int kNerBatch = 32;
struct NerBatch {
    int32_t n_mod;
    int32_t tile_begin[kNerBatch + 1];  // prefix of the modules' 16-row tiles
    int32_t n_out[kNerBatch], k_in[kNerBatch];
    const _Float16* w[kNerBatch];       // fp16 [n_out][k_in]
    const uint8_t* q[kNerBatch];        // device layout
    const uint8_t* sz[kNerBatch];
    double* part;                       // [tiles][2]
    double* sums;                       // [n_mod][2]
};
hipError_t launch_ner(const NerBatch& a, hipStream_t stream);
hipError_t launch_topk(const double* sums, int32_t n_units, int32_t n_per, int32_t k, double rel_tol, double* scores,
                       int32_t* mask, hipStream_t stream);
// g_ec terms from C = E_cat^T E_cat (lower triangle, d x d): out = (energy, captured, ratio);
// part holds d doubles
hipError_t launch_ec(const double* C, const double* sigma, int d, const double* sv, int r, double* part,
                     double* out, hipStream_t stream);

// Input second moment (offline factor solve): lower-triangle tiles x token ranges.
struct MomentArgs {
    const _Float16* x;   // [N][d] calibration activations
    int32_t N, d;
    int32_t n_tiles;     // (d / kMomentTile) (d / kMomentTile + 1) / 2
    int32_t S, kc;       // token ranges and tokens per range (a multiple of 32)
    float inv_n;
    float* part;         // [S][n_tiles][kMomentTile][kMomentTile] fp32 partial sums
    float* sigma;        // [d][d]
};
hipError_t launch_moment(const MomentArgs& a, hipStream_t stream);
// Second-moment kernel: 256 x 256 tiles (four waves of 128 x 128, 4 x 4 matrix-core blocks each),
// a ring of four 32-token LDS steps (4 x 32 KiB, one workgroup per CU).
constexpr int kMomentTile = 256;
constexpr int kMomentStages = 4;
constexpr int kMomentResident = 256;  // workgroups resident at once (one per CU)
typedef _Float16 h4x __attribute__((ext_vector_type(4)));

// Most units one restore selection ranks (their scores sit in LDS).
constexpr int kMaxScoreUnits = 4096;

// Offline factor solve (fp64).
constexpr int kSolveMaxK = 96;  // r + p columns of the range finder (LDS of the small steps)
constexpr int kMaxSolveD = 16384;  // features of a factor solve
// Most null directions of Sigma_x the solve projects out of B (the pseudo-inverse lift), the
// columns of one orthonormalisation.
constexpr int kSolveMaxNull = kSolveMaxK;
struct GemmArgs {                // C = alpha op(A) op(B) + beta C, row-major
    int32_t M, N, K;
    const double* A;
    int32_t lda, ta;              // ta: op(A) = A^T (A stored K x M)
    const double* B;
    int32_t ldb, tb;              // tb: op(B) = B^T (B stored N x K)
    double* C;
    int32_t ldc;
    double alpha, beta;
    int32_t c_lower;              // only C's lower triangle is needed
    double* part;                 // optional scratch for split-K partial products (or nullptr)
    int64_t part_cap;             // its capacity in doubles
    int32_t splits, kc;           // set by launch_gemm: K ranges of kc, one per grid z
};
// split-K: a launch with fewer tiles than kGemmWant splits K (ranges of at least kGemmMinK) over
// the grid's z dimension when a partial buffer is given, and a second kernel adds the partial
// products in range order (deterministic)
constexpr int kGemmWant = 512;
constexpr int kGemmMinK = 128;
constexpr int kSolveSplitMax = 16;  // partial-product buffer of the solve: 16 max(m, d) k doubles
hipError_t launch_gemm(const GemmArgs& g, hipStream_t stream);
hipError_t launch_cholesky(double* S, int d, int* flag, double* dg, int* drop, hipStream_t stream);
hipError_t launch_null_vectors(const double* L, int d, const int* drop, const int* list, int n0, double* N,
                               hipStream_t stream);
hipError_t launch_orth(double* X, int n, int k, double* T, double* G, double* Rinv, double* part, int64_t part_cap,
                       hipStream_t stream);
hipError_t launch_jacobi(const double* G, int k, double* w, double* V, hipStream_t stream);
hipError_t launch_colscale(double* X, int ld, int n, int r, const double* w, int mode, int by_row,
                           hipStream_t stream);
hipError_t launch_sqrt(const double* w, double* s, int r, hipStream_t stream);

}  // namespace glowq

#endif  // GLOWQ_OFFLINE_H
