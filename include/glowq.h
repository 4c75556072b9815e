/*
 * glowq.h -- C ABI of the MI355X (gfx950) library for the inference path of group-shared
 * low-rank quantisation-error correction ("GlowQ: Group-Shared LOw-Rank Approximation for
 * Quantized LLMs").
 *
 * What the path computes (token-major: X is T x d, outputs are T x O_i):
 *   W4A16 weights: 4-bit integers q in groups of 128 inputs with one fp16 scale s and one
 *   fp16 zero point z per (row, group); the dequantised weight is (q - z) * s
 *   (GlowQ paper note, "Experimental setup": W4A16, INT4 weights, g128).
 *   Low-rank compensation of the quantisation error W - W_q ~ A B adds A (B X) to the
 *   quantised product (paper note, "Research background and motivation").
 *   For an input-sharing group (Q/K/V on the attention input, gate/up on the MLP input)
 *   one right factor B_shared serves every module; the anchor (Q, or gate) forms
 *   R = X B_shared^T once and every module i, the anchor included, returns
 *   y_i = X W_hat_i^T + R A_i^T (paper note, key design 4 and the flowchart's last node).
 *   Solo modules (o_proj, down_proj) share no input and correct on the fly with a private B
 *   (key design 4).  GlowQ-S applies the correction only on selected units (restore bit).
 *
 * Conventions for every entry point:
 *   - Pointers named *_dev, and every tensor pointer of the forward calls, are DEVICE
 *     pointers on the current HIP device; the caller allocates and owns all memory.  The
 *     forward calls allocate nothing and keep no state between calls.
 *   - fp16 means IEEE binary16; tensors are dense row-major.
 *   - Tensor pointers must be 16-byte aligned; the workspace 256-byte aligned.
 *   - Every argument is validated on the host BEFORE any HIP call; a rejected call makes
 *     no HIP call and returns a negative status.  Kernels are launched asynchronously on
 *     `stream`; launch failures return GLOWQ_ERR_HIP; execution faults surface at the
 *     caller's next synchronisation.
 *   - Outputs must not alias inputs or the workspace.  One workspace must not be used by
 *     two calls that may run concurrently.
 */
#ifndef GLOWQ_H
#define GLOWQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status codes */
#define GLOWQ_OK 0
#define GLOWQ_ERR_INVALID_ARG (-1) /* null pointer, bad enum value                         */
#define GLOWQ_ERR_SHAPE (-2)       /* a size out of range (d % 128, T < 0, n_out < 1, ...)  */
#define GLOWQ_ERR_ALIGN (-3)       /* pointer not 16-byte (workspace: 256-byte) aligned    */
#define GLOWQ_ERR_UNSUPPORTED (-4) /* r > 256, r % 8 != 0, more than 8 modules            */
#define GLOWQ_ERR_WORKSPACE (-5)   /* workspace missing or smaller than required          */
#define GLOWQ_ERR_HIP (-6)         /* a HIP runtime call or kernel launch failed           */
#define GLOWQ_ERR_RANGE (-7)       /* repack: a zero point is not an integer in [-1024,1024]
                                      or a scale is not finite; solve: Sigma_x not PSD   */
#define GLOWQ_ERR_HANDOFF (-8)     /* glowq_workspace_status: a bounded wait for the shared
                                      projection expired in a call since the last check;
                                      that call's corrected outputs are invalid            */
#define GLOWQ_ERR_ROUTING (-9)     /* glowq_workspace_status: a mixture-of-experts call met
                                      routing data out of range (clamped; outputs invalid)  */

#define GLOWQ_MAX_MODULES 8
#define GLOWQ_MAX_RANK 256

#define GLOWQ_DTYPE_F32 0
#define GLOWQ_DTYPE_F16 1

/* Human-readable name of a status code (static string, never NULL). */
const char* glowq_status_string(int status);

/* Library version: major * 10000 + minor * 100 + patch. */
int glowq_version(void);

/* ---------------------------------------------------------------- weight format
 * Canonical interchange format of one INT4-g128 module (n_out x k_in, k_in % 128 == 0):
 *   q_canon : uint32 [n_out][k_in / 8]; word w of row o holds input 8w + j in bits
 *             4j..4j+3 (low nibble first), values 0..15;
 *   scales  : fp16 [n_out][k_in / 128];
 *   zeros   : fp16 [n_out][k_in / 128], integer valued, in [-1024, 1024].
 * The device layout (opaque to callers) interleaves nibbles for 128-bit loads in the
 * matrix-core operand order and pairs each zero with its scale; rows are padded to a
 * multiple of 16 with zero weights.
 */
typedef struct glowq_qweight {
    const void* q;  /* device layout words, glowq_q_bytes(n_out, k_in) bytes
                       (MX formats: glowq_mx_q_bytes(format, n_out, k_in))               */
    const void* sz; /* device layout zero/scale pairs (MX: block scales),
                       glowq_sz_bytes(n_out, k_in) bytes for every format                */
    int64_t n_out;  /* output rows O_i >= 1                                            */
    int64_t k_in;   /* input columns d, a positive multiple of 128                      */
    int32_t format; /* GLOWQ_FMT_*; 0 (a zero-initialised struct) is INT4-g128          */
    int32_t reserved; /* must be 0                                                     */
} glowq_qweight;

/* ---------------------------------------------------------------- MX weight formats
 * Microscaling weights, the MXFP4 / MXFP6 datatypes GlowQ is applied on (GlowQ arXiv page,
 * Table 13).  Encodings of the OCP Microscaling (MX) v1.0 specification: blocks of 32
 * consecutive inputs of a row share one E8M0 scale 2^(S - 127); an element is sign,
 * exponent and mantissa bits (FP4 E2M1, FP6 E2M3, FP6 E3M2; exponent field 0 subnormal).
 * The pages do not say which FP6 element they use; both are accepted.
 *   codes  : uint8 [n_out][k_in], one element code per byte in its low 4 (FP4) or 6 bits;
 *   scales : uint8 [n_out][k_in / 32], E8M0 biased exponents S.
 * The forward kernels dequantise to fp16 in registers (the gfx950 scaled conversion
 * instructions), which is exact when every element times 2^(S - 127) is an fp16 value:
 * S - 127 in [-23, 13] (MXFP4), [-21, 13] (E2M3), [-20, 11] (E3M2).  glowq_repack_mx rejects
 * other scales (including the NaN scale 255) with GLOWQ_ERR_RANGE.  Every forward entry
 * point accepts these formats except glowq_group_forward_w4a8 and glowq_moe_forward (INT4
 * only: GLOWQ_ERR_UNSUPPORTED); all modules of one call share one format.  glowq_ner_sums
 * takes INT4 weights only.
 */
#define GLOWQ_FMT_INT4_G128 0
#define GLOWQ_FMT_MXFP4 1
#define GLOWQ_FMT_MXFP6_E2M3 2
#define GLOWQ_FMT_MXFP6_E3M2 3

/* Bytes of the device-layout codes of one MX module (0 if the shape or format is invalid):
 * 1024 (MXFP4) or 1536 (MXFP6) bytes per 16 rows x 128 inputs; the scales take
 * glowq_sz_bytes(n_out, k_in) (64 bytes per 16 rows x 128 inputs). */
size_t glowq_mx_q_bytes(int32_t format, int64_t n_out, int64_t k_in);

/* Convert one MX module from codes_dev / scales_dev (the layout above) into the device layout
 * (q_dev: glowq_mx_q_bytes, sz_dev: glowq_sz_bytes).  flag_dev is a caller-provided device
 * int32 that reports a code wider than the element or a scale outside the exact range.  An
 * offline load step: it SYNCHRONISES `stream` and returns GLOWQ_ERR_RANGE on such data (the
 * layout is written regardless).  Shape rules: n_out >= 1, k_in % 128 == 0. */
int glowq_repack_mx(int32_t format, const void* codes_dev, const void* scales_dev, int64_t n_out,
                    int64_t k_in, void* q_dev, void* sz_dev, int32_t* flag_dev, hipStream_t stream);

/* Bytes of the device-layout buffers of one module (0 if the shape is invalid). */
size_t glowq_q_bytes(int64_t n_out, int64_t k_in);
size_t glowq_sz_bytes(int64_t n_out, int64_t k_in);

/* Convert one module from the canonical format (device pointers q_canon_dev, scales_dev,
 * zeros_dev) into the device layout (q_dev, sz_dev).  flag_dev is a caller-provided device
 * int32 used to report out-of-range zero points or non-finite scales.  This is the
 * offline load step: it SYNCHRONISES `stream` and returns GLOWQ_ERR_RANGE if any zero point
 * is not an integer in [-1024, 1024] or any scale is not finite (the layout is written
 * regardless).  Shape rules: n_out >= 1, k_in % 128 == 0. */
int glowq_repack(const void* q_canon_dev, const void* scales_dev, const void* zeros_dev,
                 int64_t n_out, int64_t k_in, void* q_dev, void* sz_dev, int32_t* flag_dev,
                 hipStream_t stream);

/* Export the dequantised weight (q - z) * s of one module to out_dev [n_out][k_in] as fp32
 * (exact: the product of a 5-bit integer difference and an fp16 scale fits in 24 bits) or
 * fp16 (the exact value rounded once to nearest-even).  MX modules export
 * element * 2^(S - 127), exact in both.  It runs the same in-register dequantisation
 * routines as the forward kernels.  Asynchronous on `stream`. */
int glowq_dequant(const glowq_qweight* w, void* out_dev, int32_t out_dtype, hipStream_t stream);

/* ---------------------------------------------------------------- forward
 * Workspace bytes for a call with T tokens, rank r and n_proj right projections (1 for a
 * group or solo call, m for the layerwise baseline).  Holds the projection R = X B^T (the
 * cache of key design 4 in the GlowQ paper note: formed once, consumed by every module),
 * synchronisation words and, for 17 to 64 tokens, the fp32 partial outputs of a call whose
 * input groups are split over workgroups.  It must be zero-filled once after allocation
 * (glowq_workspace_init); every call leaves it reusable.  Returns 0 when no workspace is
 * needed (r == 0 or T == 0).
 */
size_t glowq_workspace_bytes(int64_t T, int32_t r, int32_t n_proj);

/* Zero-fill a freshly allocated workspace (device, 256-byte aligned, workspace_bytes >= 8192)
 * with a fill kernel on `stream` (no memset node, so a captured graph may hold it).  A
 * workspace that is not zero when first used can hold stale synchronisation counters and
 * projection tags: the hand-off would then wait for the wrong call and report
 * GLOWQ_ERR_HANDOFF.  Asynchronous. */
int glowq_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Status of a workspace: SYNCHRONISES `stream`, reads the error word that a correcting decode
 * call raises when one of its bounded waits for the shared projection expires (its corrected
 * outputs are then wrong) and that glowq_moe_forward raises on routing data out of range, clears
 * the word and returns GLOWQ_OK (nothing raised since the last check or init),
 * GLOWQ_ERR_HANDOFF or GLOWQ_ERR_ROUTING.  Allocates nothing; not for use under graph capture. */
int glowq_workspace_status(void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Input-sharing group of m modules (1 <= m <= 8), w[0] the anchor (GlowQ paper note, key
 * design 4: the anchor of an input-sharing group computes the projection of the shared right
 * factor once and every consumer reuses it; the flowchart's last node: each module's output is
 * its quantised product plus A_i times that projection).
 *   x        : fp16 [T][d], the group's shared input (T >= 0; T == 0 is a no-op; T d <= 2^30)
 *   w        : host array of m module descriptors, every w[i].k_in == d
 *   b_shared : fp16 [r][d] shared right factor
 *   a        : host array of m device pointers, a[i] fp16 [w[i].n_out][r]
 *   r        : rank, 0 <= r <= 256, r % 8 == 0
 *   restore  : GlowQ-S bit of this group; restore == 0 or r == 0 computes the quantised
 *              product alone, and then b_shared, a and the workspace may be NULL
 *   y        : host array of m device pointers, y[i] fp16 [T][w[i].n_out]
 * Result: y[i] = fp16_RNE(X W_hat_i^T + (X b_shared^T) a[i]^T), accumulated in fp32; the
 * projection is formed once per call. */
int glowq_group_forward(const void* x, int64_t T, int64_t d, int32_t m, const glowq_qweight* w,
                        const void* b_shared, const void* const* a, int32_t r, int32_t restore,
                        void* workspace, size_t workspace_bytes, void* const* y,
                        hipStream_t stream);

/* Solo module (o_proj, down_proj; GlowQ paper note, key design 4: modules that share their
 * input with no other correct on the fly, nothing cached): y = X W_hat^T + (X b^T) a^T with its private b fp16
 * [r][d], a fp16 [n_out][r] and y fp16 [T][n_out]; nothing is kept after the call.  Same
 * rules as glowq_group_forward. */
int glowq_solo_forward(const void* x, int64_t T, int64_t d, const glowq_qweight* w, const void* b,
                       const void* a, int32_t r, int32_t restore, void* workspace,
                       size_t workspace_bytes, void* y, hipStream_t stream);

/* Allocation-free variant of glowq_group_forward, for callers that cannot allocate (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same kernels,
 * with the library's own scratch in place of the caller's workspace.  The scratch is a
 * file-scope device array of glowq_static_scratch_bytes() bytes (16 MiB), one per GPU, held
 * until the process ends; the first correcting call on a device looks up its address and
 * zero-fills it with a kernel on `stream`.  No call allocates (no hipMalloc / hipFree).
 * Calls whose workspace need, glowq_workspace_bytes(T, r, 1), exceeds the scratch return
 * GLOWQ_ERR_WORKSPACE before any HIP call (every decode call, T <= 64, fits; prefill calls fit
 * up to about T = 2048 at r = 64).  Every call on one GPU shares that GPU's array, which keeps
 * the last call's contents: calls that overlap in time on one GPU (two streams, or two
 * threads) race and give wrong results; order them on one stream or synchronise between them.
 * Hand-off expiries are flagged in the scratch and are not reported by this entry point.
 * Arguments and results as glowq_group_forward. */
size_t glowq_static_scratch_bytes(void);
int glowq_group_forward_static(const void* x, int64_t T, int64_t d, int32_t m, const glowq_qweight* w,
                               const void* b_shared, const void* const* a, int32_t r, int32_t restore,
                               void* const* y, hipStream_t stream);

/* Layerwise baseline (the comparison of the paper's latency table): every module i has
 * its own right factor b[i] fp16 [r][d] and its own projection X b[i]^T, computed in the
 * same kernels.  workspace_bytes >= glowq_workspace_bytes(T, r, m). */
int glowq_layerwise_forward(const void* x, int64_t T, int64_t d, int32_t m, const glowq_qweight* w,
                            const void* const* b, const void* const* a, int32_t r, int32_t restore,
                            void* workspace, size_t workspace_bytes, void* const* y,
                            hipStream_t stream);

/* ---------------------------------------------------------------- W4A8
 * The same group forward with 8-bit activations for the quantised product (the W4A8 rows of the
 * GlowQ arXiv page, Tables 14 and 15: INT4-g128 weights, 8-bit activations, the correction
 * applied as in W4A16).  Per token t (a row of X): scale_t = max_k |x[t, k]| / 127 (fp32),
 * code[t, k] = round-half-even(x[t, k] / scale_t) clamped to -127..127 (fp32 division), all
 * codes 0 for a zero row.  Result:
 *   y_i = fp16_RNE(scale_t * (code X W_hat_i^T) + (X b_shared^T) a[i]^T)
 * with the quantised product summed exactly per 128-input group on the int8 matrix cores
 * (nibble products minus z times the group's code sum), scaled in fp32; the projection is formed
 * once per call from the fp16 activations (the high-precision branch).  d <= 16384.
 * Workspace (always needed when T > 0), glowq_w4a8_workspace_bytes(T, d, r or 0) bytes,
 * 256-byte aligned, overwritten: the codes int8 [T][d] (within each 128-input group, position
 * 16 (4 m + g) + 8 h + b holds input 64 m + 32 h + 8 g + {0,4,1,5,2,6,3,7}[b]), then the code
 * sums int32 [T][d / 128], the scales fp32 [T] (each part starting at a multiple of 256 bytes),
 * then for a correcting call the projection.  Other rules as glowq_group_forward. */
size_t glowq_w4a8_workspace_bytes(int64_t T, int64_t d, int32_t r);
int glowq_group_forward_w4a8(const void* x, int64_t T, int64_t d, int32_t m, const glowq_qweight* w,
                             const void* b_shared, const void* const* a, int32_t r, int32_t restore,
                             void* workspace, size_t workspace_bytes, void* const* y, hipStream_t stream);

/* ---------------------------------------------------------------- MX weights x MXFP8
 * The 8-bit-activation form (GlowQ arXiv page, Tables 14-15) with the microscaling datatypes of
 * Table 13 on both operands: MXFP4 or MXFP6 (E2M3 or E3M2) weights (glowq_repack_mx) against
 * activations quantised per call to MXFP8 (OCP MX v1.0: per token and 32-input block an E8M0 scale
 * 2^(floor(log2 max|x|) - 8) and E4M3 elements, nearest value with ties to the even mantissa,
 * saturating at 448), multiplied on the gfx950 block-scaled matrix cores with both block scales
 * applied in hardware; the correction R A_i^T uses the fp16 activations (R = X B^T formed once):
 *   y_i = dequant(Xq) W_hat_i^T + [restore and r > 0] (X B^T) A_i^T.
 * Arguments, shapes and alignment as glowq_group_forward; every module must carry the same MX
 * format (GLOWQ_ERR_UNSUPPORTED for INT4-g128 or mixed formats).  The workspace (256-byte aligned,
 * not shared with concurrent calls, contents need no initialisation) holds the activation codes and
 * scales and, when correcting, the projection: glowq_mx8_workspace_bytes(T, d, r) bytes (r = 0 when
 * not correcting; 0 for an invalid shape).  Asynchronous; allocates nothing. */
size_t glowq_mx8_workspace_bytes(int64_t T, int64_t d, int32_t r);
int glowq_group_forward_mx8(const void* x, int64_t T, int64_t d, int32_t m, const glowq_qweight* w,
                            const void* b_shared, const void* const* a, int32_t r, int32_t restore,
                            void* workspace, size_t workspace_bytes, void* const* y, hipStream_t stream);

/* ---------------------------------------------------------------- mixture of experts
 * The path on an MoE layer (the GlowQ arXiv page, Figures 7-9, Qwen1.5-MoE-A2.7B: the shared
 * covariance-aligned basis of the MLP gate/up projections holds for one expert and across all
 * experts).  Tokens are routed to experts; every routed row is one token sent to one expert, and
 * the rows are listed grouped by expert: rows offsets[e] .. offsets[e + 1] - 1 belong to expert e
 * (offsets non-decreasing, offsets[0] = 0, offsets[n_exp] = n_rows).  Each expert's m modules form
 * an input-sharing group over its rows (m = 2: gate, the anchor, and up; m = 1: a solo module such
 * as down_proj).  With share == GLOWQ_MOE_SHARE_EXPERT each expert forms its projection
 * R_e = X_e B_e^T once from its own rows and its own B_e; with GLOWQ_MOE_SHARE_ALL one B serves
 * every expert and R = X B^T is formed once per token, then consumed by every expert the token is
 * routed to.  Result, for routed row j of expert e reading token t:
 *   y_i[j] = fp16_RNE(X[t] W_hat_{e,i}^T + R[.] A_{e,i}^T)
 * One launch covers every expert (its work is enumerated on the device from the offsets, so the
 * host does not need the per-expert counts).  Routing data out of range (offsets, token indices)
 * is clamped -- never read out of bounds -- and reported by glowq_workspace_status.
 */
#define GLOWQ_MOE_SHARE_EXPERT 0
#define GLOWQ_MOE_SHARE_ALL 1
#define GLOWQ_MOE_MAX_EXPERTS 256
#define GLOWQ_MOE_MAX_MODULES 4

typedef struct glowq_moe_module {
    const void* q;   /* device layout of all experts' modules: expert e at byte e * glowq_q_bytes(n_out, k_in) */
    const void* sz;  /* expert e at byte e * glowq_sz_bytes(n_out, k_in)                          */
    const void* a;   /* fp16 [n_exp][n_out][r] left factors (may be NULL when not correcting)     */
    void* y;         /* fp16 [n_rows][n_out] output, in routed-row order                           */
    int64_t n_out;   /* rows of one expert's module                                               */
    int64_t k_in;    /* == d                                                                      */
} glowq_moe_module;

/* Workspace of glowq_moe_forward: 8192 bytes of status words, then (correcting calls) the fp16
 * projection [rows][r_pad] (rows = n_rows per expert, or T shared by all) and, shared by all, its
 * split-K partials.  Zero-fill it once (glowq_workspace_init). */
size_t glowq_moe_workspace_bytes(int64_t n_rows, int64_t T, int32_t r, int32_t share);

/*   x            : fp16 [T][d]; with row_token_dev NULL row j reads x[j] (then T == n_rows)
 *   n_exp, m     : experts (1 .. 256), modules per expert (1 .. 4)
 *   mods         : host array of m module descriptors (stacked over experts)
 *   b            : fp16 [n_exp][r][d] (SHARE_EXPERT) or [r][d] (SHARE_ALL); NULL when not correcting
 *   r, restore   : rank (0 .. 256, r % 8 == 0) and the GlowQ-S bit of this call
 *   row_token_dev: device int32 [n_rows], token of each routed row, or NULL
 *   offsets_dev  : device int32 [n_exp + 1]
 *   n_rows       : routed rows (0 is a no-op)
 * Asynchronous on `stream`. */
int glowq_moe_forward(const void* x, int64_t T, int64_t d, int32_t n_exp, int32_t m, const glowq_moe_module* mods,
                      const void* b, int32_t share, int32_t r, int32_t restore, const int32_t* row_token_dev,
                      const int32_t* offsets_dev, int64_t n_rows, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* ---------------------------------------------------------------- decoder-layer schedule
 * A sequence of units run in order on one stream: per decoder layer the QKV group, the
 * o_proj solo, the gate/up group and the down_proj solo, each with the restore bit of the
 * GlowQ-S mask (paper note, key design 4).  Every unit is validated before the first
 * launch; the workspace is reused unit after unit and must hold the largest unit.
 */
#define GLOWQ_UNIT_GROUP 0
#define GLOWQ_UNIT_SOLO 1

typedef struct glowq_unit {
    int32_t kind;             /* GLOWQ_UNIT_GROUP or GLOWQ_UNIT_SOLO (then m == 1) */
    int32_t m;                /* modules                                        */
    const void* x;            /* fp16 [T][d]                                    */
    int64_t T, d;
    const glowq_qweight* w;   /* host array of m descriptors                      */
    const void* b;            /* fp16 [r][d]                                    */
    const void* const* a;     /* host array of m device pointers                */
    int32_t r;
    int32_t restore;          /* this unit's GlowQ-S bit                        */
    void* const* y;           /* host array of m device pointers                */
} glowq_unit;

int glowq_path_forward(const glowq_unit* units, int32_t n_units, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- GlowQ-S restore selection
 * Importance scores and the budgeted top-k choice of the units to restore (GlowQ paper note,
 * key design 4: units are ranked by a score -- the normalised error ratio
 * g_ner(u) = ||E_u||_F^2 / ||W_u||_F^2 with E = W - W_hat is one of the two -- and only the
 * top k are activated, layer order deciding when the signal is weak; the arXiv page, Figure 12,
 * sorts restorable groups by this ratio among other metrics).  A unit is any set of modules
 * (a group, a solo module, a whole decoder layer); its ratio is the sum of its modules' squared
 * errors over the sum of their squared weights.
 */

/* Workspace bytes of glowq_ner_sums for a module with n_out rows (0 if n_out is invalid). */
size_t glowq_ner_workspace_bytes(int64_t n_out);

/* Squared error and squared weight of one module:
 *   w_dev    : the fp16 weight W [n_out][k_in] the module was quantised from
 *   wq       : its quantised form in the device layout (glowq_repack)
 *   sums_dev : fp64 [2] output, sums_dev[0] = ||W - W_hat||_F^2, sums_dev[1] = ||W||_F^2
 * W_hat = (q - z) s is rebuilt exactly; the difference and its square are exact in fp64 and the
 * sums are taken in a fixed order (bitwise repeatable).  workspace: device memory of at least
 * glowq_ner_workspace_bytes(n_out) bytes, 256-byte aligned, overwritten.  Asynchronous. */
int glowq_ner_sums(const void* w_dev, const glowq_qweight* wq, void* workspace, size_t workspace_bytes,
                   double* sums_dev, hipStream_t stream);

/* The same for n >= 1 modules at once (a few launches for the whole set): w_devs and wqs are
 * host arrays of n entries, sums_dev fp64 [n][2] receives module i's pair at sums_dev[2 i],
 * and workspace_bytes >= the sum over the modules of glowq_ner_workspace_bytes(n_out). */
int glowq_ner_sums_batch(int32_t n, const void* const* w_devs, const glowq_qweight* wqs, void* workspace,
                         size_t workspace_bytes, double* sums_dev, hipStream_t stream);

/* Scores and restore mask of n_units units (1 <= n_units <= 4096), each made of n_per_unit
 * modules (1 .. 1024):
 *   sums_dev   : fp64 [n_units][n_per_unit][2], the glowq_ner_sums pairs of every module
 *   k          : how many units to restore, 0 <= k <= n_units
 *   scores_dev : fp64 [n_units] output, sum of the errors over sum of the weights (0 if the
 *                latter is 0), summed in module order
 *   mask_dev   : int32 [n_units] output, 1 for the k highest scores, equal scores going to
 *                the lower unit index, else 0
 * Asynchronous. */
int glowq_restore_topk(const double* sums_dev, int32_t n_units, int32_t n_per_unit, int32_t k,
                       double* scores_dev, int32_t* mask_dev, hipStream_t stream);

/* The same choice with the layer-order fallback for a weak signal (key design 4: when the scores
 * do not separate the units, restore in layer order).  rel_tol in [0, 1]: a unit's distance from
 * the best score max is counted in steps of rel_tol * max, key = floor((max - score) /
 * (rel_tol * max)) in fp64; the k units with the smallest keys are restored, equal keys going to
 * the lower unit index -- so when every score lies within one step of the best, the first k units
 * are restored.  rel_tol == 0 is glowq_restore_topk.  Asynchronous. */
int glowq_restore_select(const double* sums_dev, int32_t n_units, int32_t n_per_unit, int32_t k, double rel_tol,
                         double* scores_dev, int32_t* mask_dev, hipStream_t stream);

/* ---------------------------------------------------------------- offline factor solve
 * Input second moment of the calibration activations, the statistic the covariance-aligned fit
 * is built on (GlowQ paper note, key design 2: the usage-weighted risk E||M x||^2 equals
 * ||M Sigma_x^{1/2}||_F^2 with Sigma_x = E[x x^T]; the arXiv page, Figure 2, takes the empirical
 * input covariance of the calibration samples).
 */

/* Workspace bytes of glowq_second_moment (0 if N or d is invalid). */
size_t glowq_second_moment_workspace_bytes(int64_t N, int64_t d);

/* Sigma_x = X^T X / N:
 *   x_dev     : fp16 [N][d], one calibration token per row (N >= 1; d % 128 == 0, d <= 16384,
 *               N d <= 2^31)
 *   sigma_dev : fp32 [d][d] output, symmetric (both triangles written)
 * Products of fp16 values are exact in fp32 and accumulated in fp32 on the matrix cores per
 * token range, the ranges added in a fixed order (bitwise repeatable), then scaled by 1 / N.
 * workspace: at least glowq_second_moment_workspace_bytes(N, d) bytes, 256-byte aligned,
 * overwritten.  Asynchronous. */
int glowq_second_moment(const void* x_dev, int64_t N, int64_t d, float* sigma_dev, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes of glowq_solve_factors (0 if the sizes are invalid). */
size_t glowq_solve_workspace_bytes(int64_t m, int64_t d, int32_t k, int32_t r);

/* Shared factors of one input-sharing group (GlowQ paper note, key designs 1-3): the group's
 * quantisation errors stacked row-wise, E_cat (m x d), whitened by the input second moment,
 * then a randomized SVD with the caller's test matrix and q power iterations, balanced factors
 * and the lift back to the original variables:
 *   e_dev     : fp64 [m][d] stacked errors W_i - W_hat_i of the group's modules
 *   sigma_dev : fp64 [d][d] Sigma_x, symmetric positive semidefinite
 *   omega_dev : fp64 [d][k] test matrix (k = r + p oversampled columns, r <= k <= min(96, d))
 *   r, q      : rank, power iterations (0 <= q <= 16)
 *   a_dev     : fp64 [m][r] output A = U_r S_r^{1/2} (rows of module i at its offset in E_cat)
 *   b_dev     : fp64 [r][d] output B = S_r^{1/2} V_r^T L^{-1} (formed as S_r^{-1/2} U_r^T Q^T E_cat,
 *               the same matrix, without a triangular solve)
 *   s_dev     : fp64 [r] output, the r largest singular values of the whitened error
 * Whitening uses the Cholesky factor L of Sigma_x (Sigma_x = L L^T); the product A B is the same
 * for every square root of Sigma_x.  A singular Sigma_x (key design 3 of the paper note lifts with
 * the pseudo-inverse then): pivots at or below 1e-10 of their column's diagonal entry are zero,
 * their columns of L are dropped, and B = S_r^{1/2} V_r^T L^+ -- the rows of B are projected onto
 * the range of Sigma_x (the minimum-norm lift); at most 96 such null directions
 * (GLOWQ_ERR_UNSUPPORTED beyond).  The range finder runs on E_cat L directly (the same bases
 * as on the QR-reduced core R_e L, up to the left factor Q_e that A carries), without forming
 * it: its products are taken as products with E_cat and with L.  All arithmetic in
 * fp64.  This is an offline step: it SYNCHRONISES `stream` and returns GLOWQ_ERR_RANGE if
 * Sigma_x is not positive semidefinite (a pivot below -1e-10 of its diagonal entry).  workspace: at least glowq_solve_workspace_bytes(m, d, k, r)
 * bytes, 256-byte aligned, overwritten. */
int glowq_solve_factors(const double* e_dev, int64_t m, int64_t d, const double* sigma_dev,
                        const double* omega_dev, int32_t r, int32_t k, int32_t q, double* a_dev, double* b_dev,
                        double* s_dev, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes of glowq_ec_score (0 if the sizes are invalid). */
size_t glowq_ec_score_workspace_bytes(int64_t m, int64_t d);

/* Restore score g_ec of one unit (GlowQ paper note, key design 4): the share of the whitened
 * error's energy that its best rank r captures, sum_{j < r} s_j^2 / ||E_cat L||_F^2.
 *   e_dev     : fp64 [m][d] stacked errors of the unit's modules
 *   sigma_dev : fp64 [d][d] Sigma_x (symmetric; only the lower triangle is read)
 *   s_dev     : fp64 [r] singular values of the whitened error (as glowq_solve_factors returns
 *               them), may be NULL when r == 0; 0 <= r <= min(m, d)
 *   out_dev   : fp64 [3] output: ||E_cat L||_F^2 = trace(E_cat Sigma_x E_cat^T) (the same for
 *               every square root L of Sigma_x), sum_{j < r} s_j^2, and their ratio (0 when the
 *               energy is 0)
 * The energy is formed as sum_ij Sigma_ij (E_cat^T E_cat)_ij from the fp64 GEMM's lower triangle,
 * summed in a fixed order (bitwise repeatable).  With singular values from the randomized solve
 * the captured energy is that of its rank-r approximation, at most the exact best rank r.
 * workspace: at least glowq_ec_score_workspace_bytes(m, d) bytes, 256-byte aligned,
 * overwritten.  Asynchronous on `stream`. */
int glowq_ec_score(const double* e_dev, int64_t m, int64_t d, const double* sigma_dev, const double* s_dev,
                   int32_t r, double* out_dev, void* workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* GLOWQ_H */
