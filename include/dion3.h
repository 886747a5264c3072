/*
 * dion3.h -- C ABI of libdion3.so, the Dion3 optimizer step on AMD gfx950.
 *
 * The step (source: "Dion3: Full-Stack Orthogonal Updates", agihunt.info
 * summary, level-1 and level-3 paragraphs; the paper abstract on
 * arxivlens.com / scholarbro.com):
 *   1. score every row of the momentum matrix M (n x m) by its l1 norm;
 *   2. select the k = ceil(f n) best rows (ties: lowest row index);
 *   3. orthogonalize the selected k x m submatrix X with Gram Newton-Schulz:
 *      the quintic iteration runs on the small symmetric Gram R = X X^T
 *      (X^T X when k > m), restarting once (iteration 3 by default) from
 *      X <- Q X, R <- X X^T, Q <- I, and only then is Q multiplied back
 *      onto X; fp16 storage, fp32 accumulation;
 *   4. W[S] <- W[S] - lr * O for the selected rows only, and
 *      M[S] <- mu * M[S] (one fp32 multiply) for the selected rows only.
 *
 * Conventions for every entry point:
 *   - Matrices are row-major.  "Rows" are dim 0 (output neurons).
 *   - Every data pointer is a DEVICE pointer owned by the caller.  The
 *     library never allocates or frees device memory: scratch lives in the
 *     caller's workspace `ws` (at least dion3_workspace_size() bytes,
 *     256-byte aligned).
 *   - fp16 data is IEEE binary16 passed as uint16_t.
 *   - `stream` is a hipStream_t (NULL: the null stream).  Calls only enqueue
 *     work on `stream` and return without synchronizing.
 *   - Errors are status codes; nothing aborts or throws across the ABI.  All
 *     argument checks run before the first launch, so on any error W, M and
 *     the outputs are untouched.
 *   - NaN or Inf in M or X gives undefined results (no check is made).
 *   - Concurrent calls are safe when their workspaces and outputs are
 *     disjoint.  The library's only mutable global state is the thread-local
 *     last HIP error and the optional timing trace (dion3_trace_*).
 *   - Within one call the matrices written (W, M and, for the normalized
 *     step, V; every matrix of a megabatch) must not overlap each other in
 *     memory; W and M must not alias.  Inputs that are only read (G, and X
 *     of dion3_gram_ns) may alias outputs: they are consumed first.
 */
#ifndef DION3_H
#define DION3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define DION3_API __attribute__((visibility("default")))
#else
#define DION3_API
#endif

typedef enum {
  DION3_OK = 0,
  DION3_ERR_ARG = -1,          /* a null required pointer or an out-of-range size/parameter:
                                  any size below 1, k outside [1, n], ld < m, a schedule outside
                                  its stated ranges.  Sizes are checked in that order, so k = 0
                                  or k > n is an argument error even where n or m also exceeds
                                  DION3_MAX_DIM */
  DION3_ERR_WORKSPACE = -2,    /* ws is NULL, misaligned or smaller than dion3_workspace_size() */
  DION3_ERR_UNSUPPORTED = -3,  /* a shape beyond the library's limits (sizes that are
                                  otherwise valid): a dimension above DION3_MAX_DIM, or a
                                  zero-padded per-matrix block (the selected rows, padded to
                                  multiples of 128, or the Gram side) of 2^31 bytes or more, or
                                  a product whose 128 x 128 output tiles over the whole batch
                                  exceed 2^31 - 1; with DION3_PATH_FUSED, also a Gram side
                                  min(k, m) above 128 */
  DION3_ERR_HIP = -4           /* a HIP call or launch failed; see dion3_last_hip_error() */
} dion3_status;

#define DION3_MAX_ITERS 16
#define DION3_MAX_RESTARTS 4
#define DION3_MAX_DIM (1 << 20)   /* n, m, k each at most this */
#define DION3_MAX_BATCH 65535
#define DION3_MAX_GROUPS 64       /* shape groups in one dion3_step_groups call */

/* Newton-Schulz schedule.  Iteration t (1-based) uses the quintic
 * coefficients abc[t-1] = (a, b, c): Z = a I + b R + c R^2.  An iteration
 * listed in restart_at[0..n_restart-1] first materializes X <- Q X,
 * recomputes R <- X X^T and resets Q <- I ("Dion3: Full-Stack Orthogonal
 * Updates", agihunt.info, level-1 paragraph: one restart at the 3rd
 * iteration).  Valid: 1 <= iters <= 16, 0 <= n_restart <= 4, each restart
 * index in [2, iters], strictly increasing.  eps >= 0 is added to ||X||_F in
 * the normalization X / (||X||_F + eps). */
typedef struct {
  int32_t iters;
  int32_t n_restart;
  int32_t restart_at[DION3_MAX_RESTARTS];
  float abc[DION3_MAX_ITERS][3];
  float eps;
  int32_t method;   /* DION3_NS_GRAM (default) or DION3_NS_STANDARD */
  int32_t path;     /* DION3_PATH_AUTO (default), _TILED or _FUSED */
} dion3_ns_cfg;

/* method: DION3_NS_GRAM iterates on the Gram matrix (the level-1 paragraph);
 * DION3_NS_STANDARD runs the standard quintic iteration on X itself,
 * X <- a X + (b A + c A^2) X with A = X X^T, on the same fp16 MFMA kernels
 * (the Muon baseline the pages compare against; restarts do not apply). */
#define DION3_NS_GRAM 0
#define DION3_NS_STANDARD 1

/* path (Gram method only): how the Gram iteration is launched.
 * DION3_PATH_TILED: one tiled MFMA product per step of the iteration (about
 *   20 launches per call, every grid spread over the whole GPU).
 * DION3_PATH_FUSED: one launch, one workgroup per matrix running the whole
 *   iteration with R, Z, Q in LDS (for Gram sides up to 64 one wave runs
 *   every s x s product); only when the Gram side min(k, m) is at most 128,
 *   else DION3_ERR_UNSUPPORTED.  Its result is bitwise identical to the
 *   tiled path (same products, same accumulation order, same roundings).
 * DION3_PATH_AUTO: the fused path where it is allowed and expected to be
 *   faster (Gram side <= 128 and enough matrices or short enough rows for
 *   one workgroup each), the tiled path otherwise.
 * The standard method always runs tiled. */
#define DION3_PATH_AUTO 0
#define DION3_PATH_TILED 1
#define DION3_PATH_FUSED 2

/* Default schedule: Gram Newton-Schulz, 5 iterations of Muon's quintic
 * (3.4445, -4.7750, 2.0315), one restart at iteration 3, eps = 1e-7. */
DION3_API void dion3_ns_cfg_default(dion3_ns_cfg* cfg);

/* sizeof(dion3_ns_cfg) as this library was built, so that a binding can
 * check its own copy of the struct before passing one. */
DION3_API size_t dion3_ns_cfg_size(void);

/* k = ceil(f * n) (level-3 paragraph of the agihunt summary), computed in
 * exact rationals: f is read as the nearest fraction with denominator
 * <= 2^20 (so 0.07 * 100 gives 7, not 8).  The result is clamped to [1, n].
 * Returns -1 if n < 1 or f is not finite and positive. */
DION3_API int64_t dion3_k_from_fraction(double f, int64_t n);

/* Workspace bytes needed by dion3_row_select, dion3_gram_ns, dion3_step
 * and dion3_step_megabatch for `batch` matrices of n x m with k selected
 * rows (for dion3_gram_ns pass n = k).  Host-only; no device work. */
DION3_API dion3_status dion3_workspace_size(int32_t batch, int64_t n, int64_t m, int64_t k, size_t* bytes);

/* Steps 1-2 on `batch` matrices stored back to back: M[b] starts at
 * M + b * n * ld (fp32, row stride ld >= m).  Writes idx[b * k + j]
 * (int32, the k selected rows of matrix b in ascending order) and, when
 * scores is not NULL, scores[b * n + i] = sum_j |M[b][i][j]| (fp64). */
DION3_API dion3_status dion3_row_select(const float* M, int32_t batch, int64_t n, int64_t m, int64_t ld,
                              int64_t k, int32_t* idx, double* scores,
                              void* ws, size_t ws_bytes, void* stream);

/* Step 3 alone on `batch` fp16 matrices X[b] (k x m, contiguous, X + b*k*m):
 * normalizes each by its Frobenius norm, runs Gram Newton-Schulz with `cfg`
 * (NULL: the default) and writes O[b] (k x m fp16, contiguous). */
DION3_API dion3_status dion3_gram_ns(const uint16_t* X, uint16_t* O, int32_t batch, int64_t k, int64_t m,
                           const dion3_ns_cfg* cfg, void* ws, size_t ws_bytes, void* stream);

/* The whole step on one matrix: W and M are fp32 n x m with row stride ld.
 * lr is the final step size (the caller applies the 1/sqrt(f) scaling of
 * the level-3 paragraph); mu is the momentum decay of the selected rows.
 * Rows outside the selected set are never written.  Optional outputs (may
 * be NULL): idx_out[k] (int32 ascending) and O_out (k x m fp16, the
 * orthogonalized update before scaling by lr). */
DION3_API dion3_status dion3_step(float* W, float* M, int64_t n, int64_t m, int64_t ld, int64_t k,
                        float lr, float mu, const dion3_ns_cfg* cfg,
                        int32_t* idx_out, uint16_t* O_out,
                        void* ws, size_t ws_bytes, void* stream);

/* The whole step on `batch` same-shape matrices in one call ("megabatching",
 * level-4 paragraph of the agihunt summary, reduced to one GPU: one launch
 * sequence per shape group).  W and M are DEVICE arrays of `batch` device
 * pointers.  Optional outputs: idx_out[batch][k], O_out[batch][k][m].
 * Results equal `batch` separate dion3_step calls bit for bit. */
DION3_API dion3_status dion3_step_megabatch(float* const* W, float* const* M, int32_t batch,
                                  int64_t n, int64_t m, int64_t ld, int64_t k,
                                  float lr, float mu, const dion3_ns_cfg* cfg,
                                  int32_t* idx_out, uint16_t* O_out,
                                  void* ws, size_t ws_bytes, void* stream);

/* The step with the gradient accumulated into the momentum buffer first:
 * M <- M + G (one fp32 add per element, every row of M), then the step as in
 * dion3_step / dion3_step_megabatch on the updated M.  Error feedback keeps
 * the unselected rows of the buffer for later steps and decays only the
 * selected ones ("Dion3: Full-Stack Orthogonal Updates", agihunt.info,
 * level-3 paragraph), so the buffer is a running sum of gradients.  The
 * addition is fused into the row scoring, which reads M and G once.  G has
 * the shape and row stride of M and is not written; for the megabatch form
 * it is a DEVICE array of `batch` device pointers.  Results equal adding G
 * to M in fp32 and then calling dion3_step, bit for bit. */
DION3_API dion3_status dion3_step_accum(float* W, float* M, const float* G, int64_t n, int64_t m,
                                        int64_t ld, int64_t k, float lr, float mu,
                                        const dion3_ns_cfg* cfg, int32_t* idx_out,
                                        uint16_t* O_out, void* ws, size_t ws_bytes, void* stream);
DION3_API dion3_status dion3_step_megabatch_accum(float* const* W, float* const* M,
                                                  const float* const* G, int32_t batch, int64_t n,
                                                  int64_t m, int64_t ld, int64_t k, float lr,
                                                  float mu, const dion3_ns_cfg* cfg,
                                                  int32_t* idx_out, uint16_t* O_out, void* ws,
                                                  size_t ws_bytes, void* stream);

/* Per-neuron normalization of the update.  The pages say that Dion3
 * inherits NorMuon's per-neuron normalization ("Dion3 Cuts Muon Optimizer
 * Time by Up to 6x", quasa.io, section "Dion3's fastest path is a combined
 * systems stack") and that it runs in float32 ("Dion3: Full-Stack
 * Orthogonal Updates", agihunt.info, limitations paragraph), without a
 * formula.  Reading implemented: for the selected rows S and orthogonalized
 * rows O (k x m) of one matrix with a float32 state V (n entries, one per
 * row, caller-owned, zero before the first step):
 *   q_i = mean_j O_ij^2;  V[S_i] <- beta2 V[S_i] + (1 - beta2) q_i;
 *   U_i = O_i / (sqrt(V[S_i]) + eps)  (0 for a zero row with zero state);
 *   U <- U ||O||_F / ||U||_F  (the step keeps O's norm);
 *   W[S] <- W[S] - lr U.  Rows of V outside S are not written. */
typedef struct {
  float beta2;   /* 0 <= beta2 < 1 */
  float eps;     /* >= 0, added to sqrt(V) */
} dion3_norm_cfg;

/* The megabatch step with per-neuron normalization.  W, M, V are DEVICE
 * arrays of `batch` device pointers (V[b]: n floats); G is NULL or such an
 * array of gradients accumulated first as in dion3_step_megabatch_accum.
 * O_out, when not NULL, receives O before the normalization.  The workspace
 * is the one dion3_workspace_size gives for the same shapes.
 * DION3_ERR_ARG also for a NULL V or norm, beta2 outside [0, 1) or eps < 0. */
DION3_API dion3_status dion3_step_megabatch_norm(float* const* W, float* const* M,
                                                 const float* const* G, float* const* V,
                                                 int32_t batch, int64_t n, int64_t m, int64_t ld,
                                                 int64_t k, float lr, float mu,
                                                 const dion3_ns_cfg* cfg,
                                                 const dion3_norm_cfg* norm, int32_t* idx_out,
                                                 uint16_t* O_out, void* ws, size_t ws_bytes,
                                                 void* stream);

/* One shape group of a whole-model step (dion3_step_groups): `batch`
 * matrices of n x m (row stride ld) with k selected rows each and step size
 * lr.  W, M (and G, V when used) are DEVICE arrays of `batch` device
 * pointers, as in dion3_step_megabatch_accum / _norm.  G: NULL, or the
 * gradients accumulated first (M <- M + G).  V: the per-neuron
 * normalization states (n floats per matrix); required when the call is
 * given a dion3_norm_cfg, ignored otherwise.  idx_out ([batch][k] int32) and
 * O_out ([batch][k][m] fp16) are optional outputs as in the megabatch call. */
typedef struct {
  float* const* W;
  float* const* M;
  const float* const* G;
  float* const* V;
  int64_t n, m, ld, k;
  int32_t batch;
  float lr;
  int32_t* idx_out;
  uint16_t* O_out;
} dion3_group;

/* sizeof(dion3_group) as this library was built (for bindings). */
DION3_API size_t dion3_group_size(void);

/* Workspace bytes for dion3_step_groups over these groups and this schedule
 * (cfg NULL: the default).  Only the sizes of each group are read.  The
 * status codes are those of dion3_step_groups' shape checks. */
DION3_API dion3_status dion3_workspace_size_groups(const dion3_group* groups, int32_t ngroups,
                                                   const dion3_ns_cfg* cfg, size_t* bytes);

/* The step over a whole model's shape groups in one call (the host array
 * `groups`, 1 <= ngroups <= DION3_MAX_GROUPS).  Megabatching ("Dion3:
 * Full-Stack Orthogonal Updates", agihunt.info, level-4 paragraph) carried
 * one level further on one GPU: groups whose Gram sides are equal (s =
 * min(k, m); e.g. the attention and down-projection matrices of a
 * transformer at one fraction) may share one set of s x s matrices, where a
 * launch-round cost model says that their products (the polynomial and the
 * symmetric products of the level-2 paragraph) run no slower as one; the
 * side sets then run the iteration in step, each s x s product one launch
 * over every set and each Gram one launch over every group (the
 * multiply-backs, which write each group's own rows, run per group).  With
 * the 128-matrix batch of attention-shaped matrices and the 32 of
 * down-projection shape of a 7B-like model at f = 1/4 that is 8 symmetric,
 * 5 polynomial and 2 Gram launches per step instead of 18, 10 and 6 (the
 * two independent products that read the same polynomial also share one).
 * norm: NULL, or the
 * per-neuron normalization of dion3_step_megabatch_norm for every group.
 * Results equal calling dion3_step_megabatch (_accum, _norm) once per group
 * with the same arguments, bit for bit.  Matrices written by different
 * groups must not overlap.  All checks (every group, then the workspace)
 * run before the first launch. */
DION3_API dion3_status dion3_step_groups(const dion3_group* groups, int32_t ngroups, float mu,
                                         const dion3_ns_cfg* cfg, const dion3_norm_cfg* norm,
                                         void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the
 * megabatched step of dion3_step_megabatch with the same arguments and
 * results bit for bit, but no workspace argument.  Its scratch is a static
 * device array of DION3_STATIC_SCRATCH_BYTES in the library, one per GPU
 * (held until the process ends); the call allocates nothing.  Every call on
 * one GPU shares that GPU's array, so calls that overlap on one GPU (other
 * streams, other threads) race; serialize them.  Nothing in the array needs
 * to start at zero: every region the step reads is written first in the same
 * call.  The stream must belong to the current device.
 * DION3_ERR_WORKSPACE: the call needs more than DION3_STATIC_SCRATCH_BYTES
 * (dion3_workspace_size for the same shapes), checked before any launch.
 * DION3_ERR_ARG also when the stream belongs to another device; the other
 * status codes are dion3_step_megabatch's. */
#define DION3_STATIC_SCRATCH_BYTES (64u << 20)
DION3_API dion3_status dion3_step_megabatch_noalloc(float* const* W, float* const* M, int32_t batch,
                                                    int64_t n, int64_t m, int64_t ld, int64_t k,
                                                    float lr, float mu, const dion3_ns_cfg* cfg,
                                                    int32_t* idx_out, uint16_t* O_out,
                                                    void* stream);

/* The symmetric products of the level-2 paragraph, usable on their own.
 *
 * dion3_syrk_f16: R[b] = A[b] A[b]^T for `batch` fp16 matrices A[b]
 * (rows x cols, row stride lda, batch stride rows*lda).  R[b] is rows x rows
 * fp16 with row stride ldr (batch stride rows*ldr); only lower-triangle
 * tiles are computed and each is mirrored, so R is exactly symmetric.
 * rows and cols must be multiples of 128 and lda, ldr multiples of 8. */
DION3_API dion3_status dion3_syrk_f16(const uint16_t* A, uint16_t* R, int32_t batch, int64_t rows,
                            int64_t cols, int64_t lda, int64_t ldr, void* stream);

/* dion3_symm_f16 ("A^2 + B"): C[b] = alpha A[b] B[b] + beta D[b] + gamma I
 * for symmetric, commuting s x s fp16 matrices A[b], B[b] (so the product is
 * symmetric) and a symmetric D[b]; D may be NULL when beta == 0.  All four share row stride ld and
 * batch stride s*ld; s must be a multiple of 128, ld a multiple of 8.  Only
 * lower-triangle tiles are computed, then mirrored.  C must not alias A, B
 * or D. */
DION3_API dion3_status dion3_symm_f16(const uint16_t* A, const uint16_t* B, const uint16_t* D, uint16_t* C,
                            int32_t batch, int64_t s, int64_t ld, float alpha, float beta,
                            float gamma, void* stream);

/* Kernel timing trace, for benchmarks.  dion3_trace_enable(capacity > 0)
 * creates 2 * capacity HIP events (no device memory) and starts recording:
 * each kernel the library then launches is timed by events on the caller's
 * stream and noted with its name and the algorithmic work it does on
 * unpadded sizes (flops for the MFMA products, HBM bytes for the row
 * kernels).  Within one library call a kernel's start is the previous
 * kernel's end event, so one event is recorded per kernel and a kernel's
 * time includes its own dispatch; the first kernel of a call, and the first
 * after an untimed copy, records a start event of its own.  Records past
 * the capacity are dropped.  capacity <= 0 stops and frees the trace.
 * dion3_trace_record(i, ...) waits for record i's end event and returns its
 * kernel name (a static string), elapsed ms, flops and bytes; it returns
 * DION3_ERR_HIP when recording either event failed.  The trace is
 * process-wide; it is meant for one benchmarking thread. */
DION3_API dion3_status dion3_trace_enable(int32_t capacity);
DION3_API int32_t dion3_trace_count(void);
DION3_API void dion3_trace_reset(void);
DION3_API dion3_status dion3_trace_record(int32_t i, const char** name, double* ms, double* flops,
                                          double* bytes);

DION3_API const char* dion3_status_string(dion3_status status);

/* hipError_t of the last DION3_ERR_HIP returned on the calling thread (0 if none). */
DION3_API int dion3_last_hip_error(void);

/* Library version, for the binding's load check. */
DION3_API int dion3_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DION3_H */
