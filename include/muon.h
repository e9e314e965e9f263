/*
 * muon.h -- C ABI of the MI355X (gfx950) Muon optimizer step library.
 *
 * The library applies one optimizer step to tensors the caller owns (for
 * example PyTorch-allocated device memory), asynchronously on the caller's
 * HIP stream.  Three calls make up the hot path:
 *
 *   muon_init           -- bind a handle to a gfx950 device;
 *   muon_step_batched   -- one Muon step over a list of 2D weight matrices;
 *   adamw_step          -- one fused AdamW step over a list of tensors.
 *
 * What the Muon step computes, per matrix W of shape (rows, cols) =
 * (fan-out, fan-in), gradient G and momentum M ("About Muon: Why Not Adam",
 * kiungsong.github.io, section "The whole thing, in about forty lines", with
 * the lemma and coefficients of section "Making It Actually Run"):
 *
 *   M <- mu*M + (1-mu)*G                          momentum (moving average)
 *   Y <- (1-mu)*G + mu*M   (Y <- M if !nesterov)  Nesterov blend, updated M
 *   X <- Y / (||Y||_F + eps)                      singular values into (0,1]
 *   if rows > cols: X <- X^T                      Gram on the short side
 *   repeat ns_steps times:                        quintic Newton-Schulz
 *       A <- X X^T;  B <- b*A + c*A*A;  X <- a*X + B*X
 *   O <- X (transposed back if it was transposed)
 *   W <- (1 - lr*weight_decay)*W                  decoupled weight decay
 *   W <- W - lr*s*O    s = shape multiplier * extra_scale
 *
 * with (a,b,c) = (3.4445, -4.7750, 2.0315) every iteration unless the caller
 * passes its own table ("The Optimizer Wars: How Muon Is Replacing Adam in
 * Frontier AI Training", ai.info, section "What is Muon? ...").
 *
 * Threading: a handle may be used by one host thread at a time.  Calls only
 * enqueue work and return; they never wait for the device.  muon_step_batched
 * carries its descriptor table (one 216-byte entry per matrix plus prefix
 * arrays) into the caller's workspace in the arguments of small upload
 * kernels, 16 KB per launch (about one launch per 70 matrices), so no host
 * memory is referenced after the call returns.  A handle owns one more
 * stream (default priority).  Matrices fall in three size classes with launches
 * of their own: short side above 128; short side 33 to 128; and the fp32
 * iteration (every matrix under MUON_F32, short side at most 32 under
 * MUON_BF16).  When a call uses more than one class, the Newton-Schulz
 * launches of every class but the first in use run on that stream, ordered
 * after the caller's stream by an event and joined back into it by another
 * before the call's last launch.  For the caller the
 * call still behaves as work on its own stream, stream capture included.
 *
 * Errors: every call validates all of its arguments before it enqueues
 * anything.  Any status other than MUON_ERR_HIP means nothing was enqueued.
 * No call aborts, throws or prints.  Non-finite input values are not
 * checked: they propagate into the outputs as IEEE arithmetic dictates.
 */
#ifndef MUON_MI355X_H
#define MUON_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MUON_OK = 0,
    MUON_ERR_INVALID_ARG = 1,        /* null pointer, bad size/stride/enum  */
    MUON_ERR_UNSUPPORTED_DEVICE = 2, /* not a gfx950 device, or bad ordinal */
    MUON_ERR_WORKSPACE = 3,          /* workspace null or smaller than required */
    MUON_ERR_OVERLAP = 4,            /* param/grad/momentum ranges overlap  */
    MUON_ERR_HIP = 5,                /* a HIP runtime call failed           */
    MUON_ERR_UNALIGNED = 6,          /* pointer not aligned to its element  */
    MUON_ERR_SCRATCH = 7             /* larger than the fixed scratch of an allocation-free call */
} muon_status;

typedef enum { MUON_F32 = 0, MUON_BF16 = 1 } muon_dtype;

/* Per-matrix multiplier of the orthogonalised update
 * ("About Muon: Why Not Adam", sections "Why Muon?" and "How Do We Turn It
 * Into a Real Optimizer?"):
 *   MOONLIGHT  0.2*sqrt(max(rows, cols))  (entry RMS ~0.2; shares AdamW's lr)
 *   JORDAN     sqrt(max(1, rows/cols))
 *   BERNSTEIN  sqrt(rows/cols)            (sqrt(fan-out/fan-in))
 *   NONE       1
 * The result is multiplied by muon_hparams.extra_scale. */
typedef enum {
    MUON_SCALE_MOONLIGHT = 0,
    MUON_SCALE_JORDAN = 1,
    MUON_SCALE_BERNSTEIN = 2,
    MUON_SCALE_NONE = 3
} muon_scale_mode;

typedef struct muon_context* muon_handle;

/* One Muon matrix.  All pointers are device pointers owned by the caller.
 * Layout is row-major (rows, cols) with leading dimensions in elements
 * (ld >= cols).  A row block of a fused tensor (e.g. Q, K and V of a fused
 * QKV weight, "Why Muon Works", section 7.3) is passed as its own matrix
 * with offset pointers.
 *   param      W, F32 or BF16, updated in place.
 *   grad       G, F32 or BF16, read only.
 *   momentum   M, always F32, updated in place (caller zero-fills it before
 *              the first step).
 *   update_out optional (NULL = skip): dense rows x cols F32 array that
 *              receives O, the orthogonalised update before the multiplier.
 *   norm_out   optional (NULL = skip): one F32 that receives ||Y||_F.
 *   qk_smax    optional (NULL = no clip): device F32 array, one maximum
 *              attention logit S_max per block of qk_block_rows rows of W
 *              (a query or key projection, one block per head).  After the
 *              update every row of block h is multiplied by sqrt(gamma_h),
 *              gamma_h = tau / S_max^h if S_max^h > tau, else 1, with tau =
 *              muon_hparams.qk_tau ("The Optimizer Wars ...", section "What
 *              is MuonClip?": QK-Clip rescales W_q^h and W_k^h by sqrt of
 *              min(1, tau / S_max^h) after the Muon update).
 *   qk_block_rows  rows per head block (>= 1 when qk_smax is set). */
typedef struct {
    void* param;
    const void* grad;
    float* momentum;
    float* update_out;
    float* norm_out;
    int64_t rows, cols;
    int64_t ld_param, ld_grad, ld_mom;
    int32_t param_dtype; /* muon_dtype */
    int32_t grad_dtype;  /* muon_dtype */
    const float* qk_smax;
    int64_t qk_block_rows;
} muon_matrix;

/* Step hyperparameters, shared by every matrix of one call.
 *   coeffs: NULL = (3.4445, -4.7750, 2.0315) for every iteration; otherwise a
 *           HOST array of 3*ns_steps floats (a, b, c per iteration), read
 *           during the call only.
 *   ns_dtype: MUON_BF16 (bf16 operands, fp32 accumulation) or MUON_F32.
 *           With MUON_BF16, a matrix whose short side is at most 32 still runs
 *           the iteration in fp32: with that few singular values the bf16
 *           rounding errors do not average out, and the result would miss the
 *           bf16 iteration's usual accuracy on some inputs. */
typedef struct {
    float lr;
    float momentum;     /* mu, typically 0.95 */
    float weight_decay;
    float eps;          /* added to ||Y||_F, typically 1e-7 */
    float extra_scale;  /* typically 1 */
    int32_t nesterov;   /* 1 = Nesterov blend (default), 0 = plain momentum */
    int32_t ns_steps;   /* >= 1, typically 5 */
    int32_t ns_dtype;   /* muon_dtype */
    int32_t scale_mode; /* muon_scale_mode */
    const float* coeffs;
    float qk_tau;       /* QK-Clip threshold (100 in Kimi K2); used only by matrices with qk_smax */
} muon_hparams;

/* One AdamW tensor (flat, numel elements, contiguous).  param F32 or BF16;
 * grad F32 or BF16; exp_avg and exp_avg_sq F32.  Device pointers, caller
 * owned, updated in place. */
typedef struct {
    void* param;
    const void* grad;
    float* exp_avg;
    float* exp_avg_sq;
    int64_t numel;
    int32_t param_dtype;
    int32_t grad_dtype;
} adamw_tensor;

/* AdamW hyperparameters ("Por qué AdamW para entrenar modelos de lenguaje,
 * y qué está cambiando", gustavoai.dev, sections "Adam: las dos ideas
 * juntas", "La W: ..." and "Por qué AdamW, y por qué con esos números").
 *   step: t >= 1, already incremented by the caller (bias correction uses
 *         1 - beta^t). */
typedef struct {
    float lr;
    float beta1;        /* 0.9  */
    float beta2;        /* 0.95 */
    float eps;          /* 1e-8, added to sqrt(v_hat) */
    float weight_decay; /* 0.1, decoupled: theta -= lr*wd*theta_old */
    int64_t step;
} adamw_hparams;

/* Bind a handle to HIP device `device`.  Fails with
 * MUON_ERR_UNSUPPORTED_DEVICE unless the device is gfx950.  Release with
 * muon_destroy. */
muon_status muon_init(int device, muon_handle* out);

/* Free the handle (waits for the events of an unfinished profile). */
muon_status muon_destroy(muon_handle h);

/* Bytes of device workspace muon_step_batched needs for exactly these
 * matrices and hyperparameters (shapes and ns_dtype matter; pointers don't).
 * Same validation as muon_step_batched except for the pointers. */
muon_status muon_workspace_size(muon_handle h, const muon_matrix* mats, int n,
                                const muon_hparams* hp, size_t* bytes);

/* One Muon step over n matrices on `stream` (a hipStream_t; NULL = the
 * device's null stream).  `workspace` is caller-owned device memory of at
 * least muon_workspace_size bytes, 256-byte aligned, used only by this call's
 * kernels; it must not be shared by calls that may run concurrently.  The
 * descriptor array is host memory, read during the call only: the table the
 * kernels read is carried into the workspace in kernel arguments.  The call
 * enqueues work on `stream` and returns; it never waits on the host and keeps
 * no reference to host memory, so it may be captured in a graph (a replay
 * runs the captured shapes and pointers on the buffers' contents at replay
 * time).  Rejects:
 * n < 1, rows or cols < 1 or > 2^20, ld < cols, a null param/grad/momentum, an
 * unknown dtype or mode, ns_steps < 1 or > 1000, lr/momentum non-finite, overlapping
 * param/grad/momentum ranges within a matrix, a small or null workspace,
 * qk_block_rows outside [1, rows] when qk_smax is set, qk_tau < 0. */
muon_status muon_step_batched(muon_handle h, const muon_matrix* mats, int n,
                              const muon_hparams* hp, void* workspace,
                              size_t workspace_bytes, void* stream);

/* One AdamW step over n tensors on `stream`.  No workspace: the tensor list
 * travels in kernel arguments (groups of at most 256 tensors per launch).
 * Rejects n < 1, numel < 0, null pointers for numel > 0, unknown dtypes,
 * step < 1. */
muon_status adamw_step(muon_handle h, const adamw_tensor* ts, int n,
                       const adamw_hparams* hp, void* stream);

/* ---- per-phase timing (benchmarks) ---------------------------------------
 * While enabled, muon_step_batched records a pair of HIP events (on the
 * stream the launch goes to: the caller's, or the handle's second stream)
 * around every kernel launch it makes, and adamw_step around each of its
 * launches.  muon_profile_collect waits for every recorded event, adds up the
 * elapsed times per phase since the previous collect (or enable), fills `out`
 * and clears the record.  Launches on the two streams may overlap in time,
 * and their durations are added all the same.  Timing does not change what the
 * kernels compute.  Phases: 0 momentum, 1 norm, 2 gram, 3 poly, 4 update,
 * 5 apply, 6 adamw (matrices whose short side is at most 128, when their
 * update runs in strips, form the polynomial and the later Gram parts inside
 * the update launches: phase 4, with no phase-3 launch for them; when such
 * matrices are alone in the call and all are fp32 weights of exactly 128 rows
 * and a multiple of 128 columns, without QK-Clip or update_out, the last
 * update launch also applies the step and phase 5 records no launch). */
#define MUON_NUM_PHASES 7
typedef struct {
    float ms[MUON_NUM_PHASES];     /* summed launch durations per phase */
    int32_t launches[MUON_NUM_PHASES];
} muon_phase_times;

muon_status muon_profile_enable(muon_handle h, int enable);
muon_status muon_profile_collect(muon_handle h, muon_phase_times* out);

/* AdamW with the gradients first clipped together to a global Euclidean
 * norm ("Por qué AdamW ...", section "Por qué AdamW, y por qué con esos
 * números": before g enters m and v, if its norm exceeds 1 it is rescaled
 * to 1).  norm = ||(g_1, ..., g_n)||_2 over all numel elements of all n
 * tensors; every gradient is multiplied by max_norm / norm when norm >
 * max_norm (the gradient tensors themselves are not modified).  norm_out
 * (optional device float) receives the norm before clipping.  The reduction
 * has a fixed order, so results are bitwise repeatable.  workspace: caller
 * device memory of at least adamw_workspace_size bytes, 256-byte aligned.
 * Rejects what adamw_step rejects, max_norm <= 0 or non-finite, and a small
 * or null workspace. */
muon_status adamw_workspace_size(muon_handle h, const adamw_tensor* ts, int n, size_t* bytes);
muon_status adamw_step_clipped(muon_handle h, const adamw_tensor* ts, int n,
                               const adamw_hparams* hp, float max_norm, float* norm_out,
                               void* workspace, size_t workspace_bytes, void* stream);

/* adamw_step_clipped for callers that cannot allocate device memory: code
 * under stream capture that may not call hipMalloc, tight serving loops,
 * harnesses that forbid allocation.  Same arguments, results and validation
 * as adamw_step_clipped, without the workspace: the per-chunk partial sums
 * and the clip scale live in a fixed device array that the library holds,
 * one copy per device, for the life of the process (1 MiB + 256 bytes,
 * resolved by muon_init).  The call itself allocates nothing.
 * Limit: the tensors together may hold at most 2^18 chunks of 4096 elements
 * (2^30 elements when every numel is a multiple of 4096; each tensor counts
 * ceil(numel / 4096) chunks); beyond it the call returns MUON_ERR_SCRATCH
 * and enqueues nothing.
 * Every call on one device shares that array, which keeps the last call's
 * contents (nothing in it needs to start at zero).  Calls that may overlap in
 * time on one device -- on different streams, or through different handles
 * of that device -- race on it and must not be made. */
muon_status adamw_step_clipped_noalloc(muon_handle h, const adamw_tensor* ts, int n,
                                       const adamw_hparams* hp, float max_norm,
                                       float* norm_out, void* stream);

/* Static, human readable name of a status. */
const char* muon_status_str(muon_status s);

/* ---- single-phase entry points (test hooks) ------------------------------
 * Each runs one phase of the Newton-Schulz iteration on bf16 device buffers
 * that the caller lays out exactly as muon_step_batched's workspace does:
 * m x n row-major with leading dimension ld (elements), m and n multiples of
 * 256 and every element outside the valid region zero.  They exist so that
 * tests can compare each GEMM against the oracle's intermediate on the same
 * input.
 *   gram:   A = s2 * X X^T          (X: m x n, A: m x m)
 *   poly:   B = a*I + b*A + c*A A   (A, B: m x m, A symmetric)
 *   update: Xo = s * B X             (X, Xo: m x n, ld ldx; B: m x m, ld ldb)
 * (The quintic step a X + b A X + c A A X is (a I + b A + c A A) X: the
 * identity term rides on B's diagonal and the update is a plain product.)
 */
muon_status muon_test_gram_bf16(muon_handle h, const void* X, void* A, int64_t m,
                                int64_t n, int64_t ldx, int64_t lda, float s2, void* stream);
muon_status muon_test_poly_bf16(muon_handle h, const void* A, void* B, int64_t m,
                                int64_t lda, float a, float b, float c, void* stream);
muon_status muon_test_update_bf16(muon_handle h, const void* X, const void* B,
                                  void* Xo, int64_t m, int64_t n, int64_t ldx,
                                  int64_t ldb, float s, void* stream);

/* Test hook of the scheduler: indices into `mats` (ascending, no repeats) of
 * the matrices that hold a tile at which a grouped bf16 GEMM launch's per-XCD
 * tile range starts or ends, or that hold quarter tiles (a short last round
 * of 256-wide tiles split four ways).  Tests pick these matrices to check the
 * tile indexing where it changes.  Writes min(cap, found) indices to `out`
 * and the number found to *count.  Same validation as muon_workspace_size. */
muon_status muon_test_split_matrices(muon_handle h, const muon_matrix* mats, int n,
                                     const muon_hparams* hp, int32_t* out, int cap, int* count);

#ifdef __cplusplus
}
#endif

#endif /* MUON_MI355X_H */
