/*
 * dion.h — C ABI of the MI355X (gfx950) Dion optimizer step.
 *
 * One call performs one Dion step on a stack of `batch` same-shape m x n
 * matrices, entirely on the GPU:
 *
 *     B  = M + G                              (error-feedback buffer)
 *     P0 = B Q                                (one warm-started power-iteration step)
 *     P  = orth(P0)                           (Q-factor of the thin QR, diag > 0)
 *     R  = B^T P
 *     M <- B - (1 - mu) P R^T                 (error feedback into the momentum)
 *     Q <- R / (||r_j||_2 + eps)              (column-normalized, next step's warm start)
 *     X <- X - lr * sqrt(m / n) * P Q^T       (orthonormalized low-rank weight update)
 *
 * Passages defining the operation:
 *   - "Dion e la fine del monopolio di Adam negli optimizer AI distribuiti"
 *     (rivista.ai): only the first r singular directions are orthonormalized
 *     (the paragraph that introduces rank as a new scaling dimension); the
 *     full-versus-low-rank difference is kept and re-injected by error feedback
 *     (the paragraph on FSDP traffic); amortized power iteration with QR and
 *     Cholesky decompositions replaces Newton-Schulz, and only 2-D parameters
 *     are routed to Dion, 1-D ones to AdamW or Lion (the paragraph beginning
 *     "Tecnicamente"); the rank fraction is the cost/accuracy knob (the
 *     paragraph on the "default" optimizer).
 *   - "DASH: Faster Shampoo via Batched Block Preconditioning ..." (gist.science,
 *     "Methodologie", 1. Batched Block Preconditioning): same-shape blocks are
 *     stacked into one 3-D tensor and processed by one batched call.
 *   Readings where the pages are silent: s = sqrt(m/n); eps is used only as
 *   ||r_j|| + eps; "orth" is the unpivoted thin-QR Q-factor with a positive
 *   diagonal, reached here by Cholesky-based QR (CholeskyQR2) with an fp64
 *   fallback chain for ill-conditioned P0 (fp64 CholeskyQR2, shifted CholeskyQR3,
 *   and a Householder QR where those break down).
 *
 * Memory and ownership
 *   Every buffer is device memory owned by the caller; the library allocates
 *   no device memory and keeps no data between calls.  Layouts are row-major and
 *   contiguous: X, G, M as [batch][m][n]; Q as [batch][n][rank].
 *   X, M and Q are updated in place; G is read only.  X and G are fp32 or
 *   bf16 (independently); M and Q are fp32.  The workspace is scratch owned by
 *   the caller, at least dion_workspace_size() bytes; after the call it begins
 *   with P as fp32 [batch][m][rank] (the orthonormal factor of this step).
 *   Pointers must be 16-byte aligned (256-byte for the workspace) and the
 *   state buffers must not overlap each other or the workspace.
 *
 * Arithmetic
 *   fp32 weights (x_dtype DION_F32): P0 = B Q, the orthonormalization and R = B^T P are
 *   fp32-accurate: the contractions run on the bf16 matrix cores with each fp32 operand split
 *   exactly into three bf16 parts (six part products kept, fp32 accumulation), and
 *   ill-conditioned matrices take an fp64 chain (P0, the QR and R in fp64).  The weight pass's
 *   two rank-r products P R^T and P Q'^T, whose operands are final (no conditioning amplifies
 *   their error), split each operand into two bf16 parts (hi + lo, 16 significant bits) and
 *   keep the three part products hi hi, hi lo, lo hi: relative error at most about 3 * 2^-16
 *   per term, fp32 accumulation.
 *   bf16 weights (x_dtype DION_BF16): the three big contractions (P0 = B Q, R = B^T P and the
 *   rank-r products of the weight pass) are plain bf16 products: operands rounded once to bf16,
 *   fp32 accumulation (relative error about 2^-8), the precision bf16 weights carry.  The
 *   orthonormalization keeps the fp32-accurate arithmetic, so P^T P = I to fp32 accuracy.
 *   DION_OPT_EXACT_PRODUCTS makes every product fp32-accurate: the six-product split for the
 *   weight pass of fp32 weights and for the three big contractions of bf16 weights.
 *
 * Execution
 *   Asynchronous: the call returns without a host synchronization.  The stack
 *   may be split into chunks of whole matrices that run concurrently on the
 *   library's own streams (a per-device set of default-priority HIP streams
 *   and events, created on first use and kept): they start after the work
 *   already enqueued on `stream` (a hipStream_t, NULL = the default stream)
 *   and `stream` waits for them before anything enqueued after the call, so
 *   the call behaves as if everything ran on `stream`.  Results are bitwise
 *   reproducible for the same inputs on the same device whatever the chunking
 *   (no floating-point atomics; matrices are independent).  Calls that share
 *   a workspace must be ordered on one stream.
 *
 * Errors
 *   0 = success.  A negative status below -99 is a HIP launch error
 *   (status = -100 - hipError_t).  Other negative statuses are argument errors
 *   detected on the host before anything is enqueued; the state is then
 *   untouched.  NaN / Inf inputs are not rejected: they propagate and are
 *   reported in `flags`.
 */
#ifndef DION_MI355X_H
#define DION_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* storage type of X and G */
typedef enum { DION_F32 = 0, DION_BF16 = 1 } dion_dtype;

/* status codes */
enum {
    DION_OK = 0,
    DION_ERR_NULL = -1,       /* a required pointer is NULL */
    DION_ERR_SHAPE = -2,      /* m < 1, n < 1, batch < 0, or a size overflows */
    DION_ERR_RANK = -3,       /* rank outside [0, min(m, n)] */
    DION_ERR_HYPER = -4,      /* mu outside [0, 1), lr not finite, eps < 0 or not finite */
    DION_ERR_ALIGN = -5,      /* a pointer is not 16-byte (workspace: 256-byte) aligned */
    DION_ERR_OVERLAP = -6,    /* two of X, G, M, Q, workspace, flags overlap */
    DION_ERR_WORKSPACE = -7,  /* workspace smaller than dion_workspace_size() */
    DION_ERR_DTYPE = -8,      /* x_dtype or g_dtype not a dion_dtype */
    DION_ERR_OPTION = -9,     /* unknown option bit, contradictory options, or
                                 DION_OPT_HOUSEHOLDER with rank > 4096 */
    DION_ERR_SCRATCH = -10,   /* dion_step_batched_noalloc: the stack needs more than the
                                 DION_NOALLOC_SCRATCH_BYTES of built-in scratch */
    DION_ERR_HIP = -100       /* -100 - hipError_t for a failed HIP call */
};

/* `options` bits */
enum {
    DION_OPT_STICKY_F64 = 1,  /* matrices whose flags word has DION_FLAG_F64 set on entry
                                 skip the fp32 attempt and go straight to the fp64 chain */
    DION_OPT_FORCE_F64 = 2,   /* every matrix uses the fp64 chain */
    DION_OPT_FORCE_F32 = 4,   /* never fall back; an fp32 breakdown is reported as
                                 DION_FLAG_NONFINITE and that matrix takes the rank-0 step
                                 (see DION_FLAG_NONFINITE) */
    DION_OPT_HOUSEHOLDER = 16, /* the fp64 chain orthonormalizes P0 by its last-resort Householder
                                 QR instead of CholeskyQR (with DION_OPT_FORCE_F64: every
                                 matrix); not with DION_OPT_FORCE_F32, rank <= 4096.  The
                                 Householder QR runs one workgroup per matrix: it is slow */
    DION_OPT_SPECTRAL_SHIFT = 32, /* the shifted first pass of the fp64 chain takes its shift from
                                 a multi-power-iteration estimate of lambda_max(P0^T P0) (32
                                 start vectors, 10 normalized products; see
                                 dion_lambda_max_batched) instead of from trace(P0^T P0), which
                                 exceeds it by up to the rank.  Adds 13 launches to the fp64
                                 chain, which return at once for the matrices not shifted; not
                                 with DION_OPT_FORCE_F32 */
    DION_OPT_EXACT_PRODUCTS = 64, /* fp32-accurate products everywhere (see Arithmetic): the
                                 six-product split in the weight pass of fp32 weights, and in
                                 place of plain bf16 products for bf16 weights */
    DION_OPT_CHUNKS_SHIFT = 8 /* bits 8..11: number of concurrent chunks the stack is split into
                                 (0 = automatic, 1 = everything on `stream`); see Execution */
};

/* per-matrix `flags` bits written by the step (device int32 [batch]) */
enum {
    DION_FLAG_F64 = 1,        /* this step's P and R came from the fp64 chain */
    DION_FLAG_NONFINITE = 2,  /* a NaN/Inf was met, or the factorization broke down with no
                                 fallback left (DION_OPT_FORCE_F32, or rank > 4096 where the
                                 Householder QR does not reach): such a matrix gets M <- M + G and
                                 keeps X and Q unchanged, and its P in the workspace is undefined */
    DION_FLAG_SHIFTED = 4,    /* the fp64 chain needed the shifted first pass */
    DION_FLAG_HOUSEHOLDER = 8 /* P came from the fp64 Householder QR (the CholeskyQR passes broke
                                 down, or DION_OPT_HOUSEHOLDER) */
};

/* phases of one step, in launch order (for dion_step_batched_profiled) */
enum {
    DION_PHASE_INIT = 0,             /* per-matrix state words */
    DION_PHASE_F32_PRODUCT = 1,      /* fp32 chain: P0 = (M + G) Q */
    DION_PHASE_F32_QR = 2,           /* fp32 chain: CholeskyQR2 of P0 */
    DION_PHASE_F32_BACKPROJECT = 3,  /* fp32 chain: R = (M + G)^T P */
    DION_PHASE_F64_PRODUCT = 4,      /* fp64 chain: P0 = (M + G) Q */
    DION_PHASE_F64_QR = 5,           /* fp64 chain: (shifted) CholeskyQR */
    DION_PHASE_F64_BACKPROJECT = 6,  /* fp64 chain: R = (M + G)^T P */
    DION_PHASE_NORMS = 7,            /* column norms, next Q, fp64 -> fp32 rounding */
    DION_PHASE_UPDATE = 8,           /* M <- B - (1-mu) P R^T and X <- X - lr s P Q^T */
    DION_PHASE_FLAGS = 9,            /* per-matrix flags */
    DION_NUM_PHASES = 10
};

/*
 * Bytes of device workspace one dion_step_batched call with these sizes needs.
 * Pure host arithmetic (no HIP call).  Returns 0 for invalid sizes.
 */
size_t dion_workspace_size(int64_t m, int64_t n, int64_t batch, int64_t rank);

/*
 * One Dion step on a stack of `batch` matrices (see the top of this file).
 *   X        device, [batch][m][n], x_dtype, updated in place
 *   G        device, [batch][m][n], g_dtype, read only
 *   M        device, [batch][m][n], fp32, updated in place (momentum / error feedback)
 *   Q        device, [batch][n][rank], fp32, updated in place; may be NULL iff rank == 0
 *   m, n     matrix shape (X is m x n); batch >= 0 (0 is a no-op)
 *   rank     r in [0, min(m, n)]; r == 0 gives M <- M + G and leaves X, Q untouched
 *   mu       momentum in [0, 1); lr finite; eps >= 0 (column-norm guard)
 *   workspace, workspace_bytes   device scratch, >= dion_workspace_size(m, n, batch, rank)
 *   flags    device int32 [batch] or NULL: per-matrix DION_FLAG_* bits on exit
 *            (read on entry only with DION_OPT_STICKY_F64)
 *   options  DION_OPT_* bits
 *   stream   hipStream_t to enqueue on (NULL = default stream)
 * Returns DION_OK or a negative status (see above).
 */
int dion_step_batched(void* X, const void* G, float* M, float* Q,
                      int64_t m, int64_t n, int64_t batch, int64_t rank,
                      float mu, float lr, float eps,
                      int x_dtype, int g_dtype,
                      void* workspace, size_t workspace_bytes,
                      int32_t* flags, uint32_t options, void* stream);

/*
 * dion_step_batched with phase markers, for profiling.  `events` holds
 * DION_NUM_PHASES + 1 hipEvent_t handles created by the caller; events[i] is
 * recorded where phase i of the first chunk starts (on the stream that runs
 * that chunk) and events[DION_NUM_PHASES] after its last launch, so
 * hipEventElapsedTime(events[i], events[i + 1]) is the device time of phase i
 * for the first chunk's matrices (all matrices when the step is not split).  The single-kernel phases (the four products, the
 * update) time one kernel each.  A chain that does not run records its three
 * events back to back.  No host synchronization; same results and status
 * codes as dion_step_batched.  `events` may be NULL.
 */
int dion_step_batched_profiled(void* X, const void* G, float* M, float* Q,
                               int64_t m, int64_t n, int64_t batch, int64_t rank,
                               float mu, float lr, float eps,
                               int x_dtype, int g_dtype,
                               void* workspace, size_t workspace_bytes,
                               int32_t* flags, uint32_t options, void* stream,
                               void* const* events);

/*
 * Optional outputs of dion_step_batched_ex (any field may be NULL).
 *   events  DION_NUM_PHASES + 1 hipEvent_t handles, recorded at the phase boundaries as in
 *           dion_step_batched_profiled
 *   rmmc    device fp32 [batch]: each matrix's Relative Maximum Momentum Change over this step,
 *           max_ij |M'_ij - M_ij| / max_ij |M_ij| (M entering the step, M' leaving it; 0 where
 *           both maxima are 0, +inf where only max |M| is).  The statistic is named in
 *           "CurvaDion: Curvature-Adaptive Distributed Orthonormalization" (mlsanity.com,
 *           "Abstract (arXiv)") as a curvature proxy built from the momentum at O(d) cost per
 *           layer; the page gives no formula, and this is the reading of its name.  It is taken
 *           in the pass that writes M' (one more small launch), written on `stream`.
 */
typedef struct {
    void* const* events;
    float* rmmc;
} dion_step_outputs;

/*
 * dion_step_batched with optional outputs (`out` may be NULL).  The rmmc array must be 4-byte
 * aligned and overlap no other buffer; otherwise as dion_step_batched.
 */
int dion_step_batched_ex(void* X, const void* G, float* M, float* Q,
                         int64_t m, int64_t n, int64_t batch, int64_t rank,
                         float mu, float lr, float eps,
                         int x_dtype, int g_dtype,
                         void* workspace, size_t workspace_bytes,
                         int32_t* flags, uint32_t options, void* stream,
                         const dion_step_outputs* out);

/*
 * dion_step_batched without a caller workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, step, results and status codes as dion_step_batched, minus the workspace; the
 * scratch is a static device array of DION_NOALLOC_SCRATCH_BYTES built into the library, one per
 * GPU, held until the process ends.  Nothing is allocated by the call.
 *   - DION_ERR_SCRATCH (checked on the host before anything is enqueued) when
 *     dion_workspace_size(m, n, batch, rank) exceeds DION_NOALLOC_SCRATCH_BYTES;
 *   - the stack runs as one chunk on `stream`: chunk option bits above 1 give DION_ERR_OPTION;
 *   - every call on a GPU shares that GPU's scratch: calls that may overlap on one GPU (other
 *     streams, other threads) race and must be ordered by the caller;
 *   - the first call on a device looks up the scratch's device address (hipGetSymbolAddress);
 *     make that first call outside graph capture.
 *   - P is not returned (dion_step_batched leaves it in its workspace).
 * The scratch's contents on entry do not matter: nothing in it has to start at zero.
 */
#define DION_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int dion_step_batched_noalloc(void* X, const void* G, float* M, float* Q,
                              int64_t m, int64_t n, int64_t batch, int64_t rank,
                              float mu, float lr, float eps,
                              int x_dtype, int g_dtype,
                              int32_t* flags, uint32_t options, void* stream);

/*
 * The parameters Dion does not take.  The rivista.ai page (the paragraph
 * beginning "Tecnicamente") leaves biases and 1-D weights to optimizers such as
 * AdamW or Lion; these are the published rules, one element-wise pass each over
 * a contiguous array of n elements, in fp32 arithmetic:
 *
 *   AdamW, step t >= 1:  p <- p (1 - lr wd);  m <- b1 m + (1 - b1) g;
 *                        v <- b2 v + (1 - b2) g^2;
 *                        p <- p - lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)
 *   Lion:                c = b1 m + (1 - b1) g;  p <- p (1 - lr wd) - lr sign(c);
 *                        m <- b2 m + (1 - b2) g                       (sign(0) = 0)
 *
 *   param    device, [n], p_dtype (DION_F32 or DION_BF16; bf16 rounded to nearest
 *            even once per step), updated in place
 *   grad     device, [n], g_dtype, read only
 *   exp_avg, exp_avg_sq   device, [n], fp32, updated in place (caller-owned state,
 *            zero before the first step)
 *   n >= 0 (0 is a no-op); t >= 1; b1, b2 in [0, 1); lr, wd finite; eps finite >= 0
 * Pointers 16-byte aligned and not overlapping.  Asynchronous on `stream`
 * (NULL = default stream); no allocation.  Returns DION_OK or a negative status
 * (checked on the host before anything is enqueued).
 */
int dion_adamw_step(void* param, const void* grad, float* exp_avg, float* exp_avg_sq, int64_t n, int64_t t,
                    float lr, float beta1, float beta2, float eps, float weight_decay,
                    int p_dtype, int g_dtype, void* stream);
int dion_lion_step(void* param, const void* grad, float* exp_avg, int64_t n,
                   float lr, float beta1, float beta2, float weight_decay,
                   int p_dtype, int g_dtype, void* stream);

/*
 * Multi-power-iteration estimate of the largest eigenvalue of a stack of
 * symmetric positive semi-definite matrices, such as the Gram matrices P0^T P0 of
 * the step.  The DASH summary (gist.science, "Methodologie", 2. "Efficiënte
 * Inverse-Root Solvers", the item on multi-power-iteration scaling) estimates the
 * spectral radius by power iteration run in parallel from a pool of up to 32 start
 * vectors, in place of the Frobenius-norm scale.  Per matrix W:
 *
 *   each pool vector v, `iters` times:  v <- W v / ||W v||
 *   lambda = max over the pool of v^T W v / v^T v     (0 for a vector W maps to 0)
 *
 * The estimate never exceeds lambda_max(W) (up to rounding) and converges to it as
 * (lambda_2 / lambda_1)^(2 iters) for start vectors not orthogonal to its
 * eigenvector.  fp64 throughout.
 *
 *   W        device fp64 [batch][r][r], row-major; only the lower triangle (j <= i) is
 *            read, so the upper one may hold anything
 *   V0       device fp64 [batch][r][k], row-major (the k start vectors of a matrix side
 *            by side), or NULL: the library's start vectors, 2u - 1 with u the top 53
 *            bits of output number b*r*k + i*k + j + 1 of SplitMix64 seeded with 0 for
 *            entry (i, j) of matrix b
 *   k        pool size, 1..32;   iters  normalized products before the quotient, 0..64
 *   lambda   device fp64 [batch], written
 *   workspace  device, >= dion_lambda_max_workspace_size(r, batch, k) bytes,
 *            256-byte aligned, caller-owned scratch (contents on entry ignored)
 *   r >= 1, 0 <= batch <= 65535 (0 is a no-op)
 * W, V0 and lambda 8-byte aligned; lambda and workspace overlap nothing.
 * Asynchronous on `stream` (NULL = default stream): iters + 3 launches, no
 * allocation, no host synchronization.  Returns DION_OK or a negative status
 * (DION_ERR_SHAPE for r, batch or k, DION_ERR_HYPER for iters), checked on the host
 * before anything is enqueued.
 */
size_t dion_lambda_max_workspace_size(int64_t r, int64_t batch, int32_t k);
int dion_lambda_max_batched(const double* W, int64_t r, int64_t batch, const double* V0, int32_t k, int32_t iters,
                            double* lambda, void* workspace, size_t workspace_bytes, void* stream);

/* Static text for a status code (never NULL). */
const char* dion_strerror(int status);

/* ABI version: major * 10000 + minor * 100 + patch. */
int dion_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DION_MI355X_H */
