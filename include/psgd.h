/*
 * psgd.h -- C ABI of the PowerSGD gradient-compression library for AMD
 * Instinct MI355X (gfx950).
 *
 * The library compresses a whole model's gradient set with rank-r PowerSGD:
 * for every gradient matrix M it adds the error-feedback memory, runs one
 * warm-started power (subspace) iteration P = M Q, P_hat = GS(P),
 * Q = M^T P_hat, and replaces the memory with the residual M - P_hat Q^T.
 * Vectors and small tensors travel uncompressed.
 *
 * Sources (cited by page title and section):
 *   [N152]  anthology-of-the-sota record, note 152 (PowerSGD): "Method",
 *           "Concepts" ("Linearity of compressor", "Warm-start subspace
 *           iteration", "Error feedback").
 *   [GLOSS] inferensys glossary entry "PowerSGD": factorisation, error
 *           feedback and momentum-compression paragraphs.
 *   [PSGD+] "From PowerSGD to PowerSGD+: Low-Rank Gradient Compression for
 *           Distributed Optimization with Convergence Guarantees", Abstract.
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 * - All floating-point data is fp32 (the gradients may be bfloat16, see
 *   PSGD_FLAG_GRADS_BF16).  Device pointers are plain HIP device
 *   addresses, 16-byte aligned; the caller allocates and owns every device
 *   buffer.  The library allocates no device memory.
 * - Gradient-shaped buffers (grads, err, mom, mhat/out) are FLAT: one buffer
 *   per role for the whole model, tensor t occupying `numel(t)` elements from
 *   its plan offset (psgd_plan_tensor).  A matrix is stored row-major
 *   (rows x cols); a 4-D conv weight is viewed as (out, in*kh*kw).
 * - Packed factors: P_hat of compressed tensor t is stored column-major
 *   (rank columns of `rows` floats) from p_off(t) in the P buffer; Q likewise
 *   (rank columns of `cols` floats) from q_off(t) in the Q buffer.  The
 *   pass-through values follow the P_hat region of the P buffer, so the
 *   aggregation of P carries them.
 * - Every device-side call is asynchronous on the given stream and performs
 *   no host synchronisation; device faults surface at the caller's next
 *   synchronisation.  psgd_compress, psgd_decompress, psgd_refresh and
 *   psgd_init_q only enqueue kernels (no allocation, memset or copy), so they
 *   can be captured in a HIP graph when timing is off and the hook, if any,
 *   only enqueues work on the stream.  Calls return a status and never throw; on failure,
 *   psgd_last_error() gives a thread-local message.
 * - Thread safety: a plan is immutable after creation and may be shared by
 *   threads and streams, provided concurrent calls use distinct workspaces.
 */
#ifndef PSGD_H_
#define PSGD_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum psgd_status {
  PSGD_OK = 0,
  PSGD_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad shape, r < 1, ... */
  PSGD_ERR_UNSUPPORTED = 2, /* rank above PSGD_MAX_RANK, unknown flag        */
  PSGD_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required    */
  PSGD_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed    */
  PSGD_ERR_HOOK = 5         /* the aggregation hook returned non-zero        */
} psgd_status_t;

#define PSGD_MAX_RANK 64

/* Tensor kinds ([N152] Method: bias vectors and small tensors are sent
 * uncompressed). */
#define PSGD_KIND_VECTOR 0     /* cols <= 1: a vector, passed through          */
#define PSGD_KIND_PASSTHRU 1   /* matrix with r*(rows+cols) >= rows*cols       */
#define PSGD_KIND_COMPRESSED 2 /* matrix compressed to rank r                  */

/* Plan flags. */
#define PSGD_FLAG_MOMENTUM 1u   /* compress u <- beta*u + G instead of G ([GLOSS],
                                   momentum paragraph); needs the `mom` buffer   */
#define PSGD_FLAG_GRADS_BF16 2u /* the gradient buffer holds bfloat16 values
                                   (mixed-precision training); everything else,
                                   including the error memory, stays fp32      */

/* Pipeline stages, for psgd_timing_read. */
#define PSGD_STAGE_EF_P 0      /* EF-add (+momentum) and P = M Q            */
#define PSGD_STAGE_GS 1        /* Gram-Schmidt of P                          */
#define PSGD_STAGE_MTP 2       /* partial Q = M^T P_hat over row blocks      */
#define PSGD_STAGE_QREDUCE 3   /* fixed-order reduction of the partials      */
#define PSGD_STAGE_RESIDUAL 4  /* E = M - P_hat Q^T (+ M_hat)                */
#define PSGD_STAGE_PASSTHRU 5  /* pass-through packing / unpacking           */
#define PSGD_STAGE_REFRESH 6   /* PowerSGD+ refresh inside psgd_compress      */
#define PSGD_NSTAGES 7

typedef struct psgd_plan* psgd_plan_t;

/* Step flags (psgd_step_opts_t.flags). */
#define PSGD_STEP_NO_ERROR_FEEDBACK 1u /* ablation: compress X alone, M = X; the error
                                          memory is neither read nor accumulated ([N152]
                                          Recommendations: error feedback is not optional) */
#define PSGD_STEP_NESTEROV 2u          /* fused SGD steps along D + sgd_momentum * m
                                          (Nesterov form) instead of m */
/*
 * Deferred residual (error feedback on).  The
 * residual E = M - P_hat Q^T ([GLOSS], error-feedback paragraph) is only read
 * by the next step's EF-add, so it need not be stored: with
 * PSGD_STEP_DEFER_RESIDUAL the call leaves M itself in `err` (P_hat and Q of
 * the step are in `p` and `q` anyway) and skips the residual pass (M_hat, if
 * requested, is still written, by a write-only pass).  The next call passes
 * PSGD_STEP_RESIDUAL_DEFERRED and forms E = M_prev - P_hat_prev Q_prev^T
 * inside its EF-add pass, reading P_hat_prev and Q_prev from `p` and `q`
 * (which must hold the previous call's outputs, unchanged).  Steady state
 * passes both flags; a call with only RESIDUAL_DEFERRED ends with an explicit
 * E again (for a checkpoint).  Per element this removes the residual pass's
 * read of M and write of E: 16 instead of 24 bytes for a compress step.
 * The same E is formed, with the same operations in the same order.
 */
#define PSGD_STEP_DEFER_RESIDUAL 4u
#define PSGD_STEP_RESIDUAL_DEFERRED 8u
/*
 * Compound compression ([GLOSS]: the factors can themselves be quantised):
 * P and Q are rounded to bfloat16 values (nearest, ties to even; kept in the
 * fp32 buffers) as soon as they are formed, before their hooks, so a hook can
 * send them as bfloat16 without further loss, halving the exchanged bytes.
 * Everything after a hook uses the factors as received: the residual, and
 * with it the error memory, carries the quantisation error.  The
 * pass-through values in the P buffer are not rounded.
 */
#define PSGD_STEP_PAYLOAD_BF16 16u
/*
 * Compound compression to 8 bits (same passage): every column of P and of Q
 * (per compressed matrix, r columns each) is rounded, before its hook, to
 * OCP FP8 E4M3 values (3 fraction bits, largest finite value 448; nearest,
 * ties to even) times one power of two per column, 2^k with k the smallest
 * integer for which the column's largest magnitude is at most 448 * 2^k; the
 * values stay in the fp32 buffers, each exactly an 8-bit code times its
 * column's 2^k, so a hook can send one byte per value plus one exponent per
 * column without further loss.  An all-zero column stays zero.  As with
 * bfloat16, everything after a hook uses the factors as received and the
 * pass-through values are not rounded.  Exclusive with
 * PSGD_STEP_PAYLOAD_BF16 (PSGD_ERR_INVALID_ARG if both are set).
 */
#define PSGD_STEP_PAYLOAD_FP8 32u

/*
 * Options of one psgd_compress call; a NULL pointer means all defaults.
 *   power_iters    subspace iterations in the step (0 or 1: the single
 *                  warm-started iteration of [N152] Method; k > 1 repeats
 *                  P = M Q, P_hat = GS(P), Q = M^T P_hat k times, with both
 *                  hooks called in every iteration -- the glossary's "one or
 *                  two power iterations").
 *   refresh_iters  0 for a plain step.  k > 0 makes this a PowerSGD+ step
 *                  ([PSGD+] Abstract: the projection subspace is periodically
 *                  re-aligned with the optimal one through an SVD): after the
 *                  EF-add, every warm-start Q is replaced by k rounds of block
 *                  power iteration with orthonormalisation on M,
 *                  Q <- GS(M^T GS(M Q)), before P = M Q.  The caller chooses
 *                  the period (for example every 50th step).
 *   flags          any of PSGD_STEP_NO_ERROR_FEEDBACK, PSGD_STEP_NESTEROV,
 *                  PSGD_STEP_DEFER_RESIDUAL, PSGD_STEP_RESIDUAL_DEFERRED,
 *                  PSGD_STEP_PAYLOAD_BF16 or PSGD_STEP_PAYLOAD_FP8, or 0.
 *   params, sgd_buf, sgd_lr, sgd_momentum
 *                  fused post-compression momentum SGD ([N152] Concepts,
 *                  "Post-compression momentum"): when params is non-NULL, the
 *                  decompressed (aggregated) update D of every tensor is
 *                  applied in the residual pass as heavy-ball SGD,
 *                  m <- sgd_momentum * m + D, x <- x - sgd_lr * m (with
 *                  PSGD_STEP_NESTEROV: x <- x - sgd_lr * (D + sgd_momentum * m)),
 *                  on the flat parameter buffer `params` and the flat buffer `sgd_buf`
 *                  (both in/out, plan layout, required together).
 *   zero_cols      nullable, 4-byte aligned: ncompressed int32 in device
 *                  memory or in pinned host memory (hipHostMalloc), written
 *                  by the device.  Once the call has completed on the stream,
 *                  entry k holds how many columns of compressed matrix k's
 *                  P_hat (plan order) the Gram-Schmidt dependence rule set to
 *                  zero in this call (the last iteration's, with power_iters
 *                  > 1).  A warm start keeps such a column zero on later steps
 *                  (its Q column is M^T 0), so a non-zero count reports a drop
 *                  of the transmitted rank ([N152] Method: Gram-Schmidt of the
 *                  P factor; Concepts, "Warm-start subspace iteration").
 */
typedef struct psgd_step_opts {
  int32_t power_iters;
  int32_t refresh_iters;
  uint32_t flags;
  float sgd_lr;
  float sgd_momentum;
  float* params;
  float* sgd_buf;
  int32_t* zero_cols;
} psgd_step_opts_t;

/* Sizes derived from a plan.  Element counts are fp32 elements. */
typedef struct psgd_plan_info {
  int32_t ntensors;
  int32_t ncompressed;
  int32_t rank;
  uint32_t flags;
  size_t flat_elems;     /* elements each flat buffer must hold               */
  size_t p_elems;        /* P_hat region of the P buffer (with padding)       */
  size_t passthru_elems; /* pass-through values after the P_hat region        */
  size_t p_buffer_elems; /* p_elems + passthru_elems: size of the P buffer    */
  size_t q_elems;        /* Q buffer (with padding)                           */
  size_t payload_elems;  /* floats sent per step: sum r(m+n) + pass-through   */
  size_t dense_elems;    /* sum m*n over compressed tensors                   */
  size_t workspace_bytes;/* device workspace compress/decompress/refresh need */
} psgd_plan_info_t;

/*
 * psgd_plan_create -- describe a model's gradient set.  Host only: touches no
 * device and can run on a machine without a GPU.
 *
 *   ntensors   number of tensors (>= 0)
 *   rows,cols  per tensor, the row-major matrix view: rows = dim0,
 *              cols = product of the remaining dims (cols <= 1 for vectors,
 *              then `rows` is the length).  Every size must be >= 1.
 *   offsets    nullable.  Element offset of each tensor in the flat buffers.
 *              NULL: the plan packs the tensors in order, each start aligned
 *              to 64 elements.  Caller offsets must be >= 0 and ranges must
 *              not overlap; any alignment is accepted (unaligned rows use
 *              narrower loads).
 *   rank       r, 1 <= r <= PSGD_MAX_RANK.
 *   flags      PSGD_FLAG_MOMENTUM and / or PSGD_FLAG_GRADS_BF16, or 0.
 *   beta       momentum coefficient (used only with PSGD_FLAG_MOMENTUM).
 *   out        receives the plan; release it with psgd_plan_destroy.
 *
 * Classification ([N152] Method; the size rule is this library's reading of
 * "small tensors"): a matrix is compressed iff r*(rows+cols) < rows*cols.
 *
 * Errors: PSGD_ERR_INVALID_ARG for a NULL list or out, a size < 1 (or a
 * vector's), a size above INT32_MAX, bad offsets or a NaN beta;
 * PSGD_ERR_UNSUPPORTED for a rank above PSGD_MAX_RANK, unknown flags, or a
 * compressed matrix with 2^30 columns or more (rows are addressed with
 * 32-bit byte offsets).
 */
psgd_status_t psgd_plan_create(int32_t ntensors, const int64_t* rows, const int64_t* cols,
                               const int64_t* offsets, int32_t rank, uint32_t flags, float beta,
                               psgd_plan_t* out);

/* Releases the plan.  Only after every call that used it has completed on the
 * device (the plan owns the host copy of the tables psgd_workspace_init
 * uploads, and the timing events). */
void psgd_plan_destroy(psgd_plan_t plan);

/* Sizes of the plan's buffers; host only.  payload_elems is what one step
 * transmits: r (m + n) floats per compressed m x n matrix, the factors P_hat
 * and Q of [GLOSS] factorisation paragraph ([N152] Method: those two are
 * what the workers exchange), plus every pass-through tensor whole. */
psgd_status_t psgd_plan_get_info(psgd_plan_t plan, psgd_plan_info_t* info);

/* Where tensor `tensor` lives: kind (PSGD_KIND_*: [N152] Method sends
 * vectors and matrices that rank r would not shrink uncompressed), flat element offset,
 * P offset (P_hat start for compressed tensors; start of its values in the
 * pass-through region for others) and Q offset (-1 if not compressed).  Host
 * only.  Any output pointer may be NULL. */
psgd_status_t psgd_plan_tensor(psgd_plan_t plan, int32_t tensor, int32_t* kind, int64_t* flat_off,
                               int64_t* p_off, int64_t* q_off);

/*
 * psgd_workspace_init -- write the plan's device tables (tensor descriptors,
 * tile lists) into the first part of `workspace`, a caller-owned device buffer
 * of at least info.workspace_bytes, 256-byte aligned.  Must be called once per
 * (plan, workspace) pair before any compress / decompress / refresh that uses
 * the pair; the caller must not write to the workspace afterwards.  The rest
 * of the workspace is scratch that every call overwrites.  Asynchronous on
 * `stream`.
 */
psgd_status_t psgd_workspace_init(psgd_plan_t plan, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/*
 * Aggregation hook: called on the host, in stream order, with a device buffer
 * of `count` floats that every worker must replace by its mean over workers
 * (all-reduce-mean).  It must enqueue its work on `stream` (or make the stream
 * wait for it) and return 0, or return non-zero to abort the call.  Because
 * the compressor is linear ([N152] Concepts, "Linearity of compressor"),
 * averaging P and then Q equals compressing the averaged gradient.  A NULL
 * hook is the single-worker identity.
 */
typedef int (*psgd_reduce_fn)(float* buf, size_t count, hipStream_t stream, void* user);

/*
 * psgd_compress -- one PowerSGD step over the whole set ([N152] Method; error
 * feedback per [GLOSS] and [N152] Concepts, "Error feedback").
 *
 *   grads  flat, read-only: the stochastic gradients G, fp32 (or bfloat16
 *          with PSGD_FLAG_GRADS_BF16, widened exactly to fp32 on load).
 *   err    flat, in/out: error memory E of compressed tensors (zero at the
 *          first step).  On return: the new residual M - P_hat Q^T.  While the
 *          call runs it holds M = X + E_old; if the call fails after the first
 *          pass (a hook error or a launch failure) it is left holding M.
 *          With the deferred-residual flags it holds M on entry and / or on
 *          return instead (see PSGD_STEP_DEFER_RESIDUAL).
 *   mom    flat, in/out momentum u (all tensors), required iff the plan has
 *          PSGD_FLAG_MOMENTUM (then X = u <- beta*u + G; else X = G), else NULL.
 *   q      packed Q buffer: on entry the warm start (the previous step's Q, or a
 *          random start at the first step); on return the new Q, which is also
 *          the next step's warm start ([N152] Concepts, "Warm-start subspace
 *          iteration").
 *   p      packed P buffer (info.p_buffer_elems): receives P_hat followed by
 *          the pass-through values.
 *   mhat   nullable flat buffer: if given, receives the decompressed gradient
 *          P_hat Q^T for compressed tensors and the aggregated values of the
 *          pass-through tensors (a fused psgd_decompress).  It may alias
 *          fp32 `grads` (then G is overwritten by the update) but no other
 *          buffer.
 *   opts   nullable step options (psgd_step_opts_t): power iterations,
 *          PowerSGD+ refresh, the no-error-feedback ablation, fused
 *          post-compression momentum SGD.
 *   hook   nullable aggregation hook, called on (p, p_buffer_elems) after P is
 *          formed and on (q, q_elems) after Q is formed.  With power_iters
 *          > 1 the later iterations call it on (p, p_elems): the pass-through
 *          values are aggregated once, with the first P.
 *   workspace, workspace_bytes   initialised workspace (psgd_workspace_init).
 *
 * Errors: PSGD_ERR_INVALID_ARG for null or not 16-byte aligned buffers, a
 * missing or unexpected `mom`, negative iteration counts, `params` without
 * `sgd_buf` (or misaligned), unknown step flags, deferred-residual flags
 * without error feedback; PSGD_ERR_WORKSPACE;
 * PSGD_ERR_HOOK if a hook
 * returns non-zero (no later stage is enqueued); PSGD_ERR_HIP.
 */
psgd_status_t psgd_compress(psgd_plan_t plan, const void* grads, float* err, float* mom, float* q,
                            float* p, float* mhat, const psgd_step_opts_t* opts, psgd_reduce_fn hook,
                            void* user, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * psgd_compress_noalloc -- psgd_compress without a workspace, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Same step, same kernels,
 * same arguments and results as psgd_compress, but the scratch lives in a
 * static device array of the library, PSGD_NOALLOC_SCRATCH_BYTES per GPU,
 * which every GPU the library runs on holds until the process ends.  The
 * call allocates and frees nothing: the first call on a device looks up that
 * device's copy of the array; the plan's tables are uploaded into it (an
 * asynchronous host-to-device copy on `stream`) when the previous call on the
 * device used another plan or another stream.  The caller still owns grads,
 * err, mom, q, p and mhat.
 *
 * Every call on one GPU shares that GPU's array and finds the previous
 * call's contents there: calls that overlap on one GPU (concurrent streams
 * or threads) race, and so do calls on two streams that the caller has not
 * ordered.  Use psgd_compress with distinct workspaces for concurrent steps.
 *
 * Errors: as psgd_compress; PSGD_ERR_WORKSPACE when the plan needs more than
 * PSGD_NOALLOC_SCRATCH_BYTES of scratch (info.workspace_bytes; checked
 * before any device call); PSGD_ERR_HIP if the device's copy cannot be found.
 */
#define PSGD_NOALLOC_SCRATCH_BYTES (64ll << 20)
psgd_status_t psgd_compress_noalloc(psgd_plan_t plan, const void* grads, float* err, float* mom, float* q, float* p,
                                    float* mhat, const psgd_step_opts_t* opts, psgd_reduce_fn hook, void* user,
                                    hipStream_t stream);

/*
 * psgd_decompress -- reconstruct G ~ P_hat Q^T ([GLOSS], factorisation
 * paragraph) for every compressed tensor and copy the pass-through values
 * from the P buffer, into the flat buffer `out` (may alias the gradients).
 */
psgd_status_t psgd_decompress(psgd_plan_t plan, const float* p, const float* q, float* out,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * psgd_refresh -- PowerSGD+ subspace re-alignment ([PSGD+] Abstract), read as
 * `iters` rounds of block power iteration with orthonormalisation,
 * Q <- GS(M^T GS(M Q)), on compressed tensor `tensor` of the flat buffer `m`
 * (the compressor input), updating that tensor's columns of the packed Q
 * buffer in place.  On return its Q has orthonormal columns (dependent
 * columns are zero).  Uses the workspace scratch: not concurrent with a
 * compress call on the same workspace.  Errors: PSGD_ERR_INVALID_ARG for a
 * tensor that is not compressed, null or misaligned buffers, iters < 0.
 */
psgd_status_t psgd_refresh(psgd_plan_t plan, int32_t tensor, const float* m, float* q, int32_t iters,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * psgd_init_q -- seeded start for the warm-start factors: every compressed
 * tensor's columns of the packed Q buffer get i.i.d. N(0, 1) values.  The
 * pages warm-start each step from the previous Q ([GLOSS], temporal-coherence
 * paragraph; [N152] Method) and leave the first Q open; calling this before
 * every step gives the cold-start ablation.  Element c*n + j (row j, column c)
 * of tensor t's n x rank Q is normal number c*n + j of the stream keyed
 * (seed, t): Philox-4x64-10 block (c*n + j)/4 at counter ((c*n + j)/4, 0, 0, 0)
 * and key (seed, t) (Salmon et al., "Parallel random numbers: as easy as
 * 1, 2, 3", SC'11), words 0,1 and 2,3 turned into two normals each by the
 * Box-Muller transform in fp64 (u1 = 1 - (w0 >> 11) 2^-53, u2 = (w1 >> 11)
 * 2^-53), rounded to fp32.  The values depend only on (seed, t, c, j): every
 * worker with the same seed starts from the same Q, and a column is the
 * same at every rank.  Other parts of q are not written.  Errors:
 * PSGD_ERR_INVALID_ARG (null or misaligned q), PSGD_ERR_WORKSPACE.
 */
psgd_status_t psgd_init_q(psgd_plan_t plan, float* q, uint64_t seed, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * Diagnostics (outside the step; each reads the buffers it is given and
 * writes fp64 results in the order of the plan's compressed tensors, like
 * zero_cols; sums in a fixed order, so repeated calls agree bit for bit).
 *
 * psgd_step_stats -- after a compress with the fused decompression:
 * out[2k] = ||E_k||_F^2 and out[2k + 1] = ||M_hat_k + E_k||_F^2 = ||M_k||_F^2
 * (to the rounding of the residual) for compressed matrix k, so that
 * sqrt(out[2k] / out[2k + 1]) is the share of the compressor's input that
 * error feedback carries to later steps ([GLOSS] error-feedback paragraph:
 * e_t = G_t - compress(G_t)).  err and mhat: the flat buffers of that call
 * (with a deferred residual err holds M, not E: call it on an explicit-
 * residual step).  out: 2 * ncompressed doubles, device or pinned host
 * memory, 8-byte aligned.  Reads both buffers once.  Asynchronous on
 * `stream`; PSGD_ERR_INVALID_ARG on NULL or misaligned pointers.
 *
 * psgd_subspace_overlap -- out[k] = mean cosine of the principal angles
 * between the spans of compressed matrix k's factors in two Q buffers, e.g.
 * a copy of Q taken before a step and Q after it ([GLOSS] temporal-coherence
 * paragraph: consecutive steps' subspaces overlap with cosine similarity
 * often above 0.9).  Both factors are copied into `scratch` (caller-owned
 * device memory of 2 * q_elems floats, not overlapping q_a or q_b) and
 * orthonormalised there as the refresh orthonormalises Q (Gram-Schmidt with
 * the dependence rule: a dependent column becomes zero); the cosines are the
 * singular values of A_hat^T B_hat (cyclic Jacobi on its Gram matrix, fp64)
 * and the mean is over the r columns, a zero column counting as 0.  q_a and
 * q_b are not modified.  out: ncompressed doubles, device or pinned host
 * memory, 8-byte aligned.  Copies with hipMemcpyAsync (not for graph
 * capture).  Asynchronous on `stream`; PSGD_ERR_INVALID_ARG on NULL,
 * misaligned or overlapping pointers.
 */
psgd_status_t psgd_step_stats(psgd_plan_t plan, const float* err, const float* mhat, double* out, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);
psgd_status_t psgd_subspace_overlap(psgd_plan_t plan, const float* q_a, const float* q_b, float* scratch,
                                    double* out, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Per-stage timing with HIP events recorded on the call's stream.  While
 * enabled, every compress / decompress / refresh call records one event pair
 * per stage it runs (psgd_refresh records its products under EF_P, MTP and
 * QREDUCE and its orthonormalisations under GS).  psgd_timing_read waits for
 * the recorded events, adds the elapsed milliseconds per stage into
 * ms[PSGD_NSTAGES] (and the number of launches per stage into launches[],
 * nullable), clears the record and keeps its events for reuse.  Enabling
 * creates PSGD_TIMING_EVENTS events up front (once per plan), so that the
 * calls being timed do not create events themselves until that many are
 * pending unread; beyond it, events are created as needed.  Errors:
 * PSGD_ERR_INVALID_ARG (null plan), PSGD_ERR_HIP (event creation failed at
 * enable; timing then stays off).
 */
#define PSGD_TIMING_EVENTS 4096
psgd_status_t psgd_timing_enable(psgd_plan_t plan, int32_t enable);
/* Restricts the event pairs that enabled timing records to the stages whose
 * bit (1u << PSGD_STAGE_*) is set in mask; a new plan records every stage
 * (mask ~0u).  Fewer events per call keep host work out of launch-bound
 * calls that are being timed.  Takes effect from the next call; records
 * already taken are kept.  Errors: PSGD_ERR_INVALID_ARG (null plan). */
psgd_status_t psgd_timing_stages(psgd_plan_t plan, uint32_t mask);
psgd_status_t psgd_timing_read(psgd_plan_t plan, double* ms, int64_t* launches);

/* A plain device copy dst[i] = src[i], i < n, with 16-byte accesses (n a
 * multiple of 4, both pointers 16-byte aligned): the bandwidth ceiling and
 * the byte-counter calibration kernel. */
psgd_status_t psgd_stream_copy(float* dst, const float* src, size_t n, hipStream_t stream);

/* Streaming-bandwidth probe: the byte pattern of one pass of the step
 * without its arithmetic, to measure the practical bandwidth of that pattern
 * on the device.  Reads nin arrays in[0..nin) and writes nout arrays
 * out[0..nout) of n floats each, out_j[i] = in_0[i] + ... + in_{nin-1}[i]
 * (0 with no input); 0 <= nin <= 3, 0 <= nout <= 2, nin + nout >= 1, n a
 * multiple of 4, every array 16-byte aligned device memory.  With nout = 0
 * the sums are added atomically into sink, device memory of
 * PSGD_PROBE_SINK_FLOATS floats (several workgroups share a float; if the
 * sink was zeroed first, its total is the sum of all inputs), so that only
 * the reads reach memory.  `in` and `out` are host arrays of device pointers; an
 * output may be one of the inputs (the in-place form, each element read
 * before it is written by the same thread).  The pattern of each pass:
 * EF-add + P 2 in / 1 out (3 / 2 with momentum), M^T P_hat 1 / 0, residual
 * 1 / 1 (1 / 2 with M_hat), decompression 0 / 1; the passes write M over E,
 * u over u and E over M.
 * Asynchronous on `stream`; PSGD_ERR_INVALID_ARG on bad counts or pointers. */
#define PSGD_PROBE_SINK_FLOATS 16384
psgd_status_t psgd_stream_probe(const float* const* in, int32_t nin, float* const* out, int32_t nout, size_t n,
                                float* sink, hipStream_t stream);

/* Thread-local message describing the last failure on this thread. */
const char* psgd_last_error(void);

/* Library version string. */
const char* psgd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PSGD_H_ */
