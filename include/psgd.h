/*
 * psgd.h -- C ABI of libpsgd: PowerSGD rank-r gradient compression with error
 * feedback, as hand-written HIP kernels for AMD Instinct MI355X (gfx950).
 *
 * What one step computes (the review page "PowerSGD: Practical Low-Rank Gradient
 * Compression for Distributed Optimization", section "Proposed method"):
 *   every layer gradient is reshaped to an n x m matrix and compressed on its own;
 *   with W data-parallel workers and a warm-start factor Q (m x r) kept from the
 *   previous step:
 *     M_w  = G_w + E_w                          error feedback
 *     P    = mean_w M_w Q                       one power-iteration half step, all-reduced
 *     P    = orthonormalise(P)                  Gram-Schmidt, column order (taken in
 *                                               P's r x r Gram space in fp64: the
 *                                               modified Gram-Schmidt factor)
 *     Q    = mean_w M_w^T P                     second half step, all-reduced
 *     U    = P Q^T                              decompressed update
 *     E_w  = M_w - U                            error kept for the next step
 *   The all-reduce is linear (the page's reason it works), and the W workers live as
 *   W slices of one HBM buffer, so the all-reduce is a mean across those slices taken
 *   inside the kernels.  Tensors that are not compressed (1-D, or a matrix whose
 *   smaller side is at most r) get the plain worker mean and keep no error.
 *   psgd_ef_momentum_apply adds the momentum-SGD update the page applies to the
 *   decompressed update.
 *
 * Readings of points the page leaves open:
 *   - all-reduce means the mean over workers;
 *   - Q is shared by all workers and the next step's Q is this step's aggregated Q
 *     (not re-normalised);
 *   - the orthonormalisation drops (sets to zero) a column whose residual norm is at
 *     most 1e-4 times its norm before orthogonalisation, or is zero;
 *   - the error uses the aggregated Q (one decompressed U per matrix), or, with
 *     PSGD_FLAG_LOCAL_Q_ERROR, each worker's own Q_w;
 *   - momentum is heavy-ball, mom <- mu*mom + U, x <- x - lr*mom (Nesterov by flag);
 *   - non-finite inputs are not checked: they propagate into every output that depends
 *     on them, and a P column whose norm is not a number is dropped (set to zero).
 *
 * Memory layout.  A plan fixes a packed layout for a list of tensors:
 *   - every tensor starts at an element offset that is a multiple of 64 (256 bytes)
 *     and is stored row-major (rows x cols); psgd_plan_layer_info returns the offset;
 *   - grads and errors are [n_workers][worker_stride] (worker w's slice starts at
 *     w * worker_stride elements); update, momentum and params are [worker_stride];
 *   - p is the concatenation, in layer order, of every compressed matrix's P
 *     (rows x rank, row-major); q likewise of every Q (cols x rank, row-major); each
 *     block starts at a multiple of 4 floats (16 bytes), and psgd_plan_layer_info
 *     returns each matrix's p_offset / q_offset;
 *   - padding elements between tensors are never read for results and never written.
 *
 * Ownership.  The caller owns every buffer passed to a step, including the workspace
 * (size from psgd_plan_sizes); the library never frees caller memory.  The plan owns
 * its host tables and a small device copy of them, uploaded on the first step on a
 * device and freed by psgd_plan_destroy.
 *
 * Pointers.  Buffers passed to a step are device pointers (hipMalloc or any allocator
 * on the device the stream belongs to), 16-byte aligned.  `stream` is a hipStream_t
 * (NULL = the default stream).  errors, q (and momentum/params) are updated in place;
 * no other two buffers may overlap.
 *
 * Errors.  Argument problems are found before anything is enqueued: the call returns a
 * non-zero status and the buffers are untouched.  A failed launch returns
 * PSGD_ERR_HIP.  Steps are asynchronous: a fault inside a kernel surfaces at the
 * caller's next synchronisation of the stream.  psgd_last_error() gives a text for the
 * last failure on the calling thread.  No C++ exception crosses this interface.
 *
 * Concurrency.  A plan may be used by one stream at a time.
 */
#ifndef PSGD_H_
#define PSGD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct psgd_plan psgd_plan;

typedef enum psgd_status {
  PSGD_OK = 0,
  PSGD_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad shape, count or value */
  PSGD_ERR_UNSUPPORTED = 2, /* rank outside 1..4, unknown dtype or flag */
  PSGD_ERR_NO_MEMORY = 3,   /* host or device allocation of the plan's tables failed */
  PSGD_ERR_HIP = 4          /* a HIP call or kernel launch failed; see psgd_last_error */
} psgd_status;

typedef enum psgd_dtype {
  PSGD_F32 = 0, /* float32 gradients */
  PSGD_BF16 = 1 /* bfloat16 gradients, widened exactly to float32 on load; P, Q, E stay float32 */
} psgd_dtype;

/* Plan flags. */
#define PSGD_FLAG_NESTEROV 0x1u /* psgd_ef_momentum_apply uses x <- x - lr*(U + mu*mom) */
/* Carry the workers' mean error from one step to the next.  The first pass of a step
 * needs mean_w (G_w + E_w) = mean_w G_w + mean_w E_w; the final pass of the previous
 * step already held every E_w it stored, so it also writes their mean into the
 * workspace, and the next step's first pass then reads only the gradients (4W + 8
 * instead of 8W + 4 bytes per element).  The results are the same up to float
 * rounding order.  Contract: between consecutive steps of the plan the caller passes
 * the same `errors` and `workspace` pointers and modifies neither.  A step falls back to
 * reading all errors when it is the plan's first, follows psgd_plan_reset_carry, or
 * sees other errors/workspace pointers or another device than the previous step; a
 * failed step also forces the fallback.  The workspace grows by worker_stride floats
 * and a 256-byte state block (see "Cross-step state and graphs" below). */
#define PSGD_FLAG_CARRY_ERROR_MEAN 0x2u
/* Deferred error subtraction.  The step reads every worker's G and E once: the error
 * buffer keeps M_w = G_w + E_w of the step that wrote it (the error before subtracting
 * that step's decompressed update U), and the next step subtracts U while it adds the
 * new gradient.  A step then moves 12W + 4 bytes per element in its worker pass instead
 * of two passes over G.  The update, P and Q outputs are unchanged; only the error
 * buffer's representation differs: after a step, errors_w - P Q^T (P and Q of that step,
 * kept in the workspace) is the plain error memory E'_w, and psgd_errors_materialize
 * writes it out.  Contract and fallback as for PSGD_FLAG_CARRY_ERROR_MEAN: the same
 * errors and workspace pointers, unmodified, between steps (psgd_plan_reset_carry
 * declares that `errors` now holds plain errors).  Excludes
 * PSGD_FLAG_CARRY_ERROR_MEAN.  The workspace grows by p_elems + q_elems floats and the
 * 256-byte state block.
 *
 * Cross-step state and graphs.  Whether a step of a carry or deferred plan uses the
 * state the previous step left is decided twice: on the host (the plan's previous step
 * ran on this device with the same errors and workspace pointers and nothing reset it
 * since) and on the device, from a state word in the workspace.  The last pass of a
 * step writes the word (a key of the plan and the errors address); in-place
 * psgd_errors_materialize and psgd_plan_reset_carry_stream clear it on the stream.  A
 * step captured into a HIP graph therefore keeps working when the buffers change
 * between replays, as long as the change goes through those stream-ordered calls:
 *   - capture a step of such a plan only after one eager step on the same errors and
 *     workspace (a capture without usable state is refused with PSGD_ERR_INVALID_ARG;
 *     so is a capture of psgd_errors_materialize on a deferred plan in that case);
 *   - after writing errors or the workspace yourself, call psgd_plan_reset_carry_stream
 *     on the stream before the next replay (psgd_plan_reset_carry is host-only and
 *     reaches eager steps, not replays). */
#define PSGD_FLAG_DEFERRED_ERROR 0x4u
/* Local-Q error: each worker keeps E'_w = M_w - P Q_w^T with its own Q_w = M_w^T P
 * (the projection of M_w off span(P)) instead of M_w - P Qbar^T.  P, Qbar (the output q
 * and next warm start) and the update U = P Qbar^T are unchanged, and so is the workers'
 * mean error.  This is the form that lets a multi-GPU step finish its error locally
 * before the Q all-reduce.  One GPU pays an extra pass over every worker's G and E to form
 * the Q_w.  Excludes PSGD_FLAG_CARRY_ERROR_MEAN and PSGD_FLAG_DEFERRED_ERROR.  The
 * workspace grows by n_workers * (q_elems + Q-partial) floats. */
#define PSGD_FLAG_LOCAL_Q_ERROR 0x8u

/* One tensor of the layer list.  rows == 1 or cols == 1 marks a 1-D tensor. */
typedef struct psgd_layer {
  int64_t rows;
  int64_t cols;
} psgd_layer;

typedef struct psgd_layer_info {
  int32_t compressed;   /* 1: compressed matrix, 0: averaged, uncompressed */
  int32_t matrix_index; /* index among the compressed matrices, -1 otherwise */
  int64_t rows, cols;
  int64_t offset;   /* element offset inside a worker slice / update / momentum / params */
  int64_t p_offset; /* element offset of this matrix's P in p (-1 if uncompressed) */
  int64_t q_offset; /* element offset of this matrix's Q in q (-1 if uncompressed) */
} psgd_layer_info;

typedef struct psgd_sizes {
  int32_t n_layers, n_matrices, n_vectors;
  int32_t rank, n_workers, grad_dtype;
  int64_t worker_stride; /* elements per worker slice; also the length of update/momentum/params */
  int64_t numel;         /* sum of rows*cols over all tensors */
  int64_t matrix_numel;  /* sum of rows*cols over compressed matrices */
  int64_t vector_numel;  /* sum of rows*cols over uncompressed tensors */
  int64_t p_elems;       /* length of p: rows*rank per compressed matrix, each rounded up to 4 */
  int64_t q_elems;       /* length of q: cols*rank per compressed matrix, each rounded up to 4 */
  uint64_t workspace_bytes; /* device scratch a step needs (caller-allocated, 256-byte aligned) */
  /* fp32 bytes one worker would send per step in a real data-parallel job:
     P and Q of every compressed matrix plus every uncompressed tensor */
  uint64_t message_bytes;
  /* minimal HBM bytes of one step: per compressed element read G_w, E_w and write
     E'_w on every worker plus write U once; per uncompressed element read G_w on every
     worker and write the mean once (gradient bytes are 2 per element for bf16) */
  uint64_t model_bytes;
  /* the same for psgd_ef_momentum_apply without the update output: U is not written;
     momentum and params are read and written once per element of every tensor */
  uint64_t model_bytes_momentum;
} psgd_sizes;

/* Create a plan for `n_layers` tensors (in the order they are packed), compression
 * rank 1..4, `n_workers` >= 1 simulated workers and the gradient dtype.  Host only: no
 * HIP call is made.  Returns PSGD_ERR_INVALID_ARG for a null pointer, n_layers < 1,
 * n_workers < 1 or > 65536, a non-positive dimension or a tensor with 2^31 or more
 * elements; PSGD_ERR_UNSUPPORTED for a rank outside 1..4, an unknown dtype or flag. */
psgd_status psgd_plan_create(const psgd_layer* layers, int32_t n_layers, int32_t rank,
                             int32_t n_workers, psgd_dtype grad_dtype, uint32_t flags,
                             psgd_plan** out);

/* Sizes and byte accounting of a plan (host only). */
psgd_status psgd_plan_sizes(const psgd_plan* plan, psgd_sizes* out);

/* Placement of tensor `layer` (0-based, in the order given at creation; host only). */
psgd_status psgd_plan_layer_info(const psgd_plan* plan, int32_t layer, psgd_layer_info* out);

/* Free the plan and its device tables.  NULL is accepted.  The caller must make sure
 * no step using the plan is still running. */
psgd_status psgd_plan_destroy(psgd_plan* plan);

/* One compression step with error feedback over every tensor of the plan.
 *   grads     [n_workers][worker_stride], grad dtype, read only
 *   errors    [n_workers][worker_stride] float32; in: E, out: E' = M - U.  Only the
 *             compressed matrices' elements are read or written.
 *   q         q_elems float32; in: warm-start Q, out: the aggregated Q (next warm start)
 *   p         p_elems float32; out: orthonormalised P
 *   update    worker_stride float32; out: U = P Q^T for compressed matrices and the
 *             worker mean for the other tensors; may be NULL (not written)
 *   workspace workspace_bytes of device memory, contents need not be preserved
 * Enqueues the kernels on `stream` and returns; nothing is enqueued on error. */
psgd_status psgd_compress_step(psgd_plan* plan, const void* grads, float* errors, float* q,
                               float* p, float* update, void* workspace, void* stream);

/* The step above followed by momentum SGD on the decompressed update, fused into the
 * same final pass (EF-SGD with momentum):
 *   mom <- mu*mom + U;  x <- x - lr*mom        (Nesterov flag: x <- x - lr*(U + mu*mom))
 * for every tensor of the plan.  momentum and params are [worker_stride] float32, in
 * place.  `update` may be NULL, in which case U is not written at all.  lr and mu must be
 * finite. */
psgd_status psgd_ef_momentum_apply(psgd_plan* plan, const void* grads, float* errors, float* q,
                                   float* p, float* momentum, float* params, float lr, float mu,
                                   float* update, void* workspace, void* stream);

/* Power-iteration steps per compression step (default 1, the page's method: one
 * warm-started step per gradient).  With k > 1, after the first P, orthonormalise, Q
 * round the step repeats P = mean_w M_w Q, orthonormalise, Q = mean_w M_w^T P another
 * k - 1 times from the Q just computed, before decompressing; the worker mean of M is
 * kept in the workspace, so each extra round reads only that mean twice.  This is the
 * warm-start ablation the page's research question RQ3 and its warm-start finding
 * ("Main findings") speak of: more iterations (or a fresh Q each step, passed in `q`)
 * against one warm-started step.  Returns PSGD_ERR_INVALID_ARG outside 1..16.  Applies
 * to later steps; host only. */
psgd_status psgd_plan_set_power_iterations(psgd_plan* plan, int32_t iterations);

/* Kernel timing, for benchmarks and profiling (off by default).  While enabled, every
 * kernel a step launches is bracketed by two HIP events recorded on the launch stream;
 * psgd_plan_kernel_stats waits for the recorded events and accumulates their elapsed
 * times per kernel.  Timing adds two event records per launch.  Kernel names:
 * "k_first", "k_mgs", "k_q_partial", "k_q_reduce", "k_apply" (eager modes) or "k_update"
 * (deferred mode), "k_p_mbar" for extra power iterations, and "k_qw_partial" /
 * "k_qw_reduce" for PSGD_FLAG_LOCAL_Q_ERROR. */
typedef struct psgd_kernel_stat {
  char name[32];    /* kernel name */
  int64_t launches; /* launches timed since the last reset */
  double total_ms;  /* sum of their durations in milliseconds */
} psgd_kernel_stat;

/* Enable (non-zero) or disable timing for later steps of this plan. */
psgd_status psgd_plan_set_timing(psgd_plan* plan, int32_t enable);

/* Write up to `capacity` per-kernel statistics to `out` and their number to `count`
 * (both may be NULL/0 to only flush).  Blocks until every timed launch so far has
 * finished.  `reset` non-zero clears the statistics afterwards.  PSGD_ERR_HIP if an
 * event could not be read. */
psgd_status psgd_plan_kernel_stats(psgd_plan* plan, psgd_kernel_stat* out, int32_t capacity,
                                   int32_t* count, int32_t reset);

/* Forget the plan's cross-step state: the next step of a PSGD_FLAG_CARRY_ERROR_MEAN
 * plan reads all errors again, and the next step of a PSGD_FLAG_DEFERRED_ERROR plan
 * treats `errors` as plain errors.  Call it after writing `errors` or the workspace
 * yourself, e.g. when restoring a checkpoint. */
psgd_status psgd_plan_reset_carry(psgd_plan* plan);

/* The stream-ordered form of psgd_plan_reset_carry: clears the state word in
 * `workspace` (a device pointer, the plan's workspace) with a one-thread kernel on
 * `stream`, so that every later step on that workspace, eager or replayed from a graph,
 * treats `errors` as plain errors, and also does what psgd_plan_reset_carry does.  It
 * may itself be captured into a graph.  Plans without PSGD_FLAG_CARRY_ERROR_MEAN or
 * PSGD_FLAG_DEFERRED_ERROR (or without compressed matrices) enqueue nothing.
 * PSGD_ERR_INVALID_ARG for a NULL plan or a NULL or misaligned workspace. */
psgd_status psgd_plan_reset_carry_stream(psgd_plan* plan, void* workspace, void* stream);

/* Write the plain error memory of every compressed matrix to `out` ([n_workers]
 * [worker_stride] float32): for a PSGD_FLAG_DEFERRED_ERROR plan whose last step left
 * `errors` and `workspace` in the deferred form, out_w = errors_w - P Q^T of that step;
 * otherwise out_w = errors_w.  `out` may be `errors` (in place; the plan then treats the
 * buffer as plain, and clears the workspace's state word on the stream) or a separate
 * buffer (the plan's state is kept).  Elements of 1-D tensors and padding are not
 * written.  Asynchronous on `stream`. */
psgd_status psgd_errors_materialize(psgd_plan* plan, const float* errors, float* out, void* workspace,
                                    void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): psgd_compress_step without a workspace
 * argument and without any device allocation.  The same kernels run with the workspace
 * and the plan's device tables in a static array of the library, 64 MiB per GPU, which
 * each GPU the library runs on holds until the process ends; the first call on a GPU
 * looks up that GPU's copy of the array.  The plan's tables are copied into the array
 * (hipMemcpyAsync on `stream`) whenever the previous call on that GPU used another plan.
 * Arguments as for psgd_compress_step.  Returns PSGD_ERR_INVALID_ARG, enqueueing
 * nothing, when the plan needs more than the array holds (its workspace_bytes plus its
 * tables; ResNet-18 shapes at 16 workers and rank 2 need 46.5 MB), and PSGD_ERR_UNSUPPORTED for a
 * plan with PSGD_FLAG_CARRY_ERROR_MEAN or PSGD_FLAG_DEFERRED_ERROR (their cross-step state
 * would live in the shared array).  Every call on a GPU shares that GPU's array: calls
 * that overlap on one GPU (other streams, other threads) race and give undefined
 * results; serialise them.  No step of the plain plans needs the array cleared. */
psgd_status psgd_compress_step_noalloc(psgd_plan* plan, const void* grads, float* errors, float* q,
                                       float* p, float* update, void* stream);

/* Calibration probe: copy `bytes` (a multiple of 16) from `src` to `dst` on `stream`
 * with the same non-temporal float4 accesses the streaming passes use.  It measures the
 * copy bandwidth the device reaches, and gives hardware counters a transfer of known
 * size to be scaled against.  Device pointers, 16-byte aligned, not overlapping. */
psgd_status psgd_stream_copy(const void* src, void* dst, uint64_t bytes, void* stream);

/* Static text for a status code. */
const char* psgd_status_string(psgd_status status);

/* Text describing the last failure on the calling thread ("" if none). */
const char* psgd_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PSGD_H_ */
