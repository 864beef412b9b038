/*
 * psgd_rtopk.h -- rTop-k gradient sparsification with error feedback in libpsgd, as
 * hand-written HIP kernels for AMD Instinct MI355X (gfx950).  Status codes, dtypes,
 * the layer list and the kernel-timing record are those of psgd.h.
 *
 * What one step computes (the review page "rTop-k: A Statistical Estimation Approach
 * to Distributed SGD", section "Proposed method" and the abstract: among the entries of
 * largest magnitude, a random subset is sent -- top-k and random-k applied one after
 * the other -- and the operator is used as a compressor under error feedback):
 *   every tensor is flattened (row-major) and compressed on its own, with a top count r
 *   and a sent count k (1 <= k <= r <= numel); for each of W data-parallel workers:
 *     M_w    = G_w + E_w                       error feedback, float32
 *     T_w    = the r entries of M_w of largest magnitude
 *     S_w    = the entries of T_w whose rank is below k
 *     sent   = (index, value) of S_w           value = M_w at index, not rescaled
 *     E_w   <- M_w with the entries of S_w set to zero
 *   and U = mean_w of the sent entries scattered into a dense tensor (the all-reduce
 *   of the sparse messages; the W workers are W slices of one HBM buffer).
 *
 * Readings of points the page leaves open:
 *   - magnitude order is the order of the bit pattern of |m| as an unsigned integer (so
 *     NaN sorts above infinity); equal magnitudes are ordered by position, lower first;
 *   - the random subset is uniform; its randomness is the caller's input `ranks`: for
 *     each worker and tensor, a permutation of 0..r-1 given to the entries of T_w in
 *     ascending index order.  Entries with rank < k form S_w.  If a row of ranks is not
 *     a permutation, S_w is still the set of entries with rank < k, cut to its first k
 *     in index order, and unused output slots hold index -1 and value 0;
 *   - a tensor's sent entries are listed in ascending index order;
 *   - the update is computed in float32, adding the workers in order 0..W-1, then
 *     multiplying by 1/W.
 *
 * Memory layout.  The packed layout of psgd.h: every tensor starts at an element offset
 * that is a multiple of 64 (psgd_rtopk_plan_layer_info gives it); grads and errors are
 * [n_workers][worker_stride]; update is [worker_stride].  ranks are uint32
 * [n_workers][top_total] (tensor l at top_offset(l)); index (int32, element index inside
 * the tensor) and value (float32) are [n_workers][keep_total] (tensor l at
 * keep_offset(l)).  Padding elements are never written.
 *
 * Ownership, pointers, errors and concurrency as in psgd.h: caller-owned device
 * buffers (16-byte aligned), argument errors reported before anything is enqueued,
 * asynchronous execution on `stream`, one stream at a time per plan.  errors is updated
 * in place; no other two buffers may overlap.
 */
#ifndef PSGD_RTOPK_H_
#define PSGD_RTOPK_H_

#include "psgd.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct psgd_rtopk_plan psgd_rtopk_plan;

/* Plan flag: deferred zeroing of the sent entries.  A step then leaves the error buffer
 * holding M_w at the entries it sent (everything else is E'_w as usual), and keeps that
 * step's sent mask in the workspace; the next step's first pass reads E with those
 * entries as zero (one mask bit per element, read with E) instead of this step writing
 * them one by one.  Only the error buffer's representation differs: the lists, the
 * update and the next step's results are the same.  psgd_rtopk_errors_materialize
 * writes the plain E'.  Contract: between consecutive steps the caller passes the same
 * errors and workspace pointers and modifies neither (the workspace is then not
 * scratch).  A step applies the pending zeros only when the plan's previous step ran on
 * this device with these errors and workspace pointers and nothing reset it since (the
 * host's view), and the workspace's state word holds the plan's key for these errors
 * (the device's view: written by the step, cleared by in-place materialisation and by
 * psgd_rtopk_plan_reset_state on the stream).  So a step captured into a HIP graph keeps
 * working when the buffers change between replays through those calls; a capture
 * without usable state (no eager step yet on these buffers) is refused with
 * PSGD_ERR_INVALID_ARG. */
#define PSGD_RTOPK_FLAG_DEFERRED_ZERO 0x1u

typedef struct psgd_rtopk_layer_info {
  int64_t rows, cols;
  int64_t numel;       /* rows * cols */
  int64_t offset;      /* element offset inside a worker slice / update */
  int64_t top;         /* r: size of the top-magnitude set */
  int64_t keep;        /* k: entries sent */
  int64_t top_offset;  /* offset of this tensor's ranks inside a worker's row of ranks */
  int64_t keep_offset; /* offset of this tensor's entries inside a worker's index/value row */
} psgd_rtopk_layer_info;

typedef struct psgd_rtopk_sizes {
  int32_t n_layers, n_workers, grad_dtype, reserved;
  int64_t worker_stride; /* elements per worker slice; also the length of update */
  int64_t numel;         /* sum of numel over all tensors */
  int64_t top_total;     /* length of one worker's row of ranks: sum of r */
  int64_t keep_total;    /* length of one worker's row of index/value: sum of k */
  uint64_t workspace_bytes; /* device scratch a step needs (caller-allocated) */
  uint64_t message_bytes;   /* bytes one worker would send: keep_total * (4 + 4) */
  /* minimal bytes a step moves: read G and E, write E' per worker, write U:
     (W*(grad bytes + 8) + 4) * numel */
  uint64_t model_bytes;
} psgd_rtopk_sizes;

/* Build a plan for `n_layers` tensors with per-tensor counts top[l] = r, keep[l] = k
 * (1 <= k <= r <= rows*cols < 2^31), W = n_workers in 1..65535 workers and gradients of
 * grad_dtype.  flags: 0 or PSGD_RTOPK_FLAG_DEFERRED_ZERO (other bits:
 * PSGD_ERR_UNSUPPORTED).  Host only. */
psgd_status psgd_rtopk_plan_create(const psgd_layer* layers, int32_t n_layers, const int64_t* top,
                                   const int64_t* keep, int32_t n_workers, psgd_dtype grad_dtype,
                                   uint32_t flags, psgd_rtopk_plan** out);
psgd_status psgd_rtopk_plan_sizes(const psgd_rtopk_plan* plan, psgd_rtopk_sizes* out);
psgd_status psgd_rtopk_plan_layer_info(const psgd_rtopk_plan* plan, int32_t layer, psgd_rtopk_layer_info* out);
psgd_status psgd_rtopk_plan_destroy(psgd_rtopk_plan* plan);

/* One step for every tensor of the plan and every worker:
 *   grads     [W][worker_stride] grad_dtype, read only
 *   errors    [W][worker_stride] float32, E in, E' out (deferred-zero plans: see the flag)
 *   ranks     [W][top_total] uint32, read only
 *   index     [W][keep_total] int32 out
 *   value     [W][keep_total] float32 out
 *   update    [worker_stride] float32 out, or NULL (then not computed)
 *   workspace workspace_bytes of device memory; contents need not be preserved between
 *             steps, except for deferred-zero plans (see the flag).  Kept from step to
 *             step, it carries each segment's predicted threshold bin, which spares most
 *             steps a second read of M; any other contents give the same results
 * Asynchronous on `stream` (a hipStream_t; NULL = default stream). */
psgd_status psgd_rtopk_step(psgd_rtopk_plan* plan, const void* grads, float* errors, const uint32_t* ranks,
                            int32_t* index, float* value, float* update, void* workspace, void* stream);

/* The plain error memory E' of a deferred-zero plan: out = errors with the entries the
 * last step sent set to zero, if that step's zeros are pending in these errors (see the
 * flag), else a copy.  out may be errors (in place: only the pending entries are written,
 * and the state word is cleared on the stream, so later steps treat the buffer as plain)
 * or a separate [W][worker_stride] float32 buffer (the pending state is kept).  Elements
 * of padding are not written.  For a plan without the flag, out is a copy of errors (in
 * place: nothing to do).  Asynchronous on `stream`.  PSGD_ERR_INVALID_ARG for NULL or
 * misaligned pointers or partly overlapping buffers. */
psgd_status psgd_rtopk_errors_materialize(psgd_rtopk_plan* plan, const float* errors, float* out, void* workspace,
                                          void* stream);

/* Forget a deferred-zero plan's pending zeros (after writing errors or the workspace
 * yourself): the host's view at once, and the workspace's state word by a one-thread
 * kernel on `stream` (so replays of a captured step see it too; the call may itself be
 * captured).  Plans without the flag enqueue nothing.  PSGD_ERR_INVALID_ARG for a NULL
 * plan or a NULL or misaligned workspace. */
psgd_status psgd_rtopk_plan_reset_state(psgd_rtopk_plan* plan, void* workspace, void* stream);

/* Kernel timing as psgd_plan_set_timing / psgd_plan_kernel_stats.  Kernel names:
 * "rk_zero", "rk_ef_hist", "rk_select", "rk_mark", "rk_pick2", "rk_level3", "rk_rule",
 * "rk_final", "rk_scan_top", "rk_keep", "rk_scan_kept", "rk_emit", "rk_update". */
psgd_status psgd_rtopk_plan_set_timing(psgd_rtopk_plan* plan, int32_t enable);
psgd_status psgd_rtopk_plan_kernel_stats(psgd_rtopk_plan* plan, psgd_kernel_stat* out, int32_t capacity,
                                         int32_t* count, int32_t reset);

#ifdef __cplusplus
}
#endif

#endif /* PSGD_RTOPK_H_ */
