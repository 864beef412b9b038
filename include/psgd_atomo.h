/*
 * psgd_atomo.h -- Spectral-ATOMO gradient sparsification in libpsgd, as hand-written HIP
 * kernels for AMD Instinct MI355X (gfx950).  Status codes, the layer list and the
 * kernel-timing record are those of psgd.h.
 *
 * What one step computes (the review page "ATOMO: Communication-efficient Learning via
 * Atomic Sparsification", section "Proposed method": a gradient written as a weighted
 * sum of unit-norm atoms is sparsified without bias by keeping atom i with probability
 * p_i and dividing it by p_i; the p_i minimise the expected squared norm of the result
 * under the budget sum_i p_i = s; Spectral-ATOMO takes the atoms of a layer's gradient
 * matrix from its singular value decomposition):
 *   for each of W data-parallel workers and each layer matrix G_w (n x m, k = min(n, m)):
 *     G_w    = sum_i sigma_i u_i v_i^T          singular values descending, i < k
 *     p_i    = min(1, c * sigma_i)              c > 0 fixed by sum_i p_i = s (atoms with
 *                                               sigma_i = 0 get p_i = 0); when s is at
 *                                               least the number of nonzero sigma_i,
 *                                               every nonzero atom has p_i = 1
 *     sent   = { i : x_i < p_i }                x = the caller's uniforms in [0, 1)
 *     G_hat_w = sum over sent i of (sigma_i / p_i) u_i v_i^T
 *   and U = mean_w G_hat_w (the all-reduce of the messages; the W workers are W slices
 *   of one HBM buffer).  Tensors that are not matrices with min(n, m) >= 2 are sent
 *   whole: U = mean_w G_w.  No error feedback: the estimator is unbiased.
 *
 * Readings of points the page leaves open:
 *   - the budget s is the same for every matrix;
 *   - a sent atom travels as two factors a (n floats) and b (m floats) with
 *     G_hat_w = sum a b^T.  The factor of length k is the unit singular vector on that
 *     side (u when n <= m, else v) and the other factor is the opposite singular vector
 *     times sigma_i / p_i (computed as G^T u / p_i or G v / p_i);
 *   - a singular vector's sign is not fixed (flipping both factors leaves the atom
 *     unchanged).  Inside a cluster of (nearly) equal singular values, any orthonormal
 *     basis of the cluster's singular subspace is as valid as any other;
 *   - arithmetic is float32: the Gram matrix G G^T (or G^T G) of the short side, its
 *     reduction to tridiagonal form, bisection for its eigenvalues (sigma_i^2) and
 *     inverse iteration for the eigenvectors of the sent atoms.  The Gram matrix's
 *     products run on bf16 matrix cores with every entry split exactly into three bf16
 *     parts; the six products kept carry each x y to within about 2^-20 |x y|, and the sums
 *     accumulate in float32 (the five smaller products of a step summed apart from the
 *     running sum), which keeps the singular values as close to float64 as the float32
 *     matrix instruction does.  Singular values below about sqrt(k * 2^-24) * sigma_max
 *     carry float32 rounding of that order.
 *
 * Memory layout.  The packed layout of psgd.h: every tensor starts at an element offset
 * that is a multiple of 64 (psgd_atomo_plan_layer_info gives it); grads are
 * [n_workers][worker_stride] float32; update is [worker_stride].  Per compressed matrix
 * l, at offsets from psgd_atomo_plan_layer_info:
 *   uniforms, sigma, prob  [n_workers][sv_total] float32, k entries at sv_offset(l), in
 *                          descending-sigma order;
 *   index                  [n_workers][sv_total] int32: the first count entries are the
 *                          sent atoms' positions (ascending), the rest are -1;
 *   count                  [n_workers][n_matrices] int32, entry matrix_index(l);
 *   atoms                  [n_workers][atom_total] float32: sent atom j of matrix l at
 *                          atom_offset(l) + j * (n + m), a (n floats) then b (m floats);
 *                          the space of unsent atoms is not written.
 *
 * Ownership, pointers, errors and concurrency as in psgd.h: caller-owned device
 * buffers (16-byte aligned), argument errors reported before anything is enqueued,
 * asynchronous execution on `stream`, one stream at a time per plan.  No two buffers
 * may overlap.
 */
#ifndef PSGD_ATOMO_H_
#define PSGD_ATOMO_H_

#include "psgd.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct psgd_atomo_plan psgd_atomo_plan;

/* Largest min(rows, cols) of a compressed matrix. */
#define PSGD_ATOMO_MAX_K 1024

typedef struct psgd_atomo_layer_info {
  int64_t rows, cols;
  int64_t numel;        /* rows * cols */
  int64_t offset;       /* element offset inside a worker slice / update */
  int32_t compressed;   /* 1: a matrix with min(rows, cols) >= 2 */
  int32_t matrix_index; /* index into count's rows, or -1 */
  int64_t k;            /* min(rows, cols) for a compressed matrix, else 0 */
  int64_t sv_offset;    /* offset inside a worker's row of uniforms / sigma / prob / index */
  int64_t atom_offset;  /* offset inside a worker's row of atoms */
} psgd_atomo_layer_info;

typedef struct psgd_atomo_sizes {
  int32_t n_layers, n_workers, n_matrices, reserved;
  int64_t worker_stride;    /* elements per worker slice; also the length of update */
  int64_t numel;            /* sum of numel over all tensors */
  int64_t sv_total;         /* sum of k over the compressed matrices */
  int64_t atom_total;       /* sum of k * (rows + cols) over the compressed matrices */
  uint64_t workspace_bytes; /* device scratch a step needs (caller-allocated) */
  /* minimal bytes a step moves: read G once for the Gram matrices and once for the
     second factors, write U: (2 * W * 4 + 4) * numel */
  uint64_t model_bytes;
  double budget;            /* s */
} psgd_atomo_sizes;

/* Build a plan for `n_layers` tensors, budget s > 0 (expected atoms sent per matrix,
 * finite), W = n_workers in 1..65535 and float32 gradients.  Matrices with
 * min(rows, cols) > PSGD_ATOMO_MAX_K are rejected (PSGD_ERR_UNSUPPORTED), and so is a
 * plan with more than 65535 Gram tiles (the sum over matrices of T (T + 1) / 2 with
 * T = ceil(min(rows, cols) / 128)) or more than 65535 factor tiles (a matrix with
 * rows <= cols has ceil(cols / 256) of them, any other ceil(rows / 16)).  flags must be
 * 0.  Host only. */
psgd_status psgd_atomo_plan_create(const psgd_layer* layers, int32_t n_layers, double budget, int32_t n_workers,
                                   uint32_t flags, psgd_atomo_plan** out);
psgd_status psgd_atomo_plan_sizes(const psgd_atomo_plan* plan, psgd_atomo_sizes* out);
psgd_status psgd_atomo_plan_layer_info(const psgd_atomo_plan* plan, int32_t layer, psgd_atomo_layer_info* out);
psgd_status psgd_atomo_plan_destroy(psgd_atomo_plan* plan);

/* One step for every tensor of the plan and every worker:
 *   grads     [W][worker_stride] float32, read only
 *   uniforms  [W][sv_total] float32 in [0, 1), read only
 *   sigma     [W][sv_total] float32 out
 *   prob      [W][sv_total] float32 out
 *   index     [W][sv_total] int32 out
 *   count     [W][n_matrices] int32 out
 *   atoms     [W][atom_total] float32 out
 *   update    [worker_stride] float32 out, or NULL (then not computed)
 *   workspace workspace_bytes of device memory, contents need not be preserved
 * Asynchronous on `stream` (a hipStream_t; NULL = default stream).  Non-finite
 * gradients give non-finite results for their matrix. */
psgd_status psgd_atomo_step(psgd_atomo_plan* plan, const float* grads, const float* uniforms, float* sigma,
                            float* prob, int32_t* index, int32_t* count, float* atoms, float* update,
                            void* workspace, void* stream);

/* Kernel timing as psgd_plan_set_timing / psgd_plan_kernel_stats.  Kernel names:
 * "at_gram", "at_band", "at_chase", "at_eig", "at_sample", "at_vectors", "at_backchase",
 * "at_backband", "at_factor", "at_update". */
psgd_status psgd_atomo_plan_set_timing(psgd_atomo_plan* plan, int32_t enable);
psgd_status psgd_atomo_plan_kernel_stats(psgd_atomo_plan* plan, psgd_kernel_stat* out, int32_t capacity,
                                         int32_t* count, int32_t reset);

#ifdef __cplusplus
}
#endif

#endif /* PSGD_ATOMO_H_ */
