// gfx950 kernels of libpsgd and the two step entry points.
//
// One step (the PowerSGD review page, section "Proposed method": EF add, P = M Q from
// the warm-start Q, all-reduce, orthonormalise, Q = M^T P, all-reduce, decompress
// P Q^T, keep the error; then momentum SGD) runs as six batched launches over every
// tensor of the plan:
//
//   k_ef_mean     streams G_w and E_w of all W workers once and writes the worker
//                 mean Mbar = mean_w (G_w + E_w) (for uncompressed tensors: mean_w G_w).
//                 Because the compressor is linear and the W workers share one Q,
//                 mean_w M_w Q = Mbar Q and mean_w M_w^T P = Mbar^T P: the in-HBM
//                 all-reduce of P and Q becomes one pass over the worker slices.
//   k_p_rows      P-bar = Mbar Q_in, one wave per row, lanes across the columns.
//   k_mgs         modified Gram-Schmidt of P-bar, one workgroup per matrix.
//   k_q_partial   Q partials = Mbar^T P over row blocks and column strips.
//   k_q_reduce    Q = sum of the partials (fixed order, deterministic).
//   k_apply       streams G_w and E_w again: E'_w = (G_w + E_w) - P Q^T, writes the
//                 decompressed update once, and in the momentum entry point updates
//                 momentum and parameters in the same pass.
//
// All streaming work is HBM-bound (about one flop per byte), so no MFMA is used.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <string>

#include "plan.hpp"

namespace psgd {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

struct bf16 {
  unsigned short bits;
};

// ------------------------------------------------------------------ loads and stores
// Gradients and errors are touched once per pass and never reused from cache, so the
// streaming passes load and store them non-temporally; buffers that a later kernel of
// the same step reads again (Mbar, the carried error mean) use ordinary accesses.
__device__ __forceinline__ f4 load4(const float* p) { return *reinterpret_cast<const f4*>(p); }

__device__ __forceinline__ f4 load4_nt(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f4*>(p));
}

__device__ __forceinline__ f4 widen(const u16x4 v) {
  f4 r;
  r.x = __uint_as_float(uint32_t(v.x) << 16);
  r.y = __uint_as_float(uint32_t(v.y) << 16);
  r.z = __uint_as_float(uint32_t(v.z) << 16);
  r.w = __uint_as_float(uint32_t(v.w) << 16);
  return r;
}

__device__ __forceinline__ f4 load4_nt(const bf16* p) {
  return widen(__builtin_nontemporal_load(reinterpret_cast<const u16x4*>(p)));
}

// Store the first `valid` (>= 1) lanes of v; all four when valid >= 4.
__device__ __forceinline__ void store4(float* p, const f4 v, int64_t valid) {
  if (valid >= 4) {
    *reinterpret_cast<f4*>(p) = v;
  } else {
    p[0] = v.x;
    if (valid > 1) p[1] = v.y;
    if (valid > 2) p[2] = v.z;
  }
}

__device__ __forceinline__ void store4_nt(float* p, const f4 v, int64_t valid) {
  if (valid >= 4) {
    __builtin_nontemporal_store(v, reinterpret_cast<f4*>(p));
  } else {
    p[0] = v.x;
    if (valid > 1) p[1] = v.y;
    if (valid > 2) p[2] = v.z;
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Sum over the workgroup; every thread gets the same value (same order everywhere).
__device__ double block_sum(double v, double* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double s = 0.0;
  const int nw = blockDim.x >> 6;
  for (int i = 0; i < nw; ++i) s += red[i];
  return s;
}

// Two sums over the workgroup in one round of barriers.
__device__ void block_sum2(double& a, double& b, double* red) {
  a = wave_sum(a);
  b = wave_sum(b);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) {
    red[2 * wave] = a;
    red[2 * wave + 1] = b;
  }
  __syncthreads();
  double sa = 0.0, sb = 0.0;
  const int nw = blockDim.x >> 6;
  for (int i = 0; i < nw; ++i) {
    sa += red[2 * i];
    sb += red[2 * i + 1];
  }
  a = sa;
  b = sb;
}

// u = P Q^T at the four elements of the float4 chunk starting at element c of matrix mi
// (row-major, rank R <= 4); lanes past `valid` are zero.
__device__ __forceinline__ f4 lowrank_chunk(const MatInfo& mi, const float* __restrict__ P,
                                            const float* __restrict__ Q, int64_t c, int64_t valid, int R) {
  const float* Pm = P + mi.p_off;
  const float* Qm = Q + mi.q_off;
  const int cols = mi.cols;
  const int e0 = int(c - mi.offset);
  int i = e0 / cols;
  int j = e0 - i * cols;
  float u[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float s = 0.f;
    if (q < valid) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (k < R) s += Pm[int64_t(i) * R + k] * Qm[int64_t(j) * R + k];
    }
    u[q] = s;
    if (++j == cols) {
      j = 0;
      ++i;
    }
  }
  return f4{u[0], u[1], u[2], u[3]};
}

// ------------------------------------------------------------------ pass 1: EF add + mean
// One float4 chunk per thread, every worker's slice of it loaded before any is used.
// WT > 0: the worker count is the compile-time WT (loop fully unrolled); WT == 0: any
// worker count.  With `ebar` set (carried error mean from the previous step) only the
// gradients are read: Mbar = mean_w G_w + ebar, equal to mean_w (G_w + E_w) because the
// carried ebar is the mean of exactly the E_w stored by that step.
template <typename GT, int WT>
__global__ __launch_bounds__(kStreamThreads) void k_ef_mean(const StreamTile* __restrict__ tiles,
                                                            const GT* __restrict__ G,
                                                            const float* __restrict__ E,
                                                            const float* __restrict__ ebar,
                                                            float* __restrict__ Mbar, int W,
                                                            int64_t ld, float inv_w) {
  const StreamTile t = tiles[blockIdx.x];
  const int64_t c = t.begin + int64_t(threadIdx.x) * 4;
  if (c >= t.end) return;
  const bool with_errors = t.mat >= 0 && ebar == nullptr;
  f4 acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (WT > 0) {
    f4 g[WT];
#pragma unroll
    for (int w = 0; w < WT; ++w) g[w] = load4_nt(G + w * ld + c);
    if (with_errors) {
      f4 e[WT];
#pragma unroll
      for (int w = 0; w < WT; ++w) e[w] = load4_nt(E + w * ld + c);
#pragma unroll
      for (int w = 0; w < WT; ++w) acc += g[w] + e[w];
    } else {
#pragma unroll
      for (int w = 0; w < WT; ++w) acc += g[w];
    }
  } else {
    int w = 0;
    if (with_errors) {
      for (; w + 4 <= W; w += 4) {
        const f4 g0 = load4_nt(G + (w + 0) * ld + c), e0 = load4_nt(E + (w + 0) * ld + c);
        const f4 g1 = load4_nt(G + (w + 1) * ld + c), e1 = load4_nt(E + (w + 1) * ld + c);
        const f4 g2 = load4_nt(G + (w + 2) * ld + c), e2 = load4_nt(E + (w + 2) * ld + c);
        const f4 g3 = load4_nt(G + (w + 3) * ld + c), e3 = load4_nt(E + (w + 3) * ld + c);
        acc += g0 + e0;
        acc += g1 + e1;
        acc += g2 + e2;
        acc += g3 + e3;
      }
      for (; w < W; ++w) acc += load4_nt(G + w * ld + c) + load4_nt(E + w * ld + c);
    } else {
      for (; w + 4 <= W; w += 4) {
        const f4 g0 = load4_nt(G + (w + 0) * ld + c), g1 = load4_nt(G + (w + 1) * ld + c);
        const f4 g2 = load4_nt(G + (w + 2) * ld + c), g3 = load4_nt(G + (w + 3) * ld + c);
        acc += g0;
        acc += g1;
        acc += g2;
        acc += g3;
      }
      for (; w < W; ++w) acc += load4_nt(G + w * ld + c);
    }
  }
  acc *= inv_w;
  if (t.mat >= 0 && ebar != nullptr) acc += load4(ebar + c);
  store4(Mbar + c, acc, t.end - c);
}

// ------------------------------------------------------------------ P-bar = Mbar Q
template <int R>
__global__ __launch_bounds__(kRowThreads) void k_p_rows(const RowTile* __restrict__ tiles,
                                                        const MatInfo* __restrict__ mats,
                                                        const float* __restrict__ Mbar,
                                                        const float* __restrict__ Q,
                                                        float* __restrict__ Pbar) {
  const RowTile t = tiles[blockIdx.x];
  const MatInfo mi = mats[t.mat];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* Qm = Q + mi.q_off;
  const int cols = mi.cols;
  for (int row = t.row_begin + wave; row < t.row_end; row += kRowThreads / 64) {
    const float* mrow = Mbar + mi.offset + int64_t(row) * cols;
    float acc[R];
#pragma unroll
    for (int k = 0; k < R; ++k) acc[k] = 0.f;
    if (mi.vec4) {
#pragma unroll 4
      for (int j = lane * 4; j < cols; j += 256) {
        const f4 v = load4(mrow + j);
        const float* qj = Qm + int64_t(j) * R;
#pragma unroll
        for (int k = 0; k < R; ++k)
          acc[k] += v.x * qj[k] + v.y * qj[R + k] + v.z * qj[2 * R + k] + v.w * qj[3 * R + k];
      }
    } else {
#pragma unroll 4
      for (int j = lane; j < cols; j += 64) {
        const float v = mrow[j];
#pragma unroll
        for (int k = 0; k < R; ++k) acc[k] += v * Qm[int64_t(j) * R + k];
      }
    }
#pragma unroll
    for (int k = 0; k < R; ++k) acc[k] = wave_sum(acc[k]);
    if (lane == 0) {
#pragma unroll
      for (int k = 0; k < R; ++k) Pbar[mi.p_off + int64_t(row) * R + k] = acc[k];
    }
  }
}

// ------------------------------------------------------------------ Gram-Schmidt
// Modified Gram-Schmidt over the R columns of P-bar (rows x R, row-major), in column
// order.  Dot products and norms accumulate in double.  A column whose residual norm
// is at most 1e-4 of its norm before orthogonalisation (or zero) becomes zero.
// Each thread only touches its own rows, so only the reductions synchronise; the norm
// of a fresh column and its projection on column 0 share one reduction (both use the
// unmodified column).  `P2`, if set, receives a copy of the result.
template <int R>
__global__ __launch_bounds__(kMgsThreads) void k_mgs(const MatInfo* __restrict__ mats,
                                                     const float* __restrict__ Pbar,
                                                     float* __restrict__ P, float* __restrict__ P2) {
  __shared__ double red[2 * (kMgsThreads / 64)];
  const MatInfo mi = mats[blockIdx.x];
  const float* src = Pbar + mi.p_off;
  float* dst = P + mi.p_off;
  const int n = mi.rows;
  for (int k = 0; k < R; ++k) {
    double s = 0.0, c = 0.0;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      const int64_t o = int64_t(i) * R;
      const float v = src[o + k];
      dst[o + k] = v;
      s += double(v) * double(v);
      if (k > 0) c += double(dst[o]) * double(v);
    }
    block_sum2(s, c, red);
    const double before = sqrt(s);
    double after = before;
    if (k > 0) {
      for (int l = 0; l < k; ++l) {
        if (l > 0) {
          c = 0.0;
          for (int i = threadIdx.x; i < n; i += blockDim.x)
            c += double(dst[int64_t(i) * R + l]) * double(dst[int64_t(i) * R + k]);
          c = block_sum(c, red);
        }
        for (int i = threadIdx.x; i < n; i += blockDim.x) {
          const int64_t o = int64_t(i) * R;
          dst[o + k] = float(double(dst[o + k]) - c * double(dst[o + l]));
        }
      }
      double s2 = 0.0;
      for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const double v = dst[int64_t(i) * R + k];
        s2 += v * v;
      }
      after = sqrt(block_sum(s2, red));
    }
    const double scale = (after > 0.0 && after > 1e-4 * before) ? 1.0 / after : 0.0;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      const int64_t o = int64_t(i) * R + k;
      const float v = float(double(dst[o]) * scale);
      dst[o] = v;
      if (P2 != nullptr) P2[mi.p_off + o] = v;
    }
  }
}

// ------------------------------------------------------------------ Q = Mbar^T P
template <int R>
__global__ __launch_bounds__(kQThreads) void k_q_partial(const QTile* __restrict__ tiles,
                                                         const MatInfo* __restrict__ mats,
                                                         const float* __restrict__ Mbar,
                                                         const float* __restrict__ P,
                                                         float* __restrict__ Qpart) {
  const QTile t = tiles[blockIdx.x];
  const MatInfo mi = mats[t.mat];
  const int cols = mi.cols;
  const int r0 = t.blk * mi.rows_per_blk;
  const int r1 = min(mi.rows, r0 + mi.rows_per_blk);
  const float* Pm = P + mi.p_off;
  const float* base = Mbar + mi.offset;
  float* out = Qpart + mi.qpart_off + int64_t(t.blk) * cols * R;
  if (mi.vec4) {
    const int j = t.col_begin + int(threadIdx.x) * 4;
    if (j >= t.col_end) return;
    float acc[4][R];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int k = 0; k < R; ++k) acc[q][k] = 0.f;
#pragma unroll 8
    for (int i = r0; i < r1; ++i) {
      const f4 v = load4(base + int64_t(i) * cols + j);
#pragma unroll
      for (int k = 0; k < R; ++k) {
        const float pk = Pm[int64_t(i) * R + k];
        acc[0][k] += v.x * pk;
        acc[1][k] += v.y * pk;
        acc[2][k] += v.z * pk;
        acc[3][k] += v.w * pk;
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int k = 0; k < R; ++k) out[int64_t(j + q) * R + k] = acc[q][k];
  } else {
    const int j = t.col_begin + int(threadIdx.x);
    if (j >= t.col_end) return;
    float acc[R];
#pragma unroll
    for (int k = 0; k < R; ++k) acc[k] = 0.f;
#pragma unroll 8
    for (int i = r0; i < r1; ++i) {
      const float v = base[int64_t(i) * cols + j];
#pragma unroll
      for (int k = 0; k < R; ++k) acc[k] += v * Pm[int64_t(i) * R + k];
    }
#pragma unroll
    for (int k = 0; k < R; ++k) out[int64_t(j) * R + k] = acc[k];
  }
}

__global__ __launch_bounds__(kQRedThreads) void k_q_reduce(const MatInfo* __restrict__ mats,
                                                           const float* __restrict__ Qpart,
                                                           float* __restrict__ Q, float* __restrict__ Q2,
                                                           int R) {
  const MatInfo mi = mats[blockIdx.y];
  const int64_t n = int64_t(mi.cols) * R;
  const float* part = Qpart + mi.qpart_off;
  for (int64_t idx = int64_t(blockIdx.x) * kQRedThreads + threadIdx.x; idx < n;
       idx += int64_t(gridDim.x) * kQRedThreads) {
    float s = 0.f;
    for (int b = 0; b < mi.nblk; ++b) s += part[int64_t(b) * n + idx];
    Q[mi.q_off + idx] = s;
    if (Q2 != nullptr) Q2[mi.q_off + idx] = s;
  }
}

// ------------------------------------------------------------------ pass 2: error + update
enum ApplyMode { kCompress = 0, kMomentum = 1, kNesterov = 2 };

// One float4 chunk per thread.  For a compressed matrix: u = P Q^T at the chunk's four
// elements (rank R <= 4), E'_w = (G_w + E_w) - u for every worker, and (carry mode) the
// mean of the stored E'_w into `ebar`.  Every tensor: the update u is written once and,
// in the momentum modes, mom <- mu*mom + u; x <- x - lr*mom (or x - lr*(u + mu*mom)).
template <typename GT, int WT>
__global__ __launch_bounds__(kStreamThreads) void k_apply(
    const StreamTile* __restrict__ tiles, const MatInfo* __restrict__ mats, const GT* __restrict__ G,
    float* __restrict__ E, const float* __restrict__ Mbar, const float* __restrict__ P,
    const float* __restrict__ Q, float* __restrict__ update, float* __restrict__ mom,
    float* __restrict__ x, float* __restrict__ ebar, int W, int64_t ld, int R, int mode, float lr,
    float mu, float inv_w) {
  const StreamTile t = tiles[blockIdx.x];
  const int64_t c = t.begin + int64_t(threadIdx.x) * 4;
  if (c >= t.end) return;
  const int64_t valid = t.end - c;
  f4 uv;
  if (t.mat < 0) {  // uncompressed tensor: the update is the worker mean
    uv = load4(Mbar + c);
  } else {
    uv = lowrank_chunk(mats[t.mat], P, Q, c, valid, R);
    f4 es = {0.f, 0.f, 0.f, 0.f};
    if constexpr (WT > 0) {
      f4 g[WT], e[WT];
#pragma unroll
      for (int w = 0; w < WT; ++w) {
        g[w] = load4_nt(G + w * ld + c);
        e[w] = load4_nt(E + w * ld + c);
      }
#pragma unroll
      for (int w = 0; w < WT; ++w) {
        const f4 ew = (g[w] + e[w]) - uv;
        store4_nt(E + w * ld + c, ew, valid);
        es += ew;
      }
    } else {
      int w = 0;
      for (; w + 4 <= W; w += 4) {
        const f4 g0 = load4_nt(G + (w + 0) * ld + c), e0v = load4_nt(E + (w + 0) * ld + c);
        const f4 g1 = load4_nt(G + (w + 1) * ld + c), e1v = load4_nt(E + (w + 1) * ld + c);
        const f4 g2 = load4_nt(G + (w + 2) * ld + c), e2v = load4_nt(E + (w + 2) * ld + c);
        const f4 g3 = load4_nt(G + (w + 3) * ld + c), e3v = load4_nt(E + (w + 3) * ld + c);
        const f4 n0 = (g0 + e0v) - uv, n1 = (g1 + e1v) - uv, n2 = (g2 + e2v) - uv, n3 = (g3 + e3v) - uv;
        store4_nt(E + (w + 0) * ld + c, n0, valid);
        store4_nt(E + (w + 1) * ld + c, n1, valid);
        store4_nt(E + (w + 2) * ld + c, n2, valid);
        store4_nt(E + (w + 3) * ld + c, n3, valid);
        es += n0;
        es += n1;
        es += n2;
        es += n3;
      }
      for (; w < W; ++w) {
        const f4 n = (load4_nt(G + w * ld + c) + load4_nt(E + w * ld + c)) - uv;
        store4_nt(E + w * ld + c, n, valid);
        es += n;
      }
    }
    if (ebar != nullptr) store4(ebar + c, es * inv_w, valid);
  }
  if (update != nullptr) store4_nt(update + c, uv, valid);
  if (mode != kCompress) {
    const f4 m0 = load4_nt(mom + c), x0 = load4_nt(x + c);
    const f4 m1 = mu * m0 + uv;
    const f4 x1 = (mode == kNesterov) ? x0 - lr * (uv + mu * m1) : x0 - lr * m1;
    store4_nt(mom + c, m1, valid);
    store4_nt(x + c, x1, valid);
  }
}

// ------------------------------------------------------------------ deferred-error mode
// The error buffer holds M_w = G_w + E_w of the previous step instead of E'_w; the true
// error is that minus the previous step's P Q^T (kept in the workspace).  The single
// pass over the workers then folds the previous subtraction into this step's EF add:
// M_w(t) = G_w(t) + [M_w(t-1) - U(t-1)], stores M_w(t) back and writes Mbar.
template <typename GT, int WT>
__global__ __launch_bounds__(kStreamThreads) void k_ef_defer(
    const StreamTile* __restrict__ tiles, const MatInfo* __restrict__ mats, const GT* __restrict__ G,
    float* __restrict__ E, const float* __restrict__ Pprev, const float* __restrict__ Qprev,
    float* __restrict__ Mbar, int W, int64_t ld, int R, float inv_w, int offset_valid) {
  const StreamTile t = tiles[blockIdx.x];
  const int64_t c = t.begin + int64_t(threadIdx.x) * 4;
  if (c >= t.end) return;
  const int64_t valid = t.end - c;
  const int Wn = WT > 0 ? WT : W;
  f4 acc = {0.f, 0.f, 0.f, 0.f};
  if (t.mat < 0) {
    for (int w = 0; w < Wn; ++w) acc += load4_nt(G + w * ld + c);
    store4(Mbar + c, acc * inv_w, valid);
    return;
  }
  const f4 up = offset_valid ? lowrank_chunk(mats[t.mat], Pprev, Qprev, c, valid, R) : f4{0.f, 0.f, 0.f, 0.f};
  if constexpr (WT > 0) {
    f4 g[WT], e[WT];
#pragma unroll
    for (int w = 0; w < WT; ++w) {
      g[w] = load4_nt(G + w * ld + c);
      e[w] = load4_nt(E + w * ld + c);
    }
#pragma unroll
    for (int w = 0; w < WT; ++w) {
      const f4 m = (g[w] + e[w]) - up;
      store4_nt(E + w * ld + c, m, valid);
      acc += m;
    }
  } else {
    int w = 0;
    for (; w + 4 <= W; w += 4) {
      const f4 g0 = load4_nt(G + (w + 0) * ld + c), e0v = load4_nt(E + (w + 0) * ld + c);
      const f4 g1 = load4_nt(G + (w + 1) * ld + c), e1v = load4_nt(E + (w + 1) * ld + c);
      const f4 g2 = load4_nt(G + (w + 2) * ld + c), e2v = load4_nt(E + (w + 2) * ld + c);
      const f4 g3 = load4_nt(G + (w + 3) * ld + c), e3v = load4_nt(E + (w + 3) * ld + c);
      const f4 m0 = (g0 + e0v) - up, m1 = (g1 + e1v) - up, m2 = (g2 + e2v) - up, m3 = (g3 + e3v) - up;
      store4_nt(E + (w + 0) * ld + c, m0, valid);
      store4_nt(E + (w + 1) * ld + c, m1, valid);
      store4_nt(E + (w + 2) * ld + c, m2, valid);
      store4_nt(E + (w + 3) * ld + c, m3, valid);
      acc += m0;
      acc += m1;
      acc += m2;
      acc += m3;
    }
    for (; w < W; ++w) {
      const f4 m = (load4_nt(G + w * ld + c) + load4_nt(E + w * ld + c)) - up;
      store4_nt(E + w * ld + c, m, valid);
      acc += m;
    }
  }
  store4(Mbar + c, acc * inv_w, valid);
}

// Deferred mode's last pass: the decompressed update (P Q^T, or the mean for 1-D
// tensors) and the momentum-SGD update; no worker data is touched.  Matrix tiles are
// rows x a column strip: a thread keeps Q of its four columns in registers and walks
// the rows, reading each row of P once per wave.  The sum order over the rank matches
// lowrank_chunk, so U here equals the U the next step subtracts.
__device__ __forceinline__ void momentum_store(float* mom, float* x, int64_t c, const f4 uv, int64_t valid,
                                               int mode, float lr, float mu) {
  const f4 m0 = load4_nt(mom + c), x0 = load4_nt(x + c);
  const f4 m1 = mu * m0 + uv;
  const f4 x1 = (mode == kNesterov) ? x0 - lr * (uv + mu * m1) : x0 - lr * m1;
  store4_nt(mom + c, m1, valid);
  store4_nt(x + c, x1, valid);
}

__global__ __launch_bounds__(kQThreads) void k_update(
    const UpdTile* __restrict__ tiles, const MatInfo* __restrict__ mats, const float* __restrict__ Mbar,
    const float* __restrict__ P, const float* __restrict__ Q, float* __restrict__ update,
    float* __restrict__ mom, float* __restrict__ x, int R, int mode, float lr, float mu) {
  const UpdTile t = tiles[blockIdx.x];
  if (t.mat < 0) {
    const int64_t c = t.begin + int64_t(threadIdx.x) * 4;
    if (c >= t.end) return;
    const int64_t valid = t.end - c;
    const f4 uv = load4(Mbar + c);
    if (update != nullptr) store4_nt(update + c, uv, valid);
    if (mode != kCompress) momentum_store(mom, x, c, uv, valid, mode, lr, mu);
    return;
  }
  const MatInfo mi = mats[t.mat];
  const int cols = mi.cols;
  const float* Pm = P + mi.p_off;
  const float* Qm = Q + mi.q_off;
  if (mi.vec4) {
    const int j = t.col_begin + int(threadIdx.x) * 4;
    if (j >= cols) return;
    float qv[4][4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int k = 0; k < 4; ++k) qv[q][k] = (k < R) ? Qm[int64_t(j + q) * R + k] : 0.f;
    for (int i = t.row_begin; i < t.row_end; ++i) {
      float pr[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) pr[k] = (k < R) ? Pm[int64_t(i) * R + k] : 0.f;
      float u[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (k < R) s += pr[k] * qv[q][k];
        u[q] = s;
      }
      const f4 uv = {u[0], u[1], u[2], u[3]};
      const int64_t c = mi.offset + int64_t(i) * cols + j;
      if (update != nullptr) store4_nt(update + c, uv, 4);
      if (mode != kCompress) momentum_store(mom, x, c, uv, 4, mode, lr, mu);
    }
  } else {
    const int j = t.col_begin + int(threadIdx.x);
    if (j >= cols) return;
    float qv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) qv[k] = (k < R) ? Qm[int64_t(j) * R + k] : 0.f;
    for (int i = t.row_begin; i < t.row_end; ++i) {
      float s = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (k < R) s += Pm[int64_t(i) * R + k] * qv[k];
      const int64_t c = mi.offset + int64_t(i) * cols + j;
      if (update != nullptr) update[c] = s;
      if (mode != kCompress) {
        const float m1 = mu * mom[c] + s;
        x[c] = (mode == kNesterov) ? x[c] - lr * (s + mu * m1) : x[c] - lr * m1;
        mom[c] = m1;
      }
    }
  }
}

// out_w = errors_w - P_prev Q_prev^T for every compressed matrix (the plain error memory
// of a deferred-mode error buffer); 1-D tensors are skipped.
__global__ __launch_bounds__(kStreamThreads) void k_materialize(
    const StreamTile* __restrict__ tiles, const MatInfo* __restrict__ mats, const float* E,
    float* out, const float* __restrict__ Pprev, const float* __restrict__ Qprev, int W, int64_t ld,
    int R, int offset_valid) {
  const StreamTile t = tiles[blockIdx.x];
  const int64_t c = t.begin + int64_t(threadIdx.x) * 4;
  if (c >= t.end || t.mat < 0) return;
  const int64_t valid = t.end - c;
  const f4 up = offset_valid ? lowrank_chunk(mats[t.mat], Pprev, Qprev, c, valid, R) : f4{0.f, 0.f, 0.f, 0.f};
  for (int w = 0; w < W; ++w) store4_nt(out + w * ld + c, load4_nt(E + w * ld + c) - up, valid);
}

// ------------------------------------------------------------------ calibration copy
__global__ __launch_bounds__(256) void k_stream_copy(const float* __restrict__ src, float* __restrict__ dst,
                                                     int64_t n4) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n4; i += int64_t(gridDim.x) * 256)
    __builtin_nontemporal_store(load4_nt(src + 4 * i), reinterpret_cast<f4*>(dst + 4 * i));
}

// ------------------------------------------------------------------ host helpers
psgd_status hip_fail(const char* what, hipError_t e) {
  set_error(std::string(what) + ": " + hipGetErrorString(e));
  return PSGD_ERR_HIP;
}

uint64_t align256(uint64_t x) { return (x + 255) / 256 * 256; }

psgd_status ensure_tables(psgd_plan* plan, DeviceTables** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("hipGetDevice", e);
  auto it = plan->dev.find(dev);
  if (it != plan->dev.end()) {
    *out = &it->second;
    return PSGD_OK;
  }
  const uint64_t b_mats = align256(plan->mats.size() * sizeof(MatInfo) + 1);
  const uint64_t b_st = align256(plan->stiles.size() * sizeof(StreamTile) + 1);
  const uint64_t b_rt = align256(plan->rtiles.size() * sizeof(RowTile) + 1);
  const uint64_t b_qt = align256(plan->qtiles.size() * sizeof(QTile) + 1);
  const uint64_t b_ut = align256(plan->utiles.size() * sizeof(UpdTile) + 1);
  void* base = nullptr;
  e = hipMalloc(&base, b_mats + b_st + b_rt + b_qt + b_ut);
  if (e != hipSuccess) {
    set_error(std::string("hipMalloc of the plan's device tables: ") + hipGetErrorString(e));
    return PSGD_ERR_NO_MEMORY;
  }
  DeviceTables t;
  t.base = base;
  char* b = static_cast<char*>(base);
  t.mats = reinterpret_cast<MatInfo*>(b);
  t.stiles = reinterpret_cast<StreamTile*>(b + b_mats);
  t.rtiles = reinterpret_cast<RowTile*>(b + b_mats + b_st);
  t.qtiles = reinterpret_cast<QTile*>(b + b_mats + b_st + b_rt);
  t.utiles = reinterpret_cast<UpdTile*>(b + b_mats + b_st + b_rt + b_qt);
  struct {
    void* dst;
    const void* src;
    size_t bytes;
  } copies[] = {
      {t.mats, plan->mats.data(), plan->mats.size() * sizeof(MatInfo)},
      {t.stiles, plan->stiles.data(), plan->stiles.size() * sizeof(StreamTile)},
      {t.rtiles, plan->rtiles.data(), plan->rtiles.size() * sizeof(RowTile)},
      {t.qtiles, plan->qtiles.data(), plan->qtiles.size() * sizeof(QTile)},
      {t.utiles, plan->utiles.data(), plan->utiles.size() * sizeof(UpdTile)},
  };
  for (const auto& c : copies) {
    if (c.bytes == 0) continue;
    e = hipMemcpy(c.dst, c.src, c.bytes, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      (void)hipFree(base);
      return hip_fail("hipMemcpy of the plan's device tables", e);
    }
  }
  auto ins = plan->dev.emplace(dev, t);
  *out = &ins.first->second;
  return PSGD_OK;
}

struct Range {
  const char* name;
  uintptr_t lo, hi;
};

psgd_status check_ptr(const char* fn, const char* name, const void* p, bool nullable) {
  if (p == nullptr) {
    if (nullable) return PSGD_OK;
    set_error(std::string(fn) + ": " + name + " is NULL");
    return PSGD_ERR_INVALID_ARG;
  }
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0) {
    set_error(std::string(fn) + ": " + name + " is not 16-byte aligned");
    return PSGD_ERR_INVALID_ARG;
  }
  return PSGD_OK;
}

psgd_status take_event(psgd_plan* plan, hipEvent_t* ev) {
  if (!plan->event_pool.empty()) {
    *ev = plan->event_pool.back();
    plan->event_pool.pop_back();
    return PSGD_OK;
  }
  hipError_t e = hipEventCreate(ev);
  return e == hipSuccess ? PSGD_OK : hip_fail("hipEventCreate", e);
}

// Launch through `launch()`; with timing enabled, bracket it with two events on `st`.
template <typename F>
psgd_status launch_timed(psgd_plan* plan, hipStream_t st, int kid, F&& launch) {
  hipEvent_t a = nullptr, b = nullptr;
  if (plan->timing) {
    psgd_status s = take_event(plan, &a);
    if (s == PSGD_OK) s = take_event(plan, &b);
    if (s != PSGD_OK) {
      if (a) plan->event_pool.push_back(a);
      return s;
    }
    hipError_t e = hipEventRecord(a, st);
    if (e != hipSuccess) {
      plan->event_pool.push_back(a);
      plan->event_pool.push_back(b);
      return hip_fail("hipEventRecord", e);
    }
  }
  launch();
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && plan->timing) e = hipEventRecord(b, st);
  if (e != hipSuccess) {
    if (plan->timing) {
      plan->event_pool.push_back(a);
      plan->event_pool.push_back(b);
    }
    return hip_fail((std::string("launch ") + kKernelNames[kid]).c_str(), e);
  }
  if (plan->timing) plan->pending.push_back(PendingTiming{kid, a, b});
  return PSGD_OK;
}

// Everything one step's launches need.
struct StepArgs {
  const void* grads;
  float* errors;
  float* q;
  float* p;
  float* update;
  float* mom;
  float* x;
  float lr, mu, inv_w;
  float* Mbar;
  float* Pbar;
  float* Qpart;
  const float* ebar_in;  // carried error mean to read (carry mode, valid carry)
  float* ebar_out;       // error mean to write (carry mode)
  float* Pprev;          // previous P, Q (deferred mode)
  float* Qprev;
  int offset_valid;      // deferred mode: errors hold M of the previous step
  int W, R, mode;
  int64_t ld;
  unsigned n_st;
  hipStream_t st;
};

enum PassKind { kPassMean = 0, kPassApply = 1, kPassDefer = 2 };

template <typename GT, int WT>
void launch_pass(int which, const DeviceTables& dt, const StepArgs& a) {
  const GT* g = static_cast<const GT*>(a.grads);
  if (which == kPassMean)
    hipLaunchKernelGGL((k_ef_mean<GT, WT>), dim3(a.n_st), dim3(kStreamThreads), 0, a.st, dt.stiles, g, a.errors,
                       a.ebar_in, a.Mbar, a.W, a.ld, a.inv_w);
  else if (which == kPassApply)
    hipLaunchKernelGGL((k_apply<GT, WT>), dim3(a.n_st), dim3(kStreamThreads), 0, a.st, dt.stiles, dt.mats, g,
                       a.errors, a.Mbar, a.p, a.q, a.update, a.mom, a.x, a.ebar_out, a.W, a.ld, a.R, a.mode,
                       a.lr, a.mu, a.inv_w);
  else
    hipLaunchKernelGGL((k_ef_defer<GT, WT>), dim3(a.n_st), dim3(kStreamThreads), 0, a.st, dt.stiles, dt.mats,
                       g, a.errors, a.Pprev, a.Qprev, a.Mbar, a.W, a.ld, a.R, a.inv_w, a.offset_valid);
}

// Worker-count specialisations of the streaming passes: W in {1,2,4,8,16} unrolls fully,
// anything else takes the generic loop.
template <typename GT>
void launch_pass_w(int which, const DeviceTables& dt, const StepArgs& a) {
  switch (a.W) {
    case 1: launch_pass<GT, 1>(which, dt, a); break;
    case 2: launch_pass<GT, 2>(which, dt, a); break;
    case 4: launch_pass<GT, 4>(which, dt, a); break;
    case 8: launch_pass<GT, 8>(which, dt, a); break;
    case 16: launch_pass<GT, 16>(which, dt, a); break;
    default: launch_pass<GT, 0>(which, dt, a); break;
  }
}

template <int R>
psgd_status launch_all(psgd_plan* plan, const DeviceTables& dt, const StepArgs& a) {
  const bool deferred = (plan->flags & PSGD_FLAG_DEFERRED_ERROR) != 0;
  const bool bf = plan->dtype == PSGD_BF16;
  const unsigned n_mats = unsigned(plan->mats.size());
  hipStream_t stream = a.st;
  psgd_status s;
  auto pass = [&](int which) {
    if (bf)
      launch_pass_w<bf16>(which, dt, a);
    else
      launch_pass_w<float>(which, dt, a);
  };

  if (deferred)
    s = launch_timed(plan, stream, kKEfDefer, [&] { pass(kPassDefer); });
  else
    s = launch_timed(plan, stream, kKEfMean, [&] { pass(kPassMean); });
  if (s != PSGD_OK) return s;

  if (n_mats > 0) {
    s = launch_timed(plan, stream, kKPRows, [&] {
      hipLaunchKernelGGL(k_p_rows<R>, dim3(unsigned(plan->rtiles.size())), dim3(kRowThreads), 0, stream,
                         dt.rtiles, dt.mats, a.Mbar, a.q, a.Pbar);
    });
    if (s != PSGD_OK) return s;
    s = launch_timed(plan, stream, kKMgs, [&] {
      hipLaunchKernelGGL(k_mgs<R>, dim3(n_mats), dim3(plan->mgs_threads), 0, stream, dt.mats, a.Pbar, a.p,
                         deferred ? a.Pprev : nullptr);
    });
    if (s != PSGD_OK) return s;
    s = launch_timed(plan, stream, kKQPartial, [&] {
      hipLaunchKernelGGL(k_q_partial<R>, dim3(unsigned(plan->qtiles.size())), dim3(kQThreads), 0, stream,
                         dt.qtiles, dt.mats, a.Mbar, a.p, a.Qpart);
    });
    if (s != PSGD_OK) return s;
    const unsigned gx = unsigned((plan->max_q_elems_per_matrix + kQRedThreads - 1) / kQRedThreads);
    s = launch_timed(plan, stream, kKQReduce, [&] {
      hipLaunchKernelGGL(k_q_reduce, dim3(gx, n_mats), dim3(kQRedThreads), 0, stream, dt.mats, a.Qpart, a.q,
                         deferred ? a.Qprev : nullptr, R);
    });
    if (s != PSGD_OK) return s;
  }
  if (deferred)
    return launch_timed(plan, stream, kKUpdate, [&] {
      hipLaunchKernelGGL(k_update, dim3(unsigned(plan->utiles.size())), dim3(kQThreads), 0, stream, dt.utiles,
                         dt.mats, a.Mbar, a.p, a.q, a.update, a.mom, a.x, R, a.mode, a.lr, a.mu);
    });
  return launch_timed(plan, stream, kKApply, [&] { pass(kPassApply); });
}

// Same device, same error and workspace buffers as the step that left the state.
bool state_matches(const psgd_plan* plan, const void* errors, const void* workspace, int dev) {
  return plan->state_valid && plan->state_errors == errors && plan->state_workspace == workspace &&
         plan->state_device == dev;
}

psgd_status run_step(const char* fn, psgd_plan* plan, const void* grads, float* errors, float* q,
                     float* p, float* update, float* mom, float* x, float lr, float mu, void* workspace,
                     void* stream, int mode) {
  if (plan == nullptr) {
    set_error(std::string(fn) + ": plan is NULL");
    return PSGD_ERR_INVALID_ARG;
  }
  const bool has_mats = !plan->mats.empty();
  psgd_status s;
  if ((s = check_ptr(fn, "grads", grads, false)) != PSGD_OK) return s;
  if ((s = check_ptr(fn, "errors", errors, !has_mats)) != PSGD_OK) return s;
  if ((s = check_ptr(fn, "q", q, !has_mats)) != PSGD_OK) return s;
  if ((s = check_ptr(fn, "p", p, !has_mats)) != PSGD_OK) return s;
  if ((s = check_ptr(fn, "update", update, true)) != PSGD_OK) return s;
  if ((s = check_ptr(fn, "workspace", workspace, false)) != PSGD_OK) return s;
  if (mode != kCompress) {
    if ((s = check_ptr(fn, "momentum", mom, false)) != PSGD_OK) return s;
    if ((s = check_ptr(fn, "params", x, false)) != PSGD_OK) return s;
    if (!std::isfinite(lr) || !std::isfinite(mu)) {
      set_error(std::string(fn) + ": lr and mu must be finite");
      return PSGD_ERR_INVALID_ARG;
    }
  }
  // No two buffers may overlap (errors, q, momentum, params are in/out in place).
  const uint64_t W = uint64_t(plan->n_workers), ld = uint64_t(plan->worker_stride);
  const uint64_t gb = plan->dtype == PSGD_BF16 ? 2 : 4;
  Range rs[8];
  int nr = 0;
  auto add = [&](const char* name, const void* ptr, uint64_t bytes) {
    if (ptr != nullptr && bytes > 0)
      rs[nr++] = Range{name, reinterpret_cast<uintptr_t>(ptr), reinterpret_cast<uintptr_t>(ptr) + bytes};
  };
  add("grads", grads, W * ld * gb);
  add("errors", has_mats ? errors : nullptr, W * ld * 4);
  add("q", has_mats ? q : nullptr, uint64_t(plan->q_elems) * 4);
  add("p", has_mats ? p : nullptr, uint64_t(plan->p_elems) * 4);
  add("update", update, ld * 4);
  add("workspace", workspace, plan->workspace_bytes);
  if (mode != kCompress) {
    add("momentum", mom, ld * 4);
    add("params", x, ld * 4);
  }
  for (int i = 0; i < nr; ++i)
    for (int j = i + 1; j < nr; ++j)
      if (rs[i].lo < rs[j].hi && rs[j].lo < rs[i].hi) {
        set_error(std::string(fn) + ": buffers " + rs[i].name + " and " + rs[j].name + " overlap");
        return PSGD_ERR_INVALID_ARG;
      }

  DeviceTables* dt = nullptr;
  if ((s = ensure_tables(plan, &dt)) != PSGD_OK) return s;
  int dev = 0;
  (void)hipGetDevice(&dev);
  char* ws = static_cast<char*>(workspace);
  const bool carry = (plan->flags & PSGD_FLAG_CARRY_ERROR_MEAN) != 0;
  const bool deferred = (plan->flags & PSGD_FLAG_DEFERRED_ERROR) != 0;
  // Cross-step state (carried error mean, or the deferred offset) is used only if the
  // previous step of this plan left it on this device in these error/workspace buffers.
  const bool use_state = (carry || deferred) && state_matches(plan, errors, workspace, dev);
  plan->state_valid = false;

  StepArgs a{};
  a.grads = grads;
  a.errors = errors;
  a.q = q;
  a.p = p;
  a.update = update;
  a.mom = mom;
  a.x = x;
  a.lr = lr;
  a.mu = mu;
  a.inv_w = 1.0f / float(plan->n_workers);
  a.Mbar = reinterpret_cast<float*>(ws + plan->ws_mbar);
  a.Pbar = reinterpret_cast<float*>(ws + plan->ws_pbar);
  a.Qpart = reinterpret_cast<float*>(ws + plan->ws_qpart);
  a.ebar_out = carry ? reinterpret_cast<float*>(ws + plan->ws_ebar) : nullptr;
  a.ebar_in = (carry && use_state) ? a.ebar_out : nullptr;
  a.Pprev = deferred ? reinterpret_cast<float*>(ws + plan->ws_pprev) : nullptr;
  a.Qprev = deferred ? reinterpret_cast<float*>(ws + plan->ws_qprev) : nullptr;
  a.offset_valid = (deferred && use_state) ? 1 : 0;
  a.W = plan->n_workers;
  a.R = plan->rank;
  a.mode = mode;
  a.ld = plan->worker_stride;
  a.n_st = unsigned(plan->stiles.size());
  a.st = static_cast<hipStream_t>(stream);
  switch (plan->rank) {
    case 1: s = launch_all<1>(plan, *dt, a); break;
    case 2: s = launch_all<2>(plan, *dt, a); break;
    case 3: s = launch_all<3>(plan, *dt, a); break;
    case 4: s = launch_all<4>(plan, *dt, a); break;
    default:
      set_error(std::string(fn) + ": rank outside 1..4");
      return PSGD_ERR_UNSUPPORTED;
  }
  if (s == PSGD_OK && (carry || deferred) && has_mats) {
    plan->state_valid = true;
    plan->state_errors = errors;
    plan->state_workspace = workspace;
    plan->state_device = dev;
  }
  plan->last_step_used_state = use_state;
  return s;
}

}  // namespace
}  // namespace psgd

using namespace psgd;

extern "C" psgd_status psgd_compress_step(psgd_plan* plan, const void* grads, float* errors, float* q,
                                          float* p, float* update, void* workspace, void* stream) {
  return run_step("psgd_compress_step", plan, grads, errors, q, p, update, nullptr, nullptr, 0.f, 0.f,
                  workspace, stream, kCompress);
}

extern "C" psgd_status psgd_stream_copy(const void* src, void* dst, uint64_t bytes, void* stream) {
  psgd_status s;
  if ((s = check_ptr("psgd_stream_copy", "src", src, false)) != PSGD_OK) return s;
  if ((s = check_ptr("psgd_stream_copy", "dst", dst, false)) != PSGD_OK) return s;
  if (bytes % 16 != 0) {
    set_error("psgd_stream_copy: bytes must be a multiple of 16");
    return PSGD_ERR_INVALID_ARG;
  }
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  if (a < b + bytes && b < a + bytes) {
    set_error("psgd_stream_copy: src and dst overlap");
    return PSGD_ERR_INVALID_ARG;
  }
  if (bytes == 0) return PSGD_OK;
  // 1024 workgroups of 256 threads (4 per CU) grid-striding: the fastest shape found
  // for a plain copy on the 256-CU device.
  hipLaunchKernelGGL(k_stream_copy, dim3(1024), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const float*>(src), static_cast<float*>(dst), int64_t(bytes / 16));
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? PSGD_OK : hip_fail("launch k_stream_copy", e);
}

extern "C" psgd_status psgd_plan_reset_carry(psgd_plan* plan) {
  if (plan == nullptr) {
    set_error("psgd_plan_reset_carry: plan is NULL");
    return PSGD_ERR_INVALID_ARG;
  }
  plan->state_valid = false;
  return PSGD_OK;
}

extern "C" psgd_status psgd_errors_materialize(psgd_plan* plan, const float* errors, float* out,
                                               void* workspace, void* stream) {
  const char* fn = "psgd_errors_materialize";
  if (plan == nullptr) {
    set_error(std::string(fn) + ": plan is NULL");
    return PSGD_ERR_INVALID_ARG;
  }
  psgd_status s;
  if ((s = check_ptr(fn, "errors", errors, false)) != PSGD_OK) return s;
  if ((s = check_ptr(fn, "out", out, false)) != PSGD_OK) return s;
  if ((s = check_ptr(fn, "workspace", workspace, false)) != PSGD_OK) return s;
  const uint64_t bytes = uint64_t(plan->n_workers) * uint64_t(plan->worker_stride) * 4;
  const uintptr_t e0 = reinterpret_cast<uintptr_t>(errors), o0 = reinterpret_cast<uintptr_t>(out);
  if (out != errors && e0 < o0 + bytes && o0 < e0 + bytes) {
    set_error(std::string(fn) + ": out partly overlaps errors (pass the same pointer for in place)");
    return PSGD_ERR_INVALID_ARG;
  }
  if (plan->mats.empty()) return PSGD_OK;
  int dev = 0;
  (void)hipGetDevice(&dev);
  const bool deferred = (plan->flags & PSGD_FLAG_DEFERRED_ERROR) != 0;
  const bool offset = deferred && state_matches(plan, errors, workspace, dev);
  if (!offset && out == errors) return PSGD_OK;  // already plain, nothing to write
  DeviceTables* dt = nullptr;
  if ((s = ensure_tables(plan, &dt)) != PSGD_OK) return s;
  char* ws = static_cast<char*>(workspace);
  const float* Pprev = deferred ? reinterpret_cast<const float*>(ws + plan->ws_pprev) : nullptr;
  const float* Qprev = deferred ? reinterpret_cast<const float*>(ws + plan->ws_qprev) : nullptr;
  hipLaunchKernelGGL(k_materialize, dim3(unsigned(plan->stiles.size())), dim3(kStreamThreads), 0,
                     static_cast<hipStream_t>(stream), dt->stiles, dt->mats, errors, out, Pprev, Qprev,
                     plan->n_workers, plan->worker_stride, plan->rank, offset ? 1 : 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail("launch k_materialize", e);
  if (offset && out == errors) plan->state_valid = false;  // the buffer now holds plain errors
  return PSGD_OK;
}

extern "C" psgd_status psgd_ef_momentum_apply(psgd_plan* plan, const void* grads, float* errors,
                                              float* q, float* p, float* momentum, float* params,
                                              float lr, float mu, float* update, void* workspace,
                                              void* stream) {
  const int mode = (plan != nullptr && (plan->flags & PSGD_FLAG_NESTEROV)) ? kNesterov : kMomentum;
  return run_step("psgd_ef_momentum_apply", plan, grads, errors, q, p, update, momentum, params, lr, mu,
                  workspace, stream, mode);
}
