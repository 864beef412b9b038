// gfx950 kernels of libpsgd and the step entry points.
//
// One step (the PowerSGD review page, section "Proposed method": EF add, P = M Q from
// the warm-start Q, all-reduce, orthonormalise, Q = M^T P, all-reduce, decompress
// P Q^T, keep the error; then momentum SGD) runs as five batched launches over every
// tensor of the plan:
//
//   k_first      streams the W workers' slices of G (and E) once.  For a compressed
//                matrix it forms M_w = G_w + E_w, the worker mean Mbar, and the partial
//                row sums of P-bar = Mbar Q over its column strip.  Because the
//                compressor is linear and all workers share Q,
//                mean_w M_w Q = Mbar Q and mean_w M_w^T P = Mbar^T P: the all-reduce of
//                P and Q becomes this one pass over the worker slices.  1-D tensors get
//                the worker mean of G.
//   k_mgs        sums the P-bar partials and orthonormalises the columns, one
//                workgroup per matrix: Gram-Schmidt taken in the r x r Gram space of
//                P-bar (one fixed-order fp64 reduction of the Gram entries, then the
//                column-by-column coefficients and drop rule), which is modified
//                Gram-Schmidt in exact arithmetic.
//   k_q_partial  Q partials = Mbar^T P over row blocks and column strips.
//   k_q_reduce   Q = sum of the partials (fixed order, deterministic).
//   k_apply      streams G and E again: E'_w = (G_w + E_w) - P Q^T, writes the
//                decompressed update once and, in the momentum entry point, updates
//                momentum and parameters in the same pass.
//
// Deferred-error plans replace k_apply with k_update (U and momentum only) and fold
// the subtraction of the previous step's P Q^T into the next step's k_first.
//
// The worker passes are HBM-bound (about one flop per byte), so no MFMA is used.  They
// run one 64-lane wave per matrix row by a strip of 256 columns (float4 per lane), or per
// few rows when the worker count is small: each lane keeps Q of its four columns in
// registers, reads P one row at a time (the same address across the wave), and has every
// worker's float4 of a row in flight at once.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <map>
#include <mutex>
#include <string>
#include <type_traits>

#include "plan.hpp"

namespace psgd {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

struct bf16 {
  unsigned short bits;
};

enum ApplyMode { kCompress = 0, kMomentum = 1, kNesterov = 2 };
enum FirstPass { kFpMean = 0, kFpCarry = 1, kFpDefer = 2 };

// ------------------------------------------------------------------ loads and stores
// Gradients and errors are touched once per pass and never reused from cache, so the
// worker passes load and store them non-temporally; buffers that a later kernel of the
// same step reads again (Mbar, the carried error mean) use ordinary accesses.
// V elements per lane: 4 when a matrix's column count is even (rows 16-byte aligned, or
// 8-byte aligned and accessed as two halves), else 1.
template <int V>
using vec_t = std::conditional_t<V == 4, f4, float>;

__device__ __forceinline__ float lane(const f4& x, int q) { return x[q]; }
__device__ __forceinline__ float lane(const float& x, int) { return x; }

__device__ __forceinline__ f4 widen(const u16x4 v) {
  f4 r;
  r.x = __uint_as_float(uint32_t(v.x) << 16);
  r.y = __uint_as_float(uint32_t(v.y) << 16);
  r.z = __uint_as_float(uint32_t(v.z) << 16);
  r.w = __uint_as_float(uint32_t(v.w) << 16);
  return r;
}

__device__ __forceinline__ f2 widen(const u16x2 v) {
  f2 r;
  r.x = __uint_as_float(uint32_t(v.x) << 16);
  r.y = __uint_as_float(uint32_t(v.y) << 16);
  return r;
}

// A: the alignment of p in floats.  V = 4 with A = 2 (rows whose column count is even but
// not a multiple of 4 are only 8-byte aligned) reads and writes the four floats as two
// 8-byte halves.  Such a row ends two columns into its last lane: there hi is false and
// the upper half is neither read (it reads as zero) nor written.
template <int V, int A = V>
__device__ __forceinline__ vec_t<V> ldv(const float* p, bool hi = true) {
  if constexpr (V == 4 && A == 2) {
    const f2 a = *reinterpret_cast<const f2*>(p);
    const f2 b = hi ? *reinterpret_cast<const f2*>(p + 2) : f2{0.f, 0.f};
    return f4{a.x, a.y, b.x, b.y};
  } else if constexpr (V == 4)
    return *reinterpret_cast<const f4*>(p);
  else
    return *p;
}

template <int V, int A = V>
__device__ __forceinline__ vec_t<V> ld_nt(const float* p, bool hi = true) {
  if constexpr (V == 4 && A == 2) {
    const f2 a = __builtin_nontemporal_load(reinterpret_cast<const f2*>(p));
    const f2 b = hi ? __builtin_nontemporal_load(reinterpret_cast<const f2*>(p + 2)) : f2{0.f, 0.f};
    return f4{a.x, a.y, b.x, b.y};
  } else if constexpr (V == 4)
    return __builtin_nontemporal_load(reinterpret_cast<const f4*>(p));
  else
    return __builtin_nontemporal_load(p);
}

template <int V, int A = V>
__device__ __forceinline__ vec_t<V> ld_nt(const bf16* p, bool hi = true) {
  if constexpr (V == 4 && A == 2) {
    const f2 a = widen(__builtin_nontemporal_load(reinterpret_cast<const u16x2*>(p)));
    const f2 b = hi ? widen(__builtin_nontemporal_load(reinterpret_cast<const u16x2*>(p + 2))) : f2{0.f, 0.f};
    return f4{a.x, a.y, b.x, b.y};
  } else if constexpr (V == 4)
    return widen(__builtin_nontemporal_load(reinterpret_cast<const u16x4*>(p)));
  else
    return __uint_as_float(uint32_t(__builtin_nontemporal_load(reinterpret_cast<const unsigned short*>(p))) << 16);
}

template <int V, int A = V>
__device__ __forceinline__ void st(float* p, const vec_t<V> v, bool hi = true) {
  if constexpr (V == 4 && A == 2) {
    *reinterpret_cast<f2*>(p) = f2{v.x, v.y};
    if (hi) *reinterpret_cast<f2*>(p + 2) = f2{v.z, v.w};
  } else if constexpr (V == 4)
    *reinterpret_cast<f4*>(p) = v;
  else
    *p = v;
}

template <int V, int A = V>
__device__ __forceinline__ void st_nt(float* p, const vec_t<V> v, bool hi = true) {
  if constexpr (V == 4 && A == 2) {
    __builtin_nontemporal_store(f2{v.x, v.y}, reinterpret_cast<f2*>(p));
    if (hi) __builtin_nontemporal_store(f2{v.z, v.w}, reinterpret_cast<f2*>(p + 2));
  } else if constexpr (V == 4)
    __builtin_nontemporal_store(v, reinterpret_cast<f4*>(p));
  else
    __builtin_nontemporal_store(v, p);
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

// ------------------------------------------------------------------ reductions
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

// N sums over the workgroup in one round of barriers (red holds N * waves doubles);
// every thread gets the same values.
template <int N>
__device__ void block_sum_n(double (&v)[N], double* red) {
  const int lane_id = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int a = 0; a < N; ++a) v[a] = wave_sum(v[a]);
  __syncthreads();
  if (lane_id == 0)
#pragma unroll
    for (int a = 0; a < N; ++a) red[N * wave + a] = v[a];
  __syncthreads();
  const int nw = blockDim.x >> 6;
#pragma unroll
  for (int a = 0; a < N; ++a) {
    double t = 0.0;
    for (int i = 0; i < nw; ++i) t += red[N * i + a];
    v[a] = t;
  }
}

// ------------------------------------------------------------------ P Q^T
// The decompressed value at one element is sum_k P[i,k] Q[j,k] accumulated in k order
// from zero (one fma per term); every kernel that needs it uses exactly this order, so
// the U written by one kernel equals the U another subtracts.
__device__ __forceinline__ float pq_dot(const float* pr, const float* qr, int R) {
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (k < R) s += pr[k] * qr[k];
  return s;
}

// Q rows of four consecutive columns: 4*RR floats from a 16-byte aligned address, read
// as RR float4 loads.
template <int RR>
__device__ __forceinline__ void load_q4(float (&qv)[4][4], const float* base) {
  float flat[4 * RR];
#pragma unroll
  for (int v = 0; v < RR; ++v) {
    const f4 x = reinterpret_cast<const f4*>(base)[v];
    flat[4 * v + 0] = x.x;
    flat[4 * v + 1] = x.y;
    flat[4 * v + 2] = x.z;
    flat[4 * v + 3] = x.w;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int k = 0; k < 4; ++k) qv[q][k] = (k < RR) ? flat[q * RR + k] : 0.f;
}

// Q rows of the thread's V columns starting at j (zeros past the rank or when
// inactive).  With V = 4, j is a multiple of 4 and every Q block starts on a 16-byte
// boundary, so the 4R floats are R aligned float4 loads.
template <int V>
__device__ __forceinline__ void load_q_cols(float (&qv)[V][4], const float* Qm, int j, int R, bool active,
                                            bool hi = true) {
  if constexpr (V == 4) {
    if (active && hi) {
      const float* base = Qm + int64_t(j) * R;
      switch (R) {
        case 1: load_q4<1>(qv, base); return;
        case 2: load_q4<2>(qv, base); return;
        case 3: load_q4<3>(qv, base); return;
        default: load_q4<4>(qv, base); return;
      }
    }
  }
#pragma unroll
  for (int q = 0; q < V; ++q)
#pragma unroll
    for (int k = 0; k < 4; ++k) qv[q][k] = (active && k < R && (q < 2 || hi)) ? Qm[int64_t(j + q) * R + k] : 0.f;
}

__device__ __forceinline__ void load_p_row(float (&pr)[4], const float* Pm, int i, int R) {
#pragma unroll
  for (int k = 0; k < 4; ++k) pr[k] = (k < R) ? Pm[int64_t(i) * R + k] : 0.f;
}

template <int V>
__device__ __forceinline__ vec_t<V> pq_row(const float (&pr)[4], const float (&qv)[V][4], int R) {
  if constexpr (V == 4)
    return f4{pq_dot(pr, qv[0], R), pq_dot(pr, qv[1], R), pq_dot(pr, qv[2], R), pq_dot(pr, qv[3], R)};
  else
    return pq_dot(pr, qv[0], R);
}

// ------------------------------------------------------------------ flat chunks
// A flat matrix (rows that do not start on a 128-byte line) is streamed in runs of
// consecutive elements, four per lane from a 16-byte boundary, so that no cache line is
// split between two waves.  A lane's four elements can run from the end of one row into
// the start of the next.
struct Flat4 {
  int i0, j0;  // row and column of the lane's first element
  int nw;      // how many of the four lie in row i0; the rest continue row i0 + 1 from column 0
  int valid;   // how many lie inside the matrix (0 past its end)
};

// c: absolute element offset of the lane's first element (a multiple of 4).
__device__ __forceinline__ Flat4 flat4_at(const MatInfo& mi, int64_t c) {
  const int64_t e = c - mi.offset;
  const int64_t numel = int64_t(mi.rows) * mi.cols;
  Flat4 f;
  if (e >= numel) {
    f.i0 = mi.rows;
    f.j0 = 0;
    f.nw = 4;
    f.valid = 0;
    return f;
  }
  const int ei = int(e);
  f.i0 = ei / mi.cols;
  f.j0 = ei - f.i0 * mi.cols;
  f.nw = min(4, mi.cols - f.j0);
  f.valid = int(min<int64_t>(4, numel - e));
  return f;
}

// Q row of one column: R floats (one float4 or float2 load for R = 4 or 2; every Q
// block starts on a 16-byte boundary), zeros past the rank.
__device__ __forceinline__ void load_q_col(float (&qc)[4], const float* Qm, int col, int R) {
  const float* b = Qm + int64_t(col) * R;
  if (R == 4) {
    const f4 v = *reinterpret_cast<const f4*>(b);
    qc[0] = v.x;
    qc[1] = v.y;
    qc[2] = v.z;
    qc[3] = v.w;
  } else if (R == 2) {
    const f2 v = *reinterpret_cast<const f2*>(b);
    qc[0] = v.x;
    qc[1] = v.y;
    qc[2] = 0.f;
    qc[3] = 0.f;
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) qc[k] = (k < R) ? b[k] : 0.f;
  }
}

// P rows i0 and i0 + 1 of the lane's elements (zeros where the lane has none).
__device__ __forceinline__ void load_flat_p_rows(float (&p0)[4], float (&p1)[4], const float* Pm, const Flat4& f,
                                                 int R) {
#pragma unroll
  for (int k = 0; k < 4; ++k) p0[k] = p1[k] = 0.f;
  if (f.valid > 0) load_p_row(p0, Pm, f.i0, R);
  if (f.valid > f.nw) load_p_row(p1, Pm, f.i0 + 1, R);
}

// (P Q^T) at the lane's elements, each by pq_dot (0 past the matrix end).
__device__ __forceinline__ f4 pq_flat(const float (&p0)[4], const float (&p1)[4], const float* Qm, const Flat4& f,
                                      int R) {
  // Four elements of one row whose Q rows start on a 16-byte boundary (nearly every lane):
  // the 4R floats are R aligned float4 loads and every element uses p0.  Same products
  // and order as the column-by-column form below.
  if (f.nw == 4 && f.valid == 4 && ((f.j0 * R) & 3) == 0) {
    float qv[4][4];
    const float* base = Qm + int64_t(f.j0) * R;
    switch (R) {
      case 1: load_q4<1>(qv, base); break;
      case 2: load_q4<2>(qv, base); break;
      case 3: load_q4<3>(qv, base); break;
      default: load_q4<4>(qv, base); break;
    }
    return f4{pq_dot(p0, qv[0], R), pq_dot(p0, qv[1], R), pq_dot(p0, qv[2], R), pq_dot(p0, qv[3], R)};
  }
  f4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (q < f.valid) {
      const bool first = q < f.nw;
      float qc[4], pr[4];
      load_q_col(qc, Qm, first ? f.j0 + q : q - f.nw, R);
#pragma unroll
      for (int k = 0; k < 4; ++k) pr[k] = first ? p0[k] : p1[k];
      u[q] = pq_dot(pr, qc, R);
    }
  return u;
}

// P-bar partial row sums of one flat chunk (chunk index `chunk` within the matrix; mb
// is zero past the matrix end).  Each lane splits its share of mb Q between rows i0 and
// i0 + 1; the part in row i0 + 1 moves to the next lane, whose first element is in that
// row.  A segmented inclusive scan over the wave (lanes keyed by row, fixed order) then
// leaves each row's sum over the chunk in the row's last lane, which writes it to slot
// chunk - (first chunk of the row).  The part of the last lane in row i0 + 1 is that
// row's whole share of the chunk and is written as it is.  Every lane must call this.
__device__ __forceinline__ void flat_pbar_partial(const MatInfo& mi, const Flat4& f, const f4 mb, const float* Qm,
                                                  float* Ppart, int chunk, int R) {
  const int ln = int(threadIdx.x) & 63;
  float a[4] = {0.f, 0.f, 0.f, 0.f}, b[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (q < f.valid) {
      const bool first = q < f.nw;
      float qc[4];
      load_q_col(qc, Qm, first ? f.j0 + q : q - f.nw, R);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (first)
          a[k] += mb[q] * qc[k];
        else
          b[k] += mb[q] * qc[k];
      }
    }
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (k < R) {
      const float t = __shfl_up(b[k], 1, 64);
      if (ln > 0) a[k] += t;
    }
  const int key = f.valid > 0 ? f.i0 : mi.rows;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int kk = __shfl_up(key, o, 64);
    float t[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) t[k] = (k < R) ? __shfl_up(a[k], o, 64) : 0.f;
    if (ln >= o && kk == key)
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (k < R) a[k] += t[k];
  }
  const int next = __shfl_down(key, 1, 64);
  float* base = Ppart + mi.ppart_off;
  if ((ln == 63 || next != key) && key < mi.rows) {
    const int slot = chunk - (key * mi.cols) / kStreamTileElems;
    float* dst = base + (int64_t(slot) * mi.rows + key) * R;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (k < R) dst[k] = a[k];
  }
  if (ln == 63 && f.valid > f.nw) {
    const int row = f.i0 + 1;
    const int slot = chunk - (row * mi.cols) / kStreamTileElems;
    float* dst = base + (int64_t(slot) * mi.rows + row) * R;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (k < R) dst[k] = b[k];
  }
}

// ------------------------------------------------------------------ worker loops
// Every worker's slice of one chunk (V consecutive elements at c) is loaded before any
// is used.  WT > 0: the worker count is the compile-time WT (fully unrolled); WT == 0:
// any worker count, four at a time.

// sum_w (G_w + E_w)
template <int V, typename GT, int WT, int A = V>
__device__ __forceinline__ vec_t<V> sum_ge(const GT* G, const float* E, int W, int64_t ld, int64_t c,
                                          bool hi = true) {
  vec_t<V> acc{};
  if constexpr (WT > 0) {
    vec_t<V> g[WT], e[WT];
#pragma unroll
    for (int w = 0; w < WT; ++w) {
      g[w] = ld_nt<V, A>(G + w * ld + c, hi);
      e[w] = ld_nt<V, A>(E + w * ld + c, hi);
    }
#pragma unroll
    for (int w = 0; w < WT; ++w) acc += g[w] + e[w];
  } else {
    int w = 0;
    for (; w + 4 <= W; w += 4) {
      vec_t<V> g[4], e[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        g[k] = ld_nt<V, A>(G + (w + k) * ld + c, hi);
        e[k] = ld_nt<V, A>(E + (w + k) * ld + c, hi);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) acc += g[k] + e[k];
    }
    for (; w < W; ++w) acc += ld_nt<V, A>(G + w * ld + c, hi) + ld_nt<V, A>(E + w * ld + c, hi);
  }
  return acc;
}

// sum_w G_w
template <int V, typename GT, int WT, int A = V>
__device__ __forceinline__ vec_t<V> sum_g(const GT* G, int W, int64_t ld, int64_t c, bool hi = true) {
  vec_t<V> acc{};
  if constexpr (WT > 0) {
    vec_t<V> g[WT];
#pragma unroll
    for (int w = 0; w < WT; ++w) g[w] = ld_nt<V, A>(G + w * ld + c, hi);
#pragma unroll
    for (int w = 0; w < WT; ++w) acc += g[w];
  } else {
    int w = 0;
    for (; w + 4 <= W; w += 4) {
      vec_t<V> g[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) g[k] = ld_nt<V, A>(G + (w + k) * ld + c, hi);
#pragma unroll
      for (int k = 0; k < 4; ++k) acc += g[k];
    }
    for (; w < W; ++w) acc += ld_nt<V, A>(G + w * ld + c, hi);
  }
  return acc;
}

// E_w <- (G_w + E_w) - u for every worker; returns sum_w of the stored values.
template <int V, typename GT, int WT, int A = V>
__device__ __forceinline__ vec_t<V> update_workers(const GT* G, float* E, int W, int64_t ld, int64_t c,
                                                   const vec_t<V> u, bool hi = true) {
  vec_t<V> acc{};
  if constexpr (WT > 0) {
    vec_t<V> g[WT], e[WT];
#pragma unroll
    for (int w = 0; w < WT; ++w) {
      g[w] = ld_nt<V, A>(G + w * ld + c, hi);
      e[w] = ld_nt<V, A>(E + w * ld + c, hi);
    }
#pragma unroll
    for (int w = 0; w < WT; ++w) {
      const vec_t<V> n = (g[w] + e[w]) - u;
      st_nt<V, A>(E + w * ld + c, n, hi);
      acc += n;
    }
  } else {
    int w = 0;
    for (; w + 4 <= W; w += 4) {
      vec_t<V> g[4], e[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        g[k] = ld_nt<V, A>(G + (w + k) * ld + c, hi);
        e[k] = ld_nt<V, A>(E + (w + k) * ld + c, hi);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const vec_t<V> n = (g[k] + e[k]) - u;
        st_nt<V, A>(E + (w + k) * ld + c, n, hi);
        acc += n;
      }
    }
    for (; w < W; ++w) {
      const vec_t<V> n = (ld_nt<V, A>(G + w * ld + c, hi) + ld_nt<V, A>(E + w * ld + c, hi)) - u;
      st_nt<V, A>(E + w * ld + c, n, hi);
      acc += n;
    }
  }
  return acc;
}

// PSGD_FLAG_LOCAL_Q_ERROR: E_w <- (G_w + E_w) - P_i Q_w^T with each worker's own Q_w
// (its columns at j read from Qw + w * q_ws + q_off); returns sum_w of the stored values.
template <int V, typename GT, int WT, int A = V>
__device__ __forceinline__ vec_t<V> update_workers_local(const GT* G, float* E, int W, int64_t ld, int64_t c,
                                                         const float (&pr)[4], const float* Qw, int64_t q_ws,
                                                         int64_t q_off, int j, int R, bool hi = true) {
  vec_t<V> acc{};
  constexpr int B = 4;  // four workers in flight: each also needs its own Q_w columns
  for (int w0 = 0; w0 < W; w0 += B) {
    vec_t<V> g[B], e[B];
#pragma unroll
    for (int k = 0; k < B; ++k)
      if ((WT > 0 && WT % B == 0) || w0 + k < W) {
        g[k] = ld_nt<V, A>(G + (w0 + k) * ld + c, hi);
        e[k] = ld_nt<V, A>(E + (w0 + k) * ld + c, hi);
      }
#pragma unroll
    for (int k = 0; k < B; ++k)
      if ((WT > 0 && WT % B == 0) || w0 + k < W) {
        float qw[V][4];
        load_q_cols<V>(qw, Qw + int64_t(w0 + k) * q_ws + q_off, j, R, true, hi);
        const vec_t<V> n = (g[k] + e[k]) - pq_row<V>(pr, qw, R);
        st_nt<V, A>(E + (w0 + k) * ld + c, n, hi);
        acc += n;
      }
  }
  return acc;
}

// The last lane of a flat matrix whose size is not a multiple of 4: E_w <- (G_w + E_w) - u
// on the first `valid` elements only (the loads past them stay inside the padding before
// the next tensor); returns sum_w of the new values (unspecified past `valid`).
template <typename GT>
__device__ f4 update_workers_tail(const GT* G, float* E, int W, int64_t ld, int64_t c, const f4 u, int valid) {
  f4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int w = 0; w < W; ++w) {
    const f4 n = (ld_nt<4>(G + w * ld + c) + ld_nt<4>(E + w * ld + c)) - u;
    store4_nt(E + w * ld + c, n, valid);
    acc += n;
  }
  return acc;
}

// PSGD_FLAG_LOCAL_Q_ERROR over a flat chunk: E_w <- (G_w + E_w) - (P Q_w^T) at the
// lane's elements, only the first `valid` of them stored; returns sum_w of the new values.
template <typename GT, int WT>
__device__ __forceinline__ f4 update_workers_local_flat(const GT* G, float* E, int W, int64_t ld, int64_t c,
                                                        const float (&p0)[4], const float (&p1)[4],
                                                        const float* Qw, int64_t q_ws, int64_t q_off,
                                                        const Flat4& f, int R) {
  f4 acc = {0.f, 0.f, 0.f, 0.f};
  constexpr int B = 4;
  for (int w0 = 0; w0 < W; w0 += B) {
    f4 g[B], e[B];
#pragma unroll
    for (int k = 0; k < B; ++k)
      if ((WT > 0 && WT % B == 0) || w0 + k < W) {
        g[k] = ld_nt<4>(G + (w0 + k) * ld + c);
        e[k] = ld_nt<4>(E + (w0 + k) * ld + c);
      }
#pragma unroll
    for (int k = 0; k < B; ++k)
      if ((WT > 0 && WT % B == 0) || w0 + k < W) {
        const f4 uw = pq_flat(p0, p1, Qw + int64_t(w0 + k) * q_ws + q_off, f, R);
        const f4 n = (g[k] + e[k]) - uw;
        if (f.valid == 4)
          st_nt<4>(E + (w0 + k) * ld + c, n);
        else
          store4_nt(E + (w0 + k) * ld + c, n, f.valid);
        acc += n;
      }
  }
  return acc;
}

template <int V, int A = V>
__device__ __forceinline__ void momentum_v(float* mom, float* x, int64_t c, const vec_t<V> u, int mode, float lr,
                                           float mu, bool hi = true) {
  const vec_t<V> m0 = ld_nt<V, A>(mom + c, hi), x0 = ld_nt<V, A>(x + c, hi);
  const vec_t<V> m1 = mu * m0 + u;
  const vec_t<V> x1 = (mode == kNesterov) ? x0 - lr * (u + mu * m1) : x0 - lr * m1;
  st_nt<V, A>(mom + c, m1, hi);
  st_nt<V, A>(x + c, x1, hi);
}

__device__ __forceinline__ void momentum_masked(float* mom, float* x, int64_t c, const f4 u, int64_t valid,
                                                int mode, float lr, float mu) {
  const f4 m0 = *reinterpret_cast<const f4*>(mom + c), x0 = *reinterpret_cast<const f4*>(x + c);
  const f4 m1 = mu * m0 + u;
  const f4 x1 = (mode == kNesterov) ? x0 - lr * (u + mu * m1) : x0 - lr * m1;
  store4_nt(mom + c, m1, valid);
  store4_nt(x + c, x1, valid);
}

// ------------------------------------------------------------------ pass 1
// One wave per row of a tile: row row_begin + rb x the lanes' V columns each (a tile
// spans several rows for plans too large for one table entry per row, and at small
// worker counts).
// FP selects the first-pass form:
//   kFpMean  Mbar = mean_w (G_w + E_w)
//   kFpCarry Mbar = mean_w G_w + ebar  (ebar = mean of the errors the previous step
//            stored, carried in the workspace)
//   kFpDefer M_w = (G_w + E_w) - P_prev Q_prev^T is stored back into E; Mbar = mean_w M_w
// For every row, each lane's share of P-bar = Mbar Q over its columns is summed across
// the wave (fixed butterfly order) and lane 0 writes the strip's partial row sum.
template <int V, typename GT, int WT, int FP, int A = V>
__device__ __forceinline__ void first_matrix_tile(const UpdTile& t, const MatInfo& mi, const GT* G, float* E,
                                                  const float* ebar, const float* Pprev, const float* Qprev,
                                                  const float* Qin, float* Mbar, float* Ppart, int W, int64_t ld,
                                                  int R, float inv_w, int offset_valid, int rb) {
  const int cols = mi.cols;
  const int ln = int(threadIdx.x) & 63;
  const int j = t.col_begin + ln * V;
  const bool active = j < cols;
  const bool hi = A == V || j + 4 <= cols;
  float qv[V][4];
  load_q_cols<V>(qv, Qin + mi.q_off, j, R, active, hi);
  float qp[V][4];
  if constexpr (FP == kFpDefer) load_q_cols<V>(qp, Qprev + mi.q_off, j, R, active && offset_valid, hi);
  const int strip = t.col_begin / (kStreamThreads * V);
  float* prow = Ppart + mi.ppart_off + int64_t(strip) * mi.rows * R;
  {
    const int i = t.row_begin + rb;
    if (i >= t.row_end) return;
    float part[4] = {0.f, 0.f, 0.f, 0.f};
    if (active) {
      const int64_t c = mi.offset + int64_t(i) * cols + j;
      vec_t<V> mb;
      if constexpr (FP == kFpDefer) {
        float pp[4] = {0.f, 0.f, 0.f, 0.f};
        if (offset_valid) load_p_row(pp, Pprev + mi.p_off, i, R);
        mb = update_workers<V, GT, WT, A>(G, E, W, ld, c, pq_row<V>(pp, qp, R), hi) * inv_w;
      } else if constexpr (FP == kFpCarry) {
        mb = sum_g<V, GT, WT, A>(G, W, ld, c, hi) * inv_w + ldv<V, A>(ebar + c, hi);
      } else {
        mb = sum_ge<V, GT, WT, A>(G, E, W, ld, c, hi) * inv_w;
      }
      st<V, A>(Mbar + c, mb, hi);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float s = 0.f;
#pragma unroll
        for (int q = 0; q < V; ++q) s += lane(mb, q) * qv[q][k];
        part[k] = s;
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (k < R) {
        const float v = wave_sum(part[k]);
        if (ln == 0) prow[int64_t(i) * R + k] = v;
      }
  }
}

// The same over RP consecutive rows per wave, for small compile-time worker counts
// (WT > 0): the strip's Q rows are loaded once for all RP rows, and every worker's chunk
// of every row is in flight before the first store.  Rows past the tile's end load row
// i0 again (a valid address) and store nothing.  Per row, the arithmetic and its order
// are those of first_matrix_tile.
template <int V, typename GT, int WT, int FP, int RP, int A = V>
__device__ __forceinline__ void first_matrix_rows(const UpdTile& t, const MatInfo& mi, const GT* G, float* E,
                                                  const float* ebar, const float* Pprev, const float* Qprev,
                                                  const float* Qin, float* Mbar, float* Ppart, int64_t ld,
                                                  int R, float inv_w, int offset_valid, int rb) {
  static_assert(WT > 0, "the multi-row first pass needs a compile-time worker count");
  const int cols = mi.cols;
  const int ln = int(threadIdx.x) & 63;
  const int j = t.col_begin + ln * V;
  const bool active = j < cols;
  const bool hi = A == V || j + 4 <= cols;
  const int i0 = t.row_begin + rb * RP;
  if (i0 >= t.row_end) return;
  const int nr = min(RP, t.row_end - i0);
  float qv[V][4];
  load_q_cols<V>(qv, Qin + mi.q_off, j, R, active, hi);
  float qp[V][4];
  if constexpr (FP == kFpDefer) load_q_cols<V>(qp, Qprev + mi.q_off, j, R, active && offset_valid, hi);
  const int strip = t.col_begin / (kStreamThreads * V);
  float* prow = Ppart + mi.ppart_off + int64_t(strip) * mi.rows * R;
  float part[RP][4];
#pragma unroll
  for (int rr = 0; rr < RP; ++rr)
#pragma unroll
    for (int k = 0; k < 4; ++k) part[rr][k] = 0.f;
  if (active) {
    const int64_t c0 = mi.offset + int64_t(i0) * cols + j;
    vec_t<V> g[RP][WT], e[RP][WT];
#pragma unroll
    for (int rr = 0; rr < RP; ++rr) {
      const int64_t c = c0 + int64_t(rr < nr ? rr : 0) * cols;
#pragma unroll
      for (int w = 0; w < WT; ++w) {
        g[rr][w] = ld_nt<V, A>(G + w * ld + c, hi);
        if constexpr (FP == kFpCarry) {
          if (w == 0) e[rr][0] = ldv<V, A>(ebar + c, hi);
        } else {
          e[rr][w] = ld_nt<V, A>(E + w * ld + c, hi);
        }
      }
    }
#pragma unroll
    for (int rr = 0; rr < RP; ++rr) {
      if (rr >= nr) break;
      const int64_t c = c0 + int64_t(rr) * cols;
      vec_t<V> acc{};
      if constexpr (FP == kFpDefer) {
        float pp[4] = {0.f, 0.f, 0.f, 0.f};
        if (offset_valid) load_p_row(pp, Pprev + mi.p_off, i0 + rr, R);
        const vec_t<V> u = pq_row<V>(pp, qp, R);
#pragma unroll
        for (int w = 0; w < WT; ++w) {
          const vec_t<V> n = (g[rr][w] + e[rr][w]) - u;
          st_nt<V, A>(E + w * ld + c, n, hi);
          acc += n;
        }
        acc = acc * inv_w;
      } else if constexpr (FP == kFpCarry) {
#pragma unroll
        for (int w = 0; w < WT; ++w) acc += g[rr][w];
        acc = acc * inv_w + e[rr][0];
      } else {
#pragma unroll
        for (int w = 0; w < WT; ++w) acc += g[rr][w] + e[rr][w];
        acc = acc * inv_w;
      }
      st<V, A>(Mbar + c, acc, hi);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float s = 0.f;
#pragma unroll
        for (int q = 0; q < V; ++q) s += lane(acc, q) * qv[q][k];
        part[rr][k] = s;
      }
    }
  }
#pragma unroll
  for (int rr = 0; rr < RP; ++rr) {
    if (rr >= nr) break;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (k < R) {
        const float v = wave_sum(part[rr][k]);
        if (ln == 0) prow[int64_t(i0 + rr) * R + k] = v;
      }
  }
}

// The same for one flat chunk (chunk `chunk` of the tile), four elements per lane.
template <typename GT, int WT, int FP>
__device__ __forceinline__ void first_flat_tile(const UpdTile& t, const MatInfo& mi, const GT* G, float* E,
                                                const float* ebar, const float* Pprev, const float* Qprev,
                                                const float* Qin, float* Mbar, float* Ppart, int W, int64_t ld,
                                                int R, float inv_w, int offset_valid, int chunk) {
  const int64_t c0 = t.begin + int64_t(chunk) * kStreamTileElems;
  if (c0 >= t.end) return;
  const int64_t c = c0 + int64_t(threadIdx.x & 63) * 4;
  const Flat4 f = flat4_at(mi, c);
  f4 mb = {0.f, 0.f, 0.f, 0.f};
  if (f.valid > 0) {
    if constexpr (FP == kFpDefer) {
      f4 u = {0.f, 0.f, 0.f, 0.f};
      if (offset_valid) {
        float p0[4], p1[4];
        load_flat_p_rows(p0, p1, Pprev + mi.p_off, f, R);
        u = pq_flat(p0, p1, Qprev + mi.q_off, f, R);
      }
      mb = (f.valid == 4 ? update_workers<4, GT, WT>(G, E, W, ld, c, u)
                         : update_workers_tail<GT>(G, E, W, ld, c, u, f.valid)) * inv_w;
    } else if constexpr (FP == kFpCarry) {
      mb = sum_g<4, GT, WT>(G, W, ld, c) * inv_w + ldv<4>(ebar + c);
    } else {
      mb = sum_ge<4, GT, WT>(G, E, W, ld, c) * inv_w;
    }
    store4(Mbar + c, mb, f.valid);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (q >= f.valid) mb[q] = 0.f;
  }
  flat_pbar_partial(mi, f, mb, Qin + mi.q_off, Ppart, int((c0 - mi.offset) / kStreamTileElems), R);
}

// Worker passes run a 1-D grid of ntiles x rgroups workgroups, one wave each, with the
// row group fastest: consecutive workgroups walk down one tile's rows, so the launch
// sweeps every buffer in address order (a tile-fastest order visits one row of every
// tile first, across the whole multi-GB buffers, before the next).  A plan with 2^32 or
// more worker-pass threads takes a 2-D grid instead (tile = blockIdx.x, row group =
// blockIdx.y).
struct TileRow {
  int tile, rb;
};
__device__ __forceinline__ TileRow tile_row(int rgroups) {
  if (gridDim.y > 1) return TileRow{int(blockIdx.x), int(blockIdx.y)};
  const int id = int(blockIdx.x);
  const int ti = id / rgroups;
  return TileRow{ti, id - ti * rgroups};
}

// RP > 1 (small compile-time worker counts): each workgroup takes RP rows of its tile, or
// RP flat chunks, and rgroups is the tile's row count over RP.
template <typename GT, int WT, int FP, int RP>
__device__ __forceinline__ void first_body(const UpdTile* __restrict__ tiles, int32_t ntiles, int32_t rgroups,
                                           const MatInfo* __restrict__ mats, const GT* __restrict__ G,
                                           float* __restrict__ E, const float* __restrict__ ebar,
                                           const float* __restrict__ Pprev, const float* __restrict__ Qprev,
                                           const float* __restrict__ Qin, float* __restrict__ Mbar,
                                           float* __restrict__ Ppart, int W, int64_t ld, int R, float inv_w,
                                           int offset_valid) {
  const TileRow tr = tile_row(rgroups);
  if (tr.tile >= ntiles) return;
  const UpdTile t = tiles[tr.tile];
  const int rb = tr.rb;
  if (t.mat < 0) {  // uncompressed tensor: the worker mean of G
    if (rb != 0) return;
    const int64_t c = t.begin + int64_t(threadIdx.x & 63) * 4;
    if (c < t.end) store4(Mbar + c, sum_g<4, GT, WT>(G, W, ld, c) * inv_w, t.end - c);
    return;
  }
  const MatInfo mi = mats[t.mat];
  if (mi.flat) {
    for (int rr = 0; rr < RP; ++rr)
      first_flat_tile<GT, WT, FP>(t, mi, G, E, ebar, Pprev, Qprev, Qin, Mbar, Ppart, W, ld, R, inv_w, offset_valid,
                                  rb * RP + rr);
    return;
  }
  if constexpr (RP > 1) {
    switch (mi.vw) {
      case 4: first_matrix_rows<4, GT, WT, FP, RP>(t, mi, G, E, ebar, Pprev, Qprev, Qin, Mbar, Ppart, ld, R, inv_w,
                                                 offset_valid, rb); break;
      case 2: first_matrix_rows<4, GT, WT, FP, RP, 2>(t, mi, G, E, ebar, Pprev, Qprev, Qin, Mbar, Ppart, ld, R,
                                                    inv_w, offset_valid, rb); break;
      default: first_matrix_rows<1, GT, WT, FP, RP>(t, mi, G, E, ebar, Pprev, Qprev, Qin, Mbar, Ppart, ld, R,
                                                  inv_w, offset_valid, rb); break;
    }
    return;
  }
  switch (mi.vw) {
    case 4: first_matrix_tile<4, GT, WT, FP>(t, mi, G, E, ebar, Pprev, Qprev, Qin, Mbar, Ppart, W, ld, R, inv_w,
                                     offset_valid, rb); break;
    case 2: first_matrix_tile<4, GT, WT, FP, 2>(t, mi, G, E, ebar, Pprev, Qprev, Qin, Mbar, Ppart, W, ld, R, inv_w,
                                     offset_valid, rb); break;
    default: first_matrix_tile<1, GT, WT, FP>(t, mi, G, E, ebar, Pprev, Qprev, Qin, Mbar, Ppart, W, ld, R, inv_w,
                                     offset_valid, rb); break;
  }
}

// Cross-step state (the carried error mean, or the deferred offset) is used when the
// host allows it (use_state: the plan's previous step ran on these buffers and nothing
// reset it since) and the workspace's state word holds this plan's key for this error
// buffer (written by the last pass of the step that left the state; cleared by
// in-place materialisation and by the stream-ordered reset).  The word is read on the
// device, so a step replayed from a captured graph still sees what happened between
// replays.  Without valid state, a carry-mode pass reads every error (the plain form)
// and a deferred-mode pass subtracts nothing.
__device__ __forceinline__ int state_valid(const uint64_t* state, uint64_t key, int use_state) {
  return use_state != 0 && state != nullptr && *state == key;
}

template <typename GT, int WT, int FP, int RP>
__global__ __launch_bounds__(kStreamThreads) void k_first(const UpdTile* __restrict__ tiles, int32_t ntiles,
                                                     int32_t rgroups, const MatInfo* __restrict__ mats,
                                                     const GT* __restrict__ G, float* __restrict__ E,
                                                     const float* __restrict__ ebar,
                                                     const float* __restrict__ Pprev,
                                                     const float* __restrict__ Qprev,
                                                     const float* __restrict__ Qin, float* __restrict__ Mbar,
                                                     float* __restrict__ Ppart, int W, int64_t ld, int R,
                                                     float inv_w, const uint64_t* __restrict__ state, uint64_t key,
                                                     int use_state) {
  const int valid = state_valid(state, key, use_state);
  if constexpr (FP == kFpCarry) {
    if (!valid) {
      first_body<GT, WT, kFpMean, RP>(tiles, ntiles, rgroups, mats, G, E, ebar, Pprev, Qprev, Qin, Mbar, Ppart, W,
                                      ld, R, inv_w, 0);
      return;
    }
  }
  first_body<GT, WT, FP, RP>(tiles, ntiles, rgroups, mats, G, E, ebar, Pprev, Qprev, Qin, Mbar, Ppart, W, ld, R,
                             inv_w, FP == kFpDefer ? valid : 0);
}

// One thread stores `value` into the workspace's state word (a plain vector store).
__global__ __launch_bounds__(64) void k_state_store(uint64_t* __restrict__ state, uint64_t value) {
  if (threadIdx.x == 0) *state = value;
}

// ------------------------------------------------------------------ extra power iterations
// P-bar partial row sums of Mbar Q for one row x the wave's column strip, exactly as the
// first pass forms them, but reading the stored Mbar (extra power iterations).
template <int V, int A = V>
__device__ __forceinline__ void pbar_mbar_tile(const UpdTile& t, const MatInfo& mi, const float* Mbar,
                                               const float* Qin, float* Ppart, int R) {
  const int cols = mi.cols;
  const int j = t.col_begin + int(threadIdx.x) * V;
  const bool active = j < cols;
  const bool hi = A == V || j + 4 <= cols;
  const int i = t.row_begin + int(blockIdx.y);
  if (i >= t.row_end) return;
  float qv[V][4];
  load_q_cols<V>(qv, Qin + mi.q_off, j, R, active, hi);
  float part[4] = {0.f, 0.f, 0.f, 0.f};
  if (active) {
    const vec_t<V> mb = ldv<V, A>(Mbar + mi.offset + int64_t(i) * cols + j, hi);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < V; ++q) s += lane(mb, q) * qv[q][k];
      part[k] = s;
    }
  }
  const int strip = t.col_begin / (kStreamThreads * V);
  float* prow = Ppart + mi.ppart_off + int64_t(strip) * mi.rows * R;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (k < R) {
      const float v = wave_sum(part[k]);
      if (threadIdx.x == 0) prow[int64_t(i) * R + k] = v;
    }
}

__global__ __launch_bounds__(kStreamThreads) void k_p_mbar(const UpdTile* __restrict__ tiles,
                                                           const MatInfo* __restrict__ mats,
                                                           const float* __restrict__ Mbar,
                                                           const float* __restrict__ Qin,
                                                           float* __restrict__ Ppart, int R) {
  const UpdTile t = tiles[blockIdx.x];
  if (t.mat < 0) return;
  const MatInfo mi = mats[t.mat];
  if (mi.flat) {
    const int64_t c0 = t.begin + int64_t(blockIdx.y) * kStreamTileElems;
    if (c0 >= t.end) return;
    const int64_t c = c0 + int64_t(threadIdx.x) * 4;
    const Flat4 f = flat4_at(mi, c);
    f4 mb = {0.f, 0.f, 0.f, 0.f};
    if (f.valid > 0) {
      mb = ldv<4>(Mbar + c);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (q >= f.valid) mb[q] = 0.f;
    }
    flat_pbar_partial(mi, f, mb, Qin + mi.q_off, Ppart, int((c0 - mi.offset) / kStreamTileElems), R);
    return;
  }
  switch (mi.vw) {
    case 4: pbar_mbar_tile<4>(t, mi, Mbar, Qin, Ppart, R); break;
    case 2: pbar_mbar_tile<4, 2>(t, mi, Mbar, Qin, Ppart, R); break;
    default: pbar_mbar_tile<1>(t, mi, Mbar, Qin, Ppart, R); break;
  }
}

// ------------------------------------------------------------------ Gram-Schmidt
// P-bar = sum over column strips of the partial row sums (fixed strip order), then
// modified Gram-Schmidt over its R columns in column order.  Dot products and norms
// accumulate in double; the working column is rounded to float after each
// projection.  A column whose residual norm is at most 1e-4 of its norm before
// orthogonalisation (or zero, or not a number) becomes exactly zero.  The norm of a
// fresh column and its projection on column 0 share one reduction (both use the
// unmodified column).
// Matrices with at most kMgsRowsPerThread rows per thread keep their rows in registers;
// taller ones go through their Gram matrix (below).  `P2`, if set, receives a copy of
// the result.

// Partial slots of row i: every column strip, or for a flat matrix the chunks the row
// overlaps.
__device__ __forceinline__ int pbar_slots(const MatInfo& mi, int i) {
  if (!mi.flat) return mi.nstrips;
  return ((i + 1) * mi.cols - 1) / kStreamTileElems - (i * mi.cols) / kStreamTileElems + 1;
}

// P-bar rows i_first + u * step for u < U (zero rows from n on): each the sum of its
// partial slots in slot order.  SU slots of all U rows are loaded at once, every load
// unconditional (a slot a row does not have reads the matrix's first partial instead and
// is not added), so that they overlap.
template <int R, int U>
__device__ __forceinline__ void pbar_rows(float (&acc)[U][R], const float* src, int64_t strip_stride,
                                          const MatInfo& mi, int i_first, int step, int n) {
  constexpr int SU = (U * R >= 16) ? 1 : 16 / (U * R);
  int ns[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = i_first + u * step;
    ns[u] = i < n ? pbar_slots(mi, i) : 0;
#pragma unroll
    for (int k = 0; k < R; ++k) acc[u][k] = 0.f;
  }
  for (int s0 = 0; s0 < mi.nstrips; s0 += SU) {
    float tmp[SU][U][R];
#pragma unroll
    for (int j = 0; j < SU; ++j)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float* row =
            (s0 + j < ns[u]) ? src + (s0 + j) * strip_stride + int64_t(i_first + u * step) * R : src;
#pragma unroll
        for (int k = 0; k < R; ++k) tmp[j][u][k] = row[k];
      }
#pragma unroll
    for (int j = 0; j < SU; ++j)
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (s0 + j < ns[u])
#pragma unroll
          for (int k = 0; k < R; ++k) acc[u][k] += tmp[j][u][k];
  }
}

// Gram-Schmidt of the columns of P-bar taken in its R x R Gram space (g: the packed
// upper triangle, entry (k, l), k <= l, at k R - k (k - 1) / 2 + l - k): column by
// column, the projection coefficients R_lk on the kept earlier columns and the residual
// norm sqrt(G_kk - sum_l R_lk^2), with the drop rule (a residual norm that is zero, not a
// number, or at most 1e-4 times the column's norm before orthogonalisation drops the
// column).  In exact arithmetic this is column-by-column modified Gram-Schmidt.  Writes
// T = R^-1 with zero columns for dropped columns, so that P = P-bar T.
template <int R>
__device__ __forceinline__ void gram_gs_coeffs(const double (&g)[R * (R + 1) / 2], double (&T)[R][R]) {
  auto G = [&](int k, int l) { return g[k * R - k * (k - 1) / 2 + (l - k)]; };
  double Rm[R][R];
  bool kept[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const double before = sqrt(G(k, k));
    double ss = G(k, k);
#pragma unroll
    for (int l = 0; l < k; ++l) {
      double r = 0.0;
      if (kept[l]) {
        r = G(l, k);
#pragma unroll
        for (int m = 0; m < l; ++m) r -= Rm[m][l] * Rm[m][k];
        r /= Rm[l][l];
      }
      Rm[l][k] = r;
      ss -= r * r;
    }
    const double after = sqrt(ss > 0.0 ? ss : 0.0);
    kept[k] = after > 0.0 && after > 1e-4 * before;
    Rm[k][k] = after;
#pragma unroll
    for (int l = 0; l < R; ++l) T[l][k] = 0.0;
    if (kept[k]) {
      T[k][k] = 1.0 / after;
#pragma unroll
      for (int l = 0; l < k; ++l)
#pragma unroll
        for (int m = 0; m < R; ++m) T[m][k] -= Rm[l][k] * T[m][l] / after;
    }
  }
}

template <int R>
__global__ __launch_bounds__(kMgsThreads) void k_mgs(const MatInfo* __restrict__ mats,
                                                     const float* __restrict__ Ppart,
                                                     float* __restrict__ P, float* __restrict__ P2,
                                                     const double* __restrict__ gpart,
                                                     double* __restrict__ tmat) {
  __shared__ double red[10 * (kMgsThreads / 64)];
  const MatInfo mi = mats[blockIdx.x];
  const float* src = Ppart + mi.ppart_off;
  float* dst = P + mi.p_off;
  const int n = mi.rows;
  const int64_t strip_stride = int64_t(n) * R;
  const int bs = blockDim.x;

  if (mi.tall_blk0 < 0) {
    // as many rows per thread as the matrix needs, so that a thread with one row has
    // more of that row's partial slots in flight
    float v[kMgsRowsPerThread][R];
    const int rpt = (n + bs - 1) / bs;
    if (rpt == 1) {
      float a[1][R];
      pbar_rows<R, 1>(a, src, strip_stride, mi, int(threadIdx.x), bs, n);
#pragma unroll
      for (int r = 0; r < kMgsRowsPerThread; ++r)
#pragma unroll
        for (int k = 0; k < R; ++k) v[r][k] = r == 0 ? a[0][k] : 0.f;
    } else if (rpt == 2) {
      float a[2][R];
      pbar_rows<R, 2>(a, src, strip_stride, mi, int(threadIdx.x), bs, n);
#pragma unroll
      for (int r = 0; r < kMgsRowsPerThread; ++r)
#pragma unroll
        for (int k = 0; k < R; ++k) v[r][k] = r < 2 ? a[r][k] : 0.f;
    } else {
      pbar_rows<R, kMgsRowsPerThread>(v, src, strip_stride, mi, int(threadIdx.x), bs, n);
    }
    // The R (R + 1) / 2 Gram entries of the rows in registers, summed over the
    // workgroup in one fixed-order reduction; every thread then derives the same
    // coefficients and applies them to its rows (terms with a zero coefficient are
    // skipped, so a dropped column, even one that is not a number, leaves no trace).
    constexpr int NG = R * (R + 1) / 2;
    double g[NG];
#pragma unroll
    for (int k = 0, a = 0; k < R; ++k)
#pragma unroll
      for (int l = k; l < R; ++l, ++a) {
        double t = 0.0;
#pragma unroll
        for (int r = 0; r < kMgsRowsPerThread; ++r) t += double(v[r][k]) * double(v[r][l]);
        g[a] = t;
      }
    block_sum_n<NG>(g, red);
    double T[R][R];
    gram_gs_coeffs<R>(g, T);
#pragma unroll
    for (int r = 0; r < kMgsRowsPerThread; ++r) {
      float o[R];
#pragma unroll
      for (int k = 0; k < R; ++k) {
        double t = 0.0;
#pragma unroll
        for (int l = 0; l <= k; ++l)
          if (T[l][k] != 0.0) t += double(v[r][l]) * T[l][k];
        o[k] = float(t);
      }
#pragma unroll
      for (int k = 0; k < R; ++k) v[r][k] = o[k];
    }
#pragma unroll
    for (int r = 0; r < kMgsRowsPerThread; ++r) {
      const int i = threadIdx.x + r * bs;
      if (i < n) {
#pragma unroll
        for (int k = 0; k < R; ++k) {
          dst[int64_t(i) * R + k] = v[r][k];
          if (P2 != nullptr) P2[mi.p_off + int64_t(i) * R + k] = v[r][k];
        }
      }
    }
    return;
  }

  // Tall matrices: k_tall_rows has written P-bar into the output and one Gram partial
  // (in double) per block of kTallRows rows.  The partials are summed in a fixed order;
  // one thread takes the same Gram-space Gram-Schmidt and stores T = R^-1 (zero columns
  // for dropped ones) for k_tall_apply, which writes P = P-bar T.
  constexpr int NG = R * (R + 1) / 2;
  double g[NG];
#pragma unroll
  for (int a = 0; a < NG; ++a) g[a] = 0.0;
  for (int b = int(threadIdx.x); b < mi.tall_nblk; b += bs)
#pragma unroll
    for (int a = 0; a < NG; ++a) g[a] += gpart[int64_t(mi.tall_blk0 + b) * 10 + a];
  block_sum_n<NG>(g, red);
  if (threadIdx.x == 0) {
    double T[R][R];
    gram_gs_coeffs<R>(g, T);
    double* out = tmat + int64_t(blockIdx.x) * 16;
    for (int l = 0; l < R; ++l)
      for (int k = 0; k < R; ++k) out[l * 4 + k] = T[l][k];
  }
}

// Row pass 1 of a tall matrix, one row per thread over blocks of kTallRows rows: P-bar
// rows into P and the block's Gram partial sum_i P-bar_i^T P-bar_i (upper triangle, in
// double; thread sums across the workgroup in a fixed order).
template <int R>
__global__ __launch_bounds__(kTallRows) void k_tall_rows(const TallBlk* __restrict__ tblks,
                                                         const MatInfo* __restrict__ mats,
                                                         const float* __restrict__ Ppart, float* __restrict__ P,
                                                         double* __restrict__ gpart) {
  constexpr int NG = R * (R + 1) / 2;
  __shared__ double red[kTallRows / 64][NG];
  const TallBlk tb = tblks[blockIdx.x];
  const MatInfo mi = mats[tb.mat];
  const int n = mi.rows;
  const int i = tb.blk * kTallRows + int(threadIdx.x);
  float acc[1][R];
  pbar_rows<R, 1>(acc, Ppart + mi.ppart_off, int64_t(n) * R, mi, i, 0, n);
  double g[NG];
  int a = 0;
#pragma unroll
  for (int k = 0; k < R; ++k) {
    if (i < n) P[mi.p_off + int64_t(i) * R + k] = acc[0][k];
#pragma unroll
    for (int l = k; l < R; ++l) g[a++] = double(acc[0][k]) * double(acc[0][l]);
  }
  const int ln = int(threadIdx.x) & 63, wave = int(threadIdx.x) >> 6;
#pragma unroll
  for (int b = 0; b < NG; ++b) {
    const double v = wave_sum(g[b]);
    if (ln == 0) red[wave][b] = v;
  }
  __syncthreads();
  if (int(threadIdx.x) < NG) {
    double s = 0.0;
    for (int w = 0; w < kTallRows / 64; ++w) s += red[w][threadIdx.x];
    gpart[int64_t(blockIdx.x) * 10 + threadIdx.x] = s;
  }
}

// Row pass 2 of a tall matrix: P = P-bar T (in double, l in order), and the copy in P2.
template <int R>
__global__ __launch_bounds__(kTallRows) void k_tall_apply(const TallBlk* __restrict__ tblks,
                                                          const MatInfo* __restrict__ mats,
                                                          const double* __restrict__ tmat, float* __restrict__ P,
                                                          float* __restrict__ P2) {
  const TallBlk tb = tblks[blockIdx.x];
  const MatInfo mi = mats[tb.mat];
  const int i = tb.blk * kTallRows + int(threadIdx.x);
  if (i >= mi.rows) return;
  const double* T = tmat + int64_t(tb.mat) * 16;
  float pb[R];
#pragma unroll
  for (int k = 0; k < R; ++k) pb[k] = P[mi.p_off + int64_t(i) * R + k];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    double v = 0.0;
#pragma unroll
    for (int l = 0; l <= k; ++l)
      if (T[l * 4 + k] != 0.0) v += double(pb[l]) * T[l * 4 + k];  // a dropped column leaves no trace
    const int64_t o = mi.p_off + int64_t(i) * R + k;
    P[o] = float(v);
    if (P2 != nullptr) P2[o] = float(v);
  }
}

// ------------------------------------------------------------------ Q = Mbar^T P
// One lane's four columns j..j+3 of the row-block partial: sum over rows r0..r1-1 of
// row(i) (four floats) times P[i, :].  hi false: the row ends at j + 2 (row(i) reads the
// upper two as zero) and only columns j, j + 1 are written.
template <int R, typename RowLoad>
__device__ __forceinline__ void q_cols4(float* out, const float* Pm, int r0, int r1, int j, bool hi,
                                        RowLoad row) {
  float acc[4][R];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int k = 0; k < R; ++k) acc[q][k] = 0.f;
#pragma unroll 8
  for (int i = r0; i < r1; ++i) {
    const f4 v = row(i);
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
    if (q < 2 || hi)
#pragma unroll
      for (int k = 0; k < R; ++k) out[int64_t(j + q) * R + k] = acc[q][k];
}
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
  if (mi.vw != 1) {
    const int j = t.col_begin + int(threadIdx.x) * 4;
    if (j >= t.col_end) return;
    const bool hi = j + 4 <= cols;
    if (mi.vw == 4)
      q_cols4<R>(out, Pm, r0, r1, j, true, [&](int i) { return ldv<4>(base + int64_t(i) * cols + j); });
    else
      q_cols4<R>(out, Pm, r0, r1, j, hi, [&](int i) { return ldv<4, 2>(base + int64_t(i) * cols + j, hi); });
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

// Q = sum of the row-block partials.  Workgroup (blockIdx.x, matrix blockIdx.y) takes
// 64 elements of Q, one per lane; its waves split the row blocks (wave w sums blocks w,
// w + waves, ... in order) and the first wave adds the waves' sums in wave order.  grid.z
// walks workers when reducing the per-worker Q_w partials (strides part_ws and q_ws
// between workers; both 0 for the Q pass over Mbar).
__global__ __launch_bounds__(64 * kQRedMaxWaves) void k_q_reduce(const MatInfo* __restrict__ mats,
                                                                 const float* __restrict__ Qpart,
                                                                 float* __restrict__ Q, float* __restrict__ Q2,
                                                                 int R, int64_t part_ws, int64_t q_ws) {
  __shared__ float red[kQRedMaxWaves][64];
  const MatInfo mi = mats[blockIdx.y];
  const int64_t n = int64_t(mi.cols) * R;
  if (int64_t(blockIdx.x) * 64 >= n) return;  // the whole workgroup
  const int ln = int(threadIdx.x) & 63, wave = int(threadIdx.x) >> 6, nw = int(blockDim.x) >> 6;
  const int64_t idx = int64_t(blockIdx.x) * 64 + ln;
  const float* part = Qpart + int64_t(blockIdx.z) * part_ws + mi.qpart_off;
  float s = 0.f;
  if (idx < n) {
#pragma unroll 8
    for (int b = wave; b < mi.nblk; b += nw) s += part[int64_t(b) * n + idx];
  }
  red[wave][ln] = s;
  __syncthreads();
  if (wave == 0 && idx < n) {
    float t = red[0][ln];
    for (int w = 1; w < nw; ++w) t += red[w][ln];
    Q[int64_t(blockIdx.z) * q_ws + mi.q_off + idx] = t;
    if (Q2 != nullptr) Q2[mi.q_off + idx] = t;
  }
}

// Per-worker Q partials for PSGD_FLAG_LOCAL_Q_ERROR: Q_w = (G_w + E_w)^T P, one worker
// per grid.y, over the same row blocks and column strips as the Q pass over Mbar.
template <int R, typename GT>
__global__ __launch_bounds__(kQThreads) void k_qw_partial(const QTile* __restrict__ tiles,
                                                          const MatInfo* __restrict__ mats,
                                                          const GT* __restrict__ G, const float* __restrict__ E,
                                                          int64_t ld, const float* __restrict__ P,
                                                          float* __restrict__ Qwpart, int64_t qpart_elems) {
  const QTile t = tiles[blockIdx.x];
  const int w = blockIdx.y;
  const MatInfo mi = mats[t.mat];
  const int cols = mi.cols;
  const int r0 = t.blk * mi.rows_per_blk;
  const int r1 = min(mi.rows, r0 + mi.rows_per_blk);
  const float* Pm = P + mi.p_off;
  const GT* gb = G + int64_t(w) * ld + mi.offset;
  const float* eb = E + int64_t(w) * ld + mi.offset;
  float* out = Qwpart + int64_t(w) * qpart_elems + mi.qpart_off + int64_t(t.blk) * cols * R;
  if (mi.vw != 1) {
    const int j = t.col_begin + int(threadIdx.x) * 4;
    if (j >= t.col_end) return;
    const bool hi = j + 4 <= cols;
    if (mi.vw == 4)
      q_cols4<R>(out, Pm, r0, r1, j, true, [&](int i) {
        const int64_t c = int64_t(i) * cols + j;
        return ld_nt<4>(gb + c) + ld_nt<4>(eb + c);
      });
    else
      q_cols4<R>(out, Pm, r0, r1, j, hi, [&](int i) {
        const int64_t c = int64_t(i) * cols + j;
        return ld_nt<4, 2>(gb + c, hi) + ld_nt<4, 2>(eb + c, hi);
      });
  } else {
    const int j = t.col_begin + int(threadIdx.x);
    if (j >= t.col_end) return;
    float acc[R];
#pragma unroll
    for (int k = 0; k < R; ++k) acc[k] = 0.f;
#pragma unroll 4
    for (int i = r0; i < r1; ++i) {
      const int64_t c = int64_t(i) * cols + j;
      const float v = ld_nt<1>(gb + c) + ld_nt<1>(eb + c);
#pragma unroll
      for (int k = 0; k < R; ++k) acc[k] += v * Pm[int64_t(i) * R + k];
    }
#pragma unroll
    for (int k = 0; k < R; ++k) out[int64_t(j) * R + k] = acc[k];
  }
}

// ------------------------------------------------------------------ pass 2 (eager modes)
// Matrix tile: u = P Q^T for the thread's columns of each row; E'_w = (G_w + E_w) - u
// on every worker, the mean of the stored E'_w into `ebar` (carry mode), U once, and
// the momentum-SGD update in the momentum modes.  1-D tensors: the update is the mean.
template <int V, typename GT, int WT, bool LOCAL, int A = V>
__device__ __forceinline__ void apply_matrix_tile(const UpdTile& t, const MatInfo& mi, const GT* G, float* E,
                                                  const float* P, const float* Q, const float* Qw, int64_t q_ws,
                                                  float* update, float* mom, float* x, float* ebar, int W,
                                                  int64_t ld, int R, int mode, float lr, float mu, float inv_w,
                                                  int rb) {
  const int cols = mi.cols;
  const int j = t.col_begin + (int(threadIdx.x) & 63) * V;
  if (j >= cols) return;
  const bool hi = A == V || j + 4 <= cols;
  float qv[V][4];
  load_q_cols<V>(qv, Q + mi.q_off, j, R, true, hi);
  {
    const int i = t.row_begin + rb;
    if (i >= t.row_end) return;
    float pr[4];
    load_p_row(pr, P + mi.p_off, i, R);
    const vec_t<V> u = pq_row<V>(pr, qv, R);
    const int64_t c = mi.offset + int64_t(i) * cols + j;
    vec_t<V> es;
    if constexpr (LOCAL)
      es = update_workers_local<V, GT, WT, A>(G, E, W, ld, c, pr, Qw, q_ws, mi.q_off, j, R, hi);
    else
      es = update_workers<V, GT, WT, A>(G, E, W, ld, c, u, hi);
    if (ebar != nullptr) st<V, A>(ebar + c, es * inv_w, hi);
    if (update != nullptr) st_nt<V, A>(update + c, u, hi);
    if (mode != kCompress) momentum_v<V, A>(mom, x, c, u, mode, lr, mu, hi);
  }
}

// The same for one flat chunk (chunk rb of the tile).
template <typename GT, int WT, bool LOCAL>
__device__ __forceinline__ void apply_flat_tile(const UpdTile& t, const MatInfo& mi, const GT* G, float* E,
                                                const float* P, const float* Q, const float* Qw, int64_t q_ws,
                                                float* update, float* mom, float* x, float* ebar, int W,
                                                int64_t ld, int R, int mode, float lr, float mu, float inv_w,
                                                int rb) {
  const int64_t c0 = t.begin + int64_t(rb) * kStreamTileElems;
  if (c0 >= t.end) return;
  const int64_t c = c0 + int64_t(threadIdx.x & 63) * 4;
  const Flat4 f = flat4_at(mi, c);
  if (f.valid == 0) return;
  float p0[4], p1[4];
  load_flat_p_rows(p0, p1, P + mi.p_off, f, R);
  const f4 u = pq_flat(p0, p1, Q + mi.q_off, f, R);
  f4 es;
  if constexpr (LOCAL)
    es = update_workers_local_flat<GT, WT>(G, E, W, ld, c, p0, p1, Qw, q_ws, mi.q_off, f, R);
  else
    es = f.valid == 4 ? update_workers<4, GT, WT>(G, E, W, ld, c, u)
                      : update_workers_tail<GT>(G, E, W, ld, c, u, f.valid);
  if (f.valid == 4) {
    if (ebar != nullptr) st<4>(ebar + c, es * inv_w);
    if (update != nullptr) st_nt<4>(update + c, u);
    if (mode != kCompress) momentum_v<4>(mom, x, c, u, mode, lr, mu);
  } else {
    if (ebar != nullptr) store4(ebar + c, es * inv_w, f.valid);
    if (update != nullptr) store4_nt(update + c, u, f.valid);
    if (mode != kCompress) momentum_masked(mom, x, c, u, f.valid, mode, lr, mu);
  }
}

template <typename GT, int WT, bool LOCAL>
__global__ __launch_bounds__(kStreamThreads) void k_apply(
    const UpdTile* __restrict__ tiles, int32_t ntiles, int32_t rgroups, const MatInfo* __restrict__ mats,
    const GT* __restrict__ G,
    float* __restrict__ E, const float* __restrict__ Mbar, const float* __restrict__ P,
    const float* __restrict__ Q, const float* __restrict__ Qw, int64_t q_ws, float* __restrict__ update,
    float* __restrict__ mom, float* __restrict__ x, float* __restrict__ ebar, int W, int64_t ld, int R, int mode,
    float lr, float mu, float inv_w, uint64_t* __restrict__ state, uint64_t key) {
  if (state != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *state = key;
  const TileRow tr = tile_row(rgroups);
  if (tr.tile >= ntiles) return;
  const UpdTile t = tiles[tr.tile];
  const int rb = tr.rb;
  if (t.mat < 0) {
    if (rb != 0) return;
    const int64_t c = t.begin + int64_t(threadIdx.x & 63) * 4;
    if (c >= t.end) return;
    const int64_t valid = t.end - c;
    const f4 uv = *reinterpret_cast<const f4*>(Mbar + c);
    if (update != nullptr) store4_nt(update + c, uv, valid);
    if (mode != kCompress) momentum_masked(mom, x, c, uv, valid, mode, lr, mu);
    return;
  }
  const MatInfo mi = mats[t.mat];
  if (mi.flat) {
    apply_flat_tile<GT, WT, LOCAL>(t, mi, G, E, P, Q, Qw, q_ws, update, mom, x, ebar, W, ld, R, mode, lr, mu, inv_w,
                                   rb);
    return;
  }
  switch (mi.vw) {
    case 4: apply_matrix_tile<4, GT, WT, LOCAL>(t, mi, G, E, P, Q, Qw, q_ws, update, mom, x, ebar, W, ld, R, mode, lr, mu, inv_w, rb); break;
    case 2: apply_matrix_tile<4, GT, WT, LOCAL, 2>(t, mi, G, E, P, Q, Qw, q_ws, update, mom, x, ebar, W, ld, R, mode, lr, mu, inv_w, rb); break;
    default: apply_matrix_tile<1, GT, WT, LOCAL>(t, mi, G, E, P, Q, Qw, q_ws, update, mom, x, ebar, W, ld, R, mode, lr, mu, inv_w, rb); break;
  }
}

// ------------------------------------------------------------------ deferred-error mode
// The error buffer holds M_w = G_w + E_w of the previous step instead of E'_w; the true
// error is that minus the previous step's P Q^T (kept in the workspace).  k_first
// (kFpDefer) folds that subtraction into this step's EF add:
// M_w(t) = G_w(t) + [M_w(t-1) - U(t-1)], stores M_w(t) back and writes Mbar.
// k_update is the last pass: the decompressed update (P Q^T, or the mean for 1-D
// tensors) and the momentum-SGD update; no worker data is touched.
template <int V, int A = V>
__device__ __forceinline__ void update_matrix_tile(const UpdTile& t, const MatInfo& mi, const float* P,
                                                   const float* Q, float* update, float* mom, float* x, int R,
                                                   int mode, float lr, float mu) {
  const int cols = mi.cols;
  const int j = t.col_begin + int(threadIdx.x) * V;
  if (j >= cols) return;
  const bool hi = A == V || j + 4 <= cols;
  float qv[V][4];
  load_q_cols<V>(qv, Q + mi.q_off, j, R, true, hi);
  for (int i = t.row_begin; i < t.row_end; ++i) {
    float pr[4];
    load_p_row(pr, P + mi.p_off, i, R);
    const vec_t<V> u = pq_row<V>(pr, qv, R);
    const int64_t c = mi.offset + int64_t(i) * cols + j;
    if (update != nullptr) st_nt<V, A>(update + c, u, hi);
    if (mode != kCompress) momentum_v<V, A>(mom, x, c, u, mode, lr, mu, hi);
  }
}

// The same over a flat run: kUpdFlatRuns chunks of kUpdThreads * 4 elements.  A lane's
// next element position is its previous one moved on by the chunk length (one integer
// division per lane in all).
__device__ __forceinline__ void update_flat_tile(const UpdTile& t, const MatInfo& mi, const float* P,
                                                 const float* Q, float* update, float* mom, float* x, int R,
                                                 int mode, float lr, float mu) {
  constexpr int kStep = kUpdThreads * 4;
  const int dq = kStep / mi.cols, dr = kStep - dq * mi.cols;
  const int64_t numel = int64_t(mi.rows) * mi.cols;
  Flat4 f = flat4_at(mi, t.begin + int64_t(threadIdx.x) * 4);
  for (int64_t c = t.begin + int64_t(threadIdx.x) * 4; c < t.end; c += kStep) {
    if (c != t.begin + int64_t(threadIdx.x) * 4) {
      int j = f.j0 + dr, i = f.i0 + dq;
      if (j >= mi.cols) {
        j -= mi.cols;
        ++i;
      }
      f.i0 = i;
      f.j0 = j;
      f.nw = min(4, mi.cols - j);
      f.valid = int(min<int64_t>(4, numel - (c - mi.offset)));
    }
    float p0[4], p1[4];
    load_flat_p_rows(p0, p1, P + mi.p_off, f, R);
    const f4 u = pq_flat(p0, p1, Q + mi.q_off, f, R);
    if (f.valid == 4) {
      if (update != nullptr) st_nt<4>(update + c, u);
      if (mode != kCompress) momentum_v<4>(mom, x, c, u, mode, lr, mu);
    } else {
      if (update != nullptr) store4_nt(update + c, u, f.valid);
      if (mode != kCompress) momentum_masked(mom, x, c, u, f.valid, mode, lr, mu);
    }
  }
}

template <int R>
__global__ __launch_bounds__(kUpdThreads) void k_update(
    const UpdTile* __restrict__ tiles, const MatInfo* __restrict__ mats, const float* __restrict__ Mbar,
    const float* __restrict__ P, const float* __restrict__ Q, float* __restrict__ update,
    float* __restrict__ mom, float* __restrict__ x, int mode, float lr, float mu, uint64_t* __restrict__ state,
    uint64_t key) {
  if (state != nullptr && blockIdx.x == 0 && threadIdx.x == 0) *state = key;
  const UpdTile t = tiles[blockIdx.x];
  if (t.mat < 0) {
    const int64_t c = t.begin + int64_t(threadIdx.x) * 4;
    if (c >= t.end) return;
    const int64_t valid = t.end - c;
    const f4 uv = *reinterpret_cast<const f4*>(Mbar + c);
    if (update != nullptr) store4_nt(update + c, uv, valid);
    if (mode != kCompress) momentum_masked(mom, x, c, uv, valid, mode, lr, mu);
    return;
  }
  const MatInfo mi = mats[t.mat];
  if (mi.flat) {
    update_flat_tile(t, mi, P, Q, update, mom, x, R, mode, lr, mu);
    return;
  }
  switch (mi.vw) {
    case 4: update_matrix_tile<4>(t, mi, P, Q, update, mom, x, R, mode, lr, mu); break;
    case 2: update_matrix_tile<4, 2>(t, mi, P, Q, update, mom, x, R, mode, lr, mu); break;
    default: update_matrix_tile<1>(t, mi, P, Q, update, mom, x, R, mode, lr, mu); break;
  }
}

// out_w = errors_w - P_prev Q_prev^T for every compressed matrix (the plain error memory
// of a deferred-mode error buffer), on the worker-pass tiles; 1-D tensors are skipped.
// The subtracted value is computed exactly as the first pass subtracts it.  E and out
// may alias.
template <int V, int A = V>
__device__ __forceinline__ void materialize_tile(const UpdTile& t, const MatInfo& mi, const float* E, float* out,
                                                 const float* Pprev, const float* Qprev, int W, int64_t ld, int R,
                                                 int offset_valid) {
  const int cols = mi.cols;
  const int j = t.col_begin + int(threadIdx.x) * V;
  if (j >= cols) return;
  const bool hi = A == V || j + 4 <= cols;
  float qp[V][4];
  load_q_cols<V>(qp, Qprev + mi.q_off, j, R, offset_valid != 0, hi);
  {
    const int i = t.row_begin + int(blockIdx.y);
    if (i >= t.row_end) return;
    float pp[4] = {0.f, 0.f, 0.f, 0.f};
    if (offset_valid) load_p_row(pp, Pprev + mi.p_off, i, R);
    const vec_t<V> up = pq_row<V>(pp, qp, R);
    const int64_t c = mi.offset + int64_t(i) * cols + j;
    for (int w = 0; w < W; ++w) st_nt<V, A>(out + w * ld + c, ld_nt<V, A>(E + w * ld + c, hi) - up, hi);
  }
}

// The same for one flat chunk.
__device__ __forceinline__ void materialize_flat_tile(const UpdTile& t, const MatInfo& mi, const float* E,
                                                      float* out, const float* Pprev, const float* Qprev, int W,
                                                      int64_t ld, int R, int offset_valid) {
  const int64_t c0 = t.begin + int64_t(blockIdx.y) * kStreamTileElems;
  if (c0 >= t.end) return;
  const int64_t c = c0 + int64_t(threadIdx.x) * 4;
  const Flat4 f = flat4_at(mi, c);
  if (f.valid == 0) return;
  f4 up = {0.f, 0.f, 0.f, 0.f};
  if (offset_valid) {
    float p0[4], p1[4];
    load_flat_p_rows(p0, p1, Pprev + mi.p_off, f, R);
    up = pq_flat(p0, p1, Qprev + mi.q_off, f, R);
  }
  for (int w = 0; w < W; ++w) {
    const f4 v = ld_nt<4>(E + w * ld + c) - up;
    if (f.valid == 4)
      st_nt<4>(out + w * ld + c, v);
    else
      store4_nt(out + w * ld + c, v, f.valid);
  }
}

__global__ __launch_bounds__(kStreamThreads) void k_materialize(
    const UpdTile* __restrict__ tiles, const MatInfo* __restrict__ mats, const float* E, float* out,
    const float* __restrict__ Pprev, const float* __restrict__ Qprev, int W, int64_t ld, int R,
    const uint64_t* __restrict__ state, uint64_t key, int use_state) {
  const int offset_valid = state_valid(state, key, use_state);
  const UpdTile t = tiles[blockIdx.x];
  if (t.mat < 0) return;
  const MatInfo mi = mats[t.mat];
  if (mi.flat) {
    materialize_flat_tile(t, mi, E, out, Pprev, Qprev, W, ld, R, offset_valid);
    return;
  }
  switch (mi.vw) {
    case 4: materialize_tile<4>(t, mi, E, out, Pprev, Qprev, W, ld, R, offset_valid); break;
    case 2: materialize_tile<4, 2>(t, mi, E, out, Pprev, Qprev, W, ld, R, offset_valid); break;
    default: materialize_tile<1>(t, mi, E, out, Pprev, Qprev, W, ld, R, offset_valid); break;
  }
}

// ------------------------------------------------------------------ calibration copy
__global__ __launch_bounds__(256) void k_stream_copy(const float* __restrict__ src, float* __restrict__ dst,
                                                     int64_t n4) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n4; i += int64_t(gridDim.x) * 256)
    __builtin_nontemporal_store(ld_nt<4>(src + 4 * i), reinterpret_cast<f4*>(dst + 4 * i));
}

// ------------------------------------------------------------------ host helpers
psgd_status hip_fail(const char* what, hipError_t e) {
  set_error(std::string(what) + ": " + hipGetErrorString(e));
  return PSGD_ERR_HIP;
}

uint64_t align256(uint64_t x) { return (x + 255) / 256 * 256; }

// Layout of the plan's device tables from `base` (each table 256-byte aligned); returns
// their total size in bytes.  base may be null to only measure.
uint64_t layout_tables(const psgd_plan* plan, char* base, DeviceTables* t) {
  const uint64_t b_mats = align256(plan->mats.size() * sizeof(MatInfo) + 1);
  const uint64_t b_rt = align256(plan->s2tiles.size() * sizeof(UpdTile) + 1);
  const uint64_t b_qt = align256(plan->qtiles.size() * sizeof(QTile) + 1);
  const uint64_t b_ut = align256(plan->utiles.size() * sizeof(UpdTile) + 1);
  const uint64_t b_tb = align256(plan->tblks.size() * sizeof(TallBlk) + 1);
  if (t != nullptr) {
    t->base = base;
    t->mats = reinterpret_cast<MatInfo*>(base);
    t->s2tiles = reinterpret_cast<UpdTile*>(base + b_mats);
    t->qtiles = reinterpret_cast<QTile*>(base + b_mats + b_rt);
    t->utiles = reinterpret_cast<UpdTile*>(base + b_mats + b_rt + b_qt);
    t->tblks = reinterpret_cast<TallBlk*>(base + b_mats + b_rt + b_qt + b_ut);
  }
  return b_mats + b_rt + b_qt + b_ut + b_tb;
}

// Copy the plan's host tables to the device tables t: synchronously (stream null) or
// enqueued on `st`.
psgd_status copy_tables(const psgd_plan* plan, const DeviceTables& t, bool async, hipStream_t st) {
  struct {
    void* dst;
    const void* src;
    size_t bytes;
  } copies[] = {
      {t.mats, plan->mats.data(), plan->mats.size() * sizeof(MatInfo)},
      {t.s2tiles, plan->s2tiles.data(), plan->s2tiles.size() * sizeof(UpdTile)},
      {t.qtiles, plan->qtiles.data(), plan->qtiles.size() * sizeof(QTile)},
      {t.utiles, plan->utiles.data(), plan->utiles.size() * sizeof(UpdTile)},
      {t.tblks, plan->tblks.data(), plan->tblks.size() * sizeof(TallBlk)},
  };
  for (const auto& c : copies) {
    if (c.bytes == 0) continue;
    const hipError_t e = async ? hipMemcpyAsync(c.dst, c.src, c.bytes, hipMemcpyHostToDevice, st)
                               : hipMemcpy(c.dst, c.src, c.bytes, hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail("copy of the plan's device tables", e);
  }
  return PSGD_OK;
}

psgd_status ensure_tables(psgd_plan* plan, DeviceTables** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("hipGetDevice", e);
  auto it = plan->dev.find(dev);
  if (it != plan->dev.end()) {
    *out = &it->second;
    return PSGD_OK;
  }
  void* base = nullptr;
  e = hipMalloc(&base, layout_tables(plan, nullptr, nullptr));
  if (e != hipSuccess) {
    set_error(std::string("hipMalloc of the plan's device tables: ") + hipGetErrorString(e));
    return PSGD_ERR_NO_MEMORY;
  }
  DeviceTables t;
  layout_tables(plan, static_cast<char*>(base), &t);
  const psgd_status s = copy_tables(plan, t, false, nullptr);
  if (s != PSGD_OK) {
    (void)hipFree(base);
    return s;
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

// Launch `kernel` on `st`.  With timing enabled the launch goes through
// hipExtLaunchKernelGGL with a start and a stop event, which the runtime records with
// the kernel's own dispatch, so the elapsed time is the kernel's execution alone.
template <typename... KArgs, typename... Args>
psgd_status launch_k(psgd_plan* plan, int kid, void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t st,
                     Args... args) {
  hipEvent_t a = nullptr, b = nullptr;
  if (plan->timing) {
    psgd_status s = take_event(plan, &a);
    if (s == PSGD_OK) s = take_event(plan, &b);
    if (s != PSGD_OK) {
      if (a) plan->event_pool.push_back(a);
      return s;
    }
    hipExtLaunchKernelGGL(kernel, grid, block, 0, st, a, b, 0, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
  }
  const hipError_t e = hipGetLastError();
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
  float* Ppart;
  float* Qpart;
  double* gpart;         // tall matrices: per-block Gram partials and per-matrix T
  double* tmat;
  const float* ebar_in;  // carried error mean to read (carry mode, when the state is valid)
  float* ebar_out;       // error mean to write (carry mode)
  float* Pprev;          // previous P, Q (deferred mode)
  float* Qprev;
  float* Qwpart;         // per-worker Q partials and Q_w (local-Q error), else null
  float* Qw;
  int64_t q_ws;          // floats between workers' Q_w
  uint64_t* state;       // workspace state word (carry and deferred modes), else null
  uint64_t key;          // this plan's key for these errors
  int use_state;         // host allows the cross-step state (same buffers, not reset)
  int W, R, mode;
  int64_t ld;
  unsigned n_s2;  // worker-pass tiles
  unsigned rows_per_tile;  // grid.y of the worker passes: one workgroup per row of a tile
  hipStream_t st;
};

enum PassKind { kPassFirst = 0, kPassApply = 1 };

// One wave per workgroup (measured: four waves per workgroup were no faster at W = 4 or
// 8), one workgroup per (tile, row group); k_first takes first_pass_rows rows per group.
inline dim3 pass_grid(int32_t ntiles, int32_t rgroups) {
  if (uint64_t(ntiles) * uint64_t(rgroups) * kStreamThreads <= uint64_t(UINT32_MAX))
    return dim3(unsigned(ntiles) * unsigned(rgroups));
  return dim3(unsigned(ntiles), unsigned(rgroups));
}

template <typename GT, int WT>
psgd_status launch_pass(psgd_plan* plan, int which, int fp, const DeviceTables& dt, const StepArgs& a) {
  const GT* g = static_cast<const GT*>(a.grads);
  const int32_t ntiles = int32_t(a.n_s2);
  const dim3 block(kStreamThreads);
  if (which == kPassApply) {
    const int32_t rgroups = int32_t(a.rows_per_tile);
    return launch_k(plan, kKApply, a.Qw != nullptr ? k_apply<GT, WT, true> : k_apply<GT, WT, false>,
                    pass_grid(ntiles, rgroups), block, a.st, dt.s2tiles, ntiles, rgroups, dt.mats, g,
                    a.errors, a.Mbar, a.p, a.q, static_cast<const float*>(a.Qw), a.q_ws, a.update, a.mom, a.x,
                    a.ebar_out, a.W, a.ld, a.R, a.mode, a.lr, a.mu, a.inv_w, a.ebar_out != nullptr ? a.state : nullptr,
                    a.key);
  }
  constexpr int RP = WT > 0 ? first_pass_rows(WT, std::is_same<GT, bf16>::value) : 1;
  const int32_t rgroups = int32_t((a.rows_per_tile + RP - 1) / RP);
  auto first = fp == kFpDefer   ? k_first<GT, WT, kFpDefer, RP>
               : fp == kFpCarry ? k_first<GT, WT, kFpCarry, RP>
                                : k_first<GT, WT, kFpMean, RP>;
  return launch_k(plan, kKFirst, first, pass_grid(ntiles, rgroups), block, a.st, dt.s2tiles, ntiles,
                  rgroups, dt.mats, g, a.errors, a.ebar_in, a.Pprev, a.Qprev, a.q, a.Mbar, a.Ppart, a.W, a.ld, a.R,
                  a.inv_w, static_cast<const uint64_t*>(a.state), a.key, a.use_state);
}

// Worker-count specialisations of the worker passes: W in {1,2,4,8,16} unrolls fully,
// anything else takes the generic loop.
template <typename GT>
psgd_status launch_pass_w(psgd_plan* plan, int which, int fp, const DeviceTables& dt, const StepArgs& a) {
  switch (a.W) {
    case 1: return launch_pass<GT, 1>(plan, which, fp, dt, a);
    case 2: return launch_pass<GT, 2>(plan, which, fp, dt, a);
    case 4: return launch_pass<GT, 4>(plan, which, fp, dt, a);
    case 8: return launch_pass<GT, 8>(plan, which, fp, dt, a);
    case 16: return launch_pass<GT, 16>(plan, which, fp, dt, a);
    default: return launch_pass<GT, 0>(plan, which, fp, dt, a);
  }
}

template <int R>
psgd_status launch_all(psgd_plan* plan, const DeviceTables& dt, const StepArgs& a) {
  const bool deferred = (plan->flags & PSGD_FLAG_DEFERRED_ERROR) != 0;
  const int fp = deferred ? kFpDefer : (a.ebar_in != nullptr ? kFpCarry : kFpMean);  // carry: decided on device
  const bool bf = plan->dtype == PSGD_BF16;
  const unsigned n_mats = unsigned(plan->mats.size());
  hipStream_t stream = a.st;
  psgd_status s;
  auto pass = [&](int which) {
    return bf ? launch_pass_w<bf16>(plan, which, fp, dt, a) : launch_pass_w<float>(plan, which, fp, dt, a);
  };
  const unsigned qred_gx = unsigned((plan->max_q_elems_per_matrix + 63) / 64);
  const dim3 qred_block(unsigned(64 * plan->qred_waves));

  if ((s = pass(kPassFirst)) != PSGD_OK) return s;
  // Each round: orthonormalise P-bar, Q = Mbar^T P; rounds after the first recompute
  // the P-bar partials from the stored Mbar and the Q of the previous round.
  for (int round = 0; n_mats > 0 && round < plan->power_iterations; ++round) {
    if (round > 0) {
      s = launch_k(plan, kKPMbar, k_p_mbar, dim3(a.n_s2, a.rows_per_tile), dim3(kStreamThreads), stream,
                   dt.s2tiles, dt.mats, static_cast<const float*>(a.Mbar), static_cast<const float*>(a.q),
                   a.Ppart, R);
      if (s != PSGD_OK) return s;
    }
    const unsigned n_tall = unsigned(plan->tblks.size());
    if (n_tall > 0) {
      s = launch_k(plan, kKTallRows, k_tall_rows<R>, dim3(n_tall), dim3(kTallRows), stream, dt.tblks, dt.mats,
                   static_cast<const float*>(a.Ppart), a.p, a.gpart);
      if (s != PSGD_OK) return s;
    }
    s = launch_k(plan, kKMgs, k_mgs<R>, dim3(n_mats), dim3(plan->mgs_threads), stream, dt.mats,
                 static_cast<const float*>(a.Ppart), a.p, deferred ? a.Pprev : nullptr,
                 static_cast<const double*>(a.gpart), a.tmat);
    if (s != PSGD_OK) return s;
    if (n_tall > 0) {
      s = launch_k(plan, kKTallApply, k_tall_apply<R>, dim3(n_tall), dim3(kTallRows), stream, dt.tblks, dt.mats,
                   static_cast<const double*>(a.tmat), a.p, deferred ? a.Pprev : nullptr);
      if (s != PSGD_OK) return s;
    }
    s = launch_k(plan, kKQPartial, k_q_partial<R>, dim3(unsigned(plan->qtiles.size())), dim3(kQThreads), stream,
                 dt.qtiles, dt.mats, static_cast<const float*>(a.Mbar), static_cast<const float*>(a.p), a.Qpart);
    if (s != PSGD_OK) return s;
    s = launch_k(plan, kKQReduce, k_q_reduce, dim3(qred_gx, n_mats), qred_block, stream, dt.mats,
                 static_cast<const float*>(a.Qpart), a.q, deferred ? a.Qprev : nullptr, R, int64_t(0), int64_t(0));
    if (s != PSGD_OK) return s;
  }
  if (a.Qw != nullptr && n_mats > 0) {  // local-Q error: every worker's own Q_w = (G_w + E_w)^T P
    const dim3 qg(unsigned(plan->qtiles.size()), unsigned(a.W));
    if (bf)
      s = launch_k(plan, kKQwPartial, k_qw_partial<R, bf16>, qg, dim3(kQThreads), stream, dt.qtiles, dt.mats,
                   static_cast<const bf16*>(a.grads), static_cast<const float*>(a.errors), a.ld,
                   static_cast<const float*>(a.p), a.Qwpart, plan->qpart_elems);
    else
      s = launch_k(plan, kKQwPartial, k_qw_partial<R, float>, qg, dim3(kQThreads), stream, dt.qtiles, dt.mats,
                   static_cast<const float*>(a.grads), static_cast<const float*>(a.errors), a.ld,
                   static_cast<const float*>(a.p), a.Qwpart, plan->qpart_elems);
    if (s != PSGD_OK) return s;
    s = launch_k(plan, kKQwReduce, k_q_reduce, dim3(qred_gx, n_mats, unsigned(a.W)), qred_block, stream, dt.mats,
                 static_cast<const float*>(a.Qwpart), a.Qw, static_cast<float*>(nullptr), R, plan->qpart_elems,
                 a.q_ws);
    if (s != PSGD_OK) return s;
  }
  if (deferred)
    return launch_k(plan, kKUpdate, k_update<R>, dim3(unsigned(plan->utiles.size())), dim3(kUpdThreads), stream,
                    dt.utiles, dt.mats, static_cast<const float*>(a.Mbar), static_cast<const float*>(a.p),
                    static_cast<const float*>(a.q), a.update, a.mom, a.x, a.mode, a.lr, a.mu, a.state, a.key);
  return pass(kPassApply);
}

// Same device, same error and workspace buffers as the step that left the state.
bool state_matches(const psgd_plan* plan, const void* errors, const void* workspace, int dev) {
  return plan->state_valid && plan->state_errors == errors && plan->state_workspace == workspace &&
         plan->state_device == dev;
}

// The value the workspace's state word holds while `errors` carries this plan's
// cross-step state: the plan's random nonce mixed with the buffer address (the
// splitmix64 finaliser), never 0, the cleared value.
uint64_t state_key(const psgd_plan* plan, const void* errors) {
  uint64_t z = plan->nonce ^ (uint64_t(reinterpret_cast<uintptr_t>(errors)) * 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return (z ^ (z >> 31)) | 1u;
}

bool stream_capturing(hipStream_t st) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(st, &cs) == hipSuccess && cs == hipStreamCaptureStatusActive;
}

// A call captured into a graph keeps the host's decision (use the state or not) for every
// replay.  Captured without the state, replays would never use the state that earlier
// replays leave, so such a capture is refused: capture only after an eager step of the
// plan on the same buffers.
psgd_status check_capture(const char* fn, bool needs_state, bool use_state, hipStream_t st) {
  if (needs_state && !use_state && stream_capturing(st)) {
    set_error(std::string(fn) + ": a carry or deferred plan can be captured into a graph only after an eager "
              "step of the plan on the same errors and workspace");
    return PSGD_ERR_INVALID_ARG;
  }
  return PSGD_OK;
}

// Device tables supplied by the caller instead of the plan's own: `tables` holds the
// plan's tables when *owner == nonce, else they are copied there on the step's stream
// (after the arguments are checked) and *owner becomes nonce.
struct TableSlot {
  DeviceTables tables;
  uint64_t* owner;
};

// slot: NULL for the plan's own tables (uploaded on its first step on a device).
psgd_status run_step(const char* fn, psgd_plan* plan, const void* grads, float* errors, float* q,
                     float* p, float* update, float* mom, float* x, float lr, float mu, void* workspace,
                     void* stream, int mode, TableSlot* slot = nullptr) {
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

  int dev = 0;
  hipError_t he = hipGetDevice(&dev);
  if (he != hipSuccess) return hip_fail("hipGetDevice", he);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const bool carry = (plan->flags & PSGD_FLAG_CARRY_ERROR_MEAN) != 0;
  const bool deferred = (plan->flags & PSGD_FLAG_DEFERRED_ERROR) != 0;
  const bool cross = (carry || deferred) && has_mats;
  // Cross-step state (carried error mean, or the deferred offset) may be used only if the
  // previous step of this plan left it on this device in these error/workspace buffers;
  // the kernels also check the workspace's state word.
  const bool use_state = cross && state_matches(plan, errors, workspace, dev);
  if ((s = check_capture(fn, cross, use_state, st)) != PSGD_OK) return s;
  DeviceTables* dt = nullptr;
  if (slot == nullptr) {
    if ((s = ensure_tables(plan, &dt)) != PSGD_OK) return s;
  } else {
    dt = &slot->tables;
    if (*slot->owner != plan->nonce) {
      *slot->owner = 0;
      if ((s = copy_tables(plan, *dt, true, st)) != PSGD_OK) return s;
      *slot->owner = plan->nonce;
    }
  }
  char* ws = static_cast<char*>(workspace);
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
  a.Ppart = reinterpret_cast<float*>(ws + plan->ws_ppart);
  a.Qpart = reinterpret_cast<float*>(ws + plan->ws_qpart);
  a.gpart = reinterpret_cast<double*>(ws + plan->ws_gpart);
  a.tmat = reinterpret_cast<double*>(ws + plan->ws_tmat);
  a.ebar_out = carry ? reinterpret_cast<float*>(ws + plan->ws_ebar) : nullptr;
  a.ebar_in = a.ebar_out;
  a.Pprev = deferred ? reinterpret_cast<float*>(ws + plan->ws_pprev) : nullptr;
  a.Qprev = deferred ? reinterpret_cast<float*>(ws + plan->ws_qprev) : nullptr;
  a.state = cross ? reinterpret_cast<uint64_t*>(ws + plan->ws_state) : nullptr;
  a.key = state_key(plan, errors);
  a.use_state = use_state ? 1 : 0;
  const bool local_q = (plan->flags & PSGD_FLAG_LOCAL_Q_ERROR) != 0;
  a.Qwpart = local_q ? reinterpret_cast<float*>(ws + plan->ws_qwpart) : nullptr;
  a.Qw = local_q ? reinterpret_cast<float*>(ws + plan->ws_qw) : nullptr;
  a.q_ws = plan->q_elems;
  a.W = plan->n_workers;
  a.R = plan->rank;
  a.mode = mode;
  a.ld = plan->worker_stride;
  a.n_s2 = unsigned(plan->s2tiles.size());
  a.rows_per_tile = unsigned(plan->worker_rows_per_tile);
  a.st = st;
  switch (plan->rank) {
    case 1: s = launch_all<1>(plan, *dt, a); break;
    case 2: s = launch_all<2>(plan, *dt, a); break;
    case 3: s = launch_all<3>(plan, *dt, a); break;
    case 4: s = launch_all<4>(plan, *dt, a); break;
    default:
      set_error(std::string(fn) + ": rank outside 1..4");
      return PSGD_ERR_UNSUPPORTED;
  }
  if (s == PSGD_OK && cross) {
    plan->state_valid = true;
    plan->state_errors = errors;
    plan->state_workspace = workspace;
    plan->state_device = dev;
  }
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
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("hipGetDevice", e);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const bool deferred = (plan->flags & PSGD_FLAG_DEFERRED_ERROR) != 0;
  // The host rules out a subtraction when the plan's last step did not run on these
  // buffers (or was reset); otherwise the kernel reads the workspace's state word.
  const bool use_state = deferred && state_matches(plan, errors, workspace, dev);
  if (!use_state && out == errors) return PSGD_OK;  // already plain, nothing to write
  if ((s = check_capture(fn, deferred, use_state, st)) != PSGD_OK) return s;
  DeviceTables* dt = nullptr;
  if ((s = ensure_tables(plan, &dt)) != PSGD_OK) return s;
  char* ws = static_cast<char*>(workspace);
  const float* Pprev = deferred ? reinterpret_cast<const float*>(ws + plan->ws_pprev) : nullptr;
  const float* Qprev = deferred ? reinterpret_cast<const float*>(ws + plan->ws_qprev) : nullptr;
  uint64_t* state = deferred ? reinterpret_cast<uint64_t*>(ws + plan->ws_state) : nullptr;
  hipLaunchKernelGGL(k_materialize, dim3(unsigned(plan->s2tiles.size()), unsigned(plan->worker_rows_per_tile)),
                     dim3(kStreamThreads), 0, st, dt->s2tiles, dt->mats, errors, out, Pprev, Qprev,
                     plan->n_workers, plan->worker_stride, plan->rank, static_cast<const uint64_t*>(state),
                     state_key(plan, errors), use_state ? 1 : 0);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail("launch k_materialize", e);
  if (use_state && out == errors) {  // the buffer now holds plain errors
    plan->state_valid = false;
    hipLaunchKernelGGL(k_state_store, dim3(1), dim3(64), 0, st, state, uint64_t(0));
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail("launch k_state_store", e);
  }
  return PSGD_OK;
}

extern "C" psgd_status psgd_plan_reset_carry_stream(psgd_plan* plan, void* workspace, void* stream) {
  const char* fn = "psgd_plan_reset_carry_stream";
  if (plan == nullptr) {
    set_error(std::string(fn) + ": plan is NULL");
    return PSGD_ERR_INVALID_ARG;
  }
  psgd_status s;
  if ((s = check_ptr(fn, "workspace", workspace, false)) != PSGD_OK) return s;
  plan->state_valid = false;
  const bool cross = (plan->flags & (PSGD_FLAG_CARRY_ERROR_MEAN | PSGD_FLAG_DEFERRED_ERROR)) != 0;
  if (!cross || plan->mats.empty()) return PSGD_OK;
  hipLaunchKernelGGL(k_state_store, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                     reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) + plan->ws_state), uint64_t(0));
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? PSGD_OK : hip_fail("launch k_state_store", e);
}

extern "C" psgd_status psgd_ef_momentum_apply(psgd_plan* plan, const void* grads, float* errors,
                                              float* q, float* p, float* momentum, float* params,
                                              float lr, float mu, float* update, void* workspace,
                                              void* stream) {
  const int mode = (plan != nullptr && (plan->flags & PSGD_FLAG_NESTEROV)) ? kNesterov : kMomentum;
  return run_step("psgd_ef_momentum_apply", plan, grads, errors, q, p, update, momentum, params, lr, mu,
                  workspace, stream, mode);
}

// ------------------------------------------------------------------ no-allocation entry point
// psgd_compress_step_noalloc is for callers that cannot allocate device memory (code
// under graph capture, tight serving loops, harnesses that forbid hipMalloc).  It runs the
// kernels of psgd_compress_step with the step's workspace and the plan's device tables in
// `scratch`, one array of kNoAllocScratchBytes per GPU that the code object holds until
// the process ends.  Host code never passes `scratch` itself to a kernel or a copy (on the
// host the name is a stand-in, not a device address): on its first call on a GPU the
// entry point looks up that GPU's address of the array and uses only that.
constexpr uint64_t kNoAllocScratchBytes = uint64_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
struct NoAllocDevice {
  char* base = nullptr;      // this GPU's address of `scratch`
  uint64_t tables_of = 0;    // nonce of the plan whose device tables the array holds (0: none)
};
std::mutex g_noalloc_mutex;
std::map<int, NoAllocDevice> g_noalloc;  // per HIP device id
}  // namespace

extern "C" psgd_status psgd_compress_step_noalloc(psgd_plan* plan, const void* grads, float* errors, float* q,
                                                  float* p, float* update, void* stream) {
  const char* fn = "psgd_compress_step_noalloc";
  if (plan == nullptr) {
    set_error(std::string(fn) + ": plan is NULL");
    return PSGD_ERR_INVALID_ARG;
  }
  if (plan->flags & (PSGD_FLAG_CARRY_ERROR_MEAN | PSGD_FLAG_DEFERRED_ERROR)) {
    set_error(std::string(fn) + ": plans with PSGD_FLAG_CARRY_ERROR_MEAN or PSGD_FLAG_DEFERRED_ERROR keep state "
              "between steps in their workspace, which this entry point shares between all calls on a GPU");
    return PSGD_ERR_UNSUPPORTED;
  }
  const uint64_t tables = layout_tables(plan, nullptr, nullptr);
  const uint64_t need = tables + plan->workspace_bytes;
  if (need > kNoAllocScratchBytes) {
    set_error(std::string(fn) + ": the plan needs " + std::to_string(need) + " bytes of scratch (tables " +
              std::to_string(tables) + " + workspace " + std::to_string(plan->workspace_bytes) +
              "), more than the " + std::to_string(kNoAllocScratchBytes) + " bytes of the static array");
    return PSGD_ERR_INVALID_ARG;
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("hipGetDevice", e);
  std::lock_guard<std::mutex> lock(g_noalloc_mutex);
  NoAllocDevice& nd = g_noalloc[dev];
  if (nd.base == nullptr) {  // set-up, once per GPU, with that GPU current
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail("hipGetSymbolAddress of the scratch array", e);
    nd.base = static_cast<char*>(ptr);
  }
  TableSlot slot;
  layout_tables(plan, nd.base, &slot.tables);
  slot.owner = &nd.tables_of;
  return run_step(fn, plan, grads, errors, q, p, update, nullptr, nullptr, 0.f, 0.f, nd.base + tables, stream,
                  kCompress, &slot);
}
