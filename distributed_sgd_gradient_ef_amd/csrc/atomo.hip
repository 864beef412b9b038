// Spectral-ATOMO: the gfx950 kernels and the host side of psgd_atomo.h.  Operation: the
// review page "ATOMO: Communication-efficient Learning via Atomic Sparsification",
// section "Proposed method" -- the atoms of a layer gradient are the rank-one terms of
// its singular value decomposition; atom i is kept with probability p_i = min(1, c
// sigma_i) (sum p_i = s) and divided by p_i.
//
// A problem is one layer matrix of one worker; k = min(n, m) is its short side.  The
// singular values are the square roots of the eigenvalues of the k x k Gram matrix of
// the short side (G G^T when n <= m, else G^T G), and a sent atom needs only the one
// eigenvector on that side: the other factor is G^T u / p (or G v / p), one more pass
// over G.  Launches, each covering every problem of every worker:
//
//   at_gram       the Gram matrix, 128 x 128 output tiles of its lower block triangle
//                 (only the lower triangle is stored) on bf16 MFMA, each fp32 entry split
//                 exactly into three bf16 parts, the contraction over the long side
//                 staged through LDS
//   at_band       one workgroup per problem: reduction of the Gram matrix to a band of
//                 half-bandwidth 16 by panels of 16 columns (Householder QR of the
//                 panel in registers, two-sided blocked update of the trailing matrix's
//                 lower triangle on fp32 MFMA)
//   at_chase      one workgroup per problem: the band to tridiagonal form by bulge
//                 chasing in LDS, the sweeps pipelined three steps apart, each wave
//                 waiting only on its predecessor sweep's progress
//   at_eig        every eigenvalue of the tridiagonal matrix by bisection on Sturm
//                 counts: 64 per workgroup (one per lane; a large matrix spans several
//                 compute units), a first round of 256 probes shared by the workgroup,
//                 then four probe points per round (one per wave);
//                 sigma_i = sqrt(max(eigenvalue, 0))
//   at_sample     the closed-form probabilities (the largest atoms saturate first),
//                 the Bernoulli decisions x_i < p_i, and the list of sent atoms
//   at_vectors    inverse iteration on the tridiagonal matrix (partial pivoting, float32)
//                 for each sent atom, orthogonalised against the problem's earlier sent
//                 atoms after every solve
//   at_backchase  the sent eigenvectors back through the chase's reflectors (stage 2)
//   at_backband   and through the band reduction's panels (stage 1): the unit factor
//   at_factor     the other factor, G^T u / p or G v / p, in one pass over G
//   at_update     U = (1/W) sum over workers and their sent atoms of a b^T (and the
//                 plain mean for tensors that are not compressed)
//
// Every reduction has a fixed order, so a step is bitwise reproducible.

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <algorithm>
#include <cfloat>
#include <cmath>
#include <cstdio>
#include <map>
#include <new>
#include <string>
#include <vector>

#include "plan.hpp"
#include "psgd_atomo.h"

namespace psgd {
namespace atm {

constexpr int kMaxK = PSGD_ATOMO_MAX_K;
constexpr int kGramTile = 128;
constexpr int kGramKC = 16;
constexpr int kGramThreads = 256;
constexpr int kEigSlots = 64;    // eigenvalues per at_eig workgroup, one per lane (a matrix in slices)
constexpr int kEigWaves = 4;     // probe points per round, one per wave: each round leaves a fifth
constexpr int kEigThreads = 64 * kEigWaves;
constexpr int kSampleThreads = 1024;
constexpr int kVecThreads = 256;
constexpr int kBackThreads = 512;
constexpr int kFactorThreads = 256;
constexpr int kFactorGroup = 4;  // atoms per pass over G
constexpr int kAtUpdThreads = 256;
constexpr int kAtUpdRows = 8;

struct AtMat {
  int64_t offset;    // element offset inside a worker slice
  int64_t sv_off;    // offset in a worker's row of uniforms / sigma / prob / index
  int64_t atom_off;  // offset in a worker's row of atoms
  int64_t b_off;     // offset of the k x k Gram matrix in a worker's Gram workspace
  int64_t r_off;     // offset of the chase reflectors in a worker's reflector workspace
  int32_t rows, cols, k, left;  // left: k == rows (G G^T), else k == cols (G^T G)
  int32_t mat_index, pad;
};

struct GramTile {
  int32_t mat, ti, tj, pad;
};

// at_factor: a column range [begin, end) of a left problem (k == rows), or a row range of
// a right problem
struct FactorTile {
  int32_t mat, begin, end, pad;
};

// at_update: rows [row0, row1) x columns [col0, col0 + kAtUpdThreads) of matrix `mat`, or
// for mat < 0 the flat range [begin, end) of an uncompressed tensor
struct AtUpdTile {
  int64_t begin, end;
  int32_t mat, row0, row1, col0;
};

enum KernelId { kGram = 0, kBandK, kChase, kEig, kSample, kVectors, kBackChase, kBackBand, kFactor, kUpdate, kNumK };
const char* const kNames[kNumK] = {"at_gram",    "at_band",      "at_chase",  "at_eig",   "at_sample",
                                   "at_vectors", "at_backchase", "at_backband", "at_factor", "at_update"};

}  // namespace atm
}  // namespace psgd

struct psgd_atomo_plan {
  int32_t n_workers = 0;
  double budget = 0.0;
  std::vector<psgd_atomo_layer_info> info;
  std::vector<psgd::atm::AtMat> mats;
  std::vector<psgd::atm::GramTile> gtiles;
  std::vector<psgd::atm::FactorTile> ftiles;
  std::vector<psgd::atm::AtUpdTile> utiles;
  std::vector<int32_t> tri_list;  // matrices in decreasing k (the largest start first)
  std::vector<int32_t> eig_items;  // matrix * 16 + slice of kEigSlots eigenvalues, in decreasing k
  int32_t max_k = 0;
  int64_t worker_stride = 0, numel = 0, sv_total = 0, atom_total = 0, gram_total = 0, refl_total = 0;
  uint64_t ws_gram = 0, ws_y = 0, ws_refl = 0, ws_d = 0, ws_e = 0, ws_lam = 0, workspace_bytes = 0;
  uint64_t model_bytes = 0;
  std::map<int, void*> dev;  // device copy of the tables, per HIP device
  bool timing = false;
  std::vector<psgd::PendingTiming> pending;
  std::vector<hipEvent_t> event_pool;
  psgd::KernelStat stats[psgd::atm::kNumK];
};

namespace psgd {
namespace atm {
namespace {

// ------------------------------------------------------------------ reductions
// Sum over the 64 lanes by DPP moves (two quad permutes, two row rotates, two row
// broadcasts), a few cycles each where the shuffle butterfly waits on the LDS crossbar
// six times; lane 63 ends with the total, which every lane reads back.  All 64 lanes
// must be active (every caller is in wave-uniform control flow).  Rows that a broadcast
// does not write add zero.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}

// A DPP move that every lane reads from a lane of the wave (row rotates, quad
// permutes): bound_ctrl set, so a following add folds into one v_add_f32_dpp.
template <int CTRL>
__device__ __forceinline__ float dpp_all(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_all<0xB1>(v);   // quad_perm [1,0,3,2]: pairs
  v += dpp_all<0x4E>(v);   // quad_perm [2,3,0,1]: quads
  v += dpp_all<0x124>(v);  // row_ror:4: two quads
  v += dpp_all<0x128>(v);  // row_ror:8: the 16-lane row
  v += dpp_mov<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3: rows 0+1, 2+3
  v += dpp_mov<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3: lane 63 has all four
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Sum over the workgroup; every thread gets the total (waves added in index order).
// GUARDED = false skips the barrier that protects `red` from the previous sum's readers:
// for a caller that passes a buffer no thread has read since the last barrier.
template <typename T, bool GUARDED = true>
__device__ T block_sum(T v, T* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if constexpr (GUARDED) __syncthreads();
  if (lane == 0) red[wid] = v;
  __syncthreads();
  T s = T(0);
  const int nw = int(blockDim.x) >> 6;
  for (int i = 0; i < nw; ++i) s += red[i];
  return s;
}

__device__ __forceinline__ float block_min(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wid] = v;
  __syncthreads();
  float s = red[0];
  const int nw = int(blockDim.x) >> 6;
  for (int i = 1; i < nw; ++i) s = fminf(s, red[i]);
  return s;
}

__device__ __forceinline__ float block_max(float v, float* red) { return -block_min(-v, red); }

// ------------------------------------------------------------------ at_gram
// One 128 x 128 tile of the lower block triangle per workgroup of four waves; each wave
// computes a 64 x 64 quadrant as 2 x 2 blocks of the bf16 matrix instruction
// v_mfma_f32_32x32x16_bf16 (D += A B with A 32 x 16, B 16 x 32, fp32 accumulation).
// Lane l holds row l mod 32 of A and column l mod 32 of B, with eight contraction slots
// chosen by l / 32; A and B are filled from the same contraction index in each slot, so
// the sum covers every index once whatever order the instruction gives the slots.  The
// result D[i][j] is accumulator (i mod 4) + 4 (i / 8) of lane j + 32 ((i / 4) mod 2).
//
// fp32 entries on bf16 matrix cores: every entry is split exactly into three bf16 parts,
// x = h + m + l.  h is x with the low 16 bits of its encoding cleared (sign, exponent
// and the top 8 significant bits), m the same of x - h, and l = x - h - m, which has at
// most 8 significant bits left and so is a bf16 too; both subtractions are exact.  With
// |m| < 2^-7 |x| and |l| < 2^-14 |x|, the six products hh, hm, mh, hl, lh, mm carry x y
// up to the three left out, ml, lm and ll, together below (2^-20 + 2^-28) |x y|.  The
// rounding of the sums matters more: per block and 16-deep step the five smaller
// products are summed from zero and added to the running sum after the hh product, so
// that the running sum takes two rounded additions per step, not six.  (With all six
// products chained on the running sum, the singular values of the ResNet-18 layer
// matrices came out within 5.8e-6 sigma_max of float64; with the split sums within
// 6.2e-7, as close as with the fp32 matrix instruction, 6.8e-7.)
// (The same splitting of fp32 into bf16 parts is the bf16x6 scheme of Henry, Tang and
// Heinecke, "Leveraging the bfloat16 artificial intelligence datatype for higher-precision
// computations", ARITH 2019, there with rounded rather than truncated parts.)  The six
// products take 6 / 16 of the fp32 instruction's matrix-core time.
//
// The long side is staged through LDS in chunks of kGramKC: thread t takes short index
// a = t mod 128 and eight consecutive long indices, loads them into registers a chunk
// ahead (to clamped addresses, without conditions), and when staging zeroes the entries
// outside the matrix, splits them, and writes each part as one 16-byte row piece; a
// staged row of one part is kGramKC bf16, so a wave's operand read of 64 x 16 bytes is
// one contiguous kilobyte.
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
constexpr int kGramRowW = kGramKC / 2;                      // words per staged row of one part
constexpr int kGramGroups = kGramKC / 8 * kGramTile / kGramThreads;  // 8-index groups per thread
static_assert(kGramKC % 16 == 0 && kGramGroups >= 1, "whole 16-deep instruction steps per chunk");

// the exact three-part split of eight entries, packed two bf16 a word (even index low)
__device__ __forceinline__ void gram_split(const float (&x)[8], u4& h, u4& m, u4& l) {
  uint32_t hb[8], mb[8], lb[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t uh = __float_as_uint(x[e]) & 0xffff0000u;
    const float r = x[e] - __uint_as_float(uh);
    const uint32_t um = __float_as_uint(r) & 0xffff0000u;
    hb[e] = uh;
    mb[e] = um;
    lb[e] = __float_as_uint(r - __uint_as_float(um));
  }
  // the high halves of two words, the first one low (v_perm_b32 byte select)
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    h[q] = __builtin_amdgcn_perm(hb[2 * q + 1], hb[2 * q], 0x07060302u);
    m[q] = __builtin_amdgcn_perm(mb[2 * q + 1], mb[2 * q], 0x07060302u);
    l[q] = __builtin_amdgcn_perm(lb[2 * q + 1], lb[2 * q], 0x07060302u);
  }
}

// three waves per SIMD: the small sums' registers must not push the kernel to two
__global__ __launch_bounds__(kGramThreads) __attribute__((amdgpu_waves_per_eu(3))) void at_gram(const GramTile* __restrict__ tiles,
                                                        const AtMat* __restrict__ mats,
                                                        const float* __restrict__ G, int64_t ld,
                                                        float* __restrict__ gram, int64_t gram_ws) {
  const GramTile t = tiles[blockIdx.y];  // grid.x walks the workers: a tile of every worker
  const AtMat M = mats[t.mat];            // is dispatched before the next tile
  const int w = blockIdx.x;
  const float* g = G + int64_t(w) * ld + M.offset;
  float* B = gram + int64_t(w) * gram_ws + M.b_off;
  const int k = M.k, cols = M.cols;
  const int L = M.left ? M.cols : M.rows;  // contraction length
  const int a0 = t.ti * kGramTile, b0 = t.tj * kGramTile;
  // [operand][part][short index][words]: operand 0 the tile's rows a0.., 1 its columns b0..
  // A row's 16-byte pieces are swapped in pairs where bits 2 and 3 of the short index
  // differ, so that the lanes of one LDS pass (rows r .. r + 7 of 32 banks, or r .. r + 15
  // of 64, one piece each) meet every bank once; reads and writes of both operands place
  // the pieces the same way.
  __shared__ __align__(16) uint32_t sg[2][3][kGramTile][kGramRowW];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = (wave >> 1) * 64, wc = (wave & 1) * 64;  // the wave's quadrant
  const int half = lane >> 5, l32 = lane & 31;
  // rows (and the offset, a multiple of 64) 16-byte aligned: L and k are then multiples
  // of 4 along the contiguous direction, so a float4 is wholly inside or wholly outside
  const bool vec = M.left && (cols & 3) == 0;
  // in a diagonal tile the quadrant above the diagonal holds no stored entry: its wave
  // skips the products (the upper right blocks of the two quadrants on the diagonal are
  // computed: the wave below them, with four live blocks, sets the pace at each barrier)
  const bool live = t.ti != t.tj || wr >= wc;
  f16v acc[2][2] = {};
  const int rsw = ((lane >> 2) ^ (lane >> 3)) & 1;  // the piece swap of rows wr + 32 bi + l32
  // in a diagonal tile both operands are the same rows: only operand 0 is loaded and staged
  auto mfma_chunk = [&](auto diag_c) {
    constexpr int kOpB = decltype(diag_c)::value ? 0 : 1;
#pragma unroll
    for (int ks = 0; ks < kGramKC / 16; ++ks) {
      bf8 x[2][3], y[2][3];
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int bi = 0; bi < 2; ++bi) {
          x[bi][p] = *reinterpret_cast<const bf8*>(&sg[0][p][wr + 32 * bi + l32][4 * ((2 * ks + half) ^ rsw)]);
          y[bi][p] = *reinterpret_cast<const bf8*>(&sg[kOpB][p][wc + 32 * bi + l32][4 * ((2 * ks + half) ^ rsw)]);
        }
      // per block, the five smaller products summed from zero, then the hh product into
      // the running sum and the small sum after it: two rounded additions to the running
      // sum per step instead of six
      constexpr int kPa[5] = {2, 0, 1, 1, 0}, kPb[5] = {0, 2, 1, 0, 1};
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj) {
          f16v t = {};
#pragma unroll
          for (int q = 0; q < 5; ++q) t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x[bi][kPa[q]], y[bj][kPb[q]], t, 0, 0, 0);
          acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x[bi][0], y[bj][0], acc[bi][bj], 0, 0, 0);
          acc[bi][bj] += t;
          __builtin_amdgcn_sched_barrier(0);  // one block's small sum live at a time
        }
    }
  };
  const int ra = threadIdx.x % kGramTile, rg = threadIdx.x / kGramTile;
  const int ia = min(a0 + ra, k - 1), ib = min(b0 + ra, k - 1);  // clamped short indices
  const uint32_t oa = uint32_t(ia) * uint32_t(cols), ob = uint32_t(ib) * uint32_t(cols);  // their rows
  // path 0: G[a][c] with 16-byte aligned rows, 1: G[a][c] otherwise, 2: G[c][a]
  auto fetch = [&](auto path, auto diag_c, float (&va)[kGramGroups][8], float (&vb)[kGramGroups][8], int c0) {
    constexpr int kPath = decltype(path)::value;
    constexpr bool kB = !decltype(diag_c)::value;  // operand 1 loaded
#pragma unroll
    for (int i = 0; i < kGramGroups; ++i) {
      const int cg = c0 + 8 * (rg + i * (kGramThreads / kGramTile));  // the group's first long index
      // offsets within the matrix fit 32 bits: unsigned, they index the uniform base directly
      if constexpr (kPath == 0) {  // G[a][cg .. cg + 7]
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t c = uint32_t(min(cg + 4 * h, L - 4));
          const f4 fa = *reinterpret_cast<const f4*>(g + (oa + c));
#pragma unroll
          for (int e = 0; e < 4; ++e) va[i][4 * h + e] = fa[e];
          if constexpr (kB) {
            const f4 fb = *reinterpret_cast<const f4*>(g + (ob + c));
#pragma unroll
            for (int e = 0; e < 4; ++e) vb[i][4 * h + e] = fb[e];
          }
        }
      } else if constexpr (kPath == 1) {  // G[a][c], rows not 16-byte aligned
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t c = uint32_t(min(cg + e, L - 1));
          va[i][e] = g[oa + c];
          if constexpr (kB) vb[i][e] = g[ob + c];
        }
      } else {  // G[c][a]: consecutive threads take consecutive entries of a row
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t row = uint32_t(min(cg + e, L - 1)) * uint32_t(cols);
          va[i][e] = g[row + uint32_t(ia)];
          if constexpr (kB) vb[i][e] = g[row + uint32_t(ib)];
        }
      }
    }
  };
  // Rows past k (loaded from row k - 1) reach only Gram entries that are never stored, so
  // only the long side is masked, and only in a chunk that runs past L.
  auto stage_as = [&](auto full_c, auto diag_c, const float (&va)[kGramGroups][8], const float (&vb)[kGramGroups][8],
                      int c0) {
    constexpr bool full = decltype(full_c)::value, kB = !decltype(diag_c)::value;
#pragma unroll
    for (int i = 0; i < kGramGroups; ++i) {
      const int gi = rg + i * (kGramThreads / kGramTile), cg = c0 + 8 * gi;
      float xa[8], xb[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool cin = full || cg + e < L;
        xa[e] = cin ? va[i][e] : 0.f;
        xb[e] = cin && kB ? vb[i][e] : 0.f;
      }
      const int wo = 4 * (gi ^ (((ra >> 2) ^ (ra >> 3)) & 1));  // the piece's place in the row
      u4 h, m, l;
      gram_split(xa, h, m, l);
      *reinterpret_cast<u4*>(&sg[0][0][ra][wo]) = h;
      *reinterpret_cast<u4*>(&sg[0][1][ra][wo]) = m;
      *reinterpret_cast<u4*>(&sg[0][2][ra][wo]) = l;
      if constexpr (kB) {
        gram_split(xb, h, m, l);
        *reinterpret_cast<u4*>(&sg[1][0][ra][wo]) = h;
        *reinterpret_cast<u4*>(&sg[1][1][ra][wo]) = m;
        *reinterpret_cast<u4*>(&sg[1][2][ra][wo]) = l;
      }
    }
  };
  auto stage = [&](auto diag_c, const float (&va)[kGramGroups][8], const float (&vb)[kGramGroups][8], int c0) {
    if (c0 + kGramKC <= L)  // uniform
      stage_as(std::true_type{}, diag_c, va, vb, c0);
    else
      stage_as(std::false_type{}, diag_c, va, vb, c0);
  };
  // the skip is decided once, outside the chunk loop: a branch around the products inside
  // it made the compiler copy the accumulators between register files every chunk
  float va[kGramGroups][8], vb[kGramGroups][8];
  auto run = [&](auto with_products, auto path, auto diag_c) {
    fetch(path, diag_c, va, vb, 0);
    for (int c0 = 0; c0 < L; c0 += kGramKC) {
      stage(diag_c, va, vb, c0);
      __syncthreads();
      if (c0 + kGramKC < L) fetch(path, diag_c, va, vb, c0 + kGramKC);
      if constexpr (decltype(with_products)::value) mfma_chunk(diag_c);
      __syncthreads();
    }
  };
  auto run_diag = [&](auto with_products, auto path) {
    if (t.ti == t.tj)
      run(with_products, path, std::true_type{});
    else
      run(with_products, path, std::false_type{});
  };
  auto run_path = [&](auto with_products) {
    if (vec)
      run_diag(with_products, std::integral_constant<int, 0>{});
    else if (M.left)
      run_diag(with_products, std::integral_constant<int, 1>{});
    else
      run_diag(with_products, std::integral_constant<int, 2>{});
  };
  if (live)
    run_path(std::true_type{});
  else
    run_path(std::false_type{});
  // the tile's lower-triangle entries, row-major with leading dimension k (the upper
  // triangle is never read: the reduction works on the lower one)
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) {
      const int b = b0 + wc + 32 * bj + l32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int a = a0 + wr + 32 * bi + 8 * (v >> 2) + 4 * half + (v & 3);
        if (a < k && b <= a) B[int64_t(a) * k + b] = acc[bi][bj][v];
      }
    }
}

// ------------------------------------------------------------------ at_band / at_chase
// The Gram matrix is reduced to tridiagonal form in two stages.
//
// Stage 1 (at_band): to a band of half-bandwidth kBand, by panels of kBand columns.  For
// the panel of columns [c, c + kBand), the rows below the band (r0 = c + kBand .. k-1)
// get a Householder QR (one reflector per column, H_i = I - tau_i v_i v_i^T with
// v_i[i] = 1), accumulated as Q = I - V T V^T (T upper triangular); the trailing matrix
// A22 (rows and columns >= r0) becomes Q^T A22 Q = A22 - V Z^T - Z V^T with
// W = A22 V T, S = T^T V^T W, Z = W - V S / 2.  Only the lower triangle of the matrix is
// stored and updated: a tile above the diagonal is read as the transpose of its mirror.
// The panel's R (upper triangle, on the band) and its reflectors (below the band) stay
// in the matrix, and T goes to the block above the band, which no update touches.
//
// Stage 2 (at_chase): band to tridiagonal by bulge chasing in LDS (the lower band, with
// room for the bulges below it: 2 kBand diagonals).  Sweep j annihilates column j below
// its subdiagonal with a reflector on rows r0 = j + 1 .. j + kBand (step 0); applied from
// both sides this fills a block below the band, whose first column the next reflector,
// kBand rows further down, annihilates (step 1), and so on to the end of the matrix.
// Step s of sweep j (rows r0 = j + 1 + s kBand .. r0 + 2 kBand - 1, columns r0 - kBand ..
// r0 + kBand - 1) follows step s + 2 of sweep j - 1, which sets the entry (r0 + 31,
// r0 + 15) that it then updates; steps of two sweeps three or more apart touch disjoint
// entries.  Each wave runs its own sweeps and waits only for its predecessor sweep's
// progress, published in LDS (no workgroup barrier between steps).  Every reflector (kBand entries and tau) is kept for the back-transform, where
// the reflectors of one sweep (disjoint supports) are applied together and the sweeps in
// reverse order.
constexpr int kBand = 16;
constexpr int kVS = kBand + 1;  // LDS row stride of the panel arrays
constexpr int kBandThreads = 1024;
#ifndef PSGD_UPD_PRE
#define PSGD_UPD_PRE 2
#endif
#ifndef PSGD_X_PRE
#define PSGD_X_PRE 2
#endif
constexpr int kUpdPre = PSGD_UPD_PRE;  // update tiles in flight per wave
constexpr int kXPre = PSGD_X_PRE;      // X-pass tiles in flight per wave
constexpr int kChaseThreads = 1024;
constexpr int kChaseWaves = kChaseThreads / 64;
constexpr int kLag = 3;  // steps sweep j - 1 stays ahead of sweep j
constexpr int kChaseSpin = 1 << 16;  // polls of one wait at most (a step's wait takes tens)

// the most chase steps a sweep of a k x k problem has, and the reflector block's floats
__host__ __device__ constexpr int chase_steps_max(int k) { return (k + kBand - 1) / kBand; }
__host__ __device__ constexpr int64_t chase_block(int k) {
  return k < 3 ? 0 : int64_t(k - 2) * chase_steps_max(k) * (kBand + 1);
}
// steps of sweep j: reflectors on rows j + 1 + s kBand .. while at least two rows remain
__device__ __forceinline__ int chase_steps(int k, int j) { return j > k - 3 ? 0 : (k - 3 - j) / kBand + 1; }
// stage-1 panels: columns c = 0, kBand, ... while at least two rows lie below the band
__device__ __forceinline__ int band_panels(int k) { return k < kBand + 2 ? 0 : (k - kBand - 2) / kBand + 1; }

// Orders one wave's LDS stores before its later LDS loads, also across lanes (the
// compiler may otherwise move a lane's load above another lane's store); all lanes of the
// wave reconverge here.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Sum over each 16-lane row of the wave (every lane of the row gets it): four row rotates.
// All 64 lanes must be active.
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_all<0x128>(v);  // row_ror:8
  v += dpp_all<0x124>(v);  // row_ror:4
  v += dpp_all<0x122>(v);  // row_ror:2
  v += dpp_all<0x121>(v);  // row_ror:1
  return v;
}

// The reflector of a vector x (its first entry alpha, the squared norm of the rest sig2):
// H x = beta e_1 with H = I - tau v v^T, v[0] = 1, v[i] = x[i] * scale.  sig2 = 0 gives
// H = I (tau = 0, beta = alpha, scale = 0).
struct Refl {
  float tau, beta, scale;
};
// The hardware square root and reciprocal (about 1 ulp each) suffice: the reflector
// stays orthogonal to rounding, whatever values tau and v take.
// Branch-free: the sig2 = 0 case is selected, not branched around.
__device__ __forceinline__ Refl make_refl(float alpha, float sig2) {
  const float mu = __builtin_amdgcn_sqrtf(fmaf(alpha, alpha, sig2));
  const float beta = alpha >= 0.f ? -mu : mu;
  const bool nz = sig2 != 0.f;
  return Refl{nz ? (beta - alpha) * __builtin_amdgcn_rcpf(beta) : 0.f, nz ? beta : alpha,
              nz ? __builtin_amdgcn_rcpf(alpha - beta) : 0.f};
}

// LDS index of element (r, c) of an r x kBand matrix stored in rows of kBand floats, its
// four float4 chunks permuted by row ((c / 4) xor (r / 2) mod 4): lanes that read one
// chunk of sixteen consecutive rows as float4 then spread over all banks.
__device__ __forceinline__ int vz(int r, int c) { return r * kBand + ((((c >> 2) ^ (r >> 1)) & 3) << 2) + (c & 3); }
__device__ __forceinline__ f4 vz4(const float* b, int r, int q4) {
  return *reinterpret_cast<const f4*>(b + r * kBand + (((q4 ^ (r >> 1)) & 3) << 2));
}

// Tile loads that go straight into LDS, holding no registers while in flight: lds_dma4
// moves 4 bytes per lane to l[lane] (l the same for every lane of the wave).  Written as
// asm so that the compiler, which cannot tell the slots apart, does not wait for every
// load in flight before each LDS access; the "memory" clobber keeps it from caching LDS
// contents across the load, and the explicit waits order the slots' reads.  The update
// loads kStage tiles of 16 x 16 per wave into LDS slots at a time (the register prefetch
// holds two at 128 registers); with KR <= 8 (k <= 512) the LDS has the room.
// M0 (the LDS address of the load) is saved and restored inside the asm: the compiler
// treats M0 as reserved and does not expect an asm statement to change it.
__device__ __forceinline__ void lds_dma4(const float* g, float* l) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>(l)));  // LDS offset
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(base)
      : "memory");
}
#ifndef PSGD_BAND_STAGE
#define PSGD_BAND_STAGE 4
#endif
constexpr int kStage = PSGD_BAND_STAGE;
template <int KR>
constexpr bool kStaged = KR <= 8;
// Waits until at most N vector memory operations of the wave are outstanding.
template <int N>
__device__ __forceinline__ void vm_wait() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
// Before a slot is loaded again: the reads of what it held have completed.
__device__ __forceinline__ void lds_slot_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// KR: registers per lane for a panel column (rows lane + 64 q), so k <= 64 KR.
template <int KR>
__global__ __launch_bounds__(kBandThreads) void at_band(const int32_t* __restrict__ list,
                                                        const AtMat* __restrict__ mats, float* __restrict__ gram,
                                                        int64_t gram_ws) {
  // grid.x walks the workers, grid.y the matrices in decreasing k
  const AtMat M = mats[list[blockIdx.y]];
  const int k = M.k;
  const int np = band_panels(k);
  if (np == 0) return;  // already a band
  float* A = gram + int64_t(blockIdx.x) * gram_ws + M.b_off;
  // U: the panel in rows of kVS = kBand + 1 floats (rows read lane by lane fall in
  // different banks) and its clean reflectors, then A22 V, then Z (vz layout).  VB: V in
  // the vz layout.  Rows from m to the next multiple of 16 hold zeros.
  constexpr int kRows = 64 * KR;  // k <= kRows
  __shared__ __align__(16) float U[kRows * kVS];
  __shared__ __align__(16) float VB[kRows * kBand];
  // kStaged only: the waves' LDS slots for the update's tiles; before that, in the X
  // pass, V^T in rows of kVTld floats (a lane's four consecutive entries in one read,
  // and the rows' starts four banks apart)
  __shared__ __align__(16) float XS[kStaged<KR> ? kBandThreads / 64 * kStage * 256 : 4];
  constexpr int kVTld = kRows + 4;
  static_assert(!kStaged<KR> || kBand * kVTld <= kBandThreads / 64 * kStage * 256, "V^T fits the slots");
  __shared__ float Tm[kBand][kBand + 1];
  __shared__ float Gv[kBand][kBand + 1];  // V^T V
  __shared__ float Gx[kBand][kBand + 1];  // V^T X
  __shared__ float Sm[kBand][kBand + 1];  // (V^T X) T, then S
  __shared__ __align__(16) float vbuf[2][kMaxK];  // the current reflector (double-buffered); Gram partials
  __shared__ float hbuf[2][3];                    // its tau, scale, beta
  float* ZB = U;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform loop control
  constexpr int kRegs = KR;  // a panel column in registers: row lane + 64 q
  constexpr int kWaves = kBandThreads / 64;
  const bool vec = (k & 3) == 0;
  for (int p = 0; p < np; ++p) {
    const int c = p * kBand, r0 = c + kBand, m = k - r0;
    const int nref = min(kBand, m - 1);
    const int nb = (m + kBand - 1) / kBand;
    float* A22 = A + int64_t(r0) * k + r0;
    {  // the panel, all of a thread's loads issued together: m * kBand <= kBandThreads * KR
      float pv[KR];
#pragma unroll
      for (int q = 0; q < KR; ++q) {
        const int e = tid + q * kBandThreads, r = min(e / kBand, m - 1);
        pv[q] = A[uint32_t((r0 + r) * k + c + e % kBand)];
      }
#pragma unroll
      for (int q = 0; q < KR; ++q) {
        const int e = tid + q * kBandThreads;
        if (e < m * kBand) U[(e / kBand) * kVS + e % kBand] = pv[q];
      }
    }
    if (tid < kBand * kBand) Tm[tid / kBand][tid % kBand] = 0.f;
    __syncthreads();
    // QR of the panel: wave t holds column t in registers.  Reflector i is formed by wave
    // i from its column (in the step before, by the wave that updated it last) and put in
    // vbuf; after one barrier the waves t > i apply it, and wave i + 1 forms the next.
    // Every row of the panel arrays up to kRows is loaded and stored without a branch
    // (rows at or past m hold zeros): a load under a per-lane condition becomes a branch
    // that waits for its load before the next one goes out.
    float col[kRegs];
    {
      float cu[kRegs];
#pragma unroll
      for (int q = 0; q < kRegs; ++q) cu[q] = U[(lane + 64 * q) * kVS + wave];
#pragma unroll
      for (int q = 0; q < kRegs; ++q) col[q] = lane + 64 * q < m ? cu[q] : 0.f;
    }
    // wave w forms reflector w from its column: v (rows > w), beta at row w
    auto form = [&](int i) {
      float s2 = 0.f, alpha = 0.f;
#pragma unroll
      for (int q = 0; q < kRegs; ++q) {
        const int r = lane + 64 * q;
        if (r > i) s2 = fmaf(col[q], col[q], s2);
        if (r == i) alpha = col[q];
      }
      s2 = wave_sum(s2);
      alpha = wave_sum(alpha);  // one lane holds it
      const Refl h = make_refl(alpha, s2);
#pragma unroll
      for (int q = 0; q < kRegs; ++q) {
        const int r = lane + 64 * q;
        const float v = r > i ? col[q] * h.scale : (r == i ? 1.f : 0.f);  // 0 at or past m
        vbuf[i & 1][r] = v;
        if (r > i) col[q] = v;
        if (r == i) col[q] = h.beta;
      }
      if (lane == 0) {
        hbuf[i & 1][0] = h.tau;
        Tm[i][i] = h.tau;
      }
    };
    if (wave == 0) form(0);
    for (int i = 0; i < nref; ++i) {
      __syncthreads();
      if (wv > i) {  // wave-uniform
        // the wave that forms the next reflector is on the critical path: it goes first
        if (wv == i + 1) __builtin_amdgcn_s_setprio(2);
        const float tau = hbuf[i & 1][0];
        const float* v = vbuf[i & 1];
        // the whole reflector, all loads at once: it is zero above row i and at or past m
        float vr[kRegs];
#pragma unroll
        for (int q = 0; q < kRegs; ++q) vr[q] = v[lane + 64 * q];
        float y = 0.f;
#pragma unroll
        for (int q = 0; q < kRegs; ++q) y = fmaf(vr[q], col[q], y);
        const float f = tau * wave_sum(y);
#pragma unroll
        for (int q = 0; q < kRegs; ++q) col[q] = fmaf(-f, vr[q], col[q]);
        if (wv == i + 1) {
          if (i + 1 < nref) form(i + 1);
          __builtin_amdgcn_s_setprio(0);
        }
      }
    }
    __syncthreads();
    // the panel (R on the band, the reflectors below it) back into U and the matrix; U
    // and VB become the unit lower trapezoidal matrix V of the reflectors
#pragma unroll
    for (int q = 0; q < kRegs; ++q) U[(lane + 64 * q) * kVS + wave] = col[q];
    __syncthreads();
    for (int e = tid; e < nb * kBand * kBand; e += kBandThreads) {
      const int i = e / kBand, t = e % kBand;
      float v = 0.f;
      if (i < m) {
        const float x = U[i * kVS + t];
        A[int64_t(r0 + i) * k + c + t] = x;
        v = t < nref ? (i > t ? x : (i == t ? 1.f : 0.f)) : 0.f;
      }
      VB[vz(i, t)] = v;
      if constexpr (kStaged<KR>) XS[t * kVTld + i] = v;  // V^T for the X pass
    }
    __syncthreads();  // U (the panel) is no longer read: it becomes X
    // X = A22 V with the matrix instruction D += A B (A 16 x 4, B 4 x 16; lane l gives
    // A[l mod 16][l / 16] and B[l / 16][l mod 16]; D[i][j] is accumulator i mod 4 of lane
    // j + 16 (i / 4)).  Wave w takes the row blocks I = w, w + 16, ...: for each column
    // block J, four instructions with A[i][q] = tile(I, J)[i][4 q + e] and B[q][j] =
    // V[16 J + 4 q + e][j], e = 0..3.  Only the lower triangle is stored: tile (I, J) is
    // read from row block I for J < I (along rows), as the transpose of tile (J, I) for
    // J > I (along columns), and entry by entry from the lower triangle for J = I.  Rows
    // and columns at or beyond m read as zero (indices clamped into the matrix); the loads
    // run kXPre tiles ahead of the instructions.
    for (int I = wv; I < nb; I += kWaves) {  // wave-uniform
      const int RI = I * kBand, i = RI + li, ic = min(i, m - 1);
      const bool iok = i < m;
      f4 acc = {0.f, 0.f, 0.f, 0.f};
      float bf[kXPre][4];
      // entries outside the matrix are zeroed here, where the tile is used, not where it is
      // loaded: a selection on a loaded value would wait for the load and undo the prefetch
      auto mma = [&](const float (&a)[4], int J) {
        float b[4];
        if constexpr (kStaged<KR>) {
          const f4 x = *reinterpret_cast<const f4*>(XS + li * kVTld + J * kBand + 4 * lg);
#pragma unroll
          for (int e = 0; e < 4; ++e) b[e] = x[e];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) b[e] = VB[vz(J * kBand + 4 * lg + e, li)];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = (iok && J * kBand + 4 * lg + e < m) ? a[e] : 0.f;
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x, b[e], acc, 0, 0, 0);
        }
      };
      {  // J < I: columns below RI < m
        const float* rowp = A22 + uint32_t(ic * k + 4 * lg);
        auto ld = [&](int J, float (&a)[4]) {
          if (vec) {
            const f4 x = *reinterpret_cast<const f4*>(rowp + J * kBand);
#pragma unroll
            for (int e = 0; e < 4; ++e) a[e] = x[e];
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) a[e] = rowp[J * kBand + e];
          }
        };
#pragma unroll
        for (int d = 0; d < kXPre; ++d)
          if (d < I) ld(d, bf[d]);
        for (int J0 = 0; J0 < I; J0 += kXPre) {
#pragma unroll
          for (int d = 0; d < kXPre; ++d) {
            const int J = J0 + d;
            if (J < I) {  // wave-uniform
              mma(bf[d], J);
              if (J + kXPre < I) ld(J + kXPre, bf[d]);
            }
          }
        }
      }
      {  // J = I
        float a[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int cix = RI + 4 * lg + e;
          const bool low = i >= cix;
          const int rr = min(low ? i : cix, m - 1), cc = min(low ? cix : i, m - 1);
          a[e] = A22[uint32_t(rr * k + cc)];
        }
        mma(a, I);
      }
      {  // J > I: the transposes of stored tiles (J, I), rows 16 J + 4 lg + e
        const float* colp = A22 + ic;
        auto ld = [&](int J, float (&a)[4]) {
#pragma unroll
          for (int e = 0; e < 4; ++e) a[e] = colp[uint32_t(min(J * kBand + 4 * lg + e, m - 1) * k)];
        };
#pragma unroll
        for (int d = 0; d < kXPre; ++d)
          if (I + 1 + d < nb) ld(I + 1 + d, bf[d]);
        for (int J0 = I + 1; J0 < nb; J0 += kXPre) {
#pragma unroll
          for (int d = 0; d < kXPre; ++d) {
            const int J = J0 + d;
            if (J < nb) {  // wave-uniform
              mma(bf[d], J);
              if (J + kXPre < nb) ld(J + kXPre, bf[d]);
            }
          }
        }
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) ZB[vz(RI + 4 * lg + v, li)] = acc[v];
    }
    __syncthreads();
    // V^T V and V^T X: waves 0..3 take the 4-row chunks w, w + 4, ... (A[i][q] = V[4 ch + q][i],
    // B[q][j] = V or X [4 ch + q][j]), their partial sums go to vbuf and are added in order
    float* gpart = &vbuf[0][0];  // [4 waves][2][16 x 16]
    if (wave < 4) {
      f4 gv = {0.f, 0.f, 0.f, 0.f}, gx = {0.f, 0.f, 0.f, 0.f};
      for (int ch = wave; ch < nb * 4; ch += 4) {
        const int r = 4 * ch + lg;
        const float a = VB[vz(r, li)], x = ZB[vz(r, li)];
        gv = __builtin_amdgcn_mfma_f32_16x16x4f32(a, a, gv, 0, 0, 0);
        gx = __builtin_amdgcn_mfma_f32_16x16x4f32(a, x, gx, 0, 0, 0);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        gpart[(wave * 2) * 256 + (4 * lg + v) * kBand + li] = gv[v];
        gpart[(wave * 2 + 1) * 256 + (4 * lg + v) * kBand + li] = gx[v];
      }
    }
    __syncthreads();
    // wave 0 alone: the Gram sums, T, P = (V^T X) T and S = T^T P (16 x 16 products on the
    // matrix instruction), then one barrier for the workgroup
    if (wv == 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = lane + 64 * q;
        float sv = 0.f, sx = 0.f;
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
          sv += gpart[(w4 * 2) * 256 + e];
          sx += gpart[(w4 * 2 + 1) * 256 + e];
        }
        Gv[e / kBand][e % kBand] = sv;
        Gx[e / kBand][e % kBand] = sx;
      }
      wave_lds_sync();
      // T[i][i] = tau_i, T[0:i, i] = -tau_i T[0:i, 0:i] (V^T v_i)[0:i]: lane a (mod 16) holds
      // row a of T and of V^T V; (V^T V)[b][i] is lane i's entry b
      float gr[kBand], tr[kBand];
      const int a = lane & 15;
#pragma unroll
      for (int b = 0; b < kBand; ++b) {
        gr[b] = Gv[a][b];
        tr[b] = b == a ? Tm[a][a] : 0.f;
      }
#pragma unroll
      for (int i = 1; i < kBand; ++i) {
        float g = 0.f;
#pragma unroll
        for (int b = 0; b < i; ++b)
          g = fmaf(tr[b], __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gr[b]), i)), g);
        const float ti = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tr[i]), i));
        tr[i] = (a < i && i < nref) ? -ti * g : tr[i];
      }
#pragma unroll
      for (int b = 0; b < kBand; ++b) Tm[a][b] = tr[b];  // lanes a + 16 g store the same row
      wave_lds_sync();
      for (int e = lane; e < nref * nref; e += 64) A[int64_t(c + e / nref) * k + r0 + e % nref] = Tm[e / nref][e % nref];
      f4 pm = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cq = 0; cq < 4; ++cq)
        pm = __builtin_amdgcn_mfma_f32_16x16x4f32(Gx[li][4 * cq + lg], Tm[4 * cq + lg][li], pm, 0, 0, 0);
#pragma unroll
      for (int v = 0; v < 4; ++v) Sm[4 * lg + v][li] = pm[v];
      wave_lds_sync();
      f4 sm = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cq = 0; cq < 4; ++cq)
        sm = __builtin_amdgcn_mfma_f32_16x16x4f32(Tm[4 * cq + lg][li], Sm[4 * cq + lg][li], sm, 0, 0, 0);
      wave_lds_sync();
#pragma unroll
      for (int v = 0; v < 4; ++v) Sm[4 * lg + v][li] = -0.5f * sm[v];
    }
    __syncthreads();
    // Z = X T - V S / 2 in place of X, a 16-row block per wave: D = X_blk T + V_blk (-S / 2)
    for (int I = wave; I < nb; I += kWaves) {
      const int RI = I * kBand;
      f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cq = 0; cq < 4; ++cq) {
        const int q = 4 * cq + lg;
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ZB[vz(RI + li, q)], Tm[q][li], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(VB[vz(RI + li, q)], Sm[q][li], acc, 0, 0, 0);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) ZB[vz(RI + 4 * lg + v, li)] = acc[v];
    }
    __syncthreads();
    // A22 -= V Z^T + Z V^T on the stored (lower) tiles, I >= J: the tile is the
    // accumulator (lane li + 16 lg, register v: row 16 I + 4 lg + v, column 16 J + li),
    // then eight instructions: A[i][q] = -V[16 I + i][4 q + e], B[q][j] = Z[16 J + j][4 q + e],
    // and the same with V and Z exchanged.  A diagonal tile keeps its upper triangle.
    // Each wave takes the tiles t = w, w + 16, ... (t = I (I + 1) / 2 + J); the tiles' loads
    // run kUpdPre tiles ahead of the instructions.
    const int nt = nb * (nb + 1) / 2;
    auto tile_of = [&](int t, int& I, int& J) {
      I = int((sqrtf(8.f * float(t) + 1.f) - 1.f) * 0.5f);
      while (I * (I + 1) / 2 > t) --I;
      while ((I + 1) * (I + 2) / 2 <= t) ++I;
      J = t - I * (I + 1) / 2;
    };
    auto load_tile = [&](int I, int J, f4& acc) {
      const int col = J * kBand + li, cc = min(col, m - 1);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = I * kBand + 4 * lg + v;
        const float x = A22[uint32_t(min(r, m - 1) * k + cc)];
        acc[v] = (r < m && col < m) ? x : 0.f;
      }
    };
    if constexpr (kStaged<KR>) {
      float* stg = XS + wv * (kStage * 256);
      for (int t0 = wv; t0 < nt; t0 += kStage * kWaves) {
        lds_slot_fence();
        int Iq[kStage], Jq[kStage];
        // slot d: tile t0 + d kWaves; the lane's entry v (row 4 lg + v, column li) at
        // d 256 + 64 v + lane
#pragma unroll
        for (int d = 0; d < kStage; ++d) {
          const int t = t0 + d * kWaves;
          if (t < nt) {  // wave-uniform
            tile_of(t, Iq[d], Jq[d]);
            const int cc = min(Jq[d] * kBand + li, m - 1);
#pragma unroll
            for (int v = 0; v < 4; ++v)
              lds_dma4(A22 + uint32_t(min(Iq[d] * kBand + 4 * lg + v, m - 1) * k + cc), stg + d * 256 + 64 * v);
          }
        }
        vm_wait<0>();
#pragma unroll
        for (int d = 0; d < kStage; ++d) {
          if (t0 + d * kWaves < nt) {  // wave-uniform
            const int I = Iq[d], J = Jq[d];
            const float* sl = stg + d * 256;
            const int RI = I * kBand, RJ = J * kBand, col = RJ + li;
            // entries at or past m (loaded from clamped, finite addresses) are not zeroed:
            // an accumulator entry only reaches its own output entry, and those are not
            // stored (a selection here made the compiler branch around each load)
            f4 acc;
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[v] = sl[64 * v + lane];
            const f4 vi = vz4(VB, RI + li, lg), zi = vz4(ZB, RI + li, lg);
            const f4 vj = vz4(VB, RJ + li, lg), zj = vz4(ZB, RJ + li, lg);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(-vi[e], zj[e], acc, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(-zi[e], vj[e], acc, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int r = RI + 4 * lg + v;
              if (r < m && col < m && (I != J || 4 * lg + v >= li)) A22[uint32_t(r * k + col)] = acc[v];
            }
          }
        }
      }
    } else {
      int Iq[kUpdPre], Jq[kUpdPre];
      f4 cb[kUpdPre];
#pragma unroll
      for (int d = 0; d < kUpdPre; ++d) {
        const int t = wv + d * kWaves;
        if (t < nt) {
          tile_of(t, Iq[d], Jq[d]);
          load_tile(Iq[d], Jq[d], cb[d]);
        }
      }
      for (int t0 = wv; t0 < nt; t0 += kUpdPre * kWaves) {
#pragma unroll
        for (int d = 0; d < kUpdPre; ++d) {
          const int t = t0 + d * kWaves;
          if (t < nt) {  // wave-uniform
            const int I = Iq[d], J = Jq[d], RI = I * kBand, RJ = J * kBand, col = RJ + li;
            f4 acc = cb[d];
            const f4 vi = vz4(VB, RI + li, lg), zi = vz4(ZB, RI + li, lg);
            const f4 vj = vz4(VB, RJ + li, lg), zj = vz4(ZB, RJ + li, lg);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(-vi[e], zj[e], acc, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(-zi[e], vj[e], acc, 0, 0, 0);
            const int tn = t + kUpdPre * kWaves;
            if (tn < nt) {
              tile_of(tn, Iq[d], Jq[d]);
              load_tile(Iq[d], Jq[d], cb[d]);
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int r = RI + 4 * lg + v;
              if (r < m && col < m && (I != J || 4 * lg + v >= li)) A22[uint32_t(r * k + col)] = acc[v];
            }
          }
        }
      }
    }
    __syncthreads();
  }
}

// One chase step (sweep j, step s) by one wave.  Lane = u + 16 g; in every block the lane
// holds the four entries whose other index is t = 4 g + c, c = 0..3: L(t, u) of the
// bulge columns left of the block, D(u, t) of the diagonal block, B(u, t) of the rows
// below it.  A product with the reflector is then four in-register terms and a sum over
// the four 16-lane rows (two lane swaps).  `band` holds element (r, c), c <= r < c + 2 kBand,
// of the lower band at c kChaseLd + r: column c's 2 kBand diagonals start at
// c (kChaseLd + 1).  kChaseLd = 2 kBand + 3 leaves four unused words a column; with the
// 2 kBand - 1 of a packed layout, the lanes of one block access met in the same LDS bank
// up to four times (the diagonal block) where now at most two do.  With the kChasePad
// zeros after k columns every load of a step stays in the array without clamping.  The
// step's loads are all issued first (the blocks it reads and writes are disjoint, and no
// step running at the same time touches them), and what lies outside the matrix or the block
// is zeroed by selection.  dk[c] = kChaseLd min(u, t) + max(u, t) places element
// (r0 + u, r0 + t) of the diagonal block (lower triangle).
constexpr int kChaseLd = 2 * kBand + 3;
constexpr int kChasePad = kBand * (kChaseLd + 1);
constexpr int kChaseSink = kMaxK * (kChaseLd + 1) + kChasePad;  // 4 words per lane

// sum of v over the four 16-lane rows (each lane gets the sum for its position in the
// row): exchange rows 0<->1, 2<->3, then the halves, adding both results of each swap
__device__ __forceinline__ float rows_sum4(float v) {
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// a b + c d rounded as two products and a sum, never contracted: the lanes holding (u, t)
// and (t, u) of a symmetric update then get the same value bit for bit
__device__ __forceinline__ float sym_dot2(float a, float b, float c, float d) {
#pragma clang fp contract(off)
  return a * b + c * d;
}

// kFull: an interior step (s > 0 and two full blocks of rows from r0 on), where no entry
// lies outside the matrix and only the lanes of L's column u = kBand - 1 (not part of L)
// must not store.  Both lanes that hold a pair (u, t), (t, u) of D store the same value
// (the update is formed symmetrically, without contraction), so D needs no mask either.
// Stores that a lane must not make go to the lane's own four sink words past the band.
template <bool kFull>
__device__ __forceinline__ void chase_step(float* band, float* __restrict__ R2, int k, int j, int s, int u, int g,
                                           const int (&dk)[4], int slot_at, bool tau_lane) {
  const int r0 = j + 1 + s * kBand;
  const int len = kFull ? kBand : min(kBand, k - r0);
  const int len2 = kFull ? kBand : len == kBand ? min(kBand, k - r0 - kBand) : 0;
  const int pc = !kFull && s == 0 ? j : r0 - kBand;  // the column to clear below row r0
  const int bx = pc * kChaseLd + r0;                         // x(t) = (r0 + t, pc)
  const int bl = (pc + 1 + u) * kChaseLd + r0 + 4 * g;       // L(4 g + c, u) at + c
  const int bd = r0 * (kChaseLd + 1);                        // D(u, 4 g + c) at + dk[c]
  const int bb = (r0 + 4 * g) * kChaseLd + r0 + kBand + u;   // B(u, 4 g + c) at + c kChaseLd
  const float x0 = band[bx], xu = band[bx + u];
  float xa[4], L[4], D[4], B[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    xa[c] = band[bx + 4 * g + c];
    L[c] = band[bl + c];
    D[c] = band[bd + dk[c]];
    B[c] = band[bb + c * kChaseLd];
  }
  __builtin_amdgcn_sched_barrier(0);  // every load goes out before the first wait
  const bool in = kFull || u < len;
  const float x = in ? xu : 0.f;
  const Refl h = make_refl(x0, row_sum16(u >= 1 ? x * x : 0.f));
  const float vu = in ? (u == 0 ? 1.f : x * h.scale) : 0.f;
  const int sink = kChaseSink + 4 * (threadIdx.x & 63);
  // the reflector's slot: v[u] from every lane (the four rows write equal values), tau
  // from one lane
  R2[(int64_t(j) * chase_steps_max(k) + s) * (kBand + 1) + slot_at] = tau_lane ? h.tau : vu;
  band[in ? bx + u : sink] = u == 0 ? h.beta : 0.f;  // the four rows write equal values
  // tau = 0 (H = I) needs no branch: every update below then leaves its entries as they are
  const float tau = h.tau;
  float vv[4], pl = 0.f, pd = 0.f, pb = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int t = 4 * g + c;
    if (kFull) {
      vv[c] = t == 0 ? 1.f : xa[c] * h.scale;
    } else {
      vv[c] = t < len ? (t == 0 ? 1.f : xa[c] * h.scale) : 0.f;
      L[c] = (s > 0 && u < kBand - 1 && t < len) ? L[c] : 0.f;  // columns pc + 1 + u < r0
      D[c] = (in && t < len) ? D[c] : 0.f;
      B[c] = u < len2 ? B[c] : 0.f;
    }
    pl = fmaf(vv[c], L[c], pl);
    pd = fmaf(D[c], vv[c], pd);
    pb = fmaf(B[c], vv[c], pb);
  }
  const float yl = rows_sum4(pl);  // (v^T L)[u]
  const float pp = rows_sum4(pd);  // (D v)[u]
  const float yb = rows_sum4(pb);  // (B v)[u]
  // both sides of the diagonal block D: p = D v, w = tau p - tau^2 (v^T p) v / 2,
  // D -= v w^T + w v^T on its lower triangle; w[4 g + c] comes from lane 20 g + c
  const float vp = row_sum16(vu * pp);
  const float c2 = 0.5f * tau * tau * vp;
  const float w = fmaf(tau, pp, -c2 * vu);
  float wa[4];  // the four exchanges go out together, ahead of the stores
#pragma unroll
  for (int c = 0; c < 4; ++c) wa[c] = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (20 * g + c), __float_as_int(w)));
  const int bls = (kFull ? u < kBand - 1 : s > 0 && u < kBand - 1) ? bl : sink;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int t = 4 * g + c;
    const float dvw = sym_dot2(vu, wa[c], w, vv[c]);
    if (kFull) {
      band[bls + c] = fmaf(-tau * yl, vv[c], L[c]);
      band[bd + dk[c]] = D[c] - dvw;
      band[bb + c * kChaseLd] = fmaf(-tau * yb, vv[c], B[c]);
    } else {
      band[t < len ? bls + c : sink + c] = fmaf(-tau * yl, vv[c], L[c]);
      band[in && t < len ? bd + dk[c] : sink + c] = D[c] - dvw;
      band[u < len2 ? bb + c * kChaseLd : sink + c] = fmaf(-tau * yb, vv[c], B[c]);
    }
  }
}

__global__ __launch_bounds__(kChaseThreads) void at_chase(const int32_t* __restrict__ list,
                                                          const AtMat* __restrict__ mats,
                                                          const float* __restrict__ gram, int64_t gram_ws,
                                                          float* __restrict__ refl, int64_t refl_ws,
                                                          float* __restrict__ d_ws, float* __restrict__ e_ws,
                                                          int64_t sv_total) {
  const AtMat M = mats[list[blockIdx.y]];
  const int64_t w = blockIdx.x;
  const int k = M.k;
  const float* A = gram + w * gram_ws + M.b_off;
  float* R2 = refl + w * refl_ws + M.r_off;
  float* d = d_ws + w * sv_total + M.sv_off;
  float* e = e_ws + w * sv_total + M.sv_off;
  __shared__ float band[kChaseSink + 4 * 64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, u = lane & 15, g = lane >> 4;
  // element (c + t, c) for t <= kBand from the matrix, zero below the band and beyond
  for (int i = tid; i < k * (kChaseLd + 1) + kChasePad; i += kChaseThreads) band[i] = 0.f;
  __syncthreads();
  for (int i = tid; i < k * (kBand + 1); i += kChaseThreads) {
    const int c = i / (kBand + 1), t = i % (kBand + 1);
    if (c + t < k) band[c * kChaseLd + c + t] = A[int64_t(c + t) * k + c];
  }
  int dk[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int t = 4 * g + c;
    dk[c] = kChaseLd * min(u, t) + max(u, t);
  }
  const bool tau_lane = lane == 16;
  const int slot_at = tau_lane ? kBand : u;
  // Wave w runs the sweeps j = w, w + 16, ... in order, each step after the previous
  // sweep has finished kLag steps more (step s of sweep j once steps 0 .. s + 2 of sweep
  // j - 1 are done; steps further apart touch disjoint entries).  Progress is published
  // per wave in LDS as j * 1024 + (steps done) once the step's LDS stores are complete;
  // sweep j waits only on sweep j - 1, so the waits form a chain that ends at sweep 0.
  // Each wait is bounded all the same (kChaseSpin polls), and one that runs out stops all
  // later waits of the workgroup, so that no mistake here could leave a wave spinning.
  __shared__ int prog[kChaseWaves], bail;
  if (tid < kChaseWaves) prog[tid] = -1;
  if (tid == 0) bail = 0;
  __syncthreads();
  const int wv = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform: scalar loop control
  for (int j = wv; j <= k - 3; j += kChaseWaves) {
    const int ns = chase_steps(k, j), nprev = j > 0 ? chase_steps(k, j - 1) : 0;
    {  // the reflector slots of the steps this sweep does not have hold zeros: the
       // back-transform applies them as reflectors that change nothing, without masks
      const int smax = chase_steps_max(k);
      float* Rj = R2 + int64_t(j) * smax * (kBand + 1);
      for (int e = ns * (kBand + 1) + lane; e < smax * (kBand + 1); e += 64) Rj[e] = 0.f;
    }
    for (int st = 0; st < ns; ++st) {
      if (j > 0) {
        const int need = (j - 1) * 1024 + min(st + kLag, nprev);
#pragma nounroll
        for (int it = 0;; ++it) {
          if (__hip_atomic_load(&prog[(j - 1) % kChaseWaves], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= need ||
              __hip_atomic_load(&bail, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP))
            break;
          if (it == kChaseSpin) {
            if (lane == 0) __hip_atomic_store(&bail, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
      }
      // (j, st) made opaque to the optimiser: otherwise it strength-reduces the step's
      // lane addresses across steps into many vector adds and moves
      int js = j, ss = st;
      asm volatile("" : "+s"(js), "+s"(ss));
      if (ss > 0 && k - (js + 1 + ss * kBand) >= 2 * kBand)
        chase_step<true>(band, R2, k, js, ss, u, g, dk, slot_at, tau_lane);
      else
        chase_step<false>(band, R2, k, js, ss, u, g, dk, slot_at, tau_lane);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
      if (lane == 0) __hip_atomic_store(&prog[wv], j * 1024 + st + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
  __syncthreads();
  for (int i = tid; i < k; i += kChaseThreads) {
    d[i] = band[i * (kChaseLd + 1)];
    if (i + 1 < k) e[i] = band[i * (kChaseLd + 1) + 1];
  }
}

// ------------------------------------------------------------------ at_eig
// Number of eigenvalues of the tridiagonal (d, e^2) below x (Sturm sequence; a pivot
// smaller than pivmin is replaced by -pivmin).  The hardware reciprocal (1 ulp) is
// enough: only the signs of the pivots are used.
__device__ __forceinline__ int sturm_below(const float* sd, const float* se2, int k, float x, float pivmin) {
  float q = sd[0] - x;
  if (fabsf(q) < pivmin) q = -pivmin;
  int c = q < 0.f;
#pragma unroll 4
  for (int t = 1; t < k; ++t) {
    q = (sd[t] - x) - se2[t - 1] * __builtin_amdgcn_rcpf(q);
    if (fabsf(q) < pivmin) q = -pivmin;
    c += q < 0.f;
  }
  return c;
}

// grid (workers, items): item = matrix * 16 + slice, slices of kEigSlots eigenvalues,
// the items in decreasing k so that the longest workgroups are dispatched first
__global__ __launch_bounds__(kEigThreads) void at_eig(const int32_t* __restrict__ items, const AtMat* __restrict__ mats,
                                                      const float* __restrict__ d_ws, const float* __restrict__ e_ws,
                                                      float* __restrict__ lam_ws, float* __restrict__ sigma,
                                                      int64_t sv_total) {
  const int item = items[blockIdx.y], slice = item & 15;
  const AtMat M = mats[item >> 4];
  const int64_t w = blockIdx.x;
  const int k = M.k, tid = threadIdx.x;
  const float* d = d_ws + w * sv_total + M.sv_off;
  const float* e = e_ws + w * sv_total + M.sv_off;
  float* lam = lam_ws + w * sv_total + M.sv_off;
  float* sig = sigma + w * sv_total + M.sv_off;
  __shared__ float sd[kMaxK], se2[kMaxK];
  __shared__ float red[kEigThreads / 64];
  float lo = FLT_MAX, hi = -FLT_MAX, e2max = 0.f;
  for (int i = tid; i < k; i += kEigThreads) {
    const float di = d[i];
    const float el = i > 0 ? fabsf(e[i - 1]) : 0.f, er = i + 1 < k ? fabsf(e[i]) : 0.f;
    sd[i] = di;
    if (i + 1 < k) {
      se2[i] = er * er;
      e2max = fmaxf(e2max, er * er);
    }
    lo = fminf(lo, di - el - er);
    hi = fmaxf(hi, di + el + er);
  }
  const float glo = block_min(lo, red);
  const float ghi = block_max(hi, red);
  const float gmax = block_max(e2max, red);
  const float tnorm = fmaxf(fabsf(glo), fabsf(ghi));
  const float pivmin = FLT_MIN * fmaxf(1.f, gmax);
  const float slack = 4.f * FLT_EPSILON * tnorm + 2.f * pivmin;
  const float abstol = 4.f * FLT_EPSILON * tnorm;
  __syncthreads();
  // multisection: lane l owns eigenvalue idx; in each round wave p counts the eigenvalues
  // below a + (p + 1) h, h = (b - a) / (kEigWaves + 1), and every wave narrows (a, b) to
  // the fifth between the last probe with at most idx below it and the next one, from the
  // same counts with the same arithmetic, so all waves hold the same interval
  __shared__ int cnt[kEigWaves][64];
  const int lane = tid & 63, wave = tid >> 6;
  const int idx = slice * kEigSlots + lane;
  const bool mine = idx < k;
  float a = glo - slack, b = ghi + slack;
  {
    // one shared round first: thread t counts the eigenvalues below the probe
    // a + (t + 1) h0, h0 = (b - a) / (kEigThreads + 1), and every lane takes the probe
    // interval holding its eigenvalue (the counts do not decrease along the probes; the
    // first probe with more than idx below it is found by bisection over the probes)
    __shared__ int cs[kEigThreads];
    const float h0 = (b - a) * (1.f / float(kEigThreads + 1));
    cs[tid] = sturm_below(sd, se2, k, a + h0 * float(tid + 1), pivmin);
    __syncthreads();
    if (mine) {
      int lo = 0, hi = kEigThreads;  // the first p with cs[p] > idx lies in [lo, hi]
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (cs[mid] > idx) hi = mid;
        else lo = mid + 1;
      }
      const float na = lo > 0 ? a + h0 * float(lo) : a;
      const float nb = lo < kEigThreads ? a + h0 * float(lo + 1) : b;
      a = na;
      b = nb;
    }
  }
  for (int it = 0; it < 96; ++it) {
    const float h = (b - a) * (1.f / float(kEigWaves + 1));
    float xs[kEigWaves];
    bool split = true;
#pragma unroll
    for (int p = 0; p < kEigWaves; ++p) {
      xs[p] = a + h * float(p + 1);
      split = split && xs[p] > (p == 0 ? a : xs[p - 1]);
    }
    split = split && xs[kEigWaves - 1] < b;
    const bool active = mine && b - a > abstol && split;
    if (!__syncthreads_or(active)) break;  // the same decision in every thread
    cnt[wave][lane] = active ? sturm_below(sd, se2, k, xs[wave], pivmin) : 0;
    __syncthreads();
    if (active) {
      int p = 0;
      while (p < kEigWaves && cnt[p][lane] <= idx) ++p;
      if (p > 0) a = xs[p - 1];
      if (p < kEigWaves) b = xs[p];
    }
  }
  if (mine && wave == 0) {
    const float l = 0.5f * (a + b);
    lam[idx] = l;
    sig[k - 1 - idx] = sqrtf(fmaxf(l, 0.f));
  }
}

// ------------------------------------------------------------------ at_sample
// p_i = 1 for the j* largest atoms and c sigma_i for the rest, where j* is the first j
// (in descending order) with sigma_j (s - j) <= sum_{i >= j} sigma_i, and c = (s - j*) /
// sum_{i >= j*} sigma_i; atoms with sigma_i = 0 get 0.
__global__ __launch_bounds__(kSampleThreads) void at_sample(const AtMat* __restrict__ mats,
                                                            const float* __restrict__ sigma,
                                                            const float* __restrict__ uniforms,
                                                            float* __restrict__ prob, int32_t* __restrict__ index,
                                                            int32_t* __restrict__ count, int64_t sv_total,
                                                            int32_t n_mats, float budget) {
  const AtMat M = mats[blockIdx.x];
  const int64_t w = blockIdx.y;
  const int k = M.k, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int kWaves = kSampleThreads / 64;
  const int64_t base = w * sv_total + M.sv_off;
  __shared__ float ssum[kWaves];
  __shared__ int sint[kWaves];
  __shared__ int spos[kWaves];
  const float sg = tid < k ? sigma[base + tid] : 0.f;
  // suffix sums S_j = sum_{i >= j} sigma_i: an inclusive scan from the end, waves taken
  // from the last one down, lanes from 63 down
  float v = sg;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float n = __shfl_down(v, o, 64);
    if (lane + o < 64) v += n;
  }
  if (lane == 0) ssum[wave] = v;  // the wave's total
  __syncthreads();
  float after = 0.f;
  for (int i = kWaves - 1; i > wave; --i) after += ssum[i];
  const float S = v + after;
  // nnz and j*
  const bool nz = tid < k && sg > 0.f;
  const bool stop = nz && sg * (budget - float(tid)) <= S;
  int cand = stop ? tid : k;
  int nzc = nz ? 1 : 0;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    cand = min(cand, __shfl_xor(cand, o, 64));
    nzc += __shfl_xor(nzc, o, 64);
  }
  __syncthreads();
  if (lane == 0) {
    sint[wave] = cand;
    spos[wave] = nzc;
  }
  __syncthreads();
  int jstar = k, nnz = 0;
  for (int i = 0; i < kWaves; ++i) {
    jstar = min(jstar, sint[i]);
    nnz += spos[i];
  }
  jstar = min(jstar, nnz);
  __shared__ float s_c;
  if (tid == jstar && jstar < nnz) s_c = (budget - float(jstar)) / S;
  __syncthreads();
  const float c = jstar < nnz ? s_c : 0.f;
  float p = 0.f;
  if (tid < k && sg > 0.f) p = tid < jstar ? 1.f : fminf(1.f, c * sg);
  const bool sent = tid < k && uniforms[base + tid] < p;
  if (tid < k) prob[base + tid] = p;
  // positions of the sent atoms (ascending)
  const uint64_t ballot = __ballot(sent);
  const int below = __popcll(ballot & ((uint64_t(1) << lane) - 1));
  __syncthreads();
  if (lane == 0) spos[wave] = __popcll(ballot);
  __syncthreads();
  int before = 0, total = 0;
  for (int i = 0; i < kWaves; ++i) {
    if (i < wave) before += spos[i];
    total += spos[i];
  }
  if (tid < k) index[base + tid] = -1;
  __syncthreads();
  if (sent) index[base + before + below] = tid;
  if (tid == 0) count[w * n_mats + M.mat_index] = total;
}

// ------------------------------------------------------------------ at_vectors
// Inverse iteration for the eigenvectors of the tridiagonal (d, e) at the sent atoms'
// eigenvalues: Gaussian elimination with partial pivoting of T - lam I, then two or three
// rounds of (solve; orthogonalise each vector, in atom order, against every earlier
// atom's vector -- classical Gram-Schmidt applied twice --; normalise); the third only
// where the second solve left a residual bound above 2^-20 ||T||.  Up to vec_slots(k)
// atoms (eight up to k = 512) are solved side by side, one lane each (the elimination is a sequential
// recurrence); pivots below 2^-24 ||T|| are raised to that size.
constexpr int kVecLdsBytes = 4096 * 24;  // slots * k * (5 floats + 1 int) stays within this

__device__ __forceinline__ int vec_slots(int k) { return max(1, min(8, 4096 / k)); }
constexpr int kVecChunk = 8;  // rows of a recurrence whose loads are issued together

__global__ __launch_bounds__(kVecThreads) void at_vectors(const int32_t* __restrict__ list, const AtMat* __restrict__ mats,
                                                          const float* __restrict__ d_ws,
                                                          const float* __restrict__ e_ws,
                                                          const float* __restrict__ lam_ws,
                                                          const int32_t* __restrict__ index,
                                                          const int32_t* __restrict__ count, float* __restrict__ Y,
                                                          int64_t gram_ws, int64_t sv_total, int32_t n_mats) {
  const AtMat M = mats[list[blockIdx.y]];  // grid (workers, matrices in decreasing k)
  const int64_t w = blockIdx.x;
  const int k = M.k, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int kWaves = kVecThreads / 64;
  const int cnt = count[w * n_mats + M.mat_index];
  if (cnt == 0) return;
  const float* d = d_ws + w * sv_total + M.sv_off;
  const float* e = e_ws + w * sv_total + M.sv_off;
  const float* lam = lam_ws + w * sv_total + M.sv_off;
  const int32_t* idx = index + w * sv_total + M.sv_off;
  float* y_all = Y + w * gram_ws + M.b_off;  // sent atom j's vector at j * k
  __shared__ float sd[kMaxK], se[kMaxK], dots[kMaxK];
  __shared__ float red[kWaves];
  __shared__ float vscale[8];
  __shared__ int vconv[8];
  __shared__ __align__(16) unsigned char pool[kVecLdsBytes];
  const int ns = vec_slots(k);
  float* f0 = reinterpret_cast<float*>(pool);  // 1 / pivot
  float* f1 = f0 + ns * k;                      // first entry right of the pivot, / pivot
  float* f2 = f1 + ns * k;                      // second entry right of the pivot, / pivot
  float* fm = f2 + ns * k;                      // multiplier
  float* fy = fm + ns * k;                      // the slot's vector
  int* fsw = reinterpret_cast<int*>(fy + ns * k);  // rows swapped (0 or 1)
  float tn = 0.f;
  for (int i = tid; i < k; i += kVecThreads) {
    sd[i] = d[i];
    se[i] = i + 1 < k ? e[i] : 0.f;
    tn = fmaxf(tn, fabsf(sd[i]) + 2.f * fabsf(se[i]));
  }
  const float tiny = fmaxf(block_max(tn, red), FLT_MIN) * 0x1p-24f;
  for (int j0 = 0; j0 < cnt; j0 += ns) {
    const int ng = min(ns, cnt - j0);
    // factorisations, one lane per atom
    if (tid < ng) {
      const int s = tid;
      const float l = lam[k - 1 - idx[j0 + s]];
      float* u0 = f0 + s * k;
      float* u1 = f1 + s * k;
      float* u2 = f2 + s * k;
      float* ml = fm + s * k;
      int* sw = fsw + s * k;
      // kVecChunk rows at a time: their loads first, then the recurrence, which carries
      // only cd and c1 (the second entry right of a pivot is zero unless the rows swapped);
      // se[k - 1] is zero, so row t's super-diagonal below is se[t + 1] for every t < k - 1
      float cd = sd[0] - l, c1 = k > 1 ? se[0] : 0.f;
      auto row = [&](int t, float sub, float dn, float sp) {
        const bool swap = !(fabsf(cd) >= fabsf(sub));
        float piv = cd;
        if (fabsf(piv) < tiny) piv = piv < 0.f ? -tiny : tiny;
        const float r = __builtin_amdgcn_rcpf(swap ? sub : piv);
        const float m = (swap ? cd : sub) * r;
        u0[t] = r;  // the back substitution's row t, scaled by 1 / pivot
        u1[t] = (swap ? dn : c1) * r;
        u2[t] = swap ? sp * r : 0.f;
        ml[t] = m;
        sw[t] = swap ? 1 : 0;
        const float ncd = swap ? fmaf(-m, dn, c1) : fmaf(-m, c1, dn);
        c1 = swap ? -m * sp : sp;
        cd = ncd;
      };
      int t = 0;
      for (; t + kVecChunk <= k - 1; t += kVecChunk) {
        float sub[kVecChunk], dn[kVecChunk], sp[kVecChunk];
#pragma unroll
        for (int q = 0; q < kVecChunk; ++q) {
          sub[q] = se[t + q];
          dn[q] = sd[t + q + 1] - l;
          sp[q] = se[t + q + 1];
        }
#pragma unroll
        for (int q = 0; q < kVecChunk; ++q) row(t + q, sub[q], dn[q], sp[q]);
      }
      for (; t < k - 1; ++t) row(t, se[t], sd[t + 1] - l, se[t + 1]);
      if (fabsf(cd) < tiny) cd = cd < 0.f ? -tiny : tiny;
      u0[k - 1] = __builtin_amdgcn_rcpf(cd);
      u1[k - 1] = 0.f;
      u2[k - 1] = 0.f;
    }
    // fixed start vectors with entries in [0.5, 1.5)
    for (int e2 = tid; e2 < ng * k; e2 += kVecThreads) {
      const int s = e2 / k, i = e2 % k;
      const uint32_t h = (uint32_t(i) + 1u) * 2654435761u ^ (uint32_t(j0 + s) + 1u) * 40503u;
      fy[s * k + i] = 0.5f + float((h >> 8) & 0xffffu) / 65536.f;
    }
    __syncthreads();
    for (int it = 0; it < 3; ++it) {
      if (tid < ng) {
        const int s = tid;
        const float* u0 = f0 + s * k;
        const float* u1 = f1 + s * k;
        const float* u2 = f2 + s * k;
        const float* ml = fm + s * k;
        const int* sw = fsw + s * k;
        float* y = fy + s * k;
        // forward, kVecChunk rows at a time with their loads first (row t + 1 is read
        // before it is written, as in the one-row order): (a, b) = (cr, next) or, rows
        // swapped, (next, cr), and one fma per row
        float cr = y[0];
        auto fwd = [&](int t, float nr, float m, int sq) {
          const float a = sq ? nr : cr, b = sq ? cr : nr;
          y[t] = a;
          cr = fmaf(-m, a, b);
        };
        int t = 0;
        for (; t + kVecChunk <= k - 1; t += kVecChunk) {
          float nr[kVecChunk], mq[kVecChunk];
          int sq[kVecChunk];
#pragma unroll
          for (int q = 0; q < kVecChunk; ++q) {
            nr[q] = y[t + q + 1];
            mq[q] = ml[t + q];
            sq[q] = sw[t + q];
          }
#pragma unroll
          for (int q = 0; q < kVecChunk; ++q) fwd(t + q, nr[q], mq[q], sq[q]);
        }
        for (; t < k - 1; ++t) fwd(t, y[t + 1], ml[t], sw[t]);
        y[k - 1] = cr;
        // back substitution from the last row: z = y u0 - u1 z1 - u2 z2 (u1, u2 pre-scaled)
        float z1 = 0.f, z2 = 0.f, big = 0.f;
        auto bwd = [&](int t, float yv, float a0, float a1, float a2) {
          const float z = fmaf(-a1, z1, fmaf(-a2, z2, yv * a0));
          y[t] = z;
          z2 = z1;
          z1 = z;
          big = fmaxf(big, fabsf(z));
        };
        t = k - 1;
        for (; t >= kVecChunk - 1; t -= kVecChunk) {
          float yv[kVecChunk], a0[kVecChunk], a1[kVecChunk], a2[kVecChunk];
#pragma unroll
          for (int q = 0; q < kVecChunk; ++q) {
            yv[q] = y[t - q];
            a0[q] = u0[t - q];
            a1[q] = u1[t - q];
            a2[q] = u2[t - q];
          }
#pragma unroll
          for (int q = 0; q < kVecChunk; ++q) bwd(t - q, yv[q], a0[q], a1[q], a2[q]);
        }
        for (; t >= 0; --t) bwd(t, y[t], u0[t], u1[t], u2[t]);
        // the scale that keeps the next round from overflowing, applied below by the
        // whole workgroup.  From the second round on the solve's input has unit norm, so
        // its residual is at most 1 / big: at most 16 tiny (about 2^-20 ||T||) counts as
        // converged
        vscale[s] = big > 0.f ? 1.f / big : 0.f;
        vconv[s] = it > 0 && big * tiny >= 0x1p-4f;
      }
      __syncthreads();
      for (int e2 = tid; e2 < ng * k; e2 += kVecThreads) fy[e2] *= vscale[e2 / k];
      __syncthreads();
      for (int s = 0; s < ng; ++s) {
        const int j = j0 + s;
        float* y = fy + s * k;
        for (int pass = 0; pass < 2; ++pass) {
          for (int jj = wave; jj < j; jj += kWaves) {
            const float* yo = y_all + int64_t(jj) * k;
            float part = 0.f;
            for (int i = lane; i < k; i += 64) part = fmaf(y[i], yo[i], part);
            part = wave_sum(part);
            if (lane == 0) dots[jj] = part;
          }
          __syncthreads();
          for (int i = tid; i < k; i += kVecThreads) {
            float v = y[i];
            for (int jj = 0; jj < j; ++jj) v = fmaf(-dots[jj], y_all[int64_t(jj) * k + i], v);
            y[i] = v;
          }
          __syncthreads();
        }
        float part = 0.f;
        for (int i = tid; i < k; i += kVecThreads) part = fmaf(y[i], y[i], part);
        const float nrm = sqrtf(block_sum(part, red));
        const float inv = nrm > 0.f ? 1.f / nrm : 0.f;
        float* yo = y_all + int64_t(j) * k;
        for (int i = tid; i < k; i += kVecThreads) {
          const float v = y[i] * inv;
          y[i] = v;
          yo[i] = v;
        }
        __syncthreads();
      }
      // the third round only where an atom of the group has not converged (the same
      // decision in every thread)
      bool done = it == 1;
      for (int s = 0; s < ng; ++s) done = done && vconv[s];
      if (done) break;
    }
  }
}

// ------------------------------------------------------------------ at_backchase, at_backband
// x = Q1 Q2 y for each sent atom (one wave per atom, eight atoms per pass), written as the
// unit factor of the message: a when k == rows, b when k == cols.
//
// at_backchase applies Q2 (stage 2), the product of the chase reflectors in the order
// they were made, to y in place, sweep by sweep from the last, the reflectors of one
// sweep (disjoint row blocks) together.  Sweep j's block s covers rows j + 1 + s kBand ..
// + kBand - 1, so the wave keeps y in a window of 64 NS registers whose position p holds
// row j + 1 + p: block s is then lane group s mod 4 of register s / 4 in every sweep, and
// moving to sweep j - 1 shifts the window up by one lane (a wave-wide DPP shift, the carry
// between registers by readlane), row j entering at position 0.  Rows at or above k stay
// zero.  The reflectors reach the window through LDS, a few sweeps at a time, the next
// ones loaded into registers by all waves while the current ones are applied.
//
// at_backband applies Q1 (stage 1) panel by panel from the last: y[r0:] -= V (T (V^T
// y[r0:])), with V (unit diagonal, zero above it) and T staged in LDS from where at_band
// left them, the next panels loaded while the current one is applied, and writes x.
constexpr int kBackWaves = kBackThreads / 64;
constexpr int kBackPre = 34;                              // prefetch registers per thread
constexpr int kBackChunkFl = kBackPre * kBackThreads;     // floats one load brings
constexpr int kBackVS = kBand + 4;                        // LDS row stride of a staged V
static_assert(kMaxK * kBand <= kBackChunkFl, "a stage-1 panel (V and T) fits one load");
static_assert(16 * chase_steps_max(kMaxK) * (kBand + 1) <= kBackChunkFl, "16 sweeps fit one load");

// lane L gets lane L - 1 of v; lane 0 gets `in`
__device__ __forceinline__ float wave_shift_up(float v, float in) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(in), __float_as_int(v), 0x138, 0xf, 0xf, false));  // wave_shr:1
}

// One sweep of reflectors on the window x (NS registers): block s = 4 i + g, valid below
// n, its entries at sl[s * (kBand + 1) + u] and tau after them.
// kMask false: every block 4 i + g lies in the sweep's slot (4 NS <= chase_steps_max(k)),
// and the blocks at or past n hold zeros, so no entry needs a mask.
template <int NS, bool kMask>
__device__ __forceinline__ void back_sweep(float (&x)[NS], const float* sl, int n, int u, int g) {
  float v[NS], t[NS], d[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int s = 4 * i + g;
    if constexpr (kMask) {
      const bool ok = s < n;
      const float vs = sl[(ok ? s : 0) * (kBand + 1) + u];
      const float ts = sl[(ok ? s : 0) * (kBand + 1) + kBand];
      v[i] = ok ? vs : 0.f;
      t[i] = ok ? ts : 0.f;
    } else {
      v[i] = sl[s * (kBand + 1) + u];
      t[i] = sl[s * (kBand + 1) + kBand];
    }
  }
#pragma unroll
  for (int i = 0; i < NS; ++i) d[i] = v[i] * x[i];
#pragma unroll
  for (int i = 0; i < NS; ++i) d[i] += dpp_all<0x128>(d[i]);
#pragma unroll
  for (int i = 0; i < NS; ++i) d[i] += dpp_all<0x124>(d[i]);
#pragma unroll
  for (int i = 0; i < NS; ++i) d[i] += dpp_all<0x122>(d[i]);
#pragma unroll
  for (int i = 0; i < NS; ++i) d[i] += dpp_all<0x121>(d[i]);
#pragma unroll
  for (int i = 0; i < NS; ++i) x[i] = fmaf(-t[i] * d[i], v[i], x[i]);
}

template <int NS>
__device__ __forceinline__ void back_shift(float (&x)[NS], float yin) {
#pragma unroll
  for (int i = NS - 1; i > 0; --i)
    x[i] = wave_shift_up(x[i], __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x[i - 1]), 63)));
  x[0] = wave_shift_up(x[0], yin);
}

// The sweeps jhi down to jl of the chunk staged at `stage` (sweep jl first), on the
// window of NS = ceil(k / 64) registers, read from and written back to y.
template <int NS, bool kMask>
__device__ __forceinline__ void back_chunk_apply(float* y, const float* stage, int k, int jl, int jhi, int slot_fl) {
  const int lane = threadIdx.x & 63, u = lane & 15, g = lane >> 4;
  float x[NS];  // the window of sweep jhi starts at row jhi + 1
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int r = jhi + 1 + 64 * i + lane;
    x[i] = r < k ? y[r] : 0.f;
  }
  for (int jj = jhi; jj >= jl; --jj) {
    back_sweep<NS, kMask>(x, stage + (jj - jl) * slot_fl, chase_steps(k, jj), u, g);
    if (jj > jl) back_shift<NS>(x, y[jj]);
  }
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int r = jl + 1 + 64 * i + lane;
    if (r < k) y[r] = x[i];
  }
}

__global__ __launch_bounds__(kBackThreads) void at_backchase(const int32_t* __restrict__ list, const AtMat* __restrict__ mats,
                                                             const float* __restrict__ refl, float* __restrict__ Y,
                                                             const int32_t* __restrict__ count, int64_t gram_ws,
                                                             int64_t refl_ws, int32_t n_mats) {
  const AtMat M = mats[list[blockIdx.y]];  // grid (workers, matrices in decreasing k)
  const int64_t w = blockIdx.x;
  const int cnt = count[w * n_mats + M.mat_index];
  const int k = M.k;
  if (cnt == 0 || k < 3) return;
  const float* R2 = refl + w * refl_ws + M.r_off;
  float* y_all = Y + w * gram_ws + M.b_off;
  __shared__ float ys[kBackWaves][kMaxK];
  __shared__ __align__(16) float stage[kBackChunkFl];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sweeps = k - 2, slot_fl = chase_steps_max(k) * (kBand + 1);
  const int chunk = kBackChunkFl / slot_fl, ns = (k + 63) / 64;
  float pre[kBackPre];
  // the reflectors of sweeps [jlo, jlo + chunk) (a contiguous range of the block); every
  // load is unconditional, from an index clamped into the range
  auto load = [&](int jlo) {
    const float* src = R2 + int64_t(jlo) * slot_fl;
    const int last = min(chunk, sweeps - jlo) * slot_fl - 1;
#pragma unroll
    for (int q = 0; q < kBackPre; ++q) pre[q] = src[min(tid + q * kBackThreads, last)];
  };
  for (int j0 = 0; j0 < cnt; j0 += kBackWaves) {
    const int j = j0 + wave;
    const bool mine = j < cnt;  // wave-uniform
    float* y = ys[wave];
    float* yg = y_all + int64_t(j) * k;
    if (mine)
      for (int i = lane; i < k; i += 64) y[i] = yg[i];
    int jlo = max(0, sweeps - chunk);
    load(jlo);
    for (int jhi = sweeps - 1; jhi >= 0;) {
      __syncthreads();  // the previous chunk is no longer read
#pragma unroll
      for (int q = 0; q < kBackPre; ++q) stage[tid + q * kBackThreads] = pre[q];
      __syncthreads();
      const int jl = jlo;
      if (jl > 0) load(jlo = max(0, jl - chunk));
      if (mine) {
        switch (ns) {
#define PSGD_BACK_CASE(N)                                      \
  case N:                                                      \
    if (4 * N <= chase_steps_max(k))                           \
      back_chunk_apply<N, false>(y, stage, k, jl, jhi, slot_fl); \
    else                                                       \
      back_chunk_apply<N, true>(y, stage, k, jl, jhi, slot_fl);  \
    break;
          PSGD_BACK_CASE(1) PSGD_BACK_CASE(2) PSGD_BACK_CASE(3) PSGD_BACK_CASE(4)
          PSGD_BACK_CASE(5) PSGD_BACK_CASE(6) PSGD_BACK_CASE(7) PSGD_BACK_CASE(8)
          PSGD_BACK_CASE(9) PSGD_BACK_CASE(10) PSGD_BACK_CASE(11) PSGD_BACK_CASE(12)
          PSGD_BACK_CASE(13) PSGD_BACK_CASE(14) PSGD_BACK_CASE(15) PSGD_BACK_CASE(16)
#undef PSGD_BACK_CASE
          default: break;
        }
      }
      jhi = jl - 1;
    }
    if (mine)
      for (int i = lane; i < k; i += 64) yg[i] = y[i];
  }
}

__global__ __launch_bounds__(kBackThreads) void at_backband(const int32_t* __restrict__ list, const AtMat* __restrict__ mats,
                                                            const float* __restrict__ gram,
                                                            const float* __restrict__ Y,
                                                            const int32_t* __restrict__ count,
                                                            float* __restrict__ atoms, int64_t gram_ws,
                                                            int64_t atom_total, int32_t n_mats) {
  const AtMat M = mats[list[blockIdx.y]];  // grid (workers, matrices in decreasing k)
  const int64_t w = blockIdx.x;
  const int cnt = count[w * n_mats + M.mat_index];
  if (cnt == 0) return;
  const int k = M.k;
  const float* A = gram + w * gram_ws + M.b_off;
  const float* y_all = Y + w * gram_ws + M.b_off;
  float* at = atoms + w * atom_total;
  __shared__ float ys[kBackWaves][kMaxK];
  __shared__ __align__(16) float stage[kMaxK * kBackVS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int np = band_panels(k);
  const int64_t stride = int64_t(M.rows) + M.cols;
  // panel p: rows r < m of V, then the kBand rows of T; thread tid always takes column
  // tid mod 16 (kBackThreads is a multiple of 16), rows tid / 16 + q kBackThreads / 16.
  // The loads are unconditional, from an index inside the matrix; the masks (V's unit
  // diagonal and zeros above it, T's upper triangle) are applied when the panel is
  // stored, so no mask stays live while the loads are in flight.  With k <= 512 a panel
  // takes 16 registers per thread and two panels are in flight: the loads of panel p - 2
  // go out while panel p is applied (a third in flight measured slower).
  const int ci = tid & 15, rt = tid >> 4;
  constexpr int kRowStep = kBackThreads / 16;
  auto load = [&](auto& pre, int p) {
    constexpr int QN = sizeof(pre) / sizeof(float);
    const int c = p * kBand, r0 = c + kBand, m = k - r0;
#pragma unroll
    for (int q = 0; q < QN; ++q) {
      // row and column selected first, one product after: with a product in each arm the
      // selection became a branch around every load
      const int r = rt + q * kRowStep, a = r - m;
      const bool isv = r < m;
      const int row = isv ? r0 + r : c + min(a, kBand - 1), col = isv ? c + ci : r0 + ci;
      pre[q] = A[uint32_t(row * k + col)];
    }
  };
  // V rows at stride kBackVS, T after them
  auto store = [&](const auto& pre, int p) {
    constexpr int QN = sizeof(pre) / sizeof(float);
    const int m = k - (p * kBand + kBand), nref = min(kBand, m - 1);
#pragma unroll
    for (int q = 0; q < QN; ++q) {
      const int r = rt + q * kRowStep, a = r - m;
      const float x = pre[q];
      const float v = r < m ? (ci < nref && r > ci ? x : (ci < nref && r == ci ? 1.f : 0.f))
                            : (a <= ci && ci < nref ? x : 0.f);
      if constexpr (QN * kRowStep <= kMaxK)  // rows past the panel land in unused LDS
        stage[r * kBackVS + ci] = v;
      else if (a < kBand)
        stage[r * kBackVS + ci] = v;
    }
  };
  // y[r0:] -= V (T (V^T y[r0:])) for the staged panel p
  auto apply = [&](float* y, int p) {
    const int r0 = p * kBand + kBand, m = k - r0;
    const f4* V4 = reinterpret_cast<const f4*>(stage);
    const f4* T4 = reinterpret_cast<const f4*>(stage + m * kBackVS);
    float z[kBand];
#pragma unroll
    for (int i = 0; i < kBand; ++i) z[i] = 0.f;
    for (int r = lane; r < m; r += 64) {
      const float yr = y[r0 + r];
#pragma unroll
      for (int q4 = 0; q4 < kBand / 4; ++q4) {
        const f4 v = V4[r * (kBackVS / 4) + q4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) z[4 * q4 + e2] = fmaf(v[e2], yr, z[4 * q4 + e2]);
      }
    }
#pragma unroll
    for (int i = 0; i < kBand; ++i) z[i] = wave_sum(z[i]);
    float t[kBand];
#pragma unroll
    for (int a = 0; a < kBand; ++a) {
      float acc = 0.f;
#pragma unroll
      for (int q4 = a / 4; q4 < kBand / 4; ++q4) {
        const f4 tv = T4[a * (kBackVS / 4) + q4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) acc = fmaf(tv[e2], z[4 * q4 + e2], acc);
      }
      t[a] = acc;
    }
    for (int r = lane; r < m; r += 64) {
      float acc = 0.f;
#pragma unroll
      for (int q4 = 0; q4 < kBand / 4; ++q4) {
        const f4 v = V4[r * (kBackVS / 4) + q4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) acc = fmaf(v[e2], t[4 * q4 + e2], acc);
      }
      y[r0 + r] -= acc;
    }
  };
  for (int j0 = 0; j0 < cnt; j0 += kBackWaves) {
    const int j = j0 + wave;
    const bool mine = j < cnt;  // wave-uniform
    float* y = ys[wave];
    if (mine)
      for (int i = lane; i < k; i += 64) y[i] = y_all[int64_t(j) * k + i];
    if (k <= 64 * 8) {  // uniform
      constexpr int QP = 64 * 8 / kRowStep;  // registers of one k <= 512 panel
      static_assert(2 * QP <= kBackPre, "two k <= 512 panels fit the prefetch registers");
      float pa[QP], pb[QP];
      if (np > 0) load(pa, np - 1);
      if (np > 1) load(pb, np - 2);
      for (int p = np - 1; p >= 0; p -= 2) {
        __syncthreads();
        store(pa, p);
        __syncthreads();
        if (p >= 2) load(pa, p - 2);
        if (mine) apply(y, p);
        if (p == 0) break;
        __syncthreads();
        store(pb, p - 1);
        __syncthreads();
        if (p >= 3) load(pb, p - 3);
        if (mine) apply(y, p - 1);
      }
    } else {
      float pre[kBackPre];
      if (np > 0) load(pre, np - 1);
      for (int p = np - 1; p >= 0; --p) {
        __syncthreads();
        store(pre, p);
        __syncthreads();
        if (p > 0) load(pre, p - 1);
        if (mine) apply(y, p);
      }
    }
    if (mine) {
      float* out = at + M.atom_off + int64_t(j) * stride + (M.left ? 0 : M.rows);
      for (int i = lane; i < k; i += 64) out[i] = y[i];
    }
  }
}

// ------------------------------------------------------------------ at_factor
// The second factor of each sent atom, kFactorGroup atoms per pass over the tile of G:
//   left  (k == rows): b_j[c] = (sum_r G[r][c] u_j[r]) / p_j   (thread per column)
//   right (k == cols): a_j[r] = (sum_c G[r][c] v_j[c]) / p_j   (wave per row)
__global__ __launch_bounds__(kFactorThreads) void at_factor(const FactorTile* __restrict__ tiles,
                                                            const AtMat* __restrict__ mats,
                                                            const float* __restrict__ G, int64_t ld,
                                                            const float* __restrict__ prob,
                                                            const int32_t* __restrict__ index,
                                                            const int32_t* __restrict__ count,
                                                            float* __restrict__ atoms, int64_t sv_total,
                                                            int64_t atom_total, int32_t n_mats) {
  const FactorTile t = tiles[blockIdx.y];  // grid.x walks the workers, grid.y the tiles,
  const AtMat M = mats[t.mat];              // largest first
  const int64_t w = blockIdx.x;
  const int cnt = count[w * n_mats + M.mat_index];
  if (cnt == 0) return;
  const int n = M.rows, m = M.cols, k = M.k;
  const float* g = G + w * ld + M.offset;
  const float* pw = prob + w * sv_total + M.sv_off;
  const int32_t* iw = index + w * sv_total + M.sv_off;
  float* at = atoms + w * atom_total + M.atom_off;
  const int64_t stride = int64_t(n) + m;
  __shared__ float unit[kFactorGroup][kMaxK];
  __shared__ float rinv[kFactorGroup];
  const int tid = threadIdx.x;
  for (int j0 = 0; j0 < cnt; j0 += kFactorGroup) {
    const int ng = min(kFactorGroup, cnt - j0);
    __syncthreads();
    for (int e = tid; e < kFactorGroup * k; e += kFactorThreads) {
      const int jj = e / k, i = e % k;
      unit[jj][i] = jj < ng ? at[int64_t(j0 + jj) * stride + (M.left ? 0 : n) + i] : 0.f;
    }
    if (tid < kFactorGroup) rinv[tid] = tid < ng ? 1.f / pw[iw[j0 + tid]] : 0.f;
    __syncthreads();
    if (M.left) {
      const int c = t.begin + tid;
      if (c < t.end) {
        float acc[kFactorGroup] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 16  // sixteen rows' loads in flight per thread (8: 145 us, 32: 146 us, 16: 131 us)
        for (int r = 0; r < n; ++r) {
          const float gv = g[int64_t(r) * m + c];
#pragma unroll
          for (int jj = 0; jj < kFactorGroup; ++jj) acc[jj] = fmaf(gv, unit[jj][r], acc[jj]);
        }
        for (int jj = 0; jj < ng; ++jj) at[int64_t(j0 + jj) * stride + n + c] = acc[jj] * rinv[jj];
      }
    } else {
      const int lane = tid & 63, wave = tid >> 6;
      for (int r = t.begin + wave; r < t.end; r += kFactorThreads / 64) {
        float acc[kFactorGroup] = {0.f, 0.f, 0.f, 0.f};
        for (int c = lane; c < m; c += 64) {
          const float gv = g[int64_t(r) * m + c];
#pragma unroll
          for (int jj = 0; jj < kFactorGroup; ++jj) acc[jj] = fmaf(gv, unit[jj][c], acc[jj]);
        }
#pragma unroll
        for (int jj = 0; jj < kFactorGroup; ++jj) acc[jj] = wave_sum(acc[jj]);
        if (lane == 0)
          for (int jj = 0; jj < ng; ++jj) at[int64_t(j0 + jj) * stride + r] = acc[jj] * rinv[jj];
      }
    }
  }
}

// ------------------------------------------------------------------ at_update
__global__ __launch_bounds__(kAtUpdThreads) void at_update(const AtUpdTile* __restrict__ tiles,
                                                         const AtMat* __restrict__ mats,
                                                         const float* __restrict__ G, int64_t ld,
                                                         const int32_t* __restrict__ count,
                                                         const float* __restrict__ atoms, float* __restrict__ update,
                                                         int W, int64_t atom_total, int32_t n_mats, float inv_w) {
  const AtUpdTile t = tiles[blockIdx.x];
  const int tid = threadIdx.x;
  if (t.mat < 0) {
    for (int64_t c = t.begin + tid; c < t.end; c += kAtUpdThreads) {
      float s = 0.f;
      for (int w = 0; w < W; ++w) s += G[int64_t(w) * ld + c];
      update[c] = s * inv_w;
    }
    return;
  }
  const AtMat M = mats[t.mat];
  const int n = M.rows, m = M.cols;
  const int c = t.col0 + tid;
  if (c >= m) return;
  const int nr = t.row1 - t.row0;
  const int64_t stride = int64_t(n) + m;
  float acc[kAtUpdRows];
#pragma unroll
  for (int r = 0; r < kAtUpdRows; ++r) acc[r] = 0.f;
  for (int w = 0; w < W; ++w) {
    const int cnt = count[int64_t(w) * n_mats + M.mat_index];
    const float* aw = atoms + int64_t(w) * atom_total + M.atom_off;
    for (int j = 0; j < cnt; ++j) {
      const float* a = aw + int64_t(j) * stride;
      const float bv = a[n + c];
#pragma unroll
      for (int r = 0; r < kAtUpdRows; ++r)
        if (r < nr) acc[r] = fmaf(a[t.row0 + r], bv, acc[r]);
    }
  }
  float* u = update + M.offset;
#pragma unroll
  for (int r = 0; r < kAtUpdRows; ++r)
    if (r < nr) u[int64_t(t.row0 + r) * m + c] = acc[r] * inv_w;
}

// ------------------------------------------------------------------ host helpers
psgd_status fail(psgd_status s, const std::string& msg) {
  set_error(msg);
  return s;
}

psgd_status hip_fail(const char* what, hipError_t e) {
  return fail(PSGD_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

uint64_t a256(uint64_t x) { return (x + 255) / 256 * 256; }

struct DevTables {
  AtMat* mats;
  GramTile* gtiles;
  FactorTile* ftiles;
  AtUpdTile* utiles;
  int32_t* tri_list;
  int32_t* eig_items;
};

psgd_status device_tables(psgd_atomo_plan* plan, DevTables* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("hipGetDevice", e);
  const uint64_t bm = a256(plan->mats.size() * sizeof(AtMat) + 1);
  const uint64_t bg = a256(plan->gtiles.size() * sizeof(GramTile) + 1);
  const uint64_t bf = a256(plan->ftiles.size() * sizeof(FactorTile) + 1);
  const uint64_t bu = a256(plan->utiles.size() * sizeof(AtUpdTile) + 1);
  const uint64_t bl = a256(plan->tri_list.size() * sizeof(int32_t) + 1);
  const uint64_t be = a256(plan->eig_items.size() * sizeof(int32_t) + 1);
  auto it = plan->dev.find(dev);
  if (it == plan->dev.end()) {
    void* base = nullptr;
    e = hipMalloc(&base, bm + bg + bf + bu + bl + be);
    if (e != hipSuccess)
      return fail(PSGD_ERR_NO_MEMORY, std::string("hipMalloc of the plan's device tables: ") + hipGetErrorString(e));
    char* b = static_cast<char*>(base);
    e = hipMemcpy(b, plan->mats.data(), plan->mats.size() * sizeof(AtMat), hipMemcpyHostToDevice);
    if (e == hipSuccess)
      e = hipMemcpy(b + bm, plan->gtiles.data(), plan->gtiles.size() * sizeof(GramTile), hipMemcpyHostToDevice);
    if (e == hipSuccess)
      e = hipMemcpy(b + bm + bg, plan->ftiles.data(), plan->ftiles.size() * sizeof(FactorTile),
                    hipMemcpyHostToDevice);
    if (e == hipSuccess)
      e = hipMemcpy(b + bm + bg + bf, plan->utiles.data(), plan->utiles.size() * sizeof(AtUpdTile),
                    hipMemcpyHostToDevice);
    if (e == hipSuccess)
      e = hipMemcpy(b + bm + bg + bf + bu, plan->tri_list.data(), plan->tri_list.size() * sizeof(int32_t),
                    hipMemcpyHostToDevice);
    if (e == hipSuccess)
      e = hipMemcpy(b + bm + bg + bf + bu + bl, plan->eig_items.data(), plan->eig_items.size() * sizeof(int32_t),
                    hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      (void)hipFree(base);
      return hip_fail("hipMemcpy of the plan's device tables", e);
    }
    it = plan->dev.emplace(dev, base).first;
  }
  char* b = static_cast<char*>(it->second);
  out->mats = reinterpret_cast<AtMat*>(b);
  out->gtiles = reinterpret_cast<GramTile*>(b + bm);
  out->ftiles = reinterpret_cast<FactorTile*>(b + bm + bg);
  out->utiles = reinterpret_cast<AtUpdTile*>(b + bm + bg + bf);
  out->tri_list = reinterpret_cast<int32_t*>(b + bm + bg + bf + bu);
  out->eig_items = reinterpret_cast<int32_t*>(b + bm + bg + bf + bu + bl);
  return PSGD_OK;
}

psgd_status take_event(psgd_atomo_plan* plan, hipEvent_t* ev) {
  if (!plan->event_pool.empty()) {
    *ev = plan->event_pool.back();
    plan->event_pool.pop_back();
    return PSGD_OK;
  }
  const hipError_t e = hipEventCreate(ev);
  return e == hipSuccess ? PSGD_OK : hip_fail("hipEventCreate", e);
}

// Launch on `st`; with timing on, through hipExtLaunchKernelGGL with events the runtime
// records with the dispatch itself.
template <typename... KArgs, typename... Args>
psgd_status launch(psgd_atomo_plan* plan, int kid, void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t st,
                   Args... args) {
  if (grid.x == 0 || grid.y == 0) return PSGD_OK;
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
    return hip_fail((std::string("launch ") + kNames[kid]).c_str(), e);
  }
  if (plan->timing) plan->pending.push_back(PendingTiming{kid, a, b});
  return PSGD_OK;
}

struct Span {
  const char* name;
  uintptr_t lo, hi;
};

}  // namespace
}  // namespace atm
}  // namespace psgd

using namespace psgd;
using namespace psgd::atm;

extern "C" psgd_status psgd_atomo_plan_create(const psgd_layer* layers, int32_t n_layers, double budget,
                                              int32_t n_workers, uint32_t flags, psgd_atomo_plan** out) {
  static const char* fn = "psgd_atomo_plan_create";
  if (out == nullptr) return fail(PSGD_ERR_INVALID_ARG, std::string(fn) + ": out is NULL");
  *out = nullptr;
  if (n_layers < 1) return fail(PSGD_ERR_INVALID_ARG, std::string(fn) + ": n_layers must be >= 1");
  if (layers == nullptr) return fail(PSGD_ERR_INVALID_ARG, std::string(fn) + ": layers is NULL");
  if (n_workers < 1 || n_workers > 65535)
    return fail(PSGD_ERR_INVALID_ARG, std::string(fn) + ": n_workers must be in 1..65535");
  if (!(budget > 0.0) || !std::isfinite(budget) || budget > 1e30)
    return fail(PSGD_ERR_INVALID_ARG, std::string(fn) + ": budget must be positive and finite");
  if (flags != 0u) return fail(PSGD_ERR_UNSUPPORTED, std::string(fn) + ": flags must be 0");
  psgd_atomo_plan* plan = nullptr;
  try {
    plan = new psgd_atomo_plan();
    plan->n_workers = n_workers;
    plan->budget = budget;
    int64_t off = 0, sv = 0, atom = 0, gram = 0, refl = 0;
    for (int32_t i = 0; i < n_layers; ++i) {
      const int64_t rows = layers[i].rows, cols = layers[i].cols;
      if (rows < 1 || cols < 1 || rows > (int64_t(1) << 31) || cols > (int64_t(1) << 31) ||
          rows * cols > int64_t(0x7fffffff)) {
        delete plan;
        return fail(PSGD_ERR_INVALID_ARG, std::string(fn) + ": layer " + std::to_string(i) +
                                              " must have 1 <= rows, cols and rows * cols < 2^31");
      }
      psgd_atomo_layer_info li{};
      li.rows = rows;
      li.cols = cols;
      li.numel = rows * cols;
      li.offset = off;
      li.matrix_index = -1;
      const int64_t k = std::min(rows, cols);
      if (k >= 2) {
        if (k > kMaxK) {
          delete plan;
          return fail(PSGD_ERR_UNSUPPORTED, std::string(fn) + ": layer " + std::to_string(i) +
                                                " has min(rows, cols) above PSGD_ATOMO_MAX_K");
        }
        li.compressed = 1;
        li.matrix_index = int32_t(plan->mats.size());
        li.k = k;
        li.sv_offset = sv;
        li.atom_offset = atom;
        AtMat m{};
        m.offset = off;
        m.sv_off = sv;
        m.atom_off = atom;
        m.b_off = gram;
        m.r_off = refl;
        m.rows = int32_t(rows);
        m.cols = int32_t(cols);
        m.k = int32_t(k);
        m.left = rows <= cols ? 1 : 0;
        m.mat_index = li.matrix_index;
        plan->mats.push_back(m);
        sv += k;
        atom += k * (rows + cols);
        gram += (k * k + 63) / 64 * 64;
        refl += (chase_block(int(k)) + 63) / 64 * 64;
        plan->max_k = std::max(plan->max_k, int32_t(k));
      }
      plan->info.push_back(li);
      off += (li.numel + 63) / 64 * 64;
    }
    plan->worker_stride = off;
    plan->sv_total = sv;
    plan->atom_total = atom;
    plan->gram_total = gram;
    plan->refl_total = refl;
    plan->numel = 0;
    const uint64_t W = uint64_t(n_workers);
    uint64_t model = 0;
    for (const auto& li : plan->info) {
      plan->numel += li.numel;
      model += (li.compressed ? 8 * W + 4 : 4 * W + 4) * uint64_t(li.numel);
    }
    plan->model_bytes = model;
    // tiles
    for (size_t mi = 0; mi < plan->mats.size(); ++mi) {
      const AtMat& m = plan->mats[mi];
      const int nt = (m.k + kGramTile - 1) / kGramTile;
      for (int ti = 0; ti < nt; ++ti)
        for (int tj = 0; tj <= ti; ++tj) plan->gtiles.push_back(GramTile{int32_t(mi), ti, tj, 0});
      if (m.left) {
        for (int c = 0; c < m.cols; c += kFactorThreads)
          plan->ftiles.push_back(FactorTile{int32_t(mi), c, std::min(m.cols, c + kFactorThreads), 0});
      } else {
        const int rows_per = 4 * (kFactorThreads / 64);
        for (int r = 0; r < m.rows; r += rows_per)
          plan->ftiles.push_back(FactorTile{int32_t(mi), r, std::min(m.rows, r + rows_per), 0});
      }
      for (int r = 0; r < m.rows; r += kAtUpdRows)
        for (int c = 0; c < m.cols; c += kAtUpdThreads)
          plan->utiles.push_back(AtUpdTile{0, 0, int32_t(mi), r, std::min(m.rows, r + kAtUpdRows), c});
    }
    // the longest contractions first, so that they do not form the launch's tail (each
    // tile writes its own block of the Gram matrix; the order changes no result)
    std::stable_sort(plan->gtiles.begin(), plan->gtiles.end(), [&](const GramTile& a, const GramTile& b) {
      const AtMat& ma = plan->mats[size_t(a.mat)];
      const AtMat& mb = plan->mats[size_t(b.mat)];
      return (ma.left ? ma.cols : ma.rows) > (mb.left ? mb.cols : mb.rows);
    });
    if (plan->gtiles.size() > 65535) {  // the Gram launch's second grid dimension
      delete plan;
      return fail(PSGD_ERR_UNSUPPORTED, std::string(fn) + ": more than 65535 Gram tiles (128 x 128) in one plan");
    }
    // the largest factor tiles first (rows x columns each covers), for the same reason
    std::stable_sort(plan->ftiles.begin(), plan->ftiles.end(), [&](const FactorTile& a, const FactorTile& b) {
      const AtMat& ma = plan->mats[size_t(a.mat)];
      const AtMat& mb = plan->mats[size_t(b.mat)];
      const int64_t wa = int64_t(a.end - a.begin) * (ma.left ? ma.rows : ma.cols);
      const int64_t wb = int64_t(b.end - b.begin) * (mb.left ? mb.rows : mb.cols);
      return wa > wb;
    });
    if (plan->ftiles.size() > 65535) {  // the factor launch's second grid dimension
      delete plan;
      return fail(PSGD_ERR_UNSUPPORTED, std::string(fn) + ": more than 65535 factor tiles in one plan");
    }
    for (size_t mi = 0; mi < plan->mats.size(); ++mi) plan->tri_list.push_back(int32_t(mi));
    std::stable_sort(plan->tri_list.begin(), plan->tri_list.end(),
                     [&](int32_t x, int32_t y) { return plan->mats[size_t(x)].k > plan->mats[size_t(y)].k; });
    static_assert(kMaxK / kEigSlots <= 16, "a slice index fits four bits");
    for (const int32_t mi : plan->tri_list)
      for (int sl = 0; sl * kEigSlots < plan->mats[size_t(mi)].k; ++sl) plan->eig_items.push_back(mi * 16 + sl);
    if (plan->eig_items.size() > 65535) {  // the eigenvalue launch's second grid dimension
      delete plan;
      return fail(PSGD_ERR_UNSUPPORTED, std::string(fn) + ": more than 65535 eigenvalue slices in one plan");
    }
    for (const auto& li : plan->info)
      if (!li.compressed)
        for (int64_t b = 0; b < li.numel; b += 4096)
          plan->utiles.push_back(AtUpdTile{li.offset + b, li.offset + std::min(li.numel, b + 4096), -1, 0, 0, 0});
    // workspace
    uint64_t ws = 0;
    plan->ws_gram = ws;
    ws = a256(ws + W * uint64_t(gram) * 4);
    plan->ws_y = ws;
    ws = a256(ws + W * uint64_t(gram) * 4);
    plan->ws_refl = ws;
    ws = a256(ws + W * uint64_t(refl) * 4);
    plan->ws_d = ws;
    ws = a256(ws + W * uint64_t(sv) * 4);
    plan->ws_e = ws;
    ws = a256(ws + W * uint64_t(sv) * 4);
    plan->ws_lam = ws;
    ws = a256(ws + W * uint64_t(sv) * 4);
    plan->workspace_bytes = std::max<uint64_t>(ws, 256);
  } catch (const std::bad_alloc&) {
    delete plan;
    return fail(PSGD_ERR_NO_MEMORY, std::string(fn) + ": out of host memory");
  }
  *out = plan;
  return PSGD_OK;
}

extern "C" psgd_status psgd_atomo_plan_sizes(const psgd_atomo_plan* plan, psgd_atomo_sizes* out) {
  if (plan == nullptr || out == nullptr) return fail(PSGD_ERR_INVALID_ARG, "psgd_atomo_plan_sizes: NULL argument");
  psgd_atomo_sizes s{};
  s.n_layers = int32_t(plan->info.size());
  s.n_workers = plan->n_workers;
  s.n_matrices = int32_t(plan->mats.size());
  s.worker_stride = plan->worker_stride;
  s.numel = plan->numel;
  s.sv_total = plan->sv_total;
  s.atom_total = plan->atom_total;
  s.workspace_bytes = plan->workspace_bytes;
  s.model_bytes = plan->model_bytes;
  s.budget = plan->budget;
  *out = s;
  return PSGD_OK;
}

extern "C" psgd_status psgd_atomo_plan_layer_info(const psgd_atomo_plan* plan, int32_t layer,
                                                  psgd_atomo_layer_info* out) {
  if (plan == nullptr || out == nullptr)
    return fail(PSGD_ERR_INVALID_ARG, "psgd_atomo_plan_layer_info: NULL argument");
  if (layer < 0 || size_t(layer) >= plan->info.size())
    return fail(PSGD_ERR_INVALID_ARG, "psgd_atomo_plan_layer_info: layer index out of range");
  *out = plan->info[size_t(layer)];
  return PSGD_OK;
}

extern "C" psgd_status psgd_atomo_plan_destroy(psgd_atomo_plan* plan) {
  if (plan == nullptr) return PSGD_OK;
  psgd_status st = PSGD_OK;
  for (const PendingTiming& t : plan->pending) {
    (void)hipEventDestroy(t.start);
    (void)hipEventDestroy(t.stop);
  }
  for (hipEvent_t ev : plan->event_pool) (void)hipEventDestroy(ev);
  for (auto& kv : plan->dev) {
    int cur = 0;
    const bool have = hipGetDevice(&cur) == hipSuccess;
    if (have && cur != kv.first) (void)hipSetDevice(kv.first);
    if (hipFree(kv.second) != hipSuccess) {
      set_error("psgd_atomo_plan_destroy: hipFree of the device tables failed");
      st = PSGD_ERR_HIP;
    }
    if (have && cur != kv.first) (void)hipSetDevice(cur);
  }
  delete plan;
  return st;
}

extern "C" psgd_status psgd_atomo_plan_set_timing(psgd_atomo_plan* plan, int32_t enable) {
  if (plan == nullptr) return fail(PSGD_ERR_INVALID_ARG, "psgd_atomo_plan_set_timing: plan is NULL");
  plan->timing = enable != 0;
  return PSGD_OK;
}

extern "C" psgd_status psgd_atomo_plan_kernel_stats(psgd_atomo_plan* plan, psgd_kernel_stat* out, int32_t capacity,
                                                    int32_t* count, int32_t reset) {
  if (plan == nullptr) return fail(PSGD_ERR_INVALID_ARG, "psgd_atomo_plan_kernel_stats: plan is NULL");
  if (capacity > 0 && out == nullptr) return fail(PSGD_ERR_INVALID_ARG, "psgd_atomo_plan_kernel_stats: out is NULL");
  psgd_status st = PSGD_OK;
  for (const PendingTiming& t : plan->pending) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(t.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, t.start, t.stop);
    if (e != hipSuccess) {
      set_error(std::string("psgd_atomo_plan_kernel_stats: ") + hipGetErrorString(e));
      st = PSGD_ERR_HIP;
    } else {
      plan->stats[t.kernel].launches += 1;
      plan->stats[t.kernel].total_ms += double(ms);
    }
    plan->event_pool.push_back(t.start);
    plan->event_pool.push_back(t.stop);
  }
  plan->pending.clear();
  int32_t n = 0;
  for (int k = 0; k < kNumK; ++k) {
    if (plan->stats[k].launches == 0) continue;
    if (n < capacity) {
      psgd_kernel_stat ks{};
      std::snprintf(ks.name, sizeof(ks.name), "%s", kNames[k]);
      ks.launches = plan->stats[k].launches;
      ks.total_ms = plan->stats[k].total_ms;
      out[n] = ks;
    }
    ++n;
  }
  if (count != nullptr) *count = std::min(n, std::max<int32_t>(capacity, 0));
  if (reset)
    for (auto& k : plan->stats) k = KernelStat{};
  return st;
}

extern "C" psgd_status psgd_atomo_step(psgd_atomo_plan* plan, const float* grads, const float* uniforms,
                                       float* sigma, float* prob, int32_t* index, int32_t* count, float* atoms,
                                       float* update, void* workspace, void* stream) {
  static const char* fn = "psgd_atomo_step";
  if (plan == nullptr) return fail(PSGD_ERR_INVALID_ARG, std::string(fn) + ": plan is NULL");
  const uint64_t W = uint64_t(plan->n_workers);
  const uint64_t stride = uint64_t(plan->worker_stride);
  const uint64_t sv = uint64_t(plan->sv_total);
  const uint64_t nm = uint64_t(plan->mats.size());
  const Span spans[] = {
      {"grads", uintptr_t(grads), uintptr_t(grads) + W * stride * 4},
      {"uniforms", uintptr_t(uniforms), uintptr_t(uniforms) + W * sv * 4},
      {"sigma", uintptr_t(sigma), uintptr_t(sigma) + W * sv * 4},
      {"prob", uintptr_t(prob), uintptr_t(prob) + W * sv * 4},
      {"index", uintptr_t(index), uintptr_t(index) + W * sv * 4},
      {"count", uintptr_t(count), uintptr_t(count) + W * nm * 4},
      {"atoms", uintptr_t(atoms), uintptr_t(atoms) + W * uint64_t(plan->atom_total) * 4},
      {"update", uintptr_t(update), uintptr_t(update) + stride * 4},
      {"workspace", uintptr_t(workspace), uintptr_t(workspace) + plan->workspace_bytes},
  };
  constexpr size_t kSpans = sizeof(spans) / sizeof(spans[0]);
  for (const Span& sp : spans) {
    const std::string name(sp.name);
    const bool empty = sp.hi == sp.lo;
    const bool nullable = name == "update" || (empty && name != "grads" && name != "workspace");
    if (sp.lo == 0) {
      if (nullable) continue;
      return fail(PSGD_ERR_INVALID_ARG, std::string(fn) + ": " + sp.name + " is NULL");
    }
    if (sp.lo % 16 != 0) return fail(PSGD_ERR_INVALID_ARG, std::string(fn) + ": " + sp.name + " is not 16-byte aligned");
  }
  for (size_t i = 0; i < kSpans; ++i)
    for (size_t j = i + 1; j < kSpans; ++j) {
      const Span &a = spans[i], &b = spans[j];
      if (a.lo == 0 || b.lo == 0 || a.lo == a.hi || b.lo == b.hi) continue;
      if (a.lo < b.hi && b.lo < a.hi)
        return fail(PSGD_ERR_INVALID_ARG, std::string(fn) + ": " + a.name + " and " + b.name + " overlap");
    }
  DevTables dt{};
  psgd_status s = device_tables(plan, &dt);
  if (s != PSGD_OK) return s;

  char* ws = static_cast<char*>(workspace);
  float* gram = reinterpret_cast<float*>(ws + plan->ws_gram);
  float* Y = reinterpret_cast<float*>(ws + plan->ws_y);
  float* refl = reinterpret_cast<float*>(ws + plan->ws_refl);
  float* dd = reinterpret_cast<float*>(ws + plan->ws_d);
  float* ee = reinterpret_cast<float*>(ws + plan->ws_e);
  float* lam = reinterpret_cast<float*>(ws + plan->ws_lam);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t ld = int64_t(stride);
  const int64_t gws = plan->gram_total;
  const int64_t rws = plan->refl_total;
  const int64_t svt = plan->sv_total;
  const int64_t att = plan->atom_total;
  const int32_t nmats = int32_t(nm);
  const dim3 mgrid(static_cast<unsigned>(nm), static_cast<unsigned>(W));
  const AtMat* M = dt.mats;

  if (nm > 0) {
    if ((s = launch(plan, kGram, at_gram, dim3(unsigned(W), unsigned(plan->gtiles.size())), dim3(kGramThreads), st,
                    static_cast<const GramTile*>(dt.gtiles), M, grads, ld, gram, gws)) != PSGD_OK)
      return s;
    {
      const int32_t* list = dt.tri_list;
      const dim3 tgrid(mgrid.y, mgrid.x);  // (workers, matrices in decreasing k)
      if ((s = plan->max_k <= kMaxK / 2
                   ? launch(plan, kBandK, at_band<kMaxK / 128>, tgrid, dim3(kBandThreads), st, list, M, gram, gws)
                   : launch(plan, kBandK, at_band<kMaxK / 64>, tgrid, dim3(kBandThreads), st, list, M, gram, gws)) !=
          PSGD_OK)
        return s;
      if ((s = launch(plan, kChase, at_chase, tgrid, dim3(kChaseThreads), st, list, M,
                      static_cast<const float*>(gram), gws, refl, rws, dd, ee, svt)) != PSGD_OK)
        return s;
    }
    // eigenvalues in slices of kEigSlots per workgroup: a large matrix's bisections
    // spread over several compute units
    const dim3 egrid(unsigned(W), unsigned(plan->eig_items.size()));
    if ((s = launch(plan, kEig, at_eig, egrid, dim3(kEigThreads), st, static_cast<const int32_t*>(dt.eig_items), M,
                    static_cast<const float*>(dd),
                    static_cast<const float*>(ee), lam, sigma, svt)) != PSGD_OK)
      return s;
    if ((s = launch(plan, kSample, at_sample, mgrid, dim3(kSampleThreads), st, M, static_cast<const float*>(sigma),
                    uniforms, prob, index, count, svt, nmats, float(plan->budget))) != PSGD_OK)
      return s;
    const dim3 lgrid(mgrid.y, mgrid.x);  // (workers, matrices in decreasing k): the largest start first
    const int32_t* list = dt.tri_list;
    if ((s = launch(plan, kVectors, at_vectors, lgrid, dim3(kVecThreads), st, list, M, static_cast<const float*>(dd),
                    static_cast<const float*>(ee), static_cast<const float*>(lam),
                    static_cast<const int32_t*>(index), static_cast<const int32_t*>(count), Y, gws, svt, nmats)) !=
        PSGD_OK)
      return s;
    if ((s = launch(plan, kBackChase, at_backchase, lgrid, dim3(kBackThreads), st, list, M,
                    static_cast<const float*>(refl),
                    Y, static_cast<const int32_t*>(count), gws, rws, nmats)) != PSGD_OK)
      return s;
    if ((s = launch(plan, kBackBand, at_backband, lgrid, dim3(kBackThreads), st, list, M,
                    static_cast<const float*>(gram),
                    static_cast<const float*>(Y), static_cast<const int32_t*>(count), atoms, gws, att, nmats)) !=
        PSGD_OK)
      return s;
    if ((s = launch(plan, kFactor, at_factor, dim3(unsigned(W), unsigned(plan->ftiles.size())),
                    dim3(kFactorThreads), st, static_cast<const FactorTile*>(dt.ftiles), M, grads, ld,
                    static_cast<const float*>(prob), static_cast<const int32_t*>(index),
                    static_cast<const int32_t*>(count), atoms, svt, att, nmats)) != PSGD_OK)
      return s;
  }
  if (update != nullptr)
    s = launch(plan, kUpdate, at_update, dim3(unsigned(plan->utiles.size())), dim3(kAtUpdThreads), st,
               static_cast<const AtUpdTile*>(dt.utiles), M, grads, ld, static_cast<const int32_t*>(count),
               static_cast<const float*>(atoms), update, int(W), att, nmats, 1.0f / float(W));
  return s;
}
