// rTop-k sparsification with error feedback: the gfx950 kernels and the host side of
// psgd_rtopk.h.  Operation: the review page "rTop-k: A Statistical Estimation Approach
// to Distributed SGD", section "Proposed method" -- a random subset of the entries of
// largest magnitude is sent, and what is not sent stays in the error memory.
//
// A segment is one tensor of one worker.  A tile is kTile consecutive elements of one
// tensor (the last tile of a tensor may be shorter); the streaming launches cover every
// tile of every worker at once (grid.x = tile, grid.y = worker).  Magnitudes compare as
// the 31-bit key bits(|m|).  The top set of a segment is every entry with key above the
// r-th largest key T, plus the lowest-index entries with key T that complete r; T is
// found by a radix selection over the key in three digits (bits 30..20, 19..9, 8..0).
//
//   rk_zero       clear the three digit histograms
//   rk_ef_hist    M = G + E, stored into E; per segment, a histogram of digit 1
//                 (LDS per workgroup, flushed with atomics); and, for the digit-1 bin
//                 predicted from the previous step, the marking below
//   rk_select     per segment: the digit-1 bin b1 holding T, and how many of its
//                 entries belong to the top set; a wrong prediction sends the segment
//                 to rk_mark
//   rk_mark       (mispredicted segments) re-read M: entries above b1 -> top mask (one
//                 bit per element); entries in b1 -> the tile's candidate region (key
//                 bits 19..0 | tile offset), and a histogram of their digit 2; per-tile
//                 counts
//   rk_level3     per chunk of tiles: digit-2 bin b2 (recomputed from the histogram),
//                 then a histogram of digit 3 of the candidates in b2
//   rk_final      per chunk of tiles: T and the rule (keys >= a bound are in; when the
//                 entries equal to T are only partly in, they are tie-marked), applied
//                 to the candidates
//   rk_scan_top   per segment: scans of the per-tile tie counts (the first ties in
//                 index order are in) and of the per-tile top counts (slot bases)
//   rk_keep       per tile: each top entry's slot (its position in index order) gives
//                 its rank; rank < k -> kept mask; per-tile kept counts
//   rk_scan_kept  per segment: exclusive scan of the kept counts; unused output slots
//                 get index -1, value 0
//   rk_emit       per tile: index/value lists in index order (first k kept), E' = 0 at
//                 the sent entries (deferred-zero plans leave that to the next step's
//                 rk_ef_hist, which zeroes them as it reads E), the kept mask trimmed to
//                 what was sent, and each mask word's first list position
//   rk_update     U = (1/W) * sum over workers, in worker order, of the sent entries
//
// Every reduction that produces a float has a fixed order; every other result is an
// integer count or a set, so a step is bitwise reproducible.  The prediction only
// decides which kernel does the marking: a stale or garbage prediction costs the
// re-read, never a different result.

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <map>
#include <new>
#include <random>
#include <string>
#include <vector>

#include "plan.hpp"
#include "psgd_rtopk.h"

namespace psgd {
namespace rtk {

constexpr int kTile = 4096;               // elements per tile
constexpr int kLocalBits = 12;            // log2(kTile): offset of an entry inside its tile
constexpr int kTileThreads = 256;         // rk_ef_hist / rk_mark: 16 elements per thread
constexpr int kEfTiles = 4;               // rk_ef_hist: consecutive tiles per workgroup
constexpr int kWordThreads = kTile / 32;  // rk_update: one thread per mask word
constexpr int kSelThreads = 256;          // rk_select / rk_level3 / rk_final
constexpr int kSegThreads = 1024;         // per-segment scans
constexpr int kBins1 = 2048;              // digit 1: key bits 30..20
constexpr int kBins2 = 2048;              // digit 2: key bits 19..9
constexpr int kBins3 = 512;               // digit 3: key bits 8..0
constexpr int kChunkTiles = 16;           // tiles per workgroup in rk_level3 / rk_final
constexpr int kWaveBlock = 256;           // rk_keep / rk_emit: one wave per tile, 4 tiles per workgroup

struct RkLayer {
  int64_t offset;  // element offset in a worker slice
  int64_t numel;
  int64_t top, keep;
  int64_t top_off, keep_off;
  int32_t tile_off;  // first tile of the tensor in the tile table
  int32_t ntiles;
};

struct RkTile {
  int64_t begin;  // element offset of the tile in a worker slice
  int32_t layer;
  int32_t len;    // elements in the tile (kTile except at a tensor's end)
  int32_t chunk;  // tile number inside its tensor
  int32_t pad;
};

struct RkChunk {
  int32_t layer;
  int32_t t0, t1;  // tiles [t0, t1) of the tensor
  int32_t first;   // 1 for the tensor's first chunk (it records the segment's rule)
};

struct RkSeg {
  uint32_t b1;      // digit-1 bin holding T
  uint32_t need1;   // entries of bin b1 in the top set
  uint32_t count1;  // entries in bin b1
  uint32_t redo;    // 1: the predicted bin was not b1; rk_mark marks this segment
  uint32_t b2;       // digit-2 bin holding T
  uint32_t need2;    // entries of (b1, b2) in the top set
  uint32_t settled;  // 1: every entry of the last bin found is in (no digit 3)
  uint32_t sel_lo;   // every entry with key >= sel_lo is in the top set
  uint32_t tie_key;  // partial: the first need_t entries (index order) with this key are in
  uint32_t need_t;
  uint32_t partial;
  uint32_t ntop;   // top-set size found (r)
  uint32_t nkept;  // entries with rank < k
  uint32_t tkey;  // T of the last step whose rule was found (carried from step to step)
  uint32_t pad2, pad3;
};

enum KernelId {
  kZero = 0, kEfHist, kSelect, kMark, kPick2, kLevel3, kRule, kFinal, kScanTop, kKeep, kScanKept, kEmit, kUpdate, kNumK
};
const char* const kNames[kNumK] = {"rk_zero",     "rk_ef_hist", "rk_select",    "rk_mark", "rk_pick2",
                                   "rk_level3",   "rk_rule",    "rk_final",     "rk_scan_top", "rk_keep",
                                   "rk_scan_kept", "rk_emit",   "rk_update"};

}  // namespace rtk
}  // namespace psgd

struct psgd_rtopk_plan {
  int32_t n_workers = 0;
  psgd_dtype dtype = PSGD_F32;
  uint32_t flags = 0;
  // deferred-zero plans: the sent mask of the last step (ws_kmask) is pending in the
  // errors; the host's view of that state (these buffers, this device, not reset) and,
  // on the device, the state word at ws_state keyed by nonce and the errors address
  uint64_t nonce = 0;
  bool state_valid = false;
  const void* state_errors = nullptr;
  const void* state_workspace = nullptr;
  int state_device = -1;
  uint64_t ws_state = 0;
  std::vector<psgd_rtopk_layer_info> info;
  std::vector<psgd::rtk::RkLayer> layers;
  std::vector<psgd::rtk::RkTile> tiles;
  std::vector<psgd::rtk::RkChunk> chunks;
  int64_t worker_stride = 0, numel = 0, top_total = 0, keep_total = 0;
  int64_t n_seg = 0;
  uint64_t ws_hist1 = 0, ws_hist2 = 0, ws_hist3 = 0, ws_seg = 0, ws_pred = 0, ws_cand = 0;
  uint64_t ws_mask = 0, ws_tmask = 0, ws_kmask = 0, ws_kpos = 0, ws_ccnt4 = 0, ws_tcnt4 = 0;
  uint64_t ws_tfin = 0, ws_ttie = 0, ws_tiebase = 0, ws_tbase = 0, ws_kcnt = 0, ws_kbase = 0;
  uint64_t workspace_bytes = 0;
  uint64_t message_bytes = 0, model_bytes = 0;
  std::map<int, void*> dev;  // device copy of the layer, tile and chunk tables, per HIP device
  bool timing = false;
  std::vector<psgd::PendingTiming> pending;
  std::vector<hipEvent_t> event_pool;
  psgd::KernelStat stats[psgd::rtk::kNumK];
};

namespace psgd {
namespace rtk {
namespace {

// ------------------------------------------------------------------ device helpers
__device__ __forceinline__ uint32_t mag_key(float m) { return __float_as_uint(m) & 0x7fffffffu; }

typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

__device__ __forceinline__ v4f load_nt4(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
}

__device__ __forceinline__ void store_nt4(float* p, v4f v) {
  __builtin_nontemporal_store(v, reinterpret_cast<v4f*>(p));
}

__device__ __forceinline__ v4f load_g4(const float* p) { return load_nt4(p); }

// Four bfloat16 values widened exactly to float32.
__device__ __forceinline__ v4f load_g4(const uint16_t* p) {
  const v2u u = __builtin_nontemporal_load(reinterpret_cast<const v2u*>(p));
  v4f r;
  r.x = __uint_as_float(u.x << 16);
  r.y = __uint_as_float(u.x & 0xffff0000u);
  r.z = __uint_as_float(u.y << 16);
  r.w = __uint_as_float(u.y & 0xffff0000u);
  return r;
}

// Place bit q of an 8-bit value at bit 4q.
__device__ __forceinline__ uint32_t spread4(uint32_t x) {
  x = (x | (x << 12)) & 0x000F000Fu;
  x = (x | (x << 6)) & 0x03030303u;
  x = (x | (x << 3)) & 0x11111111u;
  return x;
}

// Wave scans and sums by DPP moves: row shifts within each 16-lane row (lanes without a
// source read zero), then the row broadcasts of lanes 15 and 31 into the rows after them.
// All 64 lanes must be active; integer sums, so the result does not depend on the order.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, ROW_MASK, 0xf, true));
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += dpp_u32<0x111, 0xf>(v);  // row_shr:1
  v += dpp_u32<0x112, 0xf>(v);  // row_shr:2
  v += dpp_u32<0x114, 0xf>(v);  // row_shr:4
  v += dpp_u32<0x118, 0xf>(v);  // row_shr:8: inclusive scan of each row
  v += dpp_u32<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_u32<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
  return uint32_t(__builtin_amdgcn_readlane(int(wave_incl_scan(v)), 63));
}

// Inclusive scan over the block (blockDim.x a multiple of 64, at most 1024); `lds`
// holds 16 words.  Every thread must call it.
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* lds) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_incl_scan(v);
  if (lane == 63) lds[wid] = v;
  __syncthreads();
  if (wid == 0) {
    const uint32_t t = wave_incl_scan(lane < nw ? lds[lane] : 0u);
    if (lane < nw) lds[lane] = t;
  }
  __syncthreads();
  if (wid > 0) v += lds[wid - 1];
  __syncthreads();
  return v;
}

// Block total of v (every thread gets it).
__device__ __forceinline__ uint32_t block_total(uint32_t v, uint32_t* lds) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_sum(v);
  if (lane == 0) lds[wid] = v;
  __syncthreads();
  uint32_t t = 0;
  for (int i = 0; i < nw; ++i) t += lds[i];
  __syncthreads();
  return t;
}


// Set bits of `bits` in order, given the running rank of the first one: those whose
// rank is below `limit` are returned.
__device__ __forceinline__ uint32_t bits_below(uint32_t bits, uint32_t& rank, uint32_t limit) {
  uint32_t out = 0;
  for (; bits != 0u; bits &= bits - 1u) {
    if (rank < limit) out |= bits & (0u - bits);
    ++rank;
  }
  return out;
}

struct Pick {
  uint32_t bin;    // the bin holding the need-th largest entry
  uint32_t above;  // entries in the bins above it
  uint32_t count;  // entries in it
};

// Walk a histogram of NB bins from the top (kSelThreads threads, NB / kSelThreads bins
// each) to the bin where the count reaches `need`.  Every thread must call it.
template <int NB>
__device__ Pick pick_bin(const uint32_t* __restrict__ h, uint32_t need, uint32_t* lds, uint32_t* sh) {
  constexpr int PER = NB / kSelThreads;
  if (threadIdx.x == 0) sh[0] = sh[1] = sh[2] = 0u;
  const int hi = NB - PER * int(threadIdx.x);
  uint32_t c[PER], tsum = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    c[j] = h[hi - 1 - j];
    tsum += c[j];
  }
  const uint32_t incl = block_incl_scan(tsum, lds);
  const uint32_t above = incl - tsum;
  if (above < need && need <= incl) {
    uint32_t acc = above;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (acc + c[j] >= need) {
        sh[0] = uint32_t(hi - 1 - j);
        sh[1] = acc;
        sh[2] = c[j];
        break;
      }
      acc += c[j];
    }
  }
  __syncthreads();
  const Pick p{sh[0], sh[1], sh[2]};
  __syncthreads();
  return p;
}

// Start of wave v's part of a tile's candidate region: the number of tile elements the
// waves before it hold (wave v holds groups v, v+4, v+8, v+12 of 256 elements), so every
// part lies inside the tile's own len elements.
__device__ __forceinline__ int wave_region(int len, int v) {
  int off = 0;
  for (int u = 0; u < v; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i) off += min(256, max(0, len - (4 * i + u) * 256));
  return off;
}

// Number of set bits of a wave-wide mask below this lane (no LDS involved).
__device__ __forceinline__ uint32_t lanes_below(uint64_t b) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(b >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(b), 0u));
}

// Marking of one tile against digit-1 bin b1, from the 16 values each thread holds
// (m[i][j] is element (i * kTileThreads + threadIdx.x) * 4 + j of the tile).  The wave
// with index v handles groups v, v+4, v+8, v+12 of 256 elements; lane l holds elements
// 4l..4l+3 of its group, so mask word q of a group (32 elements) comes from lanes
// 8q..8q+7 and is assembled by lane q from four ballots.  Entries above b1 set top-mask
// bits; entries in b1 (the candidates) go to the wave's part of the tile's region of
// `cand` (same layout as E) as (key bits 19..0) << 12 | offset in the tile, placed by
// ballot and lane count, and are then counted into the LDS histogram h2 of their digit
// 2.  Counts come from ballot popcounts and positions from mbcnt, so no LDS operation
// sits between the stores (the histogram atomics come last).  Each wave writes its own
// top and candidate counts; no barrier.
__device__ __forceinline__ void mark_tile(const float (&m)[4][4], const RkTile& t, uint32_t b1, int64_t base,
                                          int64_t trow, uint32_t* h2, uint32_t* __restrict__ mask,
                                          uint32_t* __restrict__ tmask, uint32_t* __restrict__ tcnt4,
                                          uint32_t* __restrict__ cand, uint32_t* __restrict__ ccnt4) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t wbase = base >> 5;  // begin and stride are multiples of 64
  uint32_t* out = cand + base + wave_region(t.len, wv);
  uint32_t nsure = 0, ncand = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = i * 4 + wv;
    const int e = g * 256 + lane * 4;
    uint64_t B[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t key = mag_key(m[i][j]);
      const bool ok = e + j < t.len;
      B[j] = __ballot(ok && (key >> 20) > b1);
      nsure += uint32_t(__popcll(B[j]));
      const bool c = ok && (key >> 20) == b1;
      const uint64_t bc = __ballot(c);
      if (c) out[ncand + lanes_below(bc)] = ((key & 0xfffffu) << kLocalBits) | uint32_t(e + j);
      ncand += uint32_t(__popcll(bc));
    }
    if (lane < 8 && (g * 256 + lane * 32) < t.len) {
      const int sh = lane * 8;
      const uint32_t word = spread4(uint32_t(B[0] >> sh) & 0xffu) | (spread4(uint32_t(B[1] >> sh) & 0xffu) << 1) |
                            (spread4(uint32_t(B[2] >> sh) & 0xffu) << 2) |
                            (spread4(uint32_t(B[3] >> sh) & 0xffu) << 3);
      mask[wbase + g * 8 + lane] = word;
      tmask[wbase + g * 8 + lane] = 0u;
    }
  }
  if (lane == 0) {
    tcnt4[trow * 4 + wv] = nsure;
    ccnt4[trow * 4 + wv] = ncand;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = (i * 4 + wv) * 256 + lane * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t key = mag_key(m[i][j]);
      if (e + j < t.len && (key >> 20) == b1) atomicAdd(&h2[(key >> 9) & 0x7ffu], 1u);
    }
  }
}

// ------------------------------------------------------------------ kernels
__global__ __launch_bounds__(256) void rk_zero(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) p[i] = 0u;
}

// Loads of one tile's G and E chunks (16 elements per thread).  A chunk past the tile's
// end reads the tile's first chunk instead (always in bounds) and is then ignored.  With
// `zmask` (a deferred-zero plan whose previous step's zeros are pending) the entries the
// previous step sent read as zero: their bits in that step's sent mask (base and the
// chunk start are multiples of 4, so a chunk's four bits lie in one mask word).
template <typename GT>
__device__ __forceinline__ void load_tile(const RkTile& t, const GT* G, const float* E, const uint32_t* zmask,
                                          int64_t base, v4f (&gv)[4], v4f (&ev)[4], uint32_t (&zw)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = (i * kTileThreads + int(threadIdx.x)) * 4;
    const int ec = e < t.len ? e : 0;
    gv[i] = load_g4(G + base + ec);
    ev[i] = load_nt4(E + base + ec);
    zw[i] = zmask != nullptr ? zmask[(base + ec) >> 5] : 0u;
  }
}

__device__ __forceinline__ v4f zero_sent(v4f v, uint32_t word, int e) {
  const uint32_t b = word >> (e & 31);
  v.x = (b & 1u) ? 0.f : v.x;
  v.y = (b & 2u) ? 0.f : v.y;
  v.z = (b & 4u) ? 0.f : v.z;
  v.w = (b & 8u) ? 0.f : v.w;
  return v;
}

// The state word of a deferred-zero plan's workspace holds the plan's key for the errors
// buffer while the previous step's zeros are pending there (written by rk_emit; cleared
// by in-place materialisation and the stream-ordered reset).  It is read on the device,
// so a step replayed from a captured graph sees changes made between replays.
__device__ __forceinline__ bool zeros_pending(const uint64_t* state, uint64_t key, int use_state) {
  return use_state != 0 && state != nullptr && *state == key;
}

// kEfTiles consecutive tiles of the tile table per workgroup (grid.y = worker).  The
// next tile's loads are issued before the current tile is processed.  The LDS
// histograms are flushed to the segment's global ones (and cleared) whenever the next
// tile belongs to another tensor, and after the last tile.
template <typename GT>
__global__ __launch_bounds__(kTileThreads) void rk_ef_hist(const RkTile* __restrict__ tiles, const GT* __restrict__ G,
                                                           float* __restrict__ E, const uint32_t* __restrict__ pred,
                                                           uint32_t* __restrict__ hist1, uint32_t* __restrict__ hist2,
                                                           uint32_t* __restrict__ mask, uint32_t* __restrict__ tmask,
                                                           uint32_t* __restrict__ tcnt4, uint32_t* __restrict__ cand,
                                                           uint32_t* __restrict__ ccnt4, int64_t stride, int n_layers,
                                                           int ntiles, const uint32_t* __restrict__ sent_prev,
                                                           const uint64_t* __restrict__ state, uint64_t key,
                                                           int use_state) {
  __shared__ uint32_t h1[kBins1];
  __shared__ uint32_t h2[kBins2];
  const int w = blockIdx.y;
  const int t_first = int(blockIdx.x) * kEfTiles;
  const int t_end = min(ntiles, t_first + kEfTiles);
  const uint32_t* zmask = zeros_pending(state, key, use_state) ? sent_prev : nullptr;
  RkTile t = tiles[t_first];
  v4f gv[4], ev[4];
  uint32_t zw[4];
  load_tile(t, G, E, zmask, int64_t(w) * stride + t.begin, gv, ev, zw);
  for (int b = threadIdx.x; b < kBins1; b += kTileThreads) {
    h1[b] = 0u;
    h2[b] = 0u;
  }
  __syncthreads();
  for (int ti = t_first; ti < t_end; ++ti) {
    const bool more = ti + 1 < t_end;
    const RkTile tn = more ? tiles[ti + 1] : t;
    v4f gn[4], en[4];
    uint32_t zn[4];
    if (more) load_tile(tn, G, E, zmask, int64_t(w) * stride + tn.begin, gn, en, zn);
    const int64_t s = int64_t(w) * n_layers + t.layer;
    const uint32_t bp = pred[s];
    const int64_t base = int64_t(w) * stride + t.begin;
    float m[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = (i * kTileThreads + int(threadIdx.x)) * 4;
      const int valid = max(0, min(4, t.len - e));
      v4f mv = gv[i] + (zmask != nullptr ? zero_sent(ev[i], zw[i], e) : ev[i]);
      float* ep = E + base + e;
      if (valid == 4) {
        store_nt4(ep, mv);
      } else {
        for (int j = 0; j < valid; ++j) ep[j] = mv[j];
        if (valid == 0) mv = v4f{0.f, 0.f, 0.f, 0.f};
      }
      m[i][0] = mv.x;
      m[i][1] = mv.y;
      m[i][2] = mv.z;
      m[i][3] = mv.w;
    }
    mark_tile(m, t, bp, base, int64_t(w) * ntiles + ti, h2, mask, tmask, tcnt4, cand, ccnt4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = (i * kTileThreads + int(threadIdx.x)) * 4;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (e + j < t.len) atomicAdd(&h1[mag_key(m[i][j]) >> 20], 1u);
    }
    if (!more || tn.layer != t.layer) {
      __syncthreads();
      uint32_t* g1 = hist1 + s * kBins1;
      uint32_t* g2 = hist2 + s * kBins2;
      for (int b = threadIdx.x; b < kBins1; b += kTileThreads) {
        const uint32_t c1 = h1[b], c2 = h2[b];
        if (c1) atomicAdd(g1 + b, c1);
        if (c2) atomicAdd(g2 + b, c2);
        h1[b] = 0u;
        h2[b] = 0u;
      }
      __syncthreads();
    }
    if (more) {
      t = tn;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        gv[i] = gn[i];
        ev[i] = en[i];
        zw[i] = zn[i];
      }
    }
  }
}

// Per segment: b1 from the digit-1 histogram.  If the prediction the first pass marked
// with was not b1, its digit-2 counts are discarded and rk_mark redoes the segment.
__global__ __launch_bounds__(kSelThreads) void rk_select(const RkLayer* __restrict__ layers,
                                                         const uint32_t* __restrict__ hist1,
                                                         uint32_t* __restrict__ hist2, uint32_t* __restrict__ pred,
                                                         RkSeg* __restrict__ seg, int n_layers) {
  __shared__ uint32_t lds[16], sh[3];
  const int l = blockIdx.x, w = blockIdx.y;
  const int64_t s = int64_t(w) * n_layers + l;
  const uint32_t r = uint32_t(layers[l].top);
  const Pick p = pick_bin<kBins1>(hist1 + s * kBins1, r, lds, sh);
  const bool redo = pred[s] != p.bin;
  if (redo)
    for (int b = threadIdx.x; b < kBins2; b += kSelThreads) hist2[s * kBins2 + b] = 0u;
  __syncthreads();
  if (threadIdx.x == 0) {
    RkSeg st{};
    st.b1 = p.bin;
    st.need1 = r - p.above;
    st.count1 = p.count;
    st.redo = redo ? 1u : 0u;
    st.tkey = seg[s].tkey;
    seg[s] = st;
  }
}

// Mispredicted segments only: re-read M and mark against the true b1.
__global__ __launch_bounds__(kTileThreads) void rk_mark(const RkTile* __restrict__ tiles,
                                                        const float* __restrict__ E, const RkSeg* __restrict__ seg,
                                                        uint32_t* __restrict__ hist2, uint32_t* __restrict__ mask,
                                                        uint32_t* __restrict__ tmask, uint32_t* __restrict__ tcnt4,
                                                        uint32_t* __restrict__ cand, uint32_t* __restrict__ ccnt4,
                                                        int64_t stride, int n_layers, int ntiles) {
  __shared__ uint32_t h2[kBins2];
  const RkTile t = tiles[blockIdx.x];
  const int w = blockIdx.y;
  const int64_t s = int64_t(w) * n_layers + t.layer;
  if (!seg[s].redo) return;  // uniform
  const uint32_t b1 = seg[s].b1;
  for (int b = threadIdx.x; b < kBins2; b += kTileThreads) h2[b] = 0u;
  const int64_t base = int64_t(w) * stride + t.begin;
  float m[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = (i * kTileThreads + int(threadIdx.x)) * 4;
    v4f v = *reinterpret_cast<const v4f*>(E + base + (e < t.len ? e : 0));
    if (e >= t.len) v = v4f{0.f, 0.f, 0.f, 0.f};
    m[i][0] = v.x;
    m[i][1] = v.y;
    m[i][2] = v.z;
    m[i][3] = v.w;
  }
  __syncthreads();
  mark_tile(m, t, b1, base, int64_t(w) * ntiles + blockIdx.x, h2, mask, tmask, tcnt4, cand, ccnt4);
  __syncthreads();
  uint32_t* gh = hist2 + s * kBins2;
  for (int b = threadIdx.x; b < kBins2; b += kTileThreads) {
    const uint32_t c = h2[b];
    if (c) atomicAdd(gh + b, c);
  }
}

// Per segment, once digit 2 is counted: the digit-2 bin b2 (or the segment is settled).
__global__ __launch_bounds__(kSelThreads) void rk_pick2(const uint32_t* __restrict__ hist2, RkSeg* __restrict__ seg,
                                                        int64_t n_seg) {
  __shared__ uint32_t lds[16], sh[3];
  const int64_t s = int64_t(blockIdx.y) * gridDim.x + blockIdx.x;
  const RkSeg st = seg[s];
  if (st.need1 == st.count1) {  // settled by digit 1: all of bin b1 is in
    if (threadIdx.x == 0) {
      seg[s].settled = 1u;
      seg[s].sel_lo = st.b1 << 20;
    }
    return;
  }
  const Pick p2 = pick_bin<kBins2>(hist2 + s * kBins2, st.need1, lds, sh);
  if (threadIdx.x == 0) {
    const uint32_t need2 = st.need1 - p2.above;
    seg[s].b2 = p2.bin;
    seg[s].need2 = need2;
    seg[s].settled = need2 == p2.count ? 1u : 0u;
    seg[s].sel_lo = (st.b1 << 20) | (p2.bin << 9);
  }
}

// The candidate ranges of a chunk (kChunkTiles tiles x 4 waves) flattened into one index
// space: rbeg[r] is range r's element offset in `cand`, pre[r] the number of candidates
// before it, pre[nr] the chunk's total.  Every thread must call it.
struct ChunkRanges {
  int64_t rbeg[kChunkTiles * 4];
  int64_t tbeg[kChunkTiles * 4];  // element offset of the range's tile (entries hold offsets in it)
  uint32_t pre[kChunkTiles * 4 + 1];
};

__device__ __forceinline__ uint32_t chunk_ranges(const RkChunk& ch, const RkLayer& L, const RkTile* __restrict__ tiles,
                                                 const uint32_t* __restrict__ ccnt4, int w, int64_t stride, int ntiles,
                                                 ChunkRanges& cr) {
  const int nr = (ch.t1 - ch.t0) * 4;
  if (threadIdx.x < 64) {  // one wave builds the table
    const int r = threadIdx.x;
    uint32_t n = 0;
    if (r < nr) {
      const int ti = L.tile_off + ch.t0 + (r >> 2);
      const RkTile tl = tiles[ti];
      n = ccnt4[(int64_t(w) * ntiles + ti) * 4 + (r & 3)];
      cr.tbeg[r] = int64_t(w) * stride + tl.begin;
      cr.rbeg[r] = cr.tbeg[r] + wave_region(tl.len, r & 3);
    }
    const uint32_t incl = wave_incl_scan(n);
    if (r < nr) cr.pre[r] = incl - n;
    if (r == 63) cr.pre[nr] = incl;
  }
  __syncthreads();
  return cr.pre[nr];
}

// Range holding flattened item i (pre is non-decreasing; ranges may be empty).
__device__ __forceinline__ int range_of(const ChunkRanges& cr, int nr, uint32_t i) {
  int lo = 0, hi = nr - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cr.pre[mid] <= i) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Digit 3 over the candidates whose digit 2 is b2, for segments not settled by then.
__global__ __launch_bounds__(kSelThreads) void rk_level3(const RkChunk* __restrict__ chunks,
                                                         const RkTile* __restrict__ tiles,
                                                         const RkLayer* __restrict__ layers,
                                                         const RkSeg* __restrict__ seg, uint32_t* __restrict__ hist3,
                                                         const uint32_t* __restrict__ cand,
                                                         const uint32_t* __restrict__ ccnt4, int64_t stride,
                                                         int n_layers, int ntiles) {
  __shared__ uint32_t h3[kBins3];
  const RkChunk ch = chunks[blockIdx.x];
  const int w = blockIdx.y;
  const int64_t s = int64_t(w) * n_layers + ch.layer;
  if (seg[s].settled) return;  // uniform
  const uint32_t b2 = seg[s].b2;
  for (int b = threadIdx.x; b < kBins3; b += kSelThreads) h3[b] = 0u;
  __shared__ ChunkRanges cr;
  const RkLayer L = layers[ch.layer];
  const int nr = (ch.t1 - ch.t0) * 4;
  const uint32_t total = chunk_ranges(ch, L, tiles, ccnt4, w, stride, ntiles, cr);
  for (uint32_t i = threadIdx.x; i < total; i += kSelThreads) {
    const int r = range_of(cr, nr, i);
    const uint32_t e = cand[cr.rbeg[r] + (i - cr.pre[r])];
    if ((e >> 21) == b2) atomicAdd(&h3[(e >> kLocalBits) & 0x1ffu], 1u);
  }
  __syncthreads();
  uint32_t* gh = hist3 + s * kBins3;
  for (int b = threadIdx.x; b < kBins3; b += kSelThreads) {
    const uint32_t c = h3[b];
    if (c) atomicAdd(gh + b, c);
  }
}

// Per segment, once digit 3 is counted: the rule.  Keys >= sel_lo are in; when the
// entries equal to T are only partly in, the first need_t of them in index order are.
//
// The digit-1 bin the next step marks against is predicted here from this step's T and
// the last one's: T moved on by the same amount again (at most four bins of it, else T
// as it is).  Under error feedback the top set's threshold drifts steadily from step to
// step, so T's own bin would miss about every time it crosses a bin edge.  The
// prediction decides only which kernel marks, never a result.
__device__ __forceinline__ void predict_next(RkSeg* __restrict__ seg, uint32_t* __restrict__ pred, int64_t s,
                                             uint32_t t, uint32_t t_last) {
  const int64_t d = int64_t(t) - int64_t(t_last);
  const int64_t next = (d >= -(int64_t(4) << 20) && d <= (int64_t(4) << 20)) ? int64_t(t) + d : int64_t(t);
  seg[s].tkey = t;
  pred[s] = uint32_t(min(max(next, int64_t(0)), int64_t(0x7fffffff)) >> 20);
}

__global__ __launch_bounds__(kSelThreads) void rk_rule(const uint32_t* __restrict__ hist3, RkSeg* __restrict__ seg,
                                                       uint32_t* __restrict__ pred) {
  __shared__ uint32_t lds[16], sh[3];
  const int64_t s = int64_t(blockIdx.y) * gridDim.x + blockIdx.x;
  const RkSeg st = seg[s];
  if (st.settled) {
    if (threadIdx.x == 0) {
      seg[s].partial = 0u;
      predict_next(seg, pred, s, st.sel_lo, st.tkey);
    }
    return;
  }
  const Pick p3 = pick_bin<kBins3>(hist3 + s * kBins3, st.need2, lds, sh);
  if (threadIdx.x == 0) {
    const uint32_t need3 = st.need2 - p3.above;
    const uint32_t t = st.sel_lo | p3.bin;
    if (need3 == p3.count) {
      seg[s].sel_lo = t;
      seg[s].partial = 0u;
    } else {
      seg[s].sel_lo = t + 1u;
      seg[s].tie_key = t;
      seg[s].need_t = need3;
      seg[s].partial = 1u;
    }
    predict_next(seg, pred, s, t, st.tkey);
  }
}

// Apply the segment's rule to the candidates of a chunk of tiles: top-mask bits and a
// per-tile count for those in, tie-mask bits and a per-tile tie count for the partial
// ties.  The bits are gathered in LDS bitmaps of the chunk's tiles and then ORed into
// the masks word by word (no other workgroup touches these tiles' words).
__global__ __launch_bounds__(kSelThreads) void rk_final(const RkChunk* __restrict__ chunks,
                                                        const RkTile* __restrict__ tiles,
                                                        const RkLayer* __restrict__ layers,
                                                        const RkSeg* __restrict__ seg,
                                                        const uint32_t* __restrict__ cand,
                                                        const uint32_t* __restrict__ ccnt4, uint32_t* __restrict__ mask,
                                                        uint32_t* __restrict__ tmask, uint32_t* __restrict__ tfin,
                                                        uint32_t* __restrict__ ttie, int64_t stride, int n_layers,
                                                        int ntiles) {
  constexpr int kTileWords = kTile / 32;
  __shared__ uint32_t c_in[kChunkTiles], c_tie[kChunkTiles];
  __shared__ uint32_t lm[kChunkTiles * kTileWords], lt[kChunkTiles * kTileWords];
  __shared__ ChunkRanges cr;
  const RkChunk ch = chunks[blockIdx.x];
  const int w = blockIdx.y;
  const int64_t s = int64_t(w) * n_layers + ch.layer;
  const uint32_t hi = seg[s].b1 << 20, lo = seg[s].sel_lo, tie = seg[s].tie_key;
  const bool partial = seg[s].partial != 0u;
  if (threadIdx.x < kChunkTiles) {
    c_in[threadIdx.x] = 0u;
    c_tie[threadIdx.x] = 0u;
  }
  for (int i = threadIdx.x; i < kChunkTiles * kTileWords; i += kSelThreads) {
    lm[i] = 0u;
    lt[i] = 0u;
  }
  const RkLayer L = layers[ch.layer];
  const int nr = (ch.t1 - ch.t0) * 4;
  const uint32_t total = chunk_ranges(ch, L, tiles, ccnt4, w, stride, ntiles, cr);  // (a barrier)
  for (uint32_t i = threadIdx.x; i < total; i += kSelThreads) {
    const int r = range_of(cr, nr, i);
    const uint32_t e = cand[cr.rbeg[r] + (i - cr.pre[r])];
    const uint32_t key = hi | (e >> kLocalBits);
    const uint32_t off = e & uint32_t(kTile - 1);
    const int word = (r >> 2) * kTileWords + int(off >> 5);
    if (key >= lo)
      atomicOr(&lm[word], 1u << (off & 31));
    else if (partial && key == tie)
      atomicOr(&lt[word], 1u << (off & 31));
  }
  __syncthreads();
  // tile begins are multiples of 64 elements, so a tile's mask words are its own.  The
  // candidates are distinct entries, so a tile's counts are the popcounts of its bitmap
  // words: summed per wave (a wave's 64 words lie in one tile), one LDS add per wave,
  // instead of one add per candidate on a counter that the whole wave shares
  const int nw = (ch.t1 - ch.t0) * kTileWords;
  for (int i0 = 0; i0 < nw; i0 += kSelThreads) {  // uniform: all lanes reach the sums
    const int i = i0 + int(threadIdx.x);
    uint32_t a = 0u, b = 0u;
    if (i < nw) {
      a = lm[i];
      b = lt[i];
      if ((a | b) != 0u) {
        const int64_t gw = (cr.tbeg[(i / kTileWords) * 4] >> 5) + (i % kTileWords);
        if (a) mask[gw] |= a;
        if (b) tmask[gw] |= b;
      }
    }
    const uint32_t na = wave_sum(uint32_t(__popc(a))), nb = wave_sum(uint32_t(__popc(b)));
    if ((threadIdx.x & 63) == 0 && i < nw) {
      if (na) atomicAdd(&c_in[i / kTileWords], na);
      if (nb) atomicAdd(&c_tie[i / kTileWords], nb);
    }
  }
  __syncthreads();
  if (int(threadIdx.x) < ch.t1 - ch.t0) {
    const int64_t trow = int64_t(w) * ntiles + L.tile_off + ch.t0 + threadIdx.x;
    tfin[trow] = c_in[threadIdx.x];
    ttie[trow] = c_tie[threadIdx.x];
  }
}

// Per segment: the first need_t tie entries in index order join the top set, so each
// tile takes min(its ties, what is left); then exclusive scans give every tile its
// first tie rank and its first slot.
__global__ __launch_bounds__(kSegThreads) void rk_scan_top(const RkLayer* __restrict__ layers,
                                                           const uint32_t* __restrict__ tcnt4,
                                                           const uint32_t* __restrict__ tfin,
                                                           const uint32_t* __restrict__ ttie,
                                                           uint32_t* __restrict__ tbase,
                                                           uint32_t* __restrict__ tiebase, RkSeg* __restrict__ seg,
                                                           int n_layers, int ntiles) {
  __shared__ uint32_t lds[16];
  const int l = blockIdx.x, w = blockIdx.y;
  const int64_t s = int64_t(w) * n_layers + l;
  const RkLayer L = layers[l];
  const uint32_t need_t = seg[s].partial ? seg[s].need_t : 0u;
  const int64_t row = int64_t(w) * ntiles + L.tile_off;
  uint32_t run_tie = 0, run_top = 0;
  for (int c0 = 0; c0 < L.ntiles; c0 += kSegThreads) {
    const int i = c0 + int(threadIdx.x);
    const bool ok = i < L.ntiles;
    const uint32_t vt = ok ? ttie[row + i] : 0u;
    const uint32_t tb = run_tie + block_incl_scan(vt, lds) - vt;
    const uint32_t take = tb >= need_t ? 0u : min(vt, need_t - tb);
    uint32_t v = take;
    if (ok) {
      const uint32_t* c4 = tcnt4 + (row + i) * 4;
      v += c4[0] + c4[1] + c4[2] + c4[3] + tfin[row + i];
    }
    const uint32_t incl = block_incl_scan(v, lds);
    if (ok) {
      tbase[row + i] = run_top + incl - v;
      tiebase[row + i] = tb;
    }
    run_tie += block_total(vt, lds);
    run_top += block_total(v, lds);
  }
  if (threadIdx.x == 0) seg[s].ntop = run_top;
}

// Exclusive scan of a segment's per-tile kept counts; output slots [min(total, k), k)
// get index -1, value 0.
__global__ __launch_bounds__(kSegThreads) void rk_scan_kept(const RkLayer* __restrict__ layers,
                                                            const uint32_t* __restrict__ kcnt,
                                                            uint32_t* __restrict__ kbase, RkSeg* __restrict__ seg,
                                                            int32_t* __restrict__ index, float* __restrict__ value,
                                                            int64_t keep_total, int n_layers, int ntiles) {
  __shared__ uint32_t lds[16];
  const int l = blockIdx.x, w = blockIdx.y;
  const int64_t s = int64_t(w) * n_layers + l;
  const RkLayer L = layers[l];
  const int64_t row = int64_t(w) * ntiles + L.tile_off;
  uint32_t running = 0;
  for (int c0 = 0; c0 < L.ntiles; c0 += kSegThreads) {
    const int i = c0 + int(threadIdx.x);
    const uint32_t v = i < L.ntiles ? kcnt[row + i] : 0u;
    const uint32_t incl = block_incl_scan(v, lds);
    if (i < L.ntiles) kbase[row + i] = running + incl - v;
    running += block_total(v, lds);
  }
  if (threadIdx.x == 0) seg[s].nkept = running;
  int32_t* ix = index + int64_t(w) * keep_total + L.keep_off;
  float* vx = value + int64_t(w) * keep_total + L.keep_off;
  for (int64_t p = int64_t(running) + threadIdx.x; p < L.keep; p += kSegThreads) {
    ix[p] = -1;
    vx[p] = 0.f;
  }
}

// One wave per tile, two mask words (64 elements) per lane; wave scans only.  The top
// set's words (mask, plus the tie entries whose tie rank is below need_t) in index order
// get consecutive slots from the tile's base; those whose rank is below k are kept.
__global__ __launch_bounds__(kWaveBlock) void rk_keep(const RkTile* __restrict__ tiles,
                                                      const RkLayer* __restrict__ layers,
                                                      const RkSeg* __restrict__ seg, const uint32_t* __restrict__ mask,
                                                      const uint32_t* __restrict__ tmask,
                                                      const uint32_t* __restrict__ tbase,
                                                      const uint32_t* __restrict__ tiebase,
                                                      const uint32_t* __restrict__ ranks, uint32_t* __restrict__ kmask,
                                                      uint32_t* __restrict__ kcnt, int64_t stride, int64_t top_total,
                                                      int n_layers, int ntiles) {
  const int ti = blockIdx.x * (kWaveBlock / 64) + (threadIdx.x >> 6);
  if (ti >= ntiles) return;  // whole wave
  const int lane = threadIdx.x & 63;
  const RkTile t = tiles[ti];
  const int w = blockIdx.y;
  const RkLayer L = layers[t.layer];
  const int64_t s = int64_t(w) * n_layers + t.layer;
  const uint32_t need_t = seg[s].partial ? seg[s].need_t : 0u;
  const int nwords = (t.len + 31) >> 5;
  const int q = 2 * lane;
  const int64_t wi = ((int64_t(w) * stride + t.begin) >> 5) + q;
  const int64_t trow = int64_t(w) * ntiles + ti;
  uint32_t m0 = 0, m1 = 0, t0 = 0, t1 = 0;
  if (q < nwords) {
    m0 = mask[wi];
    t0 = tmask[wi];
  }
  if (q + 1 < nwords) {
    m1 = mask[wi + 1];
    t1 = tmask[wi + 1];
  }
  const uint32_t ct = __popc(t0) + __popc(t1);
  uint32_t tr = tiebase[trow] + wave_incl_scan(ct) - ct;
  m0 |= bits_below(t0, tr, need_t);
  m1 |= bits_below(t1, tr, need_t);
  const uint32_t c = __popc(m0) + __popc(m1);
  uint32_t slot = tbase[trow] + wave_incl_scan(c) - c;
  const uint32_t* rk = ranks + int64_t(w) * top_total + L.top_off;
  const uint32_t mw[2] = {m0, m1};
  const uint32_t sw[2] = {slot, slot + uint32_t(__popc(m0))};  // slot of each word's first bit
  uint32_t kw[2] = {0u, 0u};
  // The ranks of the first two set bits of each word (nearly every word has at most
  // two) are loaded together; further bits one at a time, in order.
  bool ok[4];
  uint32_t bit[4], rv[4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t b = mw[h];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int c = 2 * h + r;
      ok[c] = b != 0u && int64_t(sw[h] + r) < L.top;
      bit[c] = b & (0u - b);
      b &= b - 1u;
    }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) rv[c] = ok[c] ? rk[sw[c >> 1] + (c & 1)] : 0u;
#pragma unroll
  for (int c = 0; c < 4; ++c)
    if (ok[c] && int64_t(rv[c]) < L.keep) kw[c >> 1] |= bit[c];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t sl = sw[h] + 2;
    uint32_t bits = mw[h];
    bits &= bits - 1u;
    bits &= bits - 1u;
    for (; bits != 0u; bits &= bits - 1u, ++sl)
      if (int64_t(sl) < L.top && int64_t(rk[sl]) < L.keep) kw[h] |= bits & (0u - bits);
  }
  const uint32_t k0 = kw[0], k1 = kw[1];
  if (q < nwords) kmask[wi] = k0;
  if (q + 1 < nwords) kmask[wi + 1] = k1;
  const uint32_t tot = wave_sum(__popc(k0) + __popc(k1));
  if (lane == 0) kcnt[trow] = tot;
}

// One wave per tile, two mask words per lane: the kept entries in index order take list
// positions from the tile's base; the first k are sent (index, value), their error is
// set to zero, and the kept mask keeps only them; each word records its first position.
__global__ __launch_bounds__(kWaveBlock) void rk_emit(const RkTile* __restrict__ tiles,
                                                      const RkLayer* __restrict__ layers, uint32_t* __restrict__ kmask,
                                                      const uint32_t* __restrict__ kbase, float* __restrict__ E,
                                                      int32_t* __restrict__ index, float* __restrict__ value,
                                                      uint32_t* __restrict__ kpos, int64_t stride, int64_t keep_total,
                                                      int ntiles, uint64_t* __restrict__ state, uint64_t key) {
  // deferred-zero plans (state != NULL): the sent entries keep their value in E, and the
  // state word says that the trimmed sent mask of this step is pending there
  const bool defer = state != nullptr;
  if (defer && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *state = key;
  const int ti = blockIdx.x * (kWaveBlock / 64) + (threadIdx.x >> 6);
  if (ti >= ntiles) return;  // whole wave
  const int lane = threadIdx.x & 63;
  const RkTile t = tiles[ti];
  const int w = blockIdx.y;
  const RkLayer L = layers[t.layer];
  const int nwords = (t.len + 31) >> 5;
  const int q = 2 * lane;
  const int64_t wi = ((int64_t(w) * stride + t.begin) >> 5) + q;
  const uint32_t k0 = q < nwords ? kmask[wi] : 0u;
  const uint32_t k1 = q + 1 < nwords ? kmask[wi + 1] : 0u;
  const uint32_t c = __popc(k0) + __popc(k1);
  const uint32_t first = kbase[int64_t(w) * ntiles + ti] + wave_incl_scan(c) - c;
  if (q >= nwords) return;
  int32_t* ix = index + int64_t(w) * keep_total + L.keep_off;
  float* vx = value + int64_t(w) * keep_total + L.keep_off;
  float* M = E + int64_t(w) * stride + L.offset;
  const int32_t e0 = t.chunk * kTile + q * 32;
  uint32_t sent[2] = {0u, 0u};
  const uint32_t kw[2] = {k0, k1};
  const uint32_t wpos[2] = {first, first + uint32_t(__popc(k0))};  // list position of each word's first bit
  if (q + 1 < nwords) kpos[wi + 1] = wpos[1];
  // The first two set bits of each word (nearly every word has at most two): their
  // values are loaded together, then listed.  Distinct bits are distinct entries, so
  // the loads may all precede the stores.
  bool cok[4];
  int32_t cidx[4];
  float cval[4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t b = kw[h];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int c = 2 * h + r;
      cok[c] = b != 0u && int64_t(wpos[h] + r) < L.keep;
      cidx[c] = e0 + 32 * h + (b != 0u ? __builtin_ctz(b) : 0);
      b &= b - 1u;
    }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) cval[c] = cok[c] ? M[cidx[c]] : 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
    if (cok[c]) {
      const uint32_t pos = wpos[c >> 1] + (c & 1);
      ix[pos] = cidx[c];
      vx[pos] = cval[c];
      if (!defer) M[cidx[c]] = 0.f;
      sent[c >> 1] |= 1u << (cidx[c] - e0 - 32 * (c >> 1));
    }
  // any further set bits, one at a time
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t pos = wpos[h] + 2;
    uint32_t bits = kw[h];
    bits &= bits - 1u;
    bits &= bits - 1u;
    for (; bits != 0u; bits &= bits - 1u, ++pos) {
      if (int64_t(pos) < L.keep) {
        const int32_t idx = e0 + 32 * h + __builtin_ctz(bits);
        ix[pos] = idx;
        vx[pos] = M[idx];
        if (!defer) M[idx] = 0.f;
        sent[h] |= bits & (0u - bits);
      }
    }
  }
  kpos[wi] = first;
  if (sent[0] != k0) kmask[wi] = sent[0];
  if (q + 1 < nwords && sent[1] != k1) kmask[wi + 1] = sent[1];
}

// Dense update, one thread per mask word: for each worker in order, the word's sent
// entries are read from the worker's value list (position = the word's first list
// position + the sent bits below) and added in LDS; the tile is then written with
// coalesced stores.
__global__ __launch_bounds__(kWordThreads) void rk_update(const RkTile* __restrict__ tiles,
                                                          const RkLayer* __restrict__ layers,
                                                          const uint32_t* __restrict__ kmask,
                                                          const uint32_t* __restrict__ kpos,
                                                          const float* __restrict__ value, float* __restrict__ update,
                                                          int W, int64_t stride, int64_t keep_total, float inv_w) {
  __shared__ float acc[kWordThreads][33];
  const RkTile t = tiles[blockIdx.x];
  const RkLayer L = layers[t.layer];
  const int nwords = (t.len + 31) >> 5;
  const int q = threadIdx.x;
#pragma unroll
  for (int j = 0; j < 32; ++j) acc[q][j] = 0.f;
  if (q < nwords) {
    const int64_t wi = (t.begin >> 5) + q;
    const int64_t wstride = stride >> 5;
    // workers in groups of 8: all mask words (then all list positions) of a group are
    // loaded before any is used
    for (int w0 = 0; w0 < W; w0 += 8) {
      uint32_t kw[8], kp[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) kw[k] = w0 + k < W ? kmask[int64_t(w0 + k) * wstride + wi] : 0u;
#pragma unroll
      for (int k = 0; k < 8; ++k) kp[k] = kw[k] != 0u ? kpos[int64_t(w0 + k) * wstride + wi] : 0u;
      // the values of the first two sent entries of each word are loaded together (nearly
      // every word has at most two); they are added in worker order as before
      float v[8][2];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float* vx = value + int64_t(w0 + k) * keep_total + L.keep_off;
        uint32_t b = kw[k];
        v[k][0] = b != 0u ? vx[kp[k]] : 0.f;
        b &= b - 1u;
        v[k][1] = b != 0u ? vx[kp[k] + 1] : 0.f;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float* vx = value + int64_t(w0 + k) * keep_total + L.keep_off;
        uint32_t bits = kw[k];
        uint32_t pos = kp[k];
        if (bits != 0u) {
          acc[q][__builtin_ctz(bits)] += v[k][0];
          bits &= bits - 1u;
          ++pos;
        }
        if (bits != 0u) {
          acc[q][__builtin_ctz(bits)] += v[k][1];
          bits &= bits - 1u;
          ++pos;
        }
        for (; bits != 0u; bits &= bits - 1u) acc[q][__builtin_ctz(bits)] += vx[pos++];
      }
    }
  }
  __syncthreads();
  float* u = update + t.begin;
  for (int e = q; e < t.len; e += kWordThreads) u[e] = acc[e >> 5][e & 31] * inv_w;
}

// The plain error memory of a deferred-zero plan: out = E with the entries the last step
// sent set to zero (when its zeros are pending), per tile and worker, 16 elements per
// thread.  In place (out == E) only the sent entries are written.
__global__ __launch_bounds__(kTileThreads) void rk_materialize(const RkTile* __restrict__ tiles,
                                                               const uint32_t* __restrict__ sent,
                                                               const float* E, float* out,
                                                               const uint64_t* __restrict__ state, uint64_t key,
                                                               int use_state, int64_t stride) {
  const RkTile t = tiles[blockIdx.x];
  const int64_t base = int64_t(blockIdx.y) * stride + t.begin;
  const bool pend = zeros_pending(state, key, use_state);
  const bool in_place = E == out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = (i * kTileThreads + int(threadIdx.x)) * 4;
    if (e >= t.len) continue;
    const int valid = min(4, t.len - e);
    const uint32_t b = pend ? (sent[(base + e) >> 5] >> (e & 31)) & 0xfu : 0u;
    if (in_place) {
      for (int j = 0; j < valid; ++j)
        if (b & (1u << j)) out[base + e + j] = 0.f;
    } else {
      for (int j = 0; j < valid; ++j) out[base + e + j] = (b & (1u << j)) ? 0.f : E[base + e + j];
    }
  }
}

// One thread stores `value` into the workspace's state word (a plain vector store).
__global__ __launch_bounds__(64) void rk_state_store(uint64_t* __restrict__ state, uint64_t value) {
  if (threadIdx.x == 0) *state = value;
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
  RkLayer* layers;
  RkTile* tiles;
  RkChunk* chunks;
};

psgd_status device_tables(psgd_rtopk_plan* plan, DevTables* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("hipGetDevice", e);
  const uint64_t bl = a256(plan->layers.size() * sizeof(RkLayer) + 1);
  const uint64_t bt = a256(plan->tiles.size() * sizeof(RkTile) + 1);
  const uint64_t bc = a256(plan->chunks.size() * sizeof(RkChunk) + 1);
  auto it = plan->dev.find(dev);
  if (it == plan->dev.end()) {
    void* base = nullptr;
    e = hipMalloc(&base, bl + bt + bc);
    if (e != hipSuccess) return fail(PSGD_ERR_NO_MEMORY, std::string("hipMalloc of the plan's device tables: ") +
                                                             hipGetErrorString(e));
    char* b = static_cast<char*>(base);
    e = hipMemcpy(b, plan->layers.data(), plan->layers.size() * sizeof(RkLayer), hipMemcpyHostToDevice);
    if (e == hipSuccess)
      e = hipMemcpy(b + bl, plan->tiles.data(), plan->tiles.size() * sizeof(RkTile), hipMemcpyHostToDevice);
    if (e == hipSuccess)
      e = hipMemcpy(b + bl + bt, plan->chunks.data(), plan->chunks.size() * sizeof(RkChunk), hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      (void)hipFree(base);
      return hip_fail("hipMemcpy of the plan's device tables", e);
    }
    it = plan->dev.emplace(dev, base).first;
  }
  char* b = static_cast<char*>(it->second);
  out->layers = reinterpret_cast<RkLayer*>(b);
  out->tiles = reinterpret_cast<RkTile*>(b + bl);
  out->chunks = reinterpret_cast<RkChunk*>(b + bl + bt);
  return PSGD_OK;
}

psgd_status take_event(psgd_rtopk_plan* plan, hipEvent_t* ev) {
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
psgd_status launch(psgd_rtopk_plan* plan, int kid, void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t st,
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
    return hip_fail((std::string("launch ") + kNames[kid]).c_str(), e);
  }
  if (plan->timing) plan->pending.push_back(PendingTiming{kid, a, b});
  return PSGD_OK;
}

struct Span {
  const char* name;
  uintptr_t lo, hi;
};

// Same device, same error and workspace buffers as the step that left pending zeros.
bool state_matches(const psgd_rtopk_plan* plan, const void* errors, const void* workspace, int dev) {
  return plan->state_valid && plan->state_errors == errors && plan->state_workspace == workspace &&
         plan->state_device == dev;
}

// The value the state word holds while `errors` has this plan's pending zeros: the plan's
// nonce mixed with the buffer address (the splitmix64 finaliser), never 0.
uint64_t state_key(const psgd_rtopk_plan* plan, const void* errors) {
  uint64_t z = plan->nonce ^ (uint64_t(reinterpret_cast<uintptr_t>(errors)) * 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return (z ^ (z >> 31)) | 1u;
}

// A captured call keeps the host's decision for every replay; without usable state the
// replays would never apply the zeros earlier replays leave pending, so such a capture
// is refused.
psgd_status check_capture(const char* fn, bool deferred, bool use_state, hipStream_t st) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (deferred && !use_state && hipStreamIsCapturing(st, &cs) == hipSuccess && cs == hipStreamCaptureStatusActive)
    return fail(PSGD_ERR_INVALID_ARG, std::string(fn) + ": a deferred-zero plan can be captured into a graph only "
                                          "after an eager step of the plan on the same errors and workspace");
  return PSGD_OK;
}

}  // namespace
}  // namespace rtk
}  // namespace psgd

using namespace psgd;
using namespace psgd::rtk;

extern "C" psgd_status psgd_rtopk_plan_create(const psgd_layer* layers, int32_t n_layers, const int64_t* top,
                                              const int64_t* keep, int32_t n_workers, psgd_dtype grad_dtype,
                                              uint32_t flags, psgd_rtopk_plan** out) {
  if (out == nullptr) return fail(PSGD_ERR_INVALID_ARG, "psgd_rtopk_plan_create: out is NULL");
  *out = nullptr;
  if (n_layers < 1) return fail(PSGD_ERR_INVALID_ARG, "psgd_rtopk_plan_create: n_layers must be >= 1");
  if (layers == nullptr || top == nullptr || keep == nullptr)
    return fail(PSGD_ERR_INVALID_ARG, "psgd_rtopk_plan_create: layers, top or keep is NULL");
  if (n_workers < 1 || n_workers > 65535)
    return fail(PSGD_ERR_INVALID_ARG, "psgd_rtopk_plan_create: n_workers must be in 1..65535");
  if (grad_dtype != PSGD_F32 && grad_dtype != PSGD_BF16)
    return fail(PSGD_ERR_UNSUPPORTED, "psgd_rtopk_plan_create: unknown grad_dtype");
  if (flags & ~uint32_t(PSGD_RTOPK_FLAG_DEFERRED_ZERO))
    return fail(PSGD_ERR_UNSUPPORTED, "psgd_rtopk_plan_create: unknown flag bits");
  psgd_rtopk_plan* plan = nullptr;
  try {
    plan = new psgd_rtopk_plan();
    plan->n_workers = n_workers;
    plan->dtype = grad_dtype;
    plan->flags = flags;
    {  // a key no other plan's state word is likely to hold: random bits, the clock, a counter
      static std::atomic<uint64_t> counter{0};
      uint64_t nonce = (++counter) * 0xD1B54A32D192ED03ull ^
                       uint64_t(std::chrono::steady_clock::now().time_since_epoch().count());
      try {
        std::random_device rd;
        nonce ^= uint64_t(rd()) << 32 | rd();
      } catch (...) {
      }
      plan->nonce = nonce;
    }
    int64_t off = 0, tile_count = 0;
    for (int32_t i = 0; i < n_layers; ++i) {
      const int64_t rows = layers[i].rows, cols = layers[i].cols;
      if (rows < 1 || cols < 1 || rows > (int64_t(1) << 31) || cols > (int64_t(1) << 31) ||
          rows * cols > int64_t(0x7fffffff)) {
        delete plan;
        return fail(PSGD_ERR_INVALID_ARG, "psgd_rtopk_plan_create: layer " + std::to_string(i) +
                                              " needs 1 <= rows*cols < 2^31");
      }
      const int64_t numel = rows * cols;
      if (keep[i] < 1 || keep[i] > top[i] || top[i] > numel) {
        delete plan;
        return fail(PSGD_ERR_INVALID_ARG, "psgd_rtopk_plan_create: layer " + std::to_string(i) +
                                              " needs 1 <= keep <= top <= rows*cols");
      }
      psgd_rtopk_layer_info li{};
      li.rows = rows;
      li.cols = cols;
      li.numel = numel;
      li.offset = off;
      li.top = top[i];
      li.keep = keep[i];
      li.top_offset = plan->top_total;
      li.keep_offset = plan->keep_total;
      RkLayer L{};
      L.offset = off;
      L.numel = numel;
      L.top = top[i];
      L.keep = keep[i];
      L.top_off = plan->top_total;
      L.keep_off = plan->keep_total;
      L.ntiles = int32_t((numel + kTile - 1) / kTile);
      L.tile_off = int32_t(tile_count);
      for (int32_t c = 0; c < L.ntiles; ++c) {
        RkTile t{};
        t.begin = off + int64_t(c) * kTile;
        t.layer = i;
        t.len = int32_t(std::min<int64_t>(kTile, numel - int64_t(c) * kTile));
        t.chunk = c;
        plan->tiles.push_back(t);
      }
      for (int32_t c = 0; c < L.ntiles; c += kChunkTiles)
        plan->chunks.push_back(RkChunk{i, c, std::min(L.ntiles, c + kChunkTiles), c == 0 ? 1 : 0});
      tile_count += L.ntiles;
      if (tile_count > int64_t(0x7fffffff)) {
        delete plan;
        return fail(PSGD_ERR_INVALID_ARG, "psgd_rtopk_plan_create: too many tiles");
      }
      plan->top_total += top[i];
      plan->keep_total += keep[i];
      plan->numel += numel;
      plan->info.push_back(li);
      plan->layers.push_back(L);
      off = (off + numel + kAlignElems - 1) / kAlignElems * kAlignElems;
    }
    plan->worker_stride = off;
    plan->n_seg = int64_t(n_workers) * n_layers;
    const uint64_t W = uint64_t(n_workers);
    const uint64_t ntiles = plan->tiles.size();
    const uint64_t words = uint64_t(plan->worker_stride / 32);
    uint64_t ws = 0;
    // the three digit histograms are contiguous: one fill clears them
    plan->ws_hist1 = ws;
    ws += uint64_t(plan->n_seg) * kBins1 * 4;
    plan->ws_hist2 = ws;
    ws += uint64_t(plan->n_seg) * kBins2 * 4;
    plan->ws_hist3 = ws;
    ws = a256(ws + uint64_t(plan->n_seg) * kBins3 * 4);
    plan->ws_seg = ws;
    ws = a256(ws + uint64_t(plan->n_seg) * sizeof(RkSeg));
    plan->ws_pred = ws;  // predicted digit-1 bin per segment (a hint only)
    ws = a256(ws + uint64_t(plan->n_seg) * 4);
    plan->ws_cand = ws;  // same layout as the error buffer, one uint32 per element
    ws = a256(ws + W * uint64_t(plan->worker_stride) * 4);
    uint64_t* word_arrays[] = {&plan->ws_mask, &plan->ws_tmask, &plan->ws_kmask, &plan->ws_kpos};
    for (uint64_t* a : word_arrays) {
      *a = ws;
      ws = a256(ws + W * words * 4);
    }
    uint64_t* wave_arrays[] = {&plan->ws_ccnt4, &plan->ws_tcnt4};  // one count per wave of a tile
    for (uint64_t* a : wave_arrays) {
      *a = ws;
      ws = a256(ws + W * ntiles * 16);
    }
    uint64_t* tile_arrays[] = {&plan->ws_tfin, &plan->ws_ttie, &plan->ws_tiebase, &plan->ws_tbase, &plan->ws_kcnt,
                               &plan->ws_kbase};
    for (uint64_t* a : tile_arrays) {
      *a = ws;
      ws = a256(ws + W * ntiles * 4);
    }
    plan->ws_state = ws;  // one 64-bit state word (deferred-zero plans)
    ws += 256;
    plan->workspace_bytes = ws;
    const uint64_t gb = grad_dtype == PSGD_BF16 ? 2 : 4;
    plan->message_bytes = uint64_t(plan->keep_total) * 8;
    plan->model_bytes = (W * (gb + 8) + 4) * uint64_t(plan->numel);
  } catch (const std::bad_alloc&) {
    delete plan;
    return fail(PSGD_ERR_NO_MEMORY, "psgd_rtopk_plan_create: out of host memory");
  }
  *out = plan;
  return PSGD_OK;
}

extern "C" psgd_status psgd_rtopk_plan_sizes(const psgd_rtopk_plan* plan, psgd_rtopk_sizes* out) {
  if (plan == nullptr || out == nullptr) return fail(PSGD_ERR_INVALID_ARG, "psgd_rtopk_plan_sizes: NULL argument");
  psgd_rtopk_sizes s{};
  s.n_layers = int32_t(plan->info.size());
  s.n_workers = plan->n_workers;
  s.grad_dtype = int32_t(plan->dtype);
  s.worker_stride = plan->worker_stride;
  s.numel = plan->numel;
  s.top_total = plan->top_total;
  s.keep_total = plan->keep_total;
  s.workspace_bytes = plan->workspace_bytes;
  s.message_bytes = plan->message_bytes;
  s.model_bytes = plan->model_bytes;
  *out = s;
  return PSGD_OK;
}

extern "C" psgd_status psgd_rtopk_plan_layer_info(const psgd_rtopk_plan* plan, int32_t layer,
                                             psgd_rtopk_layer_info* out) {
  if (plan == nullptr || out == nullptr) return fail(PSGD_ERR_INVALID_ARG, "psgd_rtopk_plan_layer_info: NULL argument");
  if (layer < 0 || size_t(layer) >= plan->info.size())
    return fail(PSGD_ERR_INVALID_ARG, "psgd_rtopk_plan_layer_info: layer index out of range");
  *out = plan->info[size_t(layer)];
  return PSGD_OK;
}

extern "C" psgd_status psgd_rtopk_plan_destroy(psgd_rtopk_plan* plan) {
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
      set_error("psgd_rtopk_plan_destroy: hipFree of the device tables failed");
      st = PSGD_ERR_HIP;
    }
    if (have && cur != kv.first) (void)hipSetDevice(cur);
  }
  delete plan;
  return st;
}

extern "C" psgd_status psgd_rtopk_plan_set_timing(psgd_rtopk_plan* plan, int32_t enable) {
  if (plan == nullptr) return fail(PSGD_ERR_INVALID_ARG, "psgd_rtopk_plan_set_timing: plan is NULL");
  plan->timing = enable != 0;
  return PSGD_OK;
}

extern "C" psgd_status psgd_rtopk_plan_kernel_stats(psgd_rtopk_plan* plan, psgd_kernel_stat* out, int32_t capacity,
                                                    int32_t* count, int32_t reset) {
  if (plan == nullptr) return fail(PSGD_ERR_INVALID_ARG, "psgd_rtopk_plan_kernel_stats: plan is NULL");
  if (capacity > 0 && out == nullptr) return fail(PSGD_ERR_INVALID_ARG, "psgd_rtopk_plan_kernel_stats: out is NULL");
  psgd_status st = PSGD_OK;
  for (const PendingTiming& t : plan->pending) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(t.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, t.start, t.stop);
    if (e != hipSuccess) {
      set_error(std::string("psgd_rtopk_plan_kernel_stats: ") + hipGetErrorString(e));
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

extern "C" psgd_status psgd_rtopk_step(psgd_rtopk_plan* plan, const void* grads, float* errors,
                                       const uint32_t* ranks, int32_t* index, float* value, float* update,
                                       void* workspace, void* stream) {
  static const char* fn = "psgd_rtopk_step";
  if (plan == nullptr) return fail(PSGD_ERR_INVALID_ARG, "psgd_rtopk_step: plan is NULL");
  const uint64_t W = uint64_t(plan->n_workers);
  const uint64_t gb = plan->dtype == PSGD_BF16 ? 2 : 4;
  const uint64_t stride = uint64_t(plan->worker_stride);
  const Span spans[] = {
      {"grads", uintptr_t(grads), uintptr_t(grads) + W * stride * gb},
      {"errors", uintptr_t(errors), uintptr_t(errors) + W * stride * 4},
      {"ranks", uintptr_t(ranks), uintptr_t(ranks) + W * uint64_t(plan->top_total) * 4},
      {"index", uintptr_t(index), uintptr_t(index) + W * uint64_t(plan->keep_total) * 4},
      {"value", uintptr_t(value), uintptr_t(value) + W * uint64_t(plan->keep_total) * 4},
      {"update", uintptr_t(update), uintptr_t(update) + stride * 4},
      {"workspace", uintptr_t(workspace), uintptr_t(workspace) + plan->workspace_bytes},
  };
  for (const Span& sp : spans) {
    const bool nullable = std::string(sp.name) == "update";
    if (sp.lo == 0) {
      if (nullable) continue;
      return fail(PSGD_ERR_INVALID_ARG, std::string(fn) + ": " + sp.name + " is NULL");
    }
    if (sp.lo % 16 != 0) return fail(PSGD_ERR_INVALID_ARG, std::string(fn) + ": " + sp.name + " is not 16-byte aligned");
  }
  for (size_t i = 0; i < sizeof(spans) / sizeof(spans[0]); ++i)
    for (size_t j = i + 1; j < sizeof(spans) / sizeof(spans[0]); ++j) {
      const Span &a = spans[i], &b = spans[j];
      if (a.lo == 0 || b.lo == 0) continue;
      if (a.lo < b.hi && b.lo < a.hi)
        return fail(PSGD_ERR_INVALID_ARG, std::string(fn) + ": " + a.name + " and " + b.name + " overlap");
    }
  int dev = 0;
  hipError_t he = hipGetDevice(&dev);
  if (he != hipSuccess) return hip_fail("hipGetDevice", he);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool deferred = (plan->flags & PSGD_RTOPK_FLAG_DEFERRED_ZERO) != 0;
  const bool use_state = deferred && state_matches(plan, errors, workspace, dev);
  psgd_status s = check_capture(fn, deferred, use_state, st);
  if (s != PSGD_OK) return s;
  DevTables dt{};
  if ((s = device_tables(plan, &dt)) != PSGD_OK) return s;
  plan->state_valid = false;

  char* ws = static_cast<char*>(workspace);
  auto u32 = [&](uint64_t off) { return reinterpret_cast<uint32_t*>(ws + off); };
  uint32_t* hist1 = u32(plan->ws_hist1);
  uint32_t* hist2 = u32(plan->ws_hist2);
  uint32_t* hist3 = u32(plan->ws_hist3);
  RkSeg* seg = reinterpret_cast<RkSeg*>(ws + plan->ws_seg);
  uint32_t* pred = u32(plan->ws_pred);
  uint32_t* cand = u32(plan->ws_cand);
  uint32_t *mask = u32(plan->ws_mask), *tmask = u32(plan->ws_tmask), *kmask = u32(plan->ws_kmask);
  uint32_t* kpos = u32(plan->ws_kpos);
  uint32_t *ccnt4 = u32(plan->ws_ccnt4), *tcnt4 = u32(plan->ws_tcnt4), *tfin = u32(plan->ws_tfin);
  uint32_t* ttie = u32(plan->ws_ttie);
  uint32_t *tiebase = u32(plan->ws_tiebase), *tbase = u32(plan->ws_tbase);
  uint32_t *kcnt = u32(plan->ws_kcnt), *kbase = u32(plan->ws_kbase);
  uint64_t* state = deferred ? reinterpret_cast<uint64_t*>(ws + plan->ws_state) : nullptr;
  const uint64_t key = state_key(plan, errors);
  const int ust = use_state ? 1 : 0;

  const int nl = int(plan->layers.size());
  const int ntiles = int(plan->tiles.size());
  const int64_t sstride = int64_t(stride);
  const dim3 tgrid(static_cast<unsigned>(ntiles), static_cast<unsigned>(W));
  const dim3 egrid(static_cast<unsigned>((ntiles + kEfTiles - 1) / kEfTiles), static_cast<unsigned>(W));
  const dim3 sgrid(static_cast<unsigned>(nl), static_cast<unsigned>(W));
  const dim3 cgrid(static_cast<unsigned>(plan->chunks.size()), static_cast<unsigned>(W));
  const int64_t nzero = int64_t(plan->n_seg) * (kBins1 + kBins2 + kBins3);
  const unsigned zblocks = unsigned(std::min<int64_t>((nzero + 255) / 256, 4096));
  const RkLayer* L = dt.layers;
  const RkTile* T = dt.tiles;
  const RkChunk* C = dt.chunks;

  if ((s = launch(plan, kZero, rk_zero, dim3(zblocks), dim3(256), st, hist1, nzero)) != PSGD_OK) return s;
  const uint32_t* cpred = pred;
  if (plan->dtype == PSGD_BF16)
    s = launch(plan, kEfHist, rk_ef_hist<uint16_t>, egrid, dim3(kTileThreads), st, T,
               static_cast<const uint16_t*>(grads), errors, cpred, hist1, hist2, mask, tmask, tcnt4, cand, ccnt4,
               sstride, nl, ntiles, static_cast<const uint32_t*>(kmask), static_cast<const uint64_t*>(state), key,
               ust);
  else
    s = launch(plan, kEfHist, rk_ef_hist<float>, egrid, dim3(kTileThreads), st, T, static_cast<const float*>(grads),
               errors, cpred, hist1, hist2, mask, tmask, tcnt4, cand, ccnt4, sstride, nl, ntiles,
               static_cast<const uint32_t*>(kmask), static_cast<const uint64_t*>(state), key, ust);
  if (s != PSGD_OK) return s;
  if ((s = launch(plan, kSelect, rk_select, sgrid, dim3(kSelThreads), st, L, static_cast<const uint32_t*>(hist1),
                  hist2, pred, seg, nl)) != PSGD_OK)
    return s;
  if ((s = launch(plan, kMark, rk_mark, tgrid, dim3(kTileThreads), st, T, static_cast<const float*>(errors),
                  static_cast<const RkSeg*>(seg), hist2, mask, tmask, tcnt4, cand, ccnt4, sstride, nl, ntiles)) !=
      PSGD_OK)
    return s;
  if ((s = launch(plan, kPick2, rk_pick2, sgrid, dim3(kSelThreads), st, static_cast<const uint32_t*>(hist2), seg,
                  plan->n_seg)) != PSGD_OK)
    return s;
  if ((s = launch(plan, kLevel3, rk_level3, cgrid, dim3(kSelThreads), st, C, T, L, static_cast<const RkSeg*>(seg),
                  hist3, static_cast<const uint32_t*>(cand), static_cast<const uint32_t*>(ccnt4), sstride, nl,
                  ntiles)) != PSGD_OK)
    return s;
  if ((s = launch(plan, kRule, rk_rule, sgrid, dim3(kSelThreads), st, static_cast<const uint32_t*>(hist3), seg,
                  pred)) != PSGD_OK)
    return s;
  if ((s = launch(plan, kFinal, rk_final, cgrid, dim3(kSelThreads), st, C, T, L, static_cast<const RkSeg*>(seg),
                  static_cast<const uint32_t*>(cand), static_cast<const uint32_t*>(ccnt4), mask, tmask, tfin, ttie,
                  sstride, nl, ntiles)) != PSGD_OK)
    return s;
  if ((s = launch(plan, kScanTop, rk_scan_top, sgrid, dim3(kSegThreads), st, L, static_cast<const uint32_t*>(tcnt4),
                  static_cast<const uint32_t*>(tfin), static_cast<const uint32_t*>(ttie), tbase, tiebase, seg, nl,
                  ntiles)) != PSGD_OK)
    return s;
  const dim3 wgrid(static_cast<unsigned>((ntiles + kWaveBlock / 64 - 1) / (kWaveBlock / 64)), static_cast<unsigned>(W));
  if ((s = launch(plan, kKeep, rk_keep, wgrid, dim3(kWaveBlock), st, T, L, static_cast<const RkSeg*>(seg),
                  static_cast<const uint32_t*>(mask), static_cast<const uint32_t*>(tmask),
                  static_cast<const uint32_t*>(tbase), static_cast<const uint32_t*>(tiebase), ranks, kmask, kcnt,
                  sstride, plan->top_total, nl, ntiles)) != PSGD_OK)
    return s;
  if ((s = launch(plan, kScanKept, rk_scan_kept, sgrid, dim3(kSegThreads), st, L, static_cast<const uint32_t*>(kcnt),
                  kbase, seg, index, value, plan->keep_total, nl, ntiles)) != PSGD_OK)
    return s;
  if ((s = launch(plan, kEmit, rk_emit, wgrid, dim3(kWaveBlock), st, T, L, kmask,
                  static_cast<const uint32_t*>(kbase), errors, index, value, kpos, sstride, plan->keep_total,
                  ntiles, state, key)) != PSGD_OK)
    return s;
  if (update != nullptr)
    s = launch(plan, kUpdate, rk_update, dim3(unsigned(ntiles)), dim3(kWordThreads), st, T, L,
               static_cast<const uint32_t*>(kmask), static_cast<const uint32_t*>(kpos),
               static_cast<const float*>(value), update, int(W), sstride, plan->keep_total, 1.0f / float(W));
  if (s == PSGD_OK && deferred) {
    plan->state_valid = true;
    plan->state_errors = errors;
    plan->state_workspace = workspace;
    plan->state_device = dev;
  }
  return s;
}

extern "C" psgd_status psgd_rtopk_errors_materialize(psgd_rtopk_plan* plan, const float* errors, float* out,
                                                     void* workspace, void* stream) {
  static const char* fn = "psgd_rtopk_errors_materialize";
  if (plan == nullptr) return fail(PSGD_ERR_INVALID_ARG, std::string(fn) + ": plan is NULL");
  const uintptr_t ptrs[] = {uintptr_t(errors), uintptr_t(out), uintptr_t(workspace)};
  for (uintptr_t p : ptrs)
    if (p == 0 || p % 16 != 0) return fail(PSGD_ERR_INVALID_ARG, std::string(fn) + ": NULL or misaligned pointer");
  const uint64_t bytes = uint64_t(plan->n_workers) * uint64_t(plan->worker_stride) * 4;
  const uintptr_t e0 = uintptr_t(errors), o0 = uintptr_t(out);
  if (out != errors && e0 < o0 + bytes && o0 < e0 + bytes)
    return fail(PSGD_ERR_INVALID_ARG, std::string(fn) + ": out partly overlaps errors (pass the same pointer for in place)");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("hipGetDevice", e);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool deferred = (plan->flags & PSGD_RTOPK_FLAG_DEFERRED_ZERO) != 0;
  const bool use_state = deferred && state_matches(plan, errors, workspace, dev);
  if (!use_state && out == errors) return PSGD_OK;  // nothing pending: already plain
  psgd_status s = check_capture(fn, deferred, use_state, st);
  if (s != PSGD_OK) return s;
  DevTables dt{};
  if ((s = device_tables(plan, &dt)) != PSGD_OK) return s;
  char* ws = static_cast<char*>(workspace);
  uint64_t* state = deferred ? reinterpret_cast<uint64_t*>(ws + plan->ws_state) : nullptr;
  hipLaunchKernelGGL(rk_materialize, dim3(unsigned(plan->tiles.size()), unsigned(plan->n_workers)),
                     dim3(kTileThreads), 0, st, static_cast<const RkTile*>(dt.tiles),
                     reinterpret_cast<const uint32_t*>(ws + plan->ws_kmask), errors, out,
                     static_cast<const uint64_t*>(state), state_key(plan, errors), use_state ? 1 : 0,
                     plan->worker_stride);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail("launch rk_materialize", e);
  if (use_state && out == errors) {  // the buffer now holds plain errors
    plan->state_valid = false;
    hipLaunchKernelGGL(rk_state_store, dim3(1), dim3(64), 0, st, state, uint64_t(0));
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail("launch rk_state_store", e);
  }
  return PSGD_OK;
}

extern "C" psgd_status psgd_rtopk_plan_reset_state(psgd_rtopk_plan* plan, void* workspace, void* stream) {
  static const char* fn = "psgd_rtopk_plan_reset_state";
  if (plan == nullptr) return fail(PSGD_ERR_INVALID_ARG, std::string(fn) + ": plan is NULL");
  if (workspace == nullptr || uintptr_t(workspace) % 16 != 0)
    return fail(PSGD_ERR_INVALID_ARG, std::string(fn) + ": workspace is NULL or misaligned");
  plan->state_valid = false;
  if (!(plan->flags & PSGD_RTOPK_FLAG_DEFERRED_ZERO)) return PSGD_OK;
  hipLaunchKernelGGL(rk_state_store, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                     reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) + plan->ws_state), uint64_t(0));
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? PSGD_OK : hip_fail("launch rk_state_store", e);
}
