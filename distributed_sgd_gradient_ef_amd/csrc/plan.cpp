// Host side of libpsgd: plan creation and validation, the packed layout, the tile
// work-lists of the batched launches, and byte accounting.  No HIP call is made here
// except freeing a plan's device tables.

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <new>
#include <random>
#include <string>

#include "plan.hpp"

namespace psgd {

static thread_local std::string g_last_error;

const char* const kKernelNames[kNumKernels] = {"k_first",      "k_mgs",         "k_q_partial",  "k_q_reduce",
                                               "k_apply",      "k_update",      "k_p_mbar",     "k_qw_partial",
                                               "k_qw_reduce",  "k_tall_rows",   "k_tall_apply"};

void set_error(const std::string& msg) { g_last_error = msg; }

static int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

}  // namespace psgd

using namespace psgd;

extern "C" const char* psgd_status_string(psgd_status s) {
  switch (s) {
    case PSGD_OK: return "ok";
    case PSGD_ERR_INVALID_ARG: return "invalid argument";
    case PSGD_ERR_UNSUPPORTED: return "unsupported";
    case PSGD_ERR_NO_MEMORY: return "out of memory";
    case PSGD_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

extern "C" const char* psgd_last_error(void) { return g_last_error.c_str(); }

static psgd_status fail(psgd_status s, const std::string& msg) {
  set_error(msg);
  return s;
}

// A tensor is compressed when it is 2-D and its smaller side exceeds the rank; a
// rank-r factorisation of anything smaller would not compress it.
static bool is_compressed(int64_t rows, int64_t cols, int rank) {
  return rows > 1 && cols > 1 && std::min(rows, cols) > rank;
}

extern "C" psgd_status psgd_plan_create(const psgd_layer* layers, int32_t n_layers, int32_t rank,
                                        int32_t n_workers, psgd_dtype grad_dtype, uint32_t flags,
                                        psgd_plan** out) {
  if (out == nullptr) return fail(PSGD_ERR_INVALID_ARG, "psgd_plan_create: out is NULL");
  *out = nullptr;
  if (layers == nullptr) return fail(PSGD_ERR_INVALID_ARG, "psgd_plan_create: layers is NULL");
  if (n_layers < 1) return fail(PSGD_ERR_INVALID_ARG, "psgd_plan_create: n_layers must be >= 1");
  if (rank < 1 || rank > 4)
    return fail(PSGD_ERR_UNSUPPORTED, "psgd_plan_create: rank must be in 1..4, got " + std::to_string(rank));
  if (n_workers < 1 || n_workers > 65536)
    return fail(PSGD_ERR_INVALID_ARG, "psgd_plan_create: n_workers must be in 1..65536");
  if (grad_dtype != PSGD_F32 && grad_dtype != PSGD_BF16)
    return fail(PSGD_ERR_UNSUPPORTED, "psgd_plan_create: unknown gradient dtype");
  if (flags & ~uint32_t(PSGD_FLAG_NESTEROV | PSGD_FLAG_CARRY_ERROR_MEAN | PSGD_FLAG_DEFERRED_ERROR |
                        PSGD_FLAG_LOCAL_Q_ERROR))
    return fail(PSGD_ERR_UNSUPPORTED, "psgd_plan_create: unknown flag bits");
  if ((flags & PSGD_FLAG_CARRY_ERROR_MEAN) && (flags & PSGD_FLAG_DEFERRED_ERROR))
    return fail(PSGD_ERR_UNSUPPORTED, "psgd_plan_create: PSGD_FLAG_CARRY_ERROR_MEAN and PSGD_FLAG_DEFERRED_ERROR exclude each other");
  if ((flags & PSGD_FLAG_LOCAL_Q_ERROR) && (flags & (PSGD_FLAG_CARRY_ERROR_MEAN | PSGD_FLAG_DEFERRED_ERROR)))
    return fail(PSGD_ERR_UNSUPPORTED,
                "psgd_plan_create: PSGD_FLAG_LOCAL_Q_ERROR excludes PSGD_FLAG_CARRY_ERROR_MEAN and PSGD_FLAG_DEFERRED_ERROR");

  psgd_plan* plan = new (std::nothrow) psgd_plan();
  if (plan == nullptr) return fail(PSGD_ERR_NO_MEMORY, "psgd_plan_create: out of host memory");
  try {
    plan->rank = rank;
    plan->n_workers = n_workers;
    plan->dtype = grad_dtype;
    plan->flags = flags;
    {  // a key no other plan's state word is likely to hold: random bits, the clock, a counter
      static std::atomic<uint64_t> counter{0};
      uint64_t nonce = (++counter) * 0x9E3779B97F4A7C15ull ^
                       uint64_t(std::chrono::steady_clock::now().time_since_epoch().count());
      try {
        std::random_device rd;
        nonce ^= uint64_t(rd()) << 32 | rd();
      } catch (...) {
      }
      plan->nonce = nonce;
    }
    const int64_t r = rank;
    int64_t off = 0, p_off = 0, q_off = 0, qpart = 0;
    for (int32_t i = 0; i < n_layers; ++i) {
      const int64_t rows = layers[i].rows, cols = layers[i].cols;
      if (rows < 1 || cols < 1) {
        delete plan;
        return fail(PSGD_ERR_INVALID_ARG, "psgd_plan_create: layer " + std::to_string(i) + " has a non-positive dimension");
      }
      if (rows > (int64_t(1) << 31) / cols || rows * cols >= (int64_t(1) << 31)) {
        delete plan;
        return fail(PSGD_ERR_INVALID_ARG, "psgd_plan_create: layer " + std::to_string(i) + " has 2^31 or more elements");
      }
      const int64_t numel = rows * cols;
      psgd_layer_info li{};
      li.rows = rows;
      li.cols = cols;
      li.offset = off;
      li.compressed = is_compressed(rows, cols, rank) ? 1 : 0;
      if (li.compressed) {
        li.matrix_index = int32_t(plan->mats.size());
        li.p_offset = p_off;
        li.q_offset = q_off;
        MatInfo mi{};
        mi.offset = off;
        mi.p_off = p_off;
        mi.q_off = q_off;
        mi.rows = int32_t(rows);
        mi.cols = int32_t(cols);
        mi.vw = (cols % 4 == 0) ? 4 : (cols % 2 == 0) ? 2 : 1;
        mi.flat = (cols >= kFlatMinCols && cols % 32 != 0) ? 1 : 0;
        if (mi.flat) {
          // a row of cols elements starting at offset o < kStreamTileElems within a chunk
          // overlaps ceil((o + cols) / kStreamTileElems) chunks
          mi.nstrips = int32_t((cols + 2 * kStreamTileElems - 2) / kStreamTileElems);
        } else {
          const int64_t strip_cols = int64_t(kStreamThreads) * (mi.vw == 1 ? 1 : 4);
          mi.nstrips = int32_t((cols + strip_cols - 1) / strip_cols);
        }
        mi.ppart_off = plan->ppart_elems;
        plan->ppart_elems += int64_t(mi.nstrips) * rows * r;
        plan->mats.push_back(mi);
        // each matrix's P and Q block starts on a 16-byte boundary
        p_off += round_up(rows * r, 4);
        q_off += round_up(cols * r, 4);
        plan->matrix_numel += numel;
        plan->max_q_elems_per_matrix = std::max(plan->max_q_elems_per_matrix, cols * r);
        plan->message_bytes += uint64_t(4) * uint64_t((rows + cols) * r);
      } else {
        li.matrix_index = -1;
        li.p_offset = -1;
        li.q_offset = -1;
        plan->vector_numel += numel;
        plan->message_bytes += uint64_t(4) * uint64_t(numel);
      }
      plan->layers.push_back(li);
      off = round_up(off + numel, kAlignElems);
      plan->numel += numel;
    }
    plan->worker_stride = off;
    plan->p_elems = p_off;
    plan->q_elems = q_off;

    // Q-pass row blocks: at most kQMaxRowBlocks, unless the matrix's share of the plan's
    // elements asks for more of the launch's kQTargetTiles tiles (a single tall, narrow
    // matrix would otherwise stream through a few workgroups).
    for (MatInfo& mi : plan->mats) {
      const int64_t rows = mi.rows, cols = mi.cols;
      const int64_t most = (rows + kQTargetRowsPerBlock - 1) / kQTargetRowsPerBlock;
      const int64_t strip = int64_t(kQThreads) * (mi.vw == 1 ? 1 : 4);
      const int64_t strips = (cols + strip - 1) / strip;
      const int64_t share = (kQTargetTiles * rows * cols + plan->matrix_numel * strips - 1) /
                            (plan->matrix_numel * strips);
      const int64_t nblk = std::min(most, std::max<int64_t>(std::min<int64_t>(most, kQMaxRowBlocks), share));
      mi.rows_per_blk = int32_t((rows + nblk - 1) / nblk);
      mi.nblk = int32_t((rows + mi.rows_per_blk - 1) / mi.rows_per_blk);
      mi.qpart_off = qpart;
      qpart += int64_t(mi.nblk) * cols * r;
      // about eight partials per wave
      plan->qred_waves = std::max(plan->qred_waves, std::min((mi.nblk + 7) / 8, kQRedMaxWaves));
    }
    plan->qpart_elems = qpart;

    // Tall matrices: blocks of kTallRows rows for the two row passes of their Gram route.
    for (size_t m = 0; m < plan->mats.size(); ++m) {
      MatInfo& mi = plan->mats[m];
      mi.tall_blk0 = -1;
      mi.tall_nblk = 0;
      if (mi.rows <= kMgsThreads * kMgsRowsPerThread) continue;
      mi.tall_blk0 = int32_t(plan->tblks.size());
      mi.tall_nblk = (mi.rows + kTallRows - 1) / kTallRows;
      for (int32_t b = 0; b < mi.tall_nblk; ++b) plan->tblks.push_back(TallBlk{int32_t(m), b});
    }

    // Work-lists: row x column-strip tiles over the compressed matrices, flat ranges
    // over the 1-D tensors.
    auto build_tiles = [&](std::vector<UpdTile>& out, int32_t rows_per_tile, int32_t flat_runs, int32_t threads) {
      for (const psgd_layer_info& li : plan->layers) {
        if (li.compressed && plan->mats[size_t(li.matrix_index)].flat) {
          // flat_runs runs of threads * 4 elements per entry
          const int64_t end = li.offset + li.rows * li.cols;
          const int64_t span = int64_t(flat_runs) * threads * 4;
          for (int64_t b = li.offset; b < end; b += span) {
            UpdTile u{};
            u.begin = b;
            u.end = std::min<int64_t>(end, b + span);
            u.mat = li.matrix_index;
            out.push_back(u);
          }
        } else if (li.compressed) {
          const MatInfo& m = plan->mats[size_t(li.matrix_index)];
          const int32_t strip = threads * (m.vw == 1 ? 1 : 4);
          for (int32_t r0 = 0; r0 < m.rows; r0 += rows_per_tile)
            for (int32_t c0 = 0; c0 < m.cols; c0 += strip) {
              UpdTile u{};
              u.mat = li.matrix_index;
              u.row_begin = r0;
              u.row_end = std::min(m.rows, r0 + rows_per_tile);
              u.col_begin = c0;
              out.push_back(u);
            }
        } else {
          const int64_t end = li.offset + li.rows * li.cols;
          for (int64_t b = li.offset; b < end; b += int64_t(threads) * 4) {
            UpdTile u{};
            u.begin = b;
            u.end = std::min<int64_t>(end, b + int64_t(threads) * 4);
            u.mat = -1;
            out.push_back(u);
          }
        }
      }
    };
    int64_t row_strips = 0;
    for (const MatInfo& m : plan->mats)
      row_strips += m.flat ? (int64_t(m.rows) * m.cols + kStreamTileElems - 1) / kStreamTileElems
                           : int64_t(m.rows) * m.nstrips;
    plan->worker_rows_per_tile = int32_t(std::max<int64_t>(first_pass_rows(n_workers, grad_dtype == PSGD_BF16),
                                                            (row_strips + kMaxWorkerTiles - 1) / kMaxWorkerTiles));
    build_tiles(plan->s2tiles, plan->worker_rows_per_tile, plan->worker_rows_per_tile, kStreamThreads);
    build_tiles(plan->utiles, kUpdRowsPerTile, kUpdFlatRuns, kUpdThreads);
    for (size_t mi = 0; mi < plan->mats.size(); ++mi) {
      const MatInfo& m = plan->mats[mi];
      const int32_t strip = kQThreads * (m.vw == 1 ? 1 : 4);
      for (int32_t b = 0; b < m.nblk; ++b)
        for (int32_t c = 0; c < m.cols; c += strip)
          plan->qtiles.push_back(QTile{int32_t(mi), b, c, std::min(m.cols, c + strip)});
    }
    // Longest row blocks first, so that they do not form the launch's tail (the Q
    // partials do not depend on the order in which tiles run).
    std::stable_sort(plan->qtiles.begin(), plan->qtiles.end(), [&](const QTile& a, const QTile& b) {
      auto len = [&](const QTile& t) {
        const MatInfo& m = plan->mats[size_t(t.mat)];
        return std::min(m.rows, (t.blk + 1) * m.rows_per_blk) - t.blk * m.rows_per_blk;
      };
      return len(a) > len(b);
    });

    // Workspace: Mbar (same layout as update), P-bar partials, Q partials; 256-byte aligned.
    uint64_t ws = 0;
    plan->ws_mbar = ws;
    ws += uint64_t(round_up(plan->worker_stride * 4, 256));
    plan->ws_ppart = ws;
    ws += uint64_t(round_up(std::max<int64_t>(plan->ppart_elems, 1) * 4, 256));
    plan->ws_qpart = ws;
    ws += uint64_t(round_up(std::max<int64_t>(plan->qpart_elems, 1) * 4, 256));
    plan->ws_ebar = ws;
    if (flags & PSGD_FLAG_CARRY_ERROR_MEAN) ws += uint64_t(round_up(plan->worker_stride * 4, 256));
    plan->ws_pprev = ws;
    if (flags & PSGD_FLAG_DEFERRED_ERROR) ws += uint64_t(round_up(std::max<int64_t>(plan->p_elems, 1) * 4, 256));
    plan->ws_qprev = ws;
    if (flags & PSGD_FLAG_DEFERRED_ERROR) ws += uint64_t(round_up(std::max<int64_t>(plan->q_elems, 1) * 4, 256));
    plan->ws_qwpart = ws;
    if (flags & PSGD_FLAG_LOCAL_Q_ERROR)
      ws += uint64_t(round_up(std::max<int64_t>(plan->qpart_elems, 1) * 4 * n_workers, 256));
    plan->ws_qw = ws;
    if (flags & PSGD_FLAG_LOCAL_Q_ERROR) ws += uint64_t(round_up(std::max<int64_t>(plan->q_elems, 1) * 4 * n_workers, 256));
    plan->ws_gpart = ws;
    ws += uint64_t(round_up(int64_t(plan->tblks.size()) * 10 * 8, 256));
    plan->ws_tmat = ws;
    if (!plan->tblks.empty()) ws += uint64_t(round_up(int64_t(plan->mats.size()) * 16 * 8, 256));
    plan->ws_state = ws;  // one 64-bit state word (carry and deferred modes)
    if (flags & (PSGD_FLAG_CARRY_ERROR_MEAN | PSGD_FLAG_DEFERRED_ERROR)) ws += 256;
    plan->workspace_bytes = ws;
    int32_t max_rows = 1;
    for (const MatInfo& m : plan->mats) max_rows = std::max(max_rows, m.rows);
    plan->mgs_threads = int32_t(std::min<int64_t>(kMgsThreads, round_up(max_rows, 64)));

    const uint64_t W = uint64_t(n_workers);
    const uint64_t gb = grad_dtype == PSGD_BF16 ? 2 : 4;
    const uint64_t mn = uint64_t(plan->matrix_numel), vn = uint64_t(plan->vector_numel);
    plan->model_bytes = (W * (gb + 8) + 4) * mn + (W * gb + 4) * vn;
    plan->model_bytes_momentum = (W * (gb + 8) + 16) * mn + (W * gb + 16) * vn;
  } catch (const std::bad_alloc&) {
    delete plan;
    return fail(PSGD_ERR_NO_MEMORY, "psgd_plan_create: out of host memory");
  }
  *out = plan;
  return PSGD_OK;
}

extern "C" psgd_status psgd_plan_sizes(const psgd_plan* plan, psgd_sizes* out) {
  if (plan == nullptr || out == nullptr) return fail(PSGD_ERR_INVALID_ARG, "psgd_plan_sizes: NULL argument");
  psgd_sizes s{};
  s.n_layers = int32_t(plan->layers.size());
  s.n_matrices = int32_t(plan->mats.size());
  s.n_vectors = s.n_layers - s.n_matrices;
  s.rank = plan->rank;
  s.n_workers = plan->n_workers;
  s.grad_dtype = int32_t(plan->dtype);
  s.worker_stride = plan->worker_stride;
  s.numel = plan->numel;
  s.matrix_numel = plan->matrix_numel;
  s.vector_numel = plan->vector_numel;
  s.p_elems = plan->p_elems;
  s.q_elems = plan->q_elems;
  s.workspace_bytes = plan->workspace_bytes;
  s.message_bytes = plan->message_bytes;
  s.model_bytes = plan->model_bytes;
  s.model_bytes_momentum = plan->model_bytes_momentum;
  *out = s;
  return PSGD_OK;
}

extern "C" psgd_status psgd_plan_layer_info(const psgd_plan* plan, int32_t layer, psgd_layer_info* out) {
  if (plan == nullptr || out == nullptr) return fail(PSGD_ERR_INVALID_ARG, "psgd_plan_layer_info: NULL argument");
  if (layer < 0 || size_t(layer) >= plan->layers.size())
    return fail(PSGD_ERR_INVALID_ARG, "psgd_plan_layer_info: layer index out of range");
  *out = plan->layers[size_t(layer)];
  return PSGD_OK;
}

extern "C" psgd_status psgd_plan_destroy(psgd_plan* plan) {
  if (plan == nullptr) return PSGD_OK;
  psgd_status st = PSGD_OK;
  for (const PendingTiming& t : plan->pending) {
    (void)hipEventDestroy(t.start);
    (void)hipEventDestroy(t.stop);
  }
  for (hipEvent_t ev : plan->event_pool) (void)hipEventDestroy(ev);
  for (auto& kv : plan->dev) {
    if (kv.second.base == nullptr) continue;
    int cur = 0;
    if (hipGetDevice(&cur) == hipSuccess && cur != kv.first) (void)hipSetDevice(kv.first);
    if (hipFree(kv.second.base) != hipSuccess) {
      set_error("psgd_plan_destroy: hipFree of the device tables failed");
      st = PSGD_ERR_HIP;
    }
    if (cur != kv.first) (void)hipSetDevice(cur);
  }
  delete plan;
  return st;
}

extern "C" psgd_status psgd_plan_set_timing(psgd_plan* plan, int32_t enable) {
  if (plan == nullptr) return fail(PSGD_ERR_INVALID_ARG, "psgd_plan_set_timing: plan is NULL");
  plan->timing = enable != 0;
  return PSGD_OK;
}

extern "C" psgd_status psgd_plan_kernel_stats(psgd_plan* plan, psgd_kernel_stat* out, int32_t capacity,
                                              int32_t* count, int32_t reset) {
  if (plan == nullptr) return fail(PSGD_ERR_INVALID_ARG, "psgd_plan_kernel_stats: plan is NULL");
  if (capacity > 0 && out == nullptr) return fail(PSGD_ERR_INVALID_ARG, "psgd_plan_kernel_stats: out is NULL");
  psgd_status st = PSGD_OK;
  for (const PendingTiming& t : plan->pending) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(t.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, t.start, t.stop);
    if (e != hipSuccess) {
      set_error(std::string("psgd_plan_kernel_stats: ") + hipGetErrorString(e));
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
  for (int k = 0; k < kNumKernels; ++k) {
    if (plan->stats[k].launches == 0) continue;
    if (n < capacity) {
      psgd_kernel_stat ks{};
      std::snprintf(ks.name, sizeof(ks.name), "%s", kKernelNames[k]);
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

extern "C" psgd_status psgd_plan_set_power_iterations(psgd_plan* plan, int32_t iterations) {
  if (plan == nullptr) return fail(PSGD_ERR_INVALID_ARG, "psgd_plan_set_power_iterations: plan is NULL");
  if (iterations < 1 || iterations > 16)
    return fail(PSGD_ERR_INVALID_ARG, "psgd_plan_set_power_iterations: iterations must be in 1..16");
  plan->power_iterations = iterations;
  return PSGD_OK;
}
