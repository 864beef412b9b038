// Internal host/device structures of libpsgd (not part of the C ABI).
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <map>
#include <string>
#include <vector>

#include "psgd.h"

namespace psgd {

constexpr int64_t kAlignElems = 64;  // every tensor starts on a 256-byte boundary

// Worker passes (the first pass and the eager error/update pass): one workgroup is one
// wave of kStreamThreads lanes.  Over a compressed matrix whose rows start on 128-byte
// lines it handles one row x a strip of kStreamThreads*4 columns (kStreamThreads
// columns when cols % 4 != 0).  Over a 1-D tensor, and over a "flat" matrix (at least
// kFlatMinCols columns, not a multiple of 32, so its rows start anywhere in a line), it
// handles kStreamTileElems consecutive elements, one float4 chunk per lane.  A tile
// table entry covers as many rows (flat chunks) as keep the table under
// kMaxWorkerTiles entries, and the launch's second grid dimension walks them, one
// workgroup each.
constexpr int kStreamThreads = 64;
constexpr int kStreamTileElems = kStreamThreads * 4;
constexpr int64_t kMaxWorkerTiles = 65536;
constexpr int kFlatMinCols = 32;
// Rows (or flat chunks) per first-pass wave at small worker counts: with few workers a
// row's loads are few, so a wave takes several rows, loads the strip's Q once for all of
// them and has every row's loads in flight together (W = 4 on the 4096- and 8192-column
// stress matrices: 2 rows for float32 gradients, 4 for bf16, measured best of 1, 2, 4 on
// one allocation).  The tile lists then hold at least this many rows per entry.
constexpr int first_pass_rows(int w, bool bf16_grads) {
  return w == 1 || w == 2 ? 4 : w == 4 ? (bf16_grads ? 4 : 2) : 1;
}

// Update-only pass (deferred mode): workgroups of kUpdThreads over kUpdRowsPerTile rows
// x a strip of kUpdThreads*4 columns, or kUpdFlatRuns runs of kUpdThreads*4 elements
// of a flat matrix, or kUpdThreads*4 elements of a 1-D tensor.  4 rows / 4 runs per
// workgroup measured best of 1, 2, 4 and 8 (ResNet-18 shapes 8.2 against 8.8 us at 8,
// LSTM shapes 41.3 against 42.9 us; 1 row: 10.7 us).
constexpr int kUpdThreads = 256;
constexpr int kUpdRowsPerTile = 4;
constexpr int kUpdFlatRuns = 4;

// Q partials = Mbar^T P over a block of rows and a strip of columns.  A matrix gets
// ceil(rows / kQTargetRowsPerBlock) row blocks, at most kQMaxRowBlocks, or more (up to
// that ceiling) when its share of the plan's elements calls for more than
// kQMaxRowBlocks of the kQTargetTiles tiles of the launch.
constexpr int kQThreads = 256;
constexpr int kQTargetRowsPerBlock = 64;
constexpr int kQMaxRowBlocks = 32;
constexpr int64_t kQTargetTiles = 2048;

// Gram-Schmidt: one workgroup per matrix.  A matrix taller than kMgsThreads *
// kMgsRowsPerThread rows is orthonormalised through its Gram matrix instead: P-bar rows
// and per-block Gram partials over blocks of kTallRows rows (one per thread), the
// coefficients in that matrix's Gram-Schmidt workgroup, and P = P-bar T over the same
// blocks.
constexpr int kMgsThreads = 1024;
constexpr int kMgsRowsPerThread = 4;
constexpr int kTallRows = 256;

// Reduction of the Q partials: a workgroup takes 64 elements of Q (one per lane) and up
// to kQRedMaxWaves waves, which split the row blocks between them.
constexpr int kQRedMaxWaves = 16;

struct MatInfo {
  int64_t offset;     // element offset of the matrix in a worker slice / Mbar / update
  int64_t p_off;      // element offset of P in p
  int64_t q_off;      // element offset of Q in q
  int64_t qpart_off;  // float offset of this matrix's Q partials in the workspace
  int64_t ppart_off;  // float offset of this matrix's P-bar partials (nstrips x rows x R)
  int32_t rows, cols;
  int32_t rows_per_blk;  // rows summed into one Q partial
  int32_t nblk;          // number of Q partials (row blocks)
  int32_t vw;            // row alignment in floats: 4 if cols % 4 == 0, 2 if even, else 1 (4 and 2
                         // run four columns per lane, 2 as two 8-byte halves; 1 one column)
  int32_t nstrips;       // P-bar partial slots per row: the column strips of the worker passes, or
                         // for a flat matrix the most flat chunks one row can overlap
  int32_t flat;          // 1: the worker passes stream the matrix in flat chunks
  int32_t tall_blk0;     // first entry of the matrix in the tall-block list, -1 if not tall
  int32_t tall_nblk;     // its number of tall blocks
};

struct TallBlk {
  int32_t mat, blk;
};

struct QTile {
  int32_t mat, blk, col_begin, col_end;
};

// Tiles of the worker and update passes: for a compressed matrix, rows
// [row_begin, row_end) x a column strip starting at col_begin; for a flat matrix and
// for an uncompressed tensor (mat < 0), the element range [begin, end) (begin a
// multiple of 4).
struct UpdTile {
  int64_t begin, end;
  int32_t mat, row_begin, row_end, col_begin;
};

struct DeviceTables {
  void* base = nullptr;
  MatInfo* mats = nullptr;
  UpdTile* s2tiles = nullptr;
  QTile* qtiles = nullptr;
  UpdTile* utiles = nullptr;
  TallBlk* tblks = nullptr;
};

void set_error(const std::string& msg);

enum KernelId {
  kKFirst = 0, kKMgs, kKQPartial, kKQReduce, kKApply, kKUpdate, kKPMbar, kKQwPartial, kKQwReduce,
  kKTallRows, kKTallApply, kNumKernels
};
extern const char* const kKernelNames[kNumKernels];

struct PendingTiming {
  int kernel;
  hipEvent_t start, stop;
};

struct KernelStat {
  int64_t launches = 0;
  double total_ms = 0.0;
};

}  // namespace psgd

struct psgd_plan {
  int32_t rank = 0;
  int32_t n_workers = 0;
  psgd_dtype dtype = PSGD_F32;
  uint32_t flags = 0;
  std::vector<psgd_layer_info> layers;
  std::vector<psgd::MatInfo> mats;
  std::vector<psgd::UpdTile> s2tiles;
  std::vector<psgd::QTile> qtiles;
  std::vector<psgd::UpdTile> utiles;
  std::vector<psgd::TallBlk> tblks;
  int64_t worker_stride = 0, numel = 0, matrix_numel = 0, vector_numel = 0;
  int64_t p_elems = 0, q_elems = 0, qpart_elems = 0, ppart_elems = 0;
  int64_t max_q_elems_per_matrix = 0;
  uint64_t ws_mbar = 0, ws_ppart = 0, ws_qpart = 0, ws_ebar = 0, ws_pprev = 0, ws_qprev = 0, workspace_bytes = 0;
  uint64_t ws_qwpart = 0, ws_qw = 0;  // per-worker Q partials and Q_w (PSGD_FLAG_LOCAL_Q_ERROR)
  uint64_t ws_gpart = 0, ws_tmat = 0;  // tall matrices: per-block Gram partials, per-matrix T (doubles)
  int32_t mgs_threads = 64;  // Gram-Schmidt block size: enough for the tallest matrix, <= kMgsThreads
  int32_t qred_waves = 1;    // waves per workgroup of the Q-partial reduction (about 8 row blocks each, <= 16)
  int32_t worker_rows_per_tile = 1;
  int32_t power_iterations = 1;  // power-iteration rounds per step (psgd_plan_set_power_iterations)
  uint64_t message_bytes = 0, model_bytes = 0, model_bytes_momentum = 0;
  std::map<int, psgd::DeviceTables> dev;  // per HIP device id
  // cross-step state: the carried error mean (PSGD_FLAG_CARRY_ERROR_MEAN) or the deferred
  // offset (PSGD_FLAG_DEFERRED_ERROR), valid for these error/workspace buffers on this device
  // (the host's view; the workspace's state word at ws_state holds the device's, keyed by
  // nonce and the errors address)
  bool state_valid = false;
  uint64_t nonce = 0;
  uint64_t ws_state = 0;
  const void* state_errors = nullptr;
  const void* state_workspace = nullptr;
  int state_device = -1;
  // kernel timing (psgd_plan_set_timing)
  bool timing = false;
  std::vector<psgd::PendingTiming> pending;
  std::vector<hipEvent_t> event_pool;
  psgd::KernelStat stats[psgd::kNumKernels];
};
