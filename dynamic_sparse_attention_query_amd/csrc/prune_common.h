// Stage bookkeeping shared by the pruning kernels: how many chunks a stage
// sees for a row and where each chunk starts.
#pragma once

#include "dsa_internal.h"

namespace dsa {

// ------------------------------------------------------------------------- //
// shared stage helpers                                                      //
// ------------------------------------------------------------------------- //
__device__ __forceinline__ int stage_input_chunks(const PruneArgs& a, int stage, int r,
                                                  const Geo& geo) {
  if (stage == 0) return geo.n1;
  return a.cnt[r * kMaxStages + stage - 1] << (a.lchunk[stage - 1] - a.lchunk[stage]);
}

// Chunk-score list of row r for `stage`. Two lists alternate by stage parity,
// so one kernel can read a stage's scores while writing the next stage's.
__device__ __forceinline__ uint32_t* stage_scores(const PruneArgs& a, int stage, int r) {
  return a.scores + (static_cast<size_t>(stage & 1) * a.R + r) * a.maxNC;
}

// Kept chunk starts of `stage` for row r (ascending, cnt[r][stage] of them).
__device__ __forceinline__ int32_t* stage_starts(const PruneArgs& a, int stage, int r) {
  return a.starts + (static_cast<size_t>(a.slot[stage]) * a.R + r) * a.maxK;
}

// First key position of chunk j of stage `stage` in row r (chunk sizes are
// powers of two, so the parent chunk and the offset inside it are shifts).
__device__ __forceinline__ int chunk_start(const PruneArgs& a, int stage, int r, int j) {
  if (stage == 0) return a.n_sink + (j << a.lchunk[0]);
  const int sh = a.lchunk[stage - 1] - a.lchunk[stage];
  const int32_t* prev = stage_starts(a, stage - 1, r);
  return prev[j >> sh] + ((j & ((1 << sh) - 1)) << a.lchunk[stage]);
}

// End of the stage-1 middle that the output of `stage` descends from: the
// current one, unless the stage reads a remembered record (mask caching),
// whose middle may predate the newest tokens.
__device__ __forceinline__ int stage_mid_end(const PruneArgs& a, int stage, int r, const Geo& geo) {
  if (stage == 0 || a.mid_end == nullptr) return geo.mid_hi;
  return a.mid_end[r * kMaxStages + stage - 1];
}

// Bookkeeping of a stage's output for row r: its kept count and, when stages
// are remembered, the middle it descends from.
__device__ __forceinline__ void record_stage(const PruneArgs& a, int stage, int r, int n_sel,
                                             const Geo& geo) {
  a.cnt[r * kMaxStages + stage] = n_sel;
  if (a.mid_end) a.mid_end[r * kMaxStages + stage] = stage_mid_end(a, stage, r, geo);
}

}  // namespace dsa
