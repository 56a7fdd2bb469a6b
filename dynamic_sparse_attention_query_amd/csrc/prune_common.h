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

// First key position of chunk j of stage `stage` in row r (chunk sizes are
// powers of two, so the parent chunk and the offset inside it are shifts).
__device__ __forceinline__ int chunk_start(const PruneArgs& a, int stage, int r, int j) {
  if (stage == 0) return a.n_sink + (j << a.lchunk[0]);
  const int sh = a.lchunk[stage - 1] - a.lchunk[stage];
  const int32_t* prev =
      a.starts + static_cast<size_t>((stage - 1) & 1) * a.R * a.maxK + static_cast<size_t>(r) * a.maxK;
  return prev[j >> sh] + ((j & ((1 << sh) - 1)) << a.lchunk[stage]);
}

}  // namespace dsa
