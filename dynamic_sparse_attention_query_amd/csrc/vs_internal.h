// Argument block of the vertical-slash index estimation (MInference page,
// 2407.02490, "Online Dynamic Index Estimation: Vertical-Slash Heads
// (Algorithm 2)" and the index building of "Vertical-Slash Hybrid Kernel
// (Appendix C.4.2)").
#pragma once

#include "dsa_internal.h"

namespace dsa {

constexpr int kVsLastQ = 64;       // estimation queries: the last 64 of the sequence
constexpr int kVsRange = 256;      // keys per workgroup of the statistics pass
constexpr int kVsWin = 128;        // columns and offsets owned by a workgroup of the sums pass
constexpr int kVsMaxKeep = 8192;   // most columns or offsets kept per head

struct VsArgs {
  KvLayout kv;                 // prefill, bf16; kv.nblk = T / 64
  const void* q;
  const void* k;
  int keep[2];                 // k_v (columns), k_s (offsets)
  double scale;                // softmax scale 1/sqrt(d)
  int nr;                      // key ranges of the statistics pass
  double* part;                // [B, Hq, nr, 64, 2] range max and exp sum per estimation query
  double* stat;                // [B, Hq, 64, 2] row max and normaliser
  uint32_t* sums;              // [B, Hq, 2, T] orderable keys: column sums, offset sums
  uint32_t* ckey[2];           // top-K candidate keys, [B * Hq * 2, T] each (ping-pong)
  int32_t* cidx[2];            // their column / offset indices
  int32_t* sel[2];             // [B, Hq, k_v] kept columns, [B, Hq, k_s] kept offsets (ascending)
  int32_t* idx;                // [B, Hq, T / 64, L] index rows
  int L;
  // the hybrid kernel's lists instead of rows (when lblk is set)
  int32_t* lblk;               // [B, Hq, T / 64, wb] ascending key-block ids, then -1
  int32_t* lcol;               // [B, Hq, T / 64, wc] ascending single columns, then -1
  int32_t* lcnt;               // [B, Hq, T / 64, 2] number of blocks, of columns
  int wb, wc;
};

hipError_t launch_vertical_slash(const VsArgs& a, hipStream_t stream);

}  // namespace dsa
