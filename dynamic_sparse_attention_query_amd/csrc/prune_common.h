// Stage bookkeeping shared by the pruning kernels: how many chunks a stage
// sees for a row and where each chunk starts.
#pragma once

#include "dsa_internal.h"
#include "topk_select.h"

namespace dsa {

// ------------------------------------------------------------------------- //
// shared stage helpers                                                      //
// ------------------------------------------------------------------------- //
__device__ __forceinline__ int stage_input_chunks(const PruneArgs& a, int stage, int r,
                                                  const Geo& geo) {
  if (stage == 0) return geo.n1;
  return a.cnt[r * kMaxStages + stage - 1] << (a.lchunk[stage - 1] - a.lchunk[stage]);
}

// Chunk-score list of row r for `stage`, written by the workgroups of head
// slice sl (decode with more than 16 kv heads; else the only slice, 0). Two
// sets of lists alternate by stage parity, so one kernel can read a stage's
// scores while writing the next stage's.
__device__ __forceinline__ uint32_t* stage_scores(const PruneArgs& a, int stage, int r, int sl = 0) {
  return a.scores + ((static_cast<size_t>(stage & 1) * a.nsl + sl) * a.R + r) * a.maxNC;
}

// Page ids of the kept chunks of `stage` for row r (paged decode), kKeptPages
// per chunk.
__device__ __forceinline__ int32_t* stage_pages(const PruneArgs& a, int stage, int r) {
  return a.kpages + (static_cast<size_t>(a.slot[stage]) * a.R + r) * a.maxK * kKeptPages;
}

// Pool rows of the positions p0 .. p0 + n - 1 of sequence b (consecutive,
// n <= page_size, so at most two pages): (page id << page_shift) | offset in
// the page, into out[0 .. n); -1 where p0 + x < 0 or x >= valid. The two
// table reads are unconditional (clamped to the row) so they go out together.
template <int N>
__device__ __forceinline__ void paged_rows_run(const KvLayout& kv, int b, int p0, int valid, int (&out)[N]) {
  const int32_t* tb = kv.block_table + static_cast<size_t>(b) * kv.max_pages;
  const int s = kv.page_shift, last = kv.max_pages - 1;
  const int q0 = max(p0, 0);
  const int pg0 = min(q0 >> s, last);
  const int id0 = tb[pg0], id1 = tb[min(pg0 + 1, last)];
#pragma unroll
  for (int x = 0; x < N; ++x) {
    const int p = p0 + x;
    const int id = (p >> s) == pg0 ? id0 : id1;
    out[x] = p < 0 || x >= valid ? -1 : (id << s) | (p & (kv.page_size - 1));
  }
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

// ------------------------------------------------------------------------- //
// inputs of a stage's top-K                                                 //
// ------------------------------------------------------------------------- //
constexpr int kMaxKeptChunks = 8192;    // keep / chunk of any stage (validated by the API)

// This thread's keys: chunks j0 .. j0+E-1 of row r's score list of `stage` (read within
// the row for every j0 of the launch; the selection masks j >= nc).
// With several head slices (a.nsl > 1) a chunk's key is the largest of its
// slices' keys: the keys are order-preserving, so that is the key of the max
// over all heads.
template <int E>
__device__ __forceinline__ void load_keys(const PruneArgs& a, int stage, int r, int j0, uint32_t (&key)[E]) {
  static_assert(E % 4 == 0, "keys are loaded four at a time");
  const uint4* sc4 = reinterpret_cast<const uint4*>(stage_scores(a, stage, r));
  const int nv = a.maxNC >> 2;
#pragma unroll
  for (int v = 0; v < E / 4; ++v) {
    const uint4 u = sc4[min((j0 >> 2) + v, nv - 1)];
    key[4 * v + 0] = u.x; key[4 * v + 1] = u.y; key[4 * v + 2] = u.z; key[4 * v + 3] = u.w;
  }
  for (int sl = 1; sl < a.nsl; ++sl) {
    const uint4* s4 = reinterpret_cast<const uint4*>(stage_scores(a, stage, r, sl));
#pragma unroll
    for (int v = 0; v < E / 4; ++v) {
      const uint4 u = s4[min((j0 >> 2) + v, nv - 1)];
      key[4 * v + 0] = max(key[4 * v + 0], u.x);
      key[4 * v + 1] = max(key[4 * v + 1], u.y);
      key[4 * v + 2] = max(key[4 * v + 2], u.z);
      key[4 * v + 3] = max(key[4 * v + 3], u.w);
    }
  }
}

// Lane group gi of a decode scoring workgroup of the launch's block bx: its
// chunk (j, or past the workgroup's share when the 16 lane groups are not a
// multiple of the heads per workgroup), kv head g and head slice sl.
struct DecodeLane {
  int sl, j0, cpw, cl, g;
  bool used;
};
__device__ __forceinline__ DecodeLane decode_lane(const PruneArgs& a, int bx, int gi) {
  DecodeLane d;
  d.cpw = 16 / a.hpw;
  d.sl = bx % a.nsl;
  d.j0 = (bx / a.nsl) * d.cpw;
  d.cl = gi / a.hpw;
  d.used = d.cl < d.cpw;
  d.cl = min(d.cl, d.cpw - 1);
  d.g = d.sl * a.hpw + (gi - (gi / a.hpw) * a.hpw);
  return d;
}

// First key position of kept chunk j of stage ps, given the kept starts of
// stage ps - 1 in sprev (chunk sizes are powers of two).
__device__ __forceinline__ int kept_start(const PruneArgs& a, int ps, int j, const int* sprev) {
  const int lgp = a.lchunk[ps];
  if (ps == 0) return a.n_sink + (j << lgp);
  const int shp = a.lchunk[ps - 1] - lgp;
  return sprev[j >> shp] + ((j & ((1 << shp) - 1)) << lgp);
}

// Longest kept list the fused decode kernels hold in LDS (per stage); rows of
// longer lists take the one-workgroup-per-row selection kernel.
constexpr int kFusedMaxKept = 1024;

// The kept starts of stage `stage` for row r (at most keep/chunk of them)
// into LDS; published by the caller's next barrier.
template <int NT = kTopkThreads>
__device__ __forceinline__ void load_kept_starts(const PruneArgs& a, int stage, int r, int* sp) {
  const int tid = threadIdx.x;
  const int kmax = a.keep[stage] >> a.lchunk[stage];
  const int32_t* src = stage_starts(a, stage, r);
  for (int i0 = 0; i0 < kmax; i0 += 4 * NT) {
    int v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * NT + tid;
      v[u] = i < kmax ? src[i] : 0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * NT + tid;
      if (i < kmax) sp[i] = v[u];
    }
  }
}

// Key rows of one chunk as seen by a lane group (lane li holds elements
// li*D/16 .. of a row). Paged K (compile-time): the chunk covers at most
// kChunkPages pages in the common case (`hoist`); their ids are loaded once,
// together, so a tournament step costs one dependent load (the row) instead
// of two (table entry, then row), and at() holds no load but the row's. A
// chunk over more pages takes the TABLE form, whose at() reads the page
// table for every row. The two forms are separate tournament bodies
// (paged_rows below): a table load inside at() behind a per-row branch made
// the compiler wait for every load in flight at the branch's join, which
// serialized a round's row loads.
constexpr int kChunkPages = 4;
template <typename T, int D, bool PAGED, bool TABLE = false>
struct ChunkRows {
  static constexpr int EPL = D / 16;
  const T* K;                   // contiguous: row 0 of (b, g), this lane's slice; paged: the pool + slice
  const int32_t* table;         // paged: this sequence's page table
  int hkv_g;                    // paged: page-pool offset of kv head g, in rows (g * page_size)
  int page_rows;                // paged: Hkv * page_size (rows per page)
  int shift, pg0;
  bool hoist;
  int pid0, pid1, pid2, pid3;       // hoisted page ids

  // pp (paged, or nullptr): the page ids of the parent chunk that starts at
  // pst, as the previous stage's top-K resolved them (kpages); the chunk's
  // pages are then taken from those registers instead of the page table,
  // which saves the dependent table load before the first row.
  __device__ __forceinline__ ChunkRows(const PruneArgs& a, int b, int g, int li, int st, int l,
                                       const int* pp = nullptr, int pst = 0) {
    const KvLayout& kv = a.kv;
    const T* base = static_cast<const T*>(a.k) + li * EPL;
    if constexpr (PAGED) {
      K = base;
      table = kv.block_table + static_cast<size_t>(b) * kv.max_pages;
      shift = kv.page_shift;
      hkv_g = g * kv.page_size;
      page_rows = kv.Hkv * kv.page_size;
      pg0 = st >> shift;
      const int npg = ((st + l - 1) >> shift) - pg0 + 1;
      hoist = !TABLE && npg <= kChunkPages;
      if (TABLE) {
        pid0 = pid1 = pid2 = pid3 = 0;
      } else if (pp != nullptr) {
        const int i0 = pg0 - (pst >> shift);     // the chunk's first page within the parent's
        auto pick = [&](int i) {
          int v = -1;
#pragma unroll
          for (int k = 0; k < kKeptPages; ++k) v = i == k ? pp[k] : v;
          return v;
        };
        pid0 = pick(i0);
        pid1 = npg > 1 ? pick(i0 + 1) : 0;
        pid2 = npg > 2 ? pick(i0 + 2) : 0;
        pid3 = npg > 3 ? pick(i0 + 3) : 0;
        hoist = hoist && pid0 >= 0 && pid1 >= 0 && pid2 >= 0 && pid3 >= 0;
      } else {
        // four loads at once (indices kept inside the table row; the ids of
        // pages past the chunk are never used)
        const int last = kv.max_pages - 1;
        pid0 = table[min(pg0, last)];
        pid1 = table[min(pg0 + 1, last)];
        pid2 = table[min(pg0 + 2, last)];
        pid3 = table[min(pg0 + 3, last)];
      }
    } else {
      K = base + (static_cast<size_t>(b) * kv.Hkv + g) * kv.T * D;
    }
  }

  __device__ __forceinline__ RowSlice<T, EPL> at(int pos) const {
    RowSlice<T, EPL> x;
    if constexpr (PAGED) {
      const int k = pos >> shift;
      int page;
      if constexpr (TABLE) {
        page = table[k];
      } else {                                  // only used when hoist holds
        const int i = k - pg0;
        page = i == 0 ? pid0 : i == 1 ? pid1 : i == 2 ? pid2 : pid3;
      }
      const size_t row = static_cast<size_t>(page) * page_rows + hkv_g + (pos - (k << shift));
      x.load(K + row * D);
    } else {
      x.load(K + static_cast<size_t>(pos) * D);
    }
    return x;
  }
};

// Calls body(rows) with the chunk's row provider: contiguous, or paged with
// the page ids in registers when the chunk spans at most kChunkPages pages,
// else paged through the page table (a divergent choice per lane group).
template <typename T, int D, bool PAGED, class Body>
__device__ __forceinline__ float paged_rows(const PruneArgs& a, int b, int g, int li, int st, int l, const int* pp,
                                            int pst, Body&& body) {
  const ChunkRows<T, D, PAGED> rows(a, b, g, li, st, l, pp, pst);
  if constexpr (PAGED) {
    if (!rows.hoist) return body(ChunkRows<T, D, true, true>(a, b, g, li, st, l));
  }
  return body(rows);
}

}  // namespace dsa
