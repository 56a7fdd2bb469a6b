// Hierarchical context pruning kernels (InfiniteHiP page, 2502.08910,
// section 3.4 "Formal Mechanism of a Single Pruning Stage" and
// "The Representative Token Selection Algorithm (SelectRep)").
//
// One prune_select call runs, for each stage i:
//   score : every (row, chunk) of the stage's input list is scored: for each
//           query head a SelectRep tournament picks one representative key;
//           the chunk score is the max over heads and block queries of the
//           representative's dot product (unscaled);
//   top-K : per row, keep the K = keep/chunk best chunks (score descending,
//           chunk index ascending), write their start positions in ascending
//           order, and after the last stage write the index row: sinks, kept
//           chunks, window, -1 padding.
// The top-K is the stage's single global synchronisation point; it runs as its
// own kernel, one workgroup per row.
// Every chunk of every stage is a contiguous run of positions: stage 1 tiles
// [n_sink, mid_hi) and each later chunk size divides the previous one.
#include <algorithm>
#include <type_traits>

#include "prune_common.h"
#include "selectrep.h"
#include "topk_select.h"

namespace dsa {

// ------------------------------------------------------------------------- //
// top-K of one row + index assembly                                         //
// ------------------------------------------------------------------------- //
// The index row of row r is sinks [0, sink_hi), the n_sel kept chunks of l
// keys (ascending), every position from win_lo (the end of the stage-1 middle
// the kept chunks descend from) up to the newest key, then -1 padding; L is a
// multiple of 64. The kept chunks are written by whoever selects them
// (write_chunk_entries); write_row_rest writes everything else, so no part of
// the row waits for another. A row that would not fit (possible only when
// stages are remembered across steps) keeps its first L entries and is
// flagged in row_status.
__device__ __forceinline__ void write_chunk_entries(int32_t* row, int L, int i0, int st, int l) {
  if (((i0 | l) & 3) == 0) {
    for (int x = 0; x < l && i0 + x < L; x += 4)
      *reinterpret_cast<int4*>(row + i0 + x) = make_int4(st + x, st + x + 1, st + x + 2, st + x + 3);
  } else {
    for (int x = 0; x < l && i0 + x < L; ++x) row[i0 + x] = st + x;
  }
}

// prow (paged decode, or nullptr): the same entries with their pages resolved
// (paged_row) into the row r of prow; b is the row's sequence.
__device__ __forceinline__ void write_row_rest(const PruneArgs& a, int r, const Geo& geo, int n_sel, int l,
                                               int win_lo, int32_t* prow = nullptr, int b = 0) {
  const int win0 = geo.sink_hi + n_sel * l;        // kept chunks fill [sink_hi, win0)
  const int end = win0 + max(0, geo.e - win_lo);
  int32_t* row = a.idx + static_cast<size_t>(r) * a.L;
  auto value = [&](int i) { return i < geo.sink_hi ? i : i < end ? win_lo + (i - win0) : -1; };
  const int n4 = a.L >> 2;
  const int head4 = (geo.sink_hi + 3) >> 2;         // 16-byte slots holding sinks
  const int tail4 = min(win0 >> 2, n4);             // first slot holding window or padding
  const int n_rest = head4 + (n4 - tail4);
  for (int k = threadIdx.x; k < n_rest; k += blockDim.x) {
    const int i4 = k < head4 ? k : tail4 + (k - head4);
    const int i = 4 * i4;
    if (i + 4 <= geo.sink_hi || i >= win0) {
      *reinterpret_cast<int4*>(row + i) = make_int4(value(i), value(i + 1), value(i + 2), value(i + 3));
      if (prow) {                                   // sinks, or window then padding: consecutive positions
        int v[4];
        const int nv = value(i) < 0 ? 0 : value(i + 3) >= 0 ? 4 : value(i + 2) >= 0 ? 3 : value(i + 1) >= 0 ? 2 : 1;
        paged_rows_run(a.kv, b, value(i), nv, v);
        *reinterpret_cast<int4*>(prow + static_cast<size_t>(r) * a.L + i) = make_int4(v[0], v[1], v[2], v[3]);
      }
    } else {                                        // a slot shared with kept-chunk entries
      int id[4];
      if (prow) {                                   // one table read per entry, all issued together
        const int32_t* tb = a.kv.block_table + static_cast<size_t>(b) * a.kv.max_pages;
#pragma unroll
        for (int u = 0; u < 4; ++u) id[u] = tb[min(max(value(i + u), 0) >> a.kv.page_shift, a.kv.max_pages - 1)];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (i + u < geo.sink_hi || i + u >= win0) {
          const int p = value(i + u);
          row[i + u] = p;
          if (prow)
            prow[static_cast<size_t>(r) * a.L + i + u] =
                p < 0 ? -1 : (id[u] << a.kv.page_shift) | (p & (a.kv.page_size - 1));
        }
    }
  }
  if (a.row_status && threadIdx.x == 0) a.row_status[r] = end > a.L ? 1 : 0;
}

// One workgroup per row: select the stage's kept chunks, write their starts
// (and their count), and after the last stage the index row. Rows of up to
// 4,096 chunks take the latency-oriented selection (select_keys: one pass
// for bins sized to the row's range, the kept indices in LDS), after which
// the threads write the kept chunks' outputs in kept order; longer rows take
// select_row, whose owning thread writes each kept chunk.
template <int E, int NT = kTopkThreads>
__global__ void __launch_bounds__(NT) k_topk(PruneArgs a, int stage) {
  constexpr bool kFast = NT == kTopkThreads && E <= 16;
  __shared__ std::conditional_t<kFast, SelectKeysLds<NT / 64>, SelectLds<NT / 64>> L;
  __shared__ int sprev[kMaxKeptChunks];
  __shared__ int skept[kFast ? E * NT : 1];           // kept indices (at most the row's E * NT chunks)

  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  int b, s, e;
  row_bounds(a.kv, r, b, s, e);
  const Geo geo = make_geo(s, e, a.n_sink, a.n_window, a.chunk[0]);
  const int lg = a.lchunk[stage], l = 1 << lg;
  const int kc = a.keep[stage] >> lg;
  const bool last = stage == a.n_stages - 1;
  const int nc = stage_input_chunks(a, stage, r, geo);

  // all loads up front: this thread's keys and the previous stage's kept starts
  const int j0 = tid * E;
  uint32_t key[E];
  load_keys<E>(a, stage, r, j0, key);
  const int sh = stage > 0 ? a.lchunk[stage - 1] - lg : 0;
  if (stage > 0) load_kept_starts<NT>(a, stage - 1, r, sprev);
  const int n_sel = nc <= kc ? nc : kc;
  int32_t* out = stage_starts(a, stage, r);
  int32_t* row = a.idx + static_cast<size_t>(r) * a.L;
  const int win_lo = last ? stage_mid_end(a, stage, r, geo) : 0;
  const bool pages = a.kv.block_table != nullptr && a.kpages != nullptr;
  // the outputs of kept chunk j in slot pos: its start, after the last stage
  // its entries of the index row (and their pool rows), before it (paged
  // decode) its page ids for the next stage
  auto emit = [&](int j, int pos) {
    const int st = stage == 0 ? a.n_sink + (j << lg) : sprev[j >> sh] + ((j & ((1 << sh) - 1)) << lg);
    out[pos] = st;
    if (last) write_chunk_entries(row, a.L, geo.sink_hi + pos * l, st, l);
    if (pages && !last) {                       // the chunk's page ids for the next stage
      const int* tb = a.kv.block_table + static_cast<size_t>(b) * a.kv.max_pages;
      const int pg0 = st >> a.kv.page_shift;
      const int npg = ((st + l - 1) >> a.kv.page_shift) - pg0 + 1;
      // all eight reads at once (clamped to the table row), then masked
      const int last_pg = a.kv.max_pages - 1;
      int v[kKeptPages];
#pragma unroll
      for (int u = 0; u < kKeptPages; ++u) v[u] = tb[min(pg0 + u, last_pg)];
#pragma unroll
      for (int u = 0; u < kKeptPages; ++u) v[u] = npg <= kKeptPages && u < npg ? v[u] : -1;
      int4* dst = reinterpret_cast<int4*>(stage_pages(a, stage, r) + pos * kKeptPages);
#pragma unroll
      for (int u = 0; u < kKeptPages / 4; ++u) dst[u] = make_int4(v[4 * u], v[4 * u + 1], v[4 * u + 2], v[4 * u + 3]);
    }
    if (pages && last && a.prow) {              // the kept entries with their pages resolved
      int32_t* prw = a.prow + static_cast<size_t>(r) * a.L;
      const int i0 = geo.sink_hi + pos * l;
      for (int x0 = 0; x0 < l && i0 + x0 < a.L; x0 += 4) {   // four entries (within two pages) at a time
        int v[4];
        paged_rows_run(a.kv, b, st + x0, min(4, l - x0), v);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (x0 + u < l && i0 + x0 + u < a.L) prw[i0 + x0 + u] = v[u];
      }
    }
  };
  if constexpr (kFast) {
    select_keys<E, NT>(key, nc, kc, L, skept);
    __syncthreads();                            // skept holds the kept chunk indices, ascending
    for (int pos = tid; pos < n_sel; pos += NT) emit(skept[pos], pos);
  } else {
    // stores only after every load has been consumed (inside the selection):
    // stores share the vector memory counter with loads, so an earlier store
    // would hold up their wait
    select_row<E, NT>(key, j0, nc, kc, L, emit);
  }
  if (tid == 0) record_stage(a, stage, r, n_sel, geo);
  if (last) write_row_rest(a, r, geo, n_sel, l, win_lo, pages ? a.prow : nullptr, b);
}

// The last stage's remembered output turned into the index row of the current
// step (mask caching, when the last stage is not due): one workgroup per row.
__global__ void __launch_bounds__(kTopkThreads) k_assemble(PruneArgs a) {
  const int r = blockIdx.x;
  const int last = a.n_stages - 1;
  int b, s, e;
  row_bounds(a.kv, r, b, s, e);
  const Geo geo = make_geo(s, e, a.n_sink, a.n_window, a.chunk[0]);
  const int l = a.chunk[last];
  const int n_sel = max(0, min(a.cnt[r * kMaxStages + last], a.keep[last] >> a.lchunk[last]));
  const int win_lo = a.mid_end[r * kMaxStages + last];
  const int32_t* starts = stage_starts(a, last, r);
  int32_t* row = a.idx + static_cast<size_t>(r) * a.L;
  for (int c = threadIdx.x; c < n_sel; c += blockDim.x)
    write_chunk_entries(row, a.L, geo.sink_hi + c * l, starts[c], l);
  write_row_rest(a, r, geo, n_sel, l, win_lo);
}

// ------------------------------------------------------------------------- //
// decode scoring: one query per row                                         //
// ------------------------------------------------------------------------- //
// One lane group's SelectRep tournaments over the chunk of chunk[stage] keys
// starting at st, on the rows of kv head g as stored.
template <typename T, int D, int G, int SPEC, bool PAGED, bool TAIL4 = false>
__device__ __forceinline__ float score_group(const PruneArgs& a, int stage, int b, int g, int li, int st,
                                             const RowSlice<T, D / 16> (&q)[G], const int* pp = nullptr,
                                             int pst = 0) {
  return paged_rows<T, D, PAGED>(a, b, g, li, st, a.chunk[stage], pp, pst, [&](const auto& rows) {
    return selectrep_group<T, D, G, SPEC, std::decay_t<decltype(rows)>, TAIL4>(a, stage, li, st, rows, q);
  });
}

// Workgroup = 16 lane groups of 16 lanes; a group owns one (chunk, kv head)
// and runs the G SelectRep tournaments of that kv head's query heads side by
// side, so each step issues G independent 16-lane row loads (256 B per row at
// bf16 d=128, fully coalesced). The first split's two representatives are
// shared by all heads. With SPEC, the 8 keys that can represent the first
// three splits (positions i*l/8) are loaded in one round and the first three
// splits are decided from them, trading up to 1/8 more row reads for two
// fewer dependent load rounds. Group results are max-reduced per chunk in
// LDS.
template <typename T, int D, int G, int SPEC, bool PAGED>
__global__ void __launch_bounds__(256, G > 4 ? 2 : ((SPEC == 8 || sizeof(T) == 4) ? 4 : 8))
k_score_decode(PruneArgs a, int stage) {
  constexpr int EPL = D / 16;
  using Row = RowSlice<T, EPL>;
  const KvLayout& kv = a.kv;
  const int r = blockIdx.y, b = r;              // one row per sequence
  const int tid = threadIdx.x;
  const int gi = tid >> 4, li = tid & 15;
  const DecodeLane dl = decode_lane(a, blockIdx.x, gi);
  const int cpw = dl.cpw, j0 = dl.j0, g = dl.g;  // chunks per workgroup, first chunk, kv head
  const int j = j0 + dl.cl;
  const T* Q = static_cast<const T*>(a.q);
  __shared__ float red[16];

  // Loads that need only the launch coordinates go out together, before the
  // checks that use them: the sequence length, the previous stage's kept
  // count, this chunk's start (read within the start list for every j of
  // the grid) and the query rows.
  const int e = seq_len_of(kv, r);
  int nc_prev = 0, st, pst = 0;
  int pp[kKeptPages];                           // paged: the parent chunk's page ids
  const bool pre = PAGED && stage > 0 && a.kpages != nullptr;
  if (stage == 0) {
    st = a.n_sink + (j << a.lchunk[0]);
  } else {
    const int sh = a.lchunk[stage - 1] - a.lchunk[stage];
    nc_prev = a.cnt[r * kMaxStages + stage - 1];
    const int jp = min(j >> sh, a.maxK - 1);
    pst = stage_starts(a, stage - 1, r)[jp];
    st = pst + ((j & ((1 << sh) - 1)) << a.lchunk[stage]);
    if (pre) {
      const int4* p4 = reinterpret_cast<const int4*>(stage_pages(a, stage - 1, r) + jp * kKeptPages);
#pragma unroll
      for (int v = 0; v < kKeptPages / 4; ++v) {
        const int4 u = p4[v];
        pp[4 * v] = u.x; pp[4 * v + 1] = u.y; pp[4 * v + 2] = u.z; pp[4 * v + 3] = u.w;
      }
    }
  }
  Row q[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) q[hh].load(Q + (static_cast<size_t>(b) * kv.Hq + g * G + hh) * D + li * EPL);

  const Geo geo = make_geo(e - 1, e, a.n_sink, a.n_window, a.chunk[0]);
  const int nc = stage == 0 ? geo.n1 : nc_prev << (a.lchunk[stage - 1] - a.lchunk[stage]);
  if (nc <= (a.keep[stage] >> a.lchunk[stage])) return;   // stage keeps everything for this row
  if (j0 >= nc) return;
  const bool active = dl.used && j < nc;

  float best = -INFINITY;
  if (active) best = score_group<T, D, G, SPEC, PAGED>(a, stage, b, g, li, st, q, pre ? pp : nullptr, pst);
  if (li == 0) red[gi] = best;
  __syncthreads();
  if (tid < cpw) {
    const int jj = j0 + tid;
    if (jj < nc) {
      float m = red[tid * a.hpw];
      for (int x = 1; x < a.hpw; ++x) m = fmaxf(m, red[tid * a.hpw + x]);
      stage_scores(a, stage, r, dl.sl)[jj] = score_key(m);
    }
  }
}

// Top-K of stage `stage - 1` fused with the SelectRep scoring of stage `stage`
// (decode, bf16). Every workgroup of the scoring launch selects the row's kept
// chunks of the previous stage itself from that stage's complete score list
// (select_keys, the latency-oriented selection), so the two steps meet at one
// kernel boundary instead of two; workgroup 0 also writes the kept starts and
// their count for the stages after. The tournaments are those of
// k_score_decode.
template <typename T, int D, int G, int SPEC, int E, bool PAGED>
__global__ void __launch_bounds__(256, 2) k_topk_score_decode(PruneArgs a, int stage) {
  constexpr int EPL = D / 16;
  using Row = RowSlice<T, EPL>;
  __shared__ SelectKeysLds<kTopkWaves> L;
  __shared__ int sprev[kFusedMaxKept];
  __shared__ int skept[kFusedMaxKept + 64];
  __shared__ float red[16];
  const KvLayout& kv = a.kv;
  const int ps = stage - 1;                     // the stage selected here
  const int r = blockIdx.y, b = r;              // one row per sequence
  const int tid = threadIdx.x;
  const int gi = tid >> 4, li = tid & 15;
  const DecodeLane dl = decode_lane(a, blockIdx.x, gi);
  const int cpw = dl.cpw, j0 = dl.j0, g = dl.g;  // chunks per workgroup, first chunk, kv head
  const T* Q = static_cast<const T*>(a.q);

  // independent loads first: sequence length, the count before stage ps,
  // this thread's keys of stage ps, the kept starts of stage ps-1, the query
  const int e = seq_len_of(kv, r);
  const int nc_before = ps > 0 ? a.cnt[r * kMaxStages + ps - 1] : 0;
  uint32_t key[E];
  load_keys<E>(a, ps, r, threadIdx.x * E, key);
  if (ps > 0) load_kept_starts(a, ps - 1, r, sprev);
  Row q[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) q[hh].load(Q + (static_cast<size_t>(b) * kv.Hq + g * G + hh) * D + li * EPL);

  const Geo geo = make_geo(e - 1, e, a.n_sink, a.n_window, a.chunk[0]);
  const int lgp = a.lchunk[ps];
  const int shp = ps > 0 ? a.lchunk[ps - 1] - lgp : 0;
  const int nc_ps = ps == 0 ? geo.n1 : nc_before << shp;
  const int kc_ps = a.keep[ps] >> lgp;
  const int n_sel = select_keys<E>(key, nc_ps, kc_ps, L, skept);
  __syncthreads();                              // the kept chunk indices are in skept
  if (blockIdx.x == 0) {                        // workgroup 0 records the stage's output
    int32_t* out = stage_starts(a, ps, r);
    for (int i = tid; i < n_sel; i += 256) out[i] = kept_start(a, ps, skept[i], sprev);
    if (tid == 0) record_stage(a, ps, r, n_sel, geo);
  }

  // stage `stage`: chunks of chunk[stage] keys tiling the kept chunks
  const int sh = lgp - a.lchunk[stage];
  const int nc = n_sel << sh;
  if (nc <= (a.keep[stage] >> a.lchunk[stage])) return;   // stage keeps everything for this row
  if (j0 >= nc) return;
  const int j = j0 + dl.cl;
  const bool active = dl.used && j < nc;
  const int st = kept_start(a, ps, skept[min(j >> sh, n_sel - 1)], sprev) +
                 ((j & ((1 << sh) - 1)) << a.lchunk[stage]);
  float best = -INFINITY;
  if (active) best = score_group<T, D, G, SPEC, PAGED, true>(a, stage, b, g, li, st, q);
  if (li == 0) red[gi] = best;
  __syncthreads();
  if (tid < cpw) {
    const int jj = j0 + tid;
    if (jj < nc) {
      float m = red[tid * a.hpw];
      for (int x = 1; x < a.hpw; ++x) m = fmaxf(m, red[tid * a.hpw + x]);
      stage_scores(a, stage, r, dl.sl)[jj] = score_key(m);
    }
  }
}

// ------------------------------------------------------------------------- //
// prefill scoring (generic FMA path): b_q queries per row                   //
// ------------------------------------------------------------------------- //
// Workgroup = 16 chunks of one row, one lane group per chunk. Heads are
// processed one after another with the head's query block staged in LDS; all
// groups evaluate in lockstep (same chunk length), each step staging its
// current key row in LDS; each lane covers b_q/16 queries.
template <typename T, int D>
__global__ void __launch_bounds__(256) k_score_prefill(PruneArgs a, int stage) {
  constexpr int EPL = D / 16;
  const KvLayout& kv = a.kv;
  const int r = blockIdx.y;
  int b, s, e;
  row_bounds(kv, r, b, s, e);
  const Geo geo = make_geo(s, e, a.n_sink, a.n_window, a.chunk[0]);
  const int nc = stage_input_chunks(a, stage, r, geo);
  const int l = a.chunk[stage];
  if (nc <= (a.keep[stage] >> a.lchunk[stage])) return;
  const int j0 = blockIdx.x * 16;
  if (j0 >= nc) return;

  const int tid = threadIdx.x, gi = tid >> 4, li = tid & 15;
  const int j = j0 + gi;
  const bool active = j < nc;
  const int bq = kv.bq;
  const int G = kv.Hq / kv.Hkv;
  __shared__ float qs[64][D + 1];
  __shared__ float ks[16][D + 4];
  const T* K = static_cast<const T*>(a.k);
  const T* Q = static_cast<const T*>(a.q);
  const int st = active ? chunk_start(a, stage, r, j) : 0;
  int n_iter = 0;
  while ((1 << n_iter) < l) ++n_iter;

  float best = -INFINITY;
  unsigned long long nvis = 0;
  for (int h = 0; h < kv.Hq; ++h) {
    const int g = h / G;
    __syncthreads();
    for (int x = tid; x < bq * D; x += 256) {
      const int t = x / D, dd = x - t * D;
      qs[t][dd] = load_one<T>(Q + ((static_cast<size_t>(b) * kv.Hq + h) * kv.T + s + t) * D + dd);
    }
    // evaluate sigma(position) for this group's row; all groups call in lockstep
    auto eval = [&](int pos) -> float {
      __syncthreads();
      if (active) {
        float kr[EPL];
        SliceLoad<T, EPL>::run(K + kv_offset(kv, b, g, pos) + li * EPL, kr);
#pragma unroll
        for (int x = 0; x < EPL; ++x) ks[gi][li * EPL + x] = kr[x];
      }
      __syncthreads();
      float m = -INFINITY;
      if (active) {
        for (int t = li; t < bq; t += 16) {
          float acc = 0.f;
#pragma unroll 8
          for (int x = 0; x < D; ++x) acc = fmaf(qs[t][x], ks[gi][x], acc);
          m = fmaxf(m, acc);
        }
      }
      return group16_max(m);
    };
    int lo = 0, hi = l - 1;
    float sa = eval(st);
    for (int it = 0; it < n_iter; ++it) {
      const int mid = (lo + hi + 1) >> 1;
      const float sm = eval(st + mid);
      if (sm > sa) { lo = mid; sa = sm; }
      else         { hi = mid - 1; }
    }
    best = fmaxf(best, sa);
  }
  (void)nvis;
  if (active && li == 0) stage_scores(a, stage, r)[j] = score_key(best);
}

// ------------------------------------------------------------------------- //
// launcher                                                                  //
// ------------------------------------------------------------------------- //
static const char* const kScoreNames[kMaxStages] = {"prune_score_stage1", "prune_score_stage2",
                                                    "prune_score_stage3", "prune_score_stage4"};
static const char* const kTopkNames[kMaxStages] = {"prune_topk_stage1", "prune_topk_stage2",
                                                   "prune_topk_stage3", "prune_topk_stage4"};
static const char* const kFusedNames[kMaxStages] = {"", "prune_topk1_score2", "prune_topk2_score3",
                                                    "prune_topk3_score4"};
constexpr int kSpecMaxChunk = 64;       // chunks this small preload their first three splits

// Speculative first round of a decode tournament: chunks of 8..64 keys load
// the 8 keys that can represent the first three splits at once, longer chunks
// the 4 of the first two (8 rows would cost too many registers for the
// stage-1 launch to keep every workgroup resident), shorter ones none.
static int spec_of(int l) { return l >= 8 && l <= kSpecMaxChunk ? 8 : l > kSpecMaxChunk ? 4 : 0; }
constexpr long long kFuseMaxWorkgroups = 2048;   // largest fused top-K + scoring launch

template <typename T, int D, int G>
static void launch_decode_score(const PruneArgs& a, int stage, int max_chunks, hipStream_t st) {
  const int cpw = 16 / a.hpw;
  if (max_chunks <= 0) return;
  dim3 grid((max_chunks + cpw - 1) / cpw * a.nsl, a.R);
  const char* nm = kScoreNames[stage];
  const int spec = spec_of(a.chunk[stage]);
  if (a.kv.block_table) {
    if (spec == 8)      DSA_LAUNCH(nm, (k_score_decode<T, D, G, 8, true>), grid, dim3(256), st, a, stage);
    else if (spec == 4) DSA_LAUNCH(nm, (k_score_decode<T, D, G, 4, true>), grid, dim3(256), st, a, stage);
    else                DSA_LAUNCH(nm, (k_score_decode<T, D, G, 0, true>), grid, dim3(256), st, a, stage);
  } else {
    if (spec == 8)      DSA_LAUNCH(nm, (k_score_decode<T, D, G, 8, false>), grid, dim3(256), st, a, stage);
    else if (spec == 4) DSA_LAUNCH(nm, (k_score_decode<T, D, G, 4, false>), grid, dim3(256), st, a, stage);
    else                DSA_LAUNCH(nm, (k_score_decode<T, D, G, 0, false>), grid, dim3(256), st, a, stage);
  }
}

void launch_topk(const PruneArgs& a, int stage, int max_chunks, hipStream_t st) {
  const char* nm = kTopkNames[stage];
  if (max_chunks <= kTopkThreads * 4) {
    DSA_LAUNCH(nm, (k_topk<4>), dim3(a.R), dim3(kTopkThreads), st, a, stage);
  } else if (max_chunks <= kTopkThreads * 16) {
    DSA_LAUNCH(nm, (k_topk<16>), dim3(a.R), dim3(kTopkThreads), st, a, stage);
  } else if (max_chunks <= 1024 * 16) {   // large rows: 16 waves, 16 keys per thread
    DSA_LAUNCH(nm, (k_topk<16, 1024>), dim3(a.R), dim3(1024), st, a, stage);
  } else {
    DSA_LAUNCH(nm, (k_topk<32, 1024>), dim3(a.R), dim3(1024), st, a, stage);
  }
}

// Top-K of stage-1 and scoring of `stage` in one launch (bf16 decode, at most
// 4096 chunks in the selected stage); false if this shape takes the separate
// kernels.
template <typename T, int D, int G>
static bool launch_decode_fused(const PruneArgs& a, int stage, int max_chunks, int sel_chunks,
                                hipStream_t st) {
  if constexpr (sizeof(T) != 2) {
    return false;
  } else {
    const int cpw = 16 / a.hpw;
    // at least one workgroup: workgroup 0 writes the selected stage's starts
    const dim3 grid(std::max(1, (max_chunks + cpw - 1) / cpw) * a.nsl, a.R);
    // every workgroup repeats the row's selection: worth it only while that
    // redundant work is small next to a kernel boundary (one sequence); a
    // batch takes the one-workgroup-per-row selection kernel instead
    if (static_cast<long long>(grid.x) * grid.y > kFuseMaxWorkgroups) return false;
    // the fused launch is for one sequence: contiguous K only
    if (a.kv.block_table) return false;
    // kept lists held in LDS: the selected stage's and the one before it
    const int ps = stage - 1;
    if ((a.keep[ps] >> a.lchunk[ps]) > kFusedMaxKept) return false;
    if (ps > 0 && (a.keep[ps - 1] >> a.lchunk[ps - 1]) > kFusedMaxKept) return false;
    const int spec = spec_of(a.chunk[stage]);
    const char* nm = kFusedNames[stage];
    if (sel_chunks <= kTopkThreads * 4) {
      if (spec == 8)      DSA_LAUNCH(nm, (k_topk_score_decode<T, D, G, 8, 4, false>), grid, dim3(256), st, a, stage);
      else if (spec == 4) DSA_LAUNCH(nm, (k_topk_score_decode<T, D, G, 4, 4, false>), grid, dim3(256), st, a, stage);
      else                DSA_LAUNCH(nm, (k_topk_score_decode<T, D, G, 0, 4, false>), grid, dim3(256), st, a, stage);
    } else if (sel_chunks <= kTopkThreads * 16) {
      if (spec == 8)      DSA_LAUNCH(nm, (k_topk_score_decode<T, D, G, 8, 16, false>), grid, dim3(256), st, a, stage);
      else if (spec == 4) DSA_LAUNCH(nm, (k_topk_score_decode<T, D, G, 4, 16, false>), grid, dim3(256), st, a, stage);
      else                DSA_LAUNCH(nm, (k_topk_score_decode<T, D, G, 0, 16, false>), grid, dim3(256), st, a, stage);
    } else {
      return false;
    }
    return true;
  }
}

// Decode: score stage 1; for every later stage, the previous stage's top-K
// and this stage's scoring (fused where possible); the last top-K writes idx
// (unless `last_topk` is false: the fused decode step selects it itself).
template <typename T, int D, int G>
static void launch_decode(const PruneArgs& a, hipStream_t st, bool last_topk = true) {
  auto chunks_of = [&](int stage) {               // longest input list of a stage
    return stage == 0 ? a.n1max : a.keep[stage - 1] / a.chunk[stage];
  };
  launch_decode_score<T, D, G>(a, 0, chunks_of(0), st);
  for (int stage = 1; stage < a.n_stages; ++stage) {
    if (!launch_decode_fused<T, D, G>(a, stage, chunks_of(stage), chunks_of(stage - 1), st)) {
      launch_topk(a, stage - 1, chunks_of(stage - 1), st);
      launch_decode_score<T, D, G>(a, stage, chunks_of(stage), st);
    }
  }
  if (last_topk) launch_topk(a, a.n_stages - 1, chunks_of(a.n_stages - 1), st);
}

int last_stage_chunks(const PruneArgs& a) {
  const int ls = a.n_stages - 1;
  return ls == 0 ? a.n1max : a.keep[ls - 1] / a.chunk[ls];
}

// Decode with remembered stages: each due stage is scored from the current
// record of the stage before it (or the whole middle for stage 1) and its
// top-K replaces its record; the top-K of a due stage whose successor is due
// too is fused into that successor's scoring as in launch_decode. When the
// last stage is not due, its record is only turned into the index row.
template <typename T, int D, int G>
static void launch_decode_cached(const PruneArgs& a, const bool* due, hipStream_t st) {
  auto chunks_of = [&](int stage) {
    return stage == 0 ? a.n1max : a.keep[stage - 1] / a.chunk[stage];
  };
  const int S = a.n_stages;
  bool pending = false;                           // a stage scored here still needs its top-K
  for (int stage = 0; stage < S; ++stage) {
    if (!due[stage]) continue;
    if (pending) {                                // stage - 1 was scored in this call
      if (!launch_decode_fused<T, D, G>(a, stage, chunks_of(stage), chunks_of(stage - 1), st)) {
        launch_topk(a, stage - 1, chunks_of(stage - 1), st);
        launch_decode_score<T, D, G>(a, stage, chunks_of(stage), st);
      }
    } else {
      launch_decode_score<T, D, G>(a, stage, chunks_of(stage), st);
    }
    pending = true;
    if (stage + 1 == S || !due[stage + 1]) {
      launch_topk(a, stage, chunks_of(stage), st);
      pending = false;
    }
  }
  if (!due[S - 1]) DSA_LAUNCH("prune_assemble", k_assemble, dim3(a.R), dim3(kTopkThreads), st, a);
}

template <typename T, int D>
static hipError_t launch_cached_typed(const PruneArgs& a, const bool* due, hipStream_t st) {
  switch (a.kv.Hq / a.kv.Hkv) {
    case 1: launch_decode_cached<T, D, 1>(a, due, st); break;
    case 2: launch_decode_cached<T, D, 2>(a, due, st); break;
    case 4: launch_decode_cached<T, D, 4>(a, due, st); break;
    case 8: launch_decode_cached<T, D, 8>(a, due, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_prune_cached(const PruneArgs& a, const bool* due, int dtype, hipStream_t st) {
  if (!a.kv.decode || !a.mid_end) return hipErrorInvalidValue;
  if (dtype == 1) {
    if (a.kv.D == 128) return launch_cached_typed<uint16_t, 128>(a, due, st);
    if (a.kv.D == 64) return launch_cached_typed<uint16_t, 64>(a, due, st);
  } else {
    if (a.kv.D == 128) return launch_cached_typed<float, 128>(a, due, st);
    if (a.kv.D == 64) return launch_cached_typed<float, 64>(a, due, st);
  }
  return hipErrorInvalidValue;
}

template <typename T, int D>
static hipError_t launch_typed(const PruneArgs& a, hipStream_t st) {
  const int G = a.kv.Hq / a.kv.Hkv;
  if (a.kv.decode) {
    switch (G) {
      case 1: launch_decode<T, D, 1>(a, st); break;
      case 2: launch_decode<T, D, 2>(a, st); break;
      case 4: launch_decode<T, D, 4>(a, st); break;
      case 8: launch_decode<T, D, 8>(a, st); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  for (int stage = 0; stage < a.n_stages; ++stage) {
    // longest input list any row can present to this stage
    const int max_chunks = stage == 0 ? a.n1max : a.keep[stage - 1] / a.chunk[stage];
    if (max_chunks > 0 &&
        !(sizeof(T) == 2 && launch_score_prefill_mfma(a, stage, max_chunks, st, kScoreNames[stage]))) {
      dim3 grid((max_chunks + 15) / 16, a.R);
      DSA_LAUNCH(kScoreNames[stage], (k_score_prefill<T, D>), grid, dim3(256), st, a, stage);
    }
    launch_topk(a, stage, max_chunks, st);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

// Plain scoring of one prefill stage on bf16 rows (the matrix-core kernel for
// query blocks of 64, else the generic one).
void launch_score_prefill_bf16(const PruneArgs& a, int stage, int max_chunks, hipStream_t st, const char* name) {
  if (max_chunks <= 0 || launch_score_prefill_mfma(a, stage, max_chunks, st, name)) return;
  const dim3 grid((max_chunks + 15) / 16, a.R);
  if (a.kv.D == 128) DSA_LAUNCH(name, (k_score_prefill<uint16_t, 128>), grid, dim3(256), st, a, stage);
  else               DSA_LAUNCH(name, (k_score_prefill<uint16_t, 64>), grid, dim3(256), st, a, stage);
}

template <typename T, int D>
static hipError_t launch_stages_typed(const PruneArgs& a, hipStream_t st) {
  switch (a.kv.Hq / a.kv.Hkv) {
    case 1: launch_decode<T, D, 1>(a, st, false); break;
    case 2: launch_decode<T, D, 2>(a, st, false); break;
    case 4: launch_decode<T, D, 4>(a, st, false); break;
    case 8: launch_decode<T, D, 8>(a, st, false); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_prune_decode_stages(const PruneArgs& a, int dtype, hipStream_t st) {
  if (!a.kv.decode) return hipErrorInvalidValue;
  if (dtype == 1) {
    if (a.kv.D == 128) return launch_stages_typed<uint16_t, 128>(a, st);
    if (a.kv.D == 64) return launch_stages_typed<uint16_t, 64>(a, st);
  } else {
    if (a.kv.D == 128) return launch_stages_typed<float, 128>(a, st);
    if (a.kv.D == 64) return launch_stages_typed<float, 64>(a, st);
  }
  return hipErrorInvalidValue;
}

// Decode pruning with its own (query, keys) per stage: as[s] holds the
// arguments of stage s (bf16 rows: the rotated copies of the chunk-indexed
// RoPE style), everything else shared. The stages run as in launch_decode.
template <int D, int G>
static void launch_decode_staged(const PruneArgs* as, hipStream_t st) {
  const PruneArgs& a = as[0];
  auto chunks_of = [&](int stage) { return stage == 0 ? a.n1max : a.keep[stage - 1] / a.chunk[stage]; };
  launch_decode_score<uint16_t, D, G>(as[0], 0, chunks_of(0), st);
  for (int stage = 1; stage < a.n_stages; ++stage) {
    if (!launch_decode_fused<uint16_t, D, G>(as[stage], stage, chunks_of(stage), chunks_of(stage - 1), st)) {
      launch_topk(as[stage - 1], stage - 1, chunks_of(stage - 1), st);
      launch_decode_score<uint16_t, D, G>(as[stage], stage, chunks_of(stage), st);
    }
  }
  launch_topk(as[a.n_stages - 1], a.n_stages - 1, chunks_of(a.n_stages - 1), st);
}

template <int D>
static hipError_t launch_staged_d(const PruneArgs* as, hipStream_t st) {
  switch (as[0].kv.Hq / as[0].kv.Hkv) {
    case 1: launch_decode_staged<D, 1>(as, st); break;
    case 2: launch_decode_staged<D, 2>(as, st); break;
    case 4: launch_decode_staged<D, 4>(as, st); break;
    case 8: launch_decode_staged<D, 8>(as, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_prune_decode_staged(const PruneArgs* as, hipStream_t st) {
  if (!as[0].kv.decode) return hipErrorInvalidValue;
  if (as[0].kv.D == 128) return launch_staged_d<128>(as, st);
  if (as[0].kv.D == 64) return launch_staged_d<64>(as, st);
  return hipErrorInvalidValue;
}

hipError_t launch_prune(const PruneArgs& a, int dtype, hipStream_t st) {
  if (dtype == 1) {
    if (a.kv.D == 128) return launch_typed<uint16_t, 128>(a, st);
    if (a.kv.D == 64) return launch_typed<uint16_t, 64>(a, st);
  } else {
    if (a.kv.D == 128) return launch_typed<float, 128>(a, st);
    if (a.kv.D == 64) return launch_typed<float, 64>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace dsa
