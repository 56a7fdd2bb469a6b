// One decode step of pruning and attention with the tail fused: the last
// stage's top-K and the gathered split attention in a single launch.
//
// The selection is the last stage's step 6 of the InfiniteHiP page's pruning
// stage (section 3.4, "Formal Mechanism of a Single Pruning Stage"); the
// attention is the split-key "Flash Decoding" pass of its "Block Sparse
// Attention Implementation", with the partial softmax merge of the InfLLM blog
// page ("Mathematical Formulation of Efficient Softmax Normalization").
//
// The index row of a sequence is cut into splits of kSplitKeys entries, the
// grid anchored where the sinks end so the kept entries fill whole splits
// (split 0 then holds the sinks and padding before entry 0); one workgroup
// owns one (split, kv head, sequence):
//   * a split that holds kept chunks of the last stage selects the row's kept
//     chunks itself from the stage's complete score list (select_keys, the
//     same selection as k_topk: score descending, lower chunk first), so the
//     selection needs no kernel of its own; splits of sinks, window or padding
//     skip it and start their loads at once;
//   * the workgroups of kv head 0 write the row's entries (the idx output);
//   * the split's K and V rows are gathered (16 lanes per 256-byte row, eight
//     rows per lane group), scored against the kv head's query heads, and an
//     unnormalised partial (local max m, sum l, o[d]) per query head is
//     written, as the split-partial decode kernel does.
// A second kernel (the split-partial merge of the separate decode path) turns
// the partials into the output. (Merging in the last-arriving workgroup was
// measured slower: the device-scope release and acquire around the arrival
// counter write back and invalidate the L2 of every XCD, about 10 us per
// step at 1M.)
#include <algorithm>

#include "prune_common.h"
#include "topk_select.h"

namespace dsa {

// The workgroup's partial (o[D], m, l) per head from each lane's share of
// o and l (already relative to the workgroup maximum M): summed over the
// wave's four lane groups by lane swaps, then over the four waves in LDS, and
// written as split sp's partial.
template <int D, int G>
__device__ __forceinline__ void write_partials(const float (&o)[G][D / 16], const float (&lsum)[G], const float (&M)[G],
                                               float (&sred)[4][G * D + G], float* part, int nsp, int sp,
                                               const KvLayout& kv, int b, int g) {
  constexpr int EPL = D / 16;
  constexpr int NO = (G * D) / 256;           // outputs per thread in the reduction (G * D >= 256)
  static_assert(G * D % 256 == 0, "whole outputs per thread");
  const int tid = threadIdx.x, li = tid & 15, lane = tid & 63, w = tid >> 6;
  // Sum over the wave's four lane groups (16-lane rows), four values at a
  // time: a row swap of values (a, b) and one of (c, d) leave the pair sums
  // of a and b, c and d interleaved by row, and a half swap of those leaves
  // in row r the total of value r, added as (r0 + r1) + (r2 + r3); each row
  // writes its value. Then over the waves in LDS.
  constexpr int NV = G * EPL + G;               // per lane: o[hh][x], then lsum[hh]
  auto val = [&](int i) -> float {
    return i < G * EPL ? o[i / EPL][i % EPL] : i < NV ? lsum[i - G * EPL] : 0.f;
  };
  const int row = lane >> 4;
#pragma unroll
  for (int i = 0; i < NV; i += 4) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(val(i)), __float_as_uint(val(i + 1)), false, false);
    const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(val(i + 2)), __float_as_uint(val(i + 3)), false, false);
    const float s01 = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    const float s23 = __uint_as_float(q[0]) + __uint_as_float(q[1]);
    const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(s01), __float_as_uint(s23), false, false);
    const float tot = __uint_as_float(t[0]) + __uint_as_float(t[1]);
    const int vi = i + row;                     // the value whose total this row holds
    if (vi < G * EPL) sred[w][(vi / EPL) * D + li * EPL + vi % EPL] = tot;
    else if (vi < NV && li == 0) sred[w][G * D + vi - G * EPL] = tot;
  }
  __syncthreads();
  float* P = part;
  const size_t head0 = static_cast<size_t>(b) * kv.Hq + g * G;
#pragma unroll
  for (int i = 0; i < NO; ++i) {
    const int oi = tid + 256 * i;
    const int hh = oi / D, dd = oi - hh * D;
    const float v = (sred[0][oi] + sred[1][oi]) + (sred[2][oi] + sred[3][oi]);
    P[((head0 + hh) * nsp + sp) * (D + 2) + dd] = v;
  }
  if (tid < G) {
    const float lt = (sred[0][G * D + tid] + sred[1][G * D + tid]) + (sred[2][G * D + tid] + sred[3][G * D + tid]);
    float* mlp = P + ((head0 + tid) * nsp + sp) * (D + 2) + D;
    mlp[0] = M[tid];
    mlp[1] = lt;
  }
}

// One split's partial softmax for the G query heads of kv head g of sequence
// b: the split's row positions are in spos (negative = padding, masked); lane
// group gi gathers the K and V rows of entries gi + 16u (16-lane 256-byte row
// loads, all issued before any arithmetic), scores them against the heads'
// queries in registers, and the workgroup writes (o[D], m, l) per head to
// part[((b * Hq + g * G + hh) * nsp + sp) * (D + 2)]: the split partials that
// k_decode_combine merges ("Flash Decoding" of the InfiniteHiP page's "Block
// Sparse Attention Implementation"; the merge of the InfLLM blog page's
// "Mathematical Formulation of Efficient Softmax Normalization").
// With sphys (paged, or nullptr) the split's rows come page-resolved
// ((page id << page_shift) | offset in the page), and the page table is not
// read.
template <int D, int G, bool PAGED, int kKeysPerGroup>
__device__ __forceinline__ void split_partial(const KvLayout& kv, const uint16_t* K, const uint16_t* V,
                                              const RowSlice<uint16_t, D / 16> (&q)[G], const int* spos,
                                              float (&smax)[16][G], float (&sred)[4][G * D + G], float* part,
                                              int nsp, int sp, int b, int g, float scale_log2,
                                              const int* sphys = nullptr) {
  constexpr int EPL = D / 16;
  using Row = RowSlice<uint16_t, EPL>;
  const int tid = threadIdx.x, gi = tid >> 4, li = tid & 15;
  // gather the split's K and V rows: lane group gi takes entries gi + 16u.
  // Every row's offset is formed first (paged: all page-table reads at once),
  // then all row loads go out together: a table read behind a per-row branch
  // would make the compiler wait for the loads in flight at every join.
  int pu[kKeysPerGroup];
  size_t off[kKeysPerGroup];
#pragma unroll
  for (int u = 0; u < kKeysPerGroup; ++u) pu[u] = spos[gi + 16 * u];
  if constexpr (PAGED) {
    const int mask = kv.page_size - 1;
    if (sphys) {
#pragma unroll
      for (int u = 0; u < kKeysPerGroup; ++u) {
        const int pr = max(sphys[gi + 16 * u], 0);
        off[u] = ((static_cast<size_t>(pr >> kv.page_shift) * kv.Hkv + g) * kv.page_size + (pr & mask)) * D;
      }
    } else {
      const int32_t* tb = kv.block_table + static_cast<size_t>(b) * kv.max_pages;
      int page[kKeysPerGroup];
#pragma unroll
      for (int u = 0; u < kKeysPerGroup; ++u) page[u] = tb[max(pu[u], 0) >> kv.page_shift];
#pragma unroll
      for (int u = 0; u < kKeysPerGroup; ++u)
        off[u] = ((static_cast<size_t>(page[u]) * kv.Hkv + g) * kv.page_size + (max(pu[u], 0) & mask)) * D;
    }
  } else {
#pragma unroll
    for (int u = 0; u < kKeysPerGroup; ++u)
      off[u] = ((static_cast<size_t>(b) * kv.Hkv + g) * kv.T + max(pu[u], 0)) * D;   // padding reads row 0
  }
  Row kr[kKeysPerGroup], vr[kKeysPerGroup];
#pragma unroll
  for (int u = 0; u < kKeysPerGroup; ++u) {
    kr[u].load(K + off[u] + li * EPL);
    vr[u].load(V + off[u] + li * EPL);
  }
  float sc[kKeysPerGroup][G];
  float mloc[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) mloc[hh] = kNegBig;
#pragma unroll
  for (int u = 0; u < kKeysPerGroup; ++u) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float d = group16_sum(kr[u].dot(q[hh])) * scale_log2;
      sc[u][hh] = pu[u] >= 0 ? d : -INFINITY;
      mloc[hh] = fmaxf(mloc[hh], sc[u][hh]);
    }
  }
  if (li == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) smax[gi][hh] = mloc[hh];
  }
  __syncthreads();
  float M[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    float m = smax[0][hh];
#pragma unroll
    for (int x = 1; x < 16; ++x) m = fmaxf(m, smax[x][hh]);
    M[hh] = m;
  }
  // this group's share of l and o = sum_u 2^(s_u - M) v_u
  float lsum[G], o[G][EPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    lsum[hh] = 0.f;
#pragma unroll
    for (int x = 0; x < EPL; ++x) o[hh][x] = 0.f;
  }
#pragma unroll
  for (int u = 0; u < kKeysPerGroup; ++u) {
    float vf[EPL];
#pragma unroll
    for (int x = 0; x < EPL / 2; ++x) {
      vf[2 * x] = __uint_as_float(vr[u].w[x] << 16);
      vf[2 * x + 1] = __uint_as_float(vr[u].w[x] & 0xffff0000u);
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      // (the hardware exponential: arguments are <= 0; below -126 it returns
      // 0 where the library routine would give a denormal, a difference
      // under 1e-38 in the sums)
      const float pz = sc[u][hh] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc[u][hh] - M[hh]);
      lsum[hh] += pz;
#pragma unroll
      for (int x = 0; x < EPL; ++x) o[hh][x] = fmaf(pz, vf[x], o[hh][x]);
    }
  }
  write_partials<D, G>(o, lsum, M, sred, part, nsp, sp, kv, b, g);
}

template <int D, int G, int E, bool PAGED, int kSplitKeys = kStepSplitKeys>
__global__ void __launch_bounds__(256, 2) k_decode_attend(StepArgs s) {
  constexpr int kKeysPerGroup = kSplitKeys / 16;
  using T = uint16_t;
  constexpr int EPL = D / 16;
  using Row = RowSlice<T, EPL>;
  __shared__ SelectKeysLds<kTopkWaves> LS;
  __shared__ int sprev[kFusedMaxKept];
  __shared__ int skept[kFusedMaxKept + 64];
  __shared__ int spos[kSplitKeys];
  __shared__ float smax[16][G];
  __shared__ float sred[4][G * D + G];

  const PruneArgs& a = s.p;
  const KvLayout& kv = a.kv;
  // workgroup order: the splits that hold kept chunks (and select) first, for
  // every kv head, then the sink / window / padding splits, so the selecting
  // workgroups are the first ones placed on the CUs
  const int b = blockIdx.z, r = b;
  int sp, g;
  {
    const int lin = blockIdx.y * gridDim.x + blockIdx.x;
    const int nk = (s.ks1 - s.ks0) * kv.Hkv;
    if (lin < nk) {
      sp = s.ks0 + lin / kv.Hkv;
      g = lin % kv.Hkv;
    } else {
      const int o = (lin - nk) / kv.Hkv;
      sp = o < s.ks0 ? o : o + (s.ks1 - s.ks0);
      g = (lin - nk) % kv.Hkv;
    }
  }
  const int tid = threadIdx.x, li = tid & 15;
  const T* Q = static_cast<const T*>(a.q);
  const T* K = static_cast<const T*>(a.k);
  const T* V = static_cast<const T*>(s.v);

  // The last stage's scores and the previous stage's kept starts are loaded
  // by every workgroup as it starts, together with the row length and kept
  // count that decide whether the workgroup selects at all: one memory round
  // trip instead of two (the loads of a workgroup that does not select are
  // not used; all are within the lists).
  const int ls = a.n_stages - 1;
  uint32_t key[E];
  load_keys<E>(a, ls, r, threadIdx.x * E, key);
  if (ls > 0) load_kept_starts(a, ls - 1, r, sprev);

  // row geometry of the last stage (uniform over the row's workgroups)
  const int e = seq_len_of(kv, b);
  const int lg = a.lchunk[ls];
  const int shp = ls > 0 ? a.lchunk[ls - 1] - lg : 0;
  const int nc_before = ls > 0 ? a.cnt[r * kMaxStages + ls - 1] : 0;
  Row q[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) q[hh].load(Q + (static_cast<size_t>(b) * kv.Hq + g * G + hh) * D + li * EPL);
  const Geo geo = make_geo(e - 1, e, a.n_sink, a.n_window, a.chunk[0]);
  const int nc = ls == 0 ? geo.n1 : nc_before << shp;
  const int kc = a.keep[ls] >> lg;
  const int n_sel = min(nc, kc);
  const int win0 = geo.sink_hi + (n_sel << lg);   // kept chunks fill [sink_hi, win0)
  const int end = win0 + max(0, e - geo.mid_hi);  // then the window [mid_hi, e)
  const int i0 = sp * kSplitKeys - s.sh0;          // (split 0 may start before entry 0)

  if (i0 < win0 && i0 + kSplitKeys > geo.sink_hi) {
    select_keys<E>(key, nc, kc, LS, skept);
    __syncthreads();                            // skept holds the kept chunk indices
  }
  if (tid < kSplitKeys) {
    const int i = i0 + tid;
    int p = -1;
    if (i < 0) {
      p = -1;
    } else if (i < geo.sink_hi) {
      p = i;
    } else if (i < win0) {
      const int c = i - geo.sink_hi;
      p = kept_start(a, ls, skept[c >> lg], sprev) + (c & ((1 << lg) - 1));
    } else if (i < end) {
      p = geo.mid_hi + (i - win0);
    }
    if (g == 0 && i >= 0 && i < a.L) a.idx[static_cast<size_t>(r) * a.L + i] = p;
    spos[tid] = p;
  }
  __syncthreads();

  split_partial<D, G, PAGED, kKeysPerGroup>(kv, K, V, q, spos, smax, sred, s.part, s.nsp, sp, b, g, s.scale_log2);
}

// Split partials over index rows given in memory (the two-call decode path:
// dsa_sparse_attn after a separate prune_select): the same splits of
// kStepSplitKeys entries and the same gather and reduction as the fused step,
// with the positions read from the row (entries past the row, negative or
// after the query are padding).
template <int D, int G, bool PAGED>
__global__ void __launch_bounds__(256, 2) k_decode_rows(AttnArgs a) {
  constexpr int kKeysPerGroup = kStepSplitKeys / 16;
  constexpr int EPL = D / 16;
  using Row = RowSlice<uint16_t, EPL>;
  __shared__ int spos[kStepSplitKeys];
  __shared__ int sphys[PAGED ? kStepSplitKeys : 1];
  __shared__ float smax[16][G];
  __shared__ float sred[4][G * D + G];
  const KvLayout& kv = a.kv;
  const int sp = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, li = tid & 15;
  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  Row q[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) q[hh].load(Q + (static_cast<size_t>(b) * kv.Hq + g * G + hh) * D + li * EPL);
  const int tq = seq_len_of(kv, b) - 1;
  const bool phys = PAGED && a.prow != nullptr;
  if (tid < kStepSplitKeys) {
    const int i = sp * kStepSplitKeys + tid;
    int p = -1, pr = -1;
    if (i < a.L) {
      p = a.idx[static_cast<size_t>(b) * a.L + i];
      if (phys) pr = a.prow[static_cast<size_t>(b) * a.L + i];
      if (p < 0 || p > tq) p = -1;
    }
    spos[tid] = p;
    if constexpr (PAGED) sphys[tid] = pr;
  }
  __syncthreads();
  split_partial<D, G, PAGED, kKeysPerGroup>(kv, static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v),
                                            q, spos, smax, sred, a.part, a.n_splits, sp, b, g, a.scale_log2,
                                            phys ? sphys : nullptr);
}

// ------------------------------------------------------------------------- //
// launcher                                                                  //
// ------------------------------------------------------------------------- //
// True if the fused tail was launched; false if this shape takes the separate
// selection, partial and merge kernels.
template <int D, int G>
static bool launch_attend_typed(const StepArgs& s, int sel_chunks, hipStream_t st) {
  const PruneArgs& a = s.p;
  const dim3 grid(s.nsp, a.kv.Hkv, a.kv.B);
  const int ls = a.n_stages - 1;
  if (static_cast<long long>(grid.x) * grid.y * grid.z > 2048) return false;
  if ((a.keep[ls] >> a.lchunk[ls]) > kFusedMaxKept) return false;
  if (ls > 0 && (a.keep[ls - 1] >> a.lchunk[ls - 1]) > kFusedMaxKept) return false;
  const bool paged = a.kv.block_table != nullptr;
  const char* nm = "decode_topk_attend_partial";
  if (sel_chunks <= kTopkThreads * 4) {
    if (paged) DSA_LAUNCH(nm, (k_decode_attend<D, G, 4, true>), grid, dim3(256), st, s);
    else       DSA_LAUNCH(nm, (k_decode_attend<D, G, 4, false>), grid, dim3(256), st, s);
  } else if (sel_chunks <= kTopkThreads * 16) {
    if (paged) DSA_LAUNCH(nm, (k_decode_attend<D, G, 16, true>), grid, dim3(256), st, s);
    else       DSA_LAUNCH(nm, (k_decode_attend<D, G, 16, false>), grid, dim3(256), st, s);
  } else {
    return false;
  }
  AttnArgs m{};
  m.kv = a.kv;
  m.out = s.out;
  m.part = s.part;
  m.n_splits = s.nsp;
  launch_decode_combine(m, st);
  return true;
}

// Split partials over spans of a.kps entries, several chunks of
// kStepSplitKeys each: the dense decode (entry i is key position i) and index
// rows longer than one chunk per split. Each lane group keeps an online
// softmax (running max, sum and output) over its own entries, gi + 16u of
// every chunk, so the chunks need no barrier; at the end the groups' maxima
// meet in LDS, each group rescales its sums to the workgroup maximum, and the
// partial is written as the one-chunk splits write theirs.
template <int D, int G, bool PAGED, bool ROWS>
__global__ void __launch_bounds__(256, 2) k_decode_span(AttnArgs a) {
  constexpr int KPG = kStepSplitKeys / 16;
  constexpr int EPL = D / 16;
  using Row = RowSlice<uint16_t, EPL>;
  __shared__ float smax[16][G];
  __shared__ float sred[4][G * D + G];
  const KvLayout& kv = a.kv;
  const int sp = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, gi = tid >> 4, li = tid & 15;
  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* K = static_cast<const uint16_t*>(a.k);
  const uint16_t* V = static_cast<const uint16_t*>(a.v);
  Row q[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) q[hh].load(Q + (static_cast<size_t>(b) * kv.Hq + g * G + hh) * D + li * EPL);
  const int tq = seq_len_of(kv, b) - 1;
  const int n_total = ROWS ? a.L : tq + 1;      // (dense: the keys after the query are not visited)
  const int k_begin = sp * a.kps;
  const int k_end = min(n_total, k_begin + a.kps);
  const int32_t* row = ROWS ? a.idx + static_cast<size_t>(b) * a.L : nullptr;
  float m[G], l[G], o[G][EPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m[hh] = kNegBig;
    l[hh] = 0.f;
#pragma unroll
    for (int x = 0; x < EPL; ++x) o[hh][x] = 0.f;
  }
  for (int base = k_begin; base < k_end; base += kStepSplitKeys) {
    // positions, then (paged) pages, then rows, each step's loads issued
    // together (no load behind a per-row branch: its join would wait for
    // every load in flight)
    int pu[KPG];
#pragma unroll
    for (int u = 0; u < KPG; ++u) {
      const int i = base + gi + 16 * u;
      int p = ROWS ? row[min(i, k_end - 1)] : i;
      if (i >= k_end || p < 0 || p > tq) p = -1;
      pu[u] = p;
    }
    size_t off[KPG];
    if constexpr (PAGED) {
      const int32_t* tb = kv.block_table + static_cast<size_t>(b) * kv.max_pages;
      int page[KPG];
#pragma unroll
      for (int u = 0; u < KPG; ++u) page[u] = tb[max(pu[u], 0) >> kv.page_shift];
#pragma unroll
      for (int u = 0; u < KPG; ++u)
        off[u] = ((static_cast<size_t>(page[u]) * kv.Hkv + g) * kv.page_size + (max(pu[u], 0) & (kv.page_size - 1))) *
                 D;
    } else {
#pragma unroll
      for (int u = 0; u < KPG; ++u)
        off[u] = ((static_cast<size_t>(b) * kv.Hkv + g) * kv.T + max(pu[u], 0)) * D;   // padding reads row 0
    }
    Row kr[KPG], vr[KPG];
#pragma unroll
    for (int u = 0; u < KPG; ++u) {
      kr[u].load(K + off[u] + li * EPL);
      vr[u].load(V + off[u] + li * EPL);
    }
    float sc[KPG][G], mc[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) mc[hh] = m[hh];
#pragma unroll
    for (int u = 0; u < KPG; ++u) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float d = group16_sum(kr[u].dot(q[hh])) * a.scale_log2;
        sc[u][hh] = pu[u] >= 0 ? d : -INFINITY;
        mc[hh] = fmaxf(mc[hh], sc[u][hh]);
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {              // the group's sums relative to its new maximum
      const float alpha = __builtin_amdgcn_exp2f(m[hh] - mc[hh]);
      l[hh] *= alpha;
#pragma unroll
      for (int x = 0; x < EPL; ++x) o[hh][x] *= alpha;
      m[hh] = mc[hh];
    }
#pragma unroll
    for (int u = 0; u < KPG; ++u) {
      float vf[EPL];
#pragma unroll
      for (int x = 0; x < EPL / 2; ++x) {
        vf[2 * x] = __uint_as_float(vr[u].w[x] << 16);
        vf[2 * x + 1] = __uint_as_float(vr[u].w[x] & 0xffff0000u);
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float pz = sc[u][hh] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc[u][hh] - m[hh]);
        l[hh] += pz;
#pragma unroll
        for (int x = 0; x < EPL; ++x) o[hh][x] = fmaf(pz, vf[x], o[hh][x]);
      }
    }
  }
  if (li == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) smax[gi][hh] = m[hh];
  }
  __syncthreads();
  float M[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    float mm = smax[0][hh];
#pragma unroll
    for (int x = 1; x < 16; ++x) mm = fmaxf(mm, smax[x][hh]);
    M[hh] = mm;
    const float f = __builtin_amdgcn_exp2f(m[hh] - mm);
    l[hh] *= f;
#pragma unroll
    for (int x = 0; x < EPL; ++x) o[hh][x] *= f;
  }
  write_partials<D, G>(o, l, M, sred, a.part, a.n_splits, sp, kv, b, g);
}

// Split partials over index rows (bf16, d = 128, 2 to 8 query heads per kv
// head) and their merge; a.n_splits must be ceil(a.L / kStepSplitKeys).
template <int G>
static void launch_rows_typed(const AttnArgs& a, hipStream_t st) {
  const dim3 grid(a.n_splits, a.kv.Hkv, a.kv.B);
  const char* nm = "attn_decode_partial";
  if (a.kv.block_table) DSA_LAUNCH(nm, (k_decode_rows<128, G, true>), grid, dim3(256), st, a);
  else                  DSA_LAUNCH(nm, (k_decode_rows<128, G, false>), grid, dim3(256), st, a);
  launch_decode_combine(a, st);
}

bool launch_decode_rows(const AttnArgs& a, hipStream_t st) {
  if (!a.kv.decode || a.kv.D != 128 || !a.idx) return false;
  switch (a.kv.Hq / a.kv.Hkv) {
    case 2: launch_rows_typed<2>(a, st); return true;
    case 4: launch_rows_typed<4>(a, st); return true;
    case 8: launch_rows_typed<8>(a, st); return true;
    default: return false;
  }
}

// Split partials over spans of a.kps entries (the dense decode when a.idx is
// null, else index rows) and their merge; bf16, d = 128, 2-8 query heads per
// kv head, else false.
template <int G>
static void launch_span_typed(const AttnArgs& a, hipStream_t st) {
  const dim3 grid(a.n_splits, a.kv.Hkv, a.kv.B);
  const char* nm = a.idx ? "attn_decode_partial" : "dense_decode_partial";
  const bool paged = a.kv.block_table != nullptr;
  if (a.idx) {
    if (paged) DSA_LAUNCH(nm, (k_decode_span<128, G, true, true>), grid, dim3(256), st, a);
    else       DSA_LAUNCH(nm, (k_decode_span<128, G, false, true>), grid, dim3(256), st, a);
  } else {
    if (paged) DSA_LAUNCH(nm, (k_decode_span<128, G, true, false>), grid, dim3(256), st, a);
    else       DSA_LAUNCH(nm, (k_decode_span<128, G, false, false>), grid, dim3(256), st, a);
  }
  launch_decode_combine(a, st);
}

bool launch_decode_span(const AttnArgs& a, hipStream_t st) {
  if (!a.kv.decode || a.kv.D != 128) return false;
  switch (a.kv.Hq / a.kv.Hkv) {
    case 2: launch_span_typed<2>(a, st); return true;
    case 4: launch_span_typed<4>(a, st); return true;
    case 8: launch_span_typed<8>(a, st); return true;
    default: return false;
  }
}

bool launch_decode_attend(const StepArgs& s, int sel_chunks, hipStream_t st) {
  const PruneArgs& a = s.p;
  if (a.kv.D != 128) return false;
  switch (a.kv.Hq / a.kv.Hkv) {
    case 2: return launch_attend_typed<128, 2>(s, sel_chunks, st);
    case 4: return launch_attend_typed<128, 4>(s, sel_chunks, st);
    case 8: return launch_attend_typed<128, 8>(s, sel_chunks, st);
    default: return false;
  }
}

}  // namespace dsa
