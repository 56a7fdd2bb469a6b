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
#include "prune_common.h"

namespace dsa {

// ------------------------------------------------------------------------- //
// top-K of one row + index assembly                                         //
// ------------------------------------------------------------------------- //
constexpr int kTopkThreads = 256;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kTopkMaxE = 128;          // rows of up to 32768 chunks (128 KiB of keys in LDS)

__device__ __forceinline__ uint32_t wave_and_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v &= static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), o, 64));
  return v;
}
__device__ __forceinline__ uint32_t wave_or_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), o, 64));
  return v;
}
// number of lanes below this one whose bit is set in `mask`
__device__ __forceinline__ int lanes_below(unsigned long long mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0));
}

// Run by all 256 threads of one workgroup. The row's keys are staged in LDS;
// thread t handles keys j = x*256 + t (x < E), so for each x a wave covers 64
// consecutive chunk indices and wave ballots give counts and in-order ranks
// without shuffles. The K-th largest key tau is found by a
// most-significant-first bit search over the bits that vary across the row's
// keys (one barrier per bit); then every key > tau is kept plus the
// lowest-index keys == tau until K are kept.
template <int MAXE>
__device__ void topk_row(const PruneArgs& a, int stage, int r, const Geo& geo, int nc) {
  constexpr int NXW = MAXE * kTopkWaves;          // (x, wave) slots in index order
  const int l = a.chunk[stage];
  const int kc = a.keep[stage] >> a.lchunk[stage];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  __shared__ uint32_t red[2][kTopkWaves];
  __shared__ int cnt[2][kTopkWaves];
  __shared__ int wgt[NXW], weq[NXW];              // per-slot counts of keys > tau, == tau
  __shared__ int bgt[NXW], beq[NXW];              // exclusive prefixes of the same
  __shared__ int s_ngt;
  __shared__ uint32_t skey[MAXE * kTopkThreads];
  int32_t* out = a.starts + static_cast<size_t>(stage & 1) * a.R * a.maxK + static_cast<size_t>(r) * a.maxK;
  int n_sel;
  if (nc <= kc) {
    int32_t* sel = reinterpret_cast<int32_t*>(skey);
    for (int j = tid; j < nc; j += kTopkThreads) {
      const int p = chunk_start(a, stage, r, j);
      out[j] = p;
      sel[j] = p;
    }
    n_sel = nc;
  } else {
    // keys are padded with 0 (below every real key) so every pass below is
    // branch-free over all MAXE slots
    const uint32_t* sc = a.scores + static_cast<size_t>(r) * a.maxNC;
    uint32_t vand = 0xffffffffu, vor = 0u;
    constexpr int LB = MAXE < 8 ? MAXE : 8;         // loads issued per batch
#pragma unroll
    for (int x0 = 0; x0 < MAXE; x0 += LB) {
      uint32_t kreg[LB];
#pragma unroll
      for (int u = 0; u < LB; ++u) {
        const int j = (x0 + u) * kTopkThreads + tid;
        kreg[u] = j < nc ? sc[j] : 0u;
      }
#pragma unroll
      for (int u = 0; u < LB; ++u) {
        skey[(x0 + u) * kTopkThreads + tid] = kreg[u];
        if (kreg[u] != 0u) { vand &= kreg[u]; vor |= kreg[u]; }
      }
    }
    vand = wave_and_u32(vand);
    vor = wave_or_u32(vor);
    if (lane == 0) { red[0][w] = vand; red[1][w] = vor; }
    __syncthreads();
    vand = 0xffffffffu;
    vor = 0u;
#pragma unroll
    for (int i = 0; i < kTopkWaves; ++i) { vand &= red[0][i]; vor |= red[1][i]; }
    const uint32_t varying = vand ^ vor;
    uint32_t tau = vand;
    int par = 0;
    for (int bit = 31; bit >= 0; --bit) {
      if (!((varying >> bit) & 1u)) continue;
      const uint32_t c = tau | (1u << bit);
      int n = 0;
#pragma unroll
      for (int x = 0; x < MAXE; ++x) n += __popcll(__ballot(skey[x * kTopkThreads + tid] >= c));
      if (lane == 0) cnt[par][w] = n;
      __syncthreads();
      int tot = 0;
#pragma unroll
      for (int i = 0; i < kTopkWaves; ++i) tot += cnt[par][i];
      if (tot >= kc) tau = c;
      par ^= 1;
    }
    // per (x, wave) slot: counts of keys > tau and == tau
#pragma unroll
    for (int x = 0; x < MAXE; ++x) {
      const uint32_t k = skey[x * kTopkThreads + tid];
      const int ng = __popcll(__ballot(k > tau));
      const int ne = __popcll(__ballot(k == tau));
      if (lane == 0) { wgt[x * kTopkWaves + w] = ng; weq[x * kTopkWaves + w] = ne; }
    }
    __syncthreads();
    if (w == 0) {                                    // exclusive scans over the slots
      int cg = 0, ce = 0;
      for (int i0 = 0; i0 < NXW; i0 += 64) {
        const int i = i0 + lane;
        const int g0 = i < NXW ? wgt[i] : 0, e0 = i < NXW ? weq[i] : 0;
        int g = g0, e = e0;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int gu = __shfl_up(g, o, 64), eu = __shfl_up(e, o, 64);
          if (lane >= o) { g += gu; e += eu; }
        }
        if (i < NXW) { bgt[i] = cg + g - g0; beq[i] = ce + e - e0; }
        cg += __shfl(g, 63, 64);
        ce += __shfl(e, 63, 64);
      }
      if (lane == 0) s_ngt = cg;
    }
    __syncthreads();
    const int need = kc - s_ngt;                    // >= 1 keys equal to tau are kept
    int rank[MAXE];
#pragma unroll
    for (int x = 0; x < MAXE; ++x) {
      const uint32_t k = skey[x * kTopkThreads + tid];
      const int bq_eq = beq[x * kTopkWaves + w], bq_gt = bgt[x * kTopkWaves + w];
      const unsigned long long eqm = __ballot(k == tau);
      const bool take = (k > tau) || (k == tau && bq_eq + lanes_below(eqm) < need);
      const unsigned long long tm = __ballot(take);
      rank[x] = take ? bq_gt + min(need, bq_eq) + lanes_below(tm) : -1;
    }
    __syncthreads();                                // skey is reused for the kept list
    int32_t* sel = reinterpret_cast<int32_t*>(skey);
    constexpr int PB = MAXE < 8 ? MAXE : 8;         // start lookups issued per batch
#pragma unroll
    for (int x0 = 0; x0 < MAXE; x0 += PB) {
      int pos[PB];
#pragma unroll
      for (int u = 0; u < PB; ++u)                  // unconditional, so the loads batch
        pos[u] = chunk_start(a, stage, r, min((x0 + u) * kTopkThreads + tid, nc - 1));
#pragma unroll
      for (int u = 0; u < PB; ++u) {
        if (rank[x0 + u] >= 0) {
          out[rank[x0 + u]] = pos[u];
          sel[rank[x0 + u]] = pos[u];
        }
      }
    }
    n_sel = kc;
  }
  if (tid == 0) a.cnt[r * kMaxStages + stage] = n_sel;
  if (stage != a.n_stages - 1) return;

  // final stage: write the index row from the kept starts in LDS
  __syncthreads();
  const int32_t* sel = reinterpret_cast<const int32_t*>(skey);
  int32_t* row = a.idx + static_cast<size_t>(r) * a.L;
  const int n_pr = n_sel * l;
  const int n_win = max(0, geo.e - geo.mid_hi);
  for (int i = tid; i < a.L; i += kTopkThreads) {
    int v;
    if (i < geo.sink_hi) {
      v = i;
    } else if (i < geo.sink_hi + n_pr) {
      const int k = i - geo.sink_hi;
      const int c = k >> a.lchunk[stage];
      v = sel[c] + (k & (l - 1));
    } else if (i < geo.sink_hi + n_pr + n_win) {
      v = geo.mid_hi + (i - geo.sink_hi - n_pr);
    } else {
      v = -1;
    }
    row[i] = v;
  }
}

template <int MAXE>
__global__ void __launch_bounds__(kTopkThreads) k_topk(PruneArgs a, int stage) {
  const int r = blockIdx.x;
  int b, s, e;
  row_bounds(a.kv, r, b, s, e);
  const Geo geo = make_geo(s, e, a.n_sink, a.n_window, a.chunk[0]);
  topk_row<MAXE>(a, stage, r, geo, stage_input_chunks(a, stage, r, geo));
}

// ------------------------------------------------------------------------- //
// decode scoring: one query per row                                         //
// ------------------------------------------------------------------------- //
// Workgroup = 16 lane groups of 16 lanes; a group owns one (chunk, kv head)
// and runs the G SelectRep tournaments of that kv head's query heads side by
// side, so each step issues G independent 16-lane row loads (256 B per row at
// bf16 d=128, fully coalesced). The first split's two representatives are
// shared by all heads. With SPEC, the 8 keys that can represent the first
// three splits (positions i*l/8) are loaded in one round and the first three
// splits are decided from them, trading up to 1/8 more row reads for two
// fewer dependent load rounds. Group results are max-reduced per chunk in
// LDS.
template <typename T, int D, int G, bool SPEC>
__global__ void __launch_bounds__(256, G > 4 ? 2 : ((SPEC || sizeof(T) == 4) ? 4 : 8))
k_score_decode(PruneArgs a, int stage) {
  constexpr int EPL = D / 16;
  const KvLayout& kv = a.kv;
  const int r = blockIdx.y;
  int b, s, e;
  row_bounds(kv, r, b, s, e);
  const Geo geo = make_geo(s, e, a.n_sink, a.n_window, a.chunk[0]);
  const int nc = stage_input_chunks(a, stage, r, geo);
  const int l = a.chunk[stage];
  if (nc <= (a.keep[stage] >> a.lchunk[stage])) return;   // stage keeps everything for this row
  const int cpw = 16 / kv.Hkv;                  // chunks per workgroup
  const int j0 = blockIdx.x * cpw;
  if (j0 >= nc) return;

  const int tid = threadIdx.x;
  const int gi = tid >> 4, li = tid & 15;
  const int cl = gi / kv.Hkv, g = gi - cl * kv.Hkv;
  const int j = j0 + cl;
  const bool active = j < nc;
  __shared__ float red[16];

  float best = -INFINITY;
  if (active) {
    const T* K = static_cast<const T*>(a.k);
    const T* Q = static_cast<const T*>(a.q);
    const int st = chunk_start(a, stage, r, j);
    using Row = RowSlice<T, EPL>;
    Row q[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) q[hh].load(Q + (static_cast<size_t>(b) * kv.Hq + g * G + hh) * D + li * EPL);
    auto dot = [&](const Row& kr, int hh) { return group16_sum(kr.dot(q[hh])); };
    auto row_at = [&](int pos) {
      Row x;
      x.load(K + kv_offset(kv, b, g, pos) + li * EPL);
      return x;
    };

    float sa[G];
    int lo[G], hi[G];
    unsigned long long nvis = 0;
    int width;                                   // size of every head's remaining range
    if (l == 1) {
      const Row k0 = row_at(st);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) { sa[hh] = dot(k0, hh); lo[hh] = hi[hh] = 0; }
      nvis = 1;
      width = 1;
    } else if (SPEC && l >= 8) {
      const int u = l >> 3;
      float sc8[G][8];
      {
        Row kr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) kr[i] = row_at(st + i * u);
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int hh = 0; hh < G; ++hh) sc8[hh][i] = dot(kr[i], hh);
      }
      int a1[G], a2[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        int A = 0;
        float s0 = sc8[hh][0];
        if (sc8[hh][4] > s0) { A = 4; s0 = sc8[hh][4]; }
        a1[hh] = A;
        const float s2 = A ? sc8[hh][6] : sc8[hh][2];
        if (s2 > s0) { A += 2; s0 = s2; }
        a2[hh] = A;
        const float s3 = A == 0 ? sc8[hh][1] : A == 2 ? sc8[hh][3] : A == 4 ? sc8[hh][5] : sc8[hh][7];
        if (s3 > s0) { A += 1; s0 = s3; }
        lo[hh] = A * u;
        hi[hh] = A * u + u - 1;
        sa[hh] = s0;
      }
      if (a.visited) {
        nvis = 2;                                 // split 1: keys 0 and l/2
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {          // splits 2 and 3: distinct midpoints
          bool f2 = true, f3 = true;
#pragma unroll
          for (int h2 = 0; h2 < hh; ++h2) {
            f2 = f2 && (a1[h2] != a1[hh]);
            f3 = f3 && (a2[h2] != a2[hh]);
          }
          nvis += (f2 ? 1 : 0) + (f3 ? 1 : 0);
        }
      }
      width = u;
    } else {
      const int mid0 = l >> 1;
      const Row k0 = row_at(st), k1 = row_at(st + mid0);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float a0 = dot(k0, hh), a1 = dot(k1, hh);
        if (a1 > a0) { lo[hh] = mid0; hi[hh] = l - 1; sa[hh] = a1; }
        else         { lo[hh] = 0;    hi[hh] = mid0 - 1; sa[hh] = a0; }
      }
      nvis = 2;
      width = mid0;
    }
    for (int wdt = width >> 1; wdt >= 1; wdt >>= 1) {   // remaining splits
      Row kk[G];
      int mid[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        mid[hh] = (lo[hh] + hi[hh] + 1) >> 1;
        kk[hh] = row_at(st + mid[hh]);
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float acc = dot(kk[hh], hh);
        if (acc > sa[hh]) { lo[hh] = mid[hh]; sa[hh] = acc; }
        else              { hi[hh] = mid[hh] - 1; }
      }
      if (a.visited) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          bool fresh = true;
#pragma unroll
          for (int h2 = 0; h2 < hh; ++h2) fresh = fresh && (mid[h2] != mid[hh]);
          nvis += fresh ? 1 : 0;
        }
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) best = fmaxf(best, sa[hh]);
    if (a.visited && li == 0) atomicAdd(a.visited + stage, nvis);
  }
  if (li == 0) red[gi] = best;
  __syncthreads();
  if (tid < cpw) {
    const int jj = j0 + tid;
    if (jj < nc) {
      float m = red[tid * kv.Hkv];
      for (int x = 1; x < kv.Hkv; ++x) m = fmaxf(m, red[tid * kv.Hkv + x]);
      a.scores[static_cast<size_t>(r) * a.maxNC + jj] = score_key(m);
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
  if (active && li == 0) a.scores[static_cast<size_t>(r) * a.maxNC + j] = score_key(best);
}

// ------------------------------------------------------------------------- //
// launcher                                                                  //
// ------------------------------------------------------------------------- //
static const char* const kScoreNames[kMaxStages] = {"prune_score_stage1", "prune_score_stage2",
                                                    "prune_score_stage3", "prune_score_stage4"};
static const char* const kTopkNames[kMaxStages] = {"prune_topk_stage1", "prune_topk_stage2",
                                                   "prune_topk_stage3", "prune_topk_stage4"};
constexpr int kSpecMaxChunk = 64;       // chunks this small preload their first three splits

template <typename T, int D, int G>
static void launch_decode_score(const PruneArgs& a, int stage, int max_chunks, hipStream_t st) {
  const int cpw = 16 / a.kv.Hkv;
  if (max_chunks <= 0) return;
  dim3 grid((max_chunks + cpw - 1) / cpw, a.R);
  const char* nm = kScoreNames[stage];
  if (a.chunk[stage] >= 8 && a.chunk[stage] <= kSpecMaxChunk)
    DSA_LAUNCH(nm, (k_score_decode<T, D, G, true>), grid, dim3(256), st, a, stage);
  else
    DSA_LAUNCH(nm, (k_score_decode<T, D, G, false>), grid, dim3(256), st, a, stage);
}

static void launch_topk(const PruneArgs& a, int stage, int max_chunks, hipStream_t st) {
  const char* nm = kTopkNames[stage];
  if (max_chunks <= kTopkThreads * 4) {
    DSA_LAUNCH(nm, (k_topk<4>), dim3(a.R), dim3(kTopkThreads), st, a, stage);
  } else if (max_chunks <= kTopkThreads * 16) {
    DSA_LAUNCH(nm, (k_topk<16>), dim3(a.R), dim3(kTopkThreads), st, a, stage);
  } else if (max_chunks <= kTopkThreads * 64) {
    DSA_LAUNCH(nm, (k_topk<64>), dim3(a.R), dim3(kTopkThreads), st, a, stage);
  } else {
    DSA_LAUNCH(nm, (k_topk<kTopkMaxE>), dim3(a.R), dim3(kTopkThreads), st, a, stage);
  }
}

template <typename T, int D>
static hipError_t launch_typed(const PruneArgs& a, hipStream_t st) {
  const int G = a.kv.Hq / a.kv.Hkv;
  for (int stage = 0; stage < a.n_stages; ++stage) {
    // longest input list any row can present to this stage
    const int max_chunks = stage == 0 ? a.n1max : a.keep[stage - 1] / a.chunk[stage];
    if (a.kv.decode) {
      switch (G) {
        case 1: launch_decode_score<T, D, 1>(a, stage, max_chunks, st); break;
        case 2: launch_decode_score<T, D, 2>(a, stage, max_chunks, st); break;
        case 4: launch_decode_score<T, D, 4>(a, stage, max_chunks, st); break;
        case 8: launch_decode_score<T, D, 8>(a, stage, max_chunks, st); break;
        default: return hipErrorInvalidValue;
      }
      launch_topk(a, stage, max_chunks, st);
    } else {
      if (max_chunks > 0 &&
          !(sizeof(T) == 2 && launch_score_prefill_mfma(a, stage, max_chunks, st, kScoreNames[stage]))) {
        dim3 grid((max_chunks + 15) / 16, a.R);
        DSA_LAUNCH(kScoreNames[stage], (k_score_prefill<T, D>), grid, dim3(256), st, a, stage);
      }
      launch_topk(a, stage, max_chunks, st);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
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
