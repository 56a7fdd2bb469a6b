// Hierarchical context pruning kernels (InfiniteHiP page, 2502.08910,
// section 3.4 "Formal Mechanism of a Single Pruning Stage" and
// "The Representative Token Selection Algorithm (SelectRep)").
//
// One prune_select call runs, for each stage i:
//   score_i : every (row, chunk) of the stage's input list is scored: for each
//             query head a SelectRep tournament picks one representative key,
//             the chunk score is the max over heads and block queries of the
//             representative's dot product (unscaled);
//   topk_i  : one workgroup per row keeps the K = keep/chunk best chunks
//             (score descending, chunk index ascending), writes their start
//             positions in ascending order, and after the last stage writes
//             the index row: sinks, kept chunks, window, -1 padding.
// Every chunk of every stage is a contiguous run of positions: stage 1 tiles
// [n_sink, mid_hi) and each later chunk size divides the previous one.
#include "dsa_internal.h"

namespace dsa {

// ------------------------------------------------------------------------- //
// shared stage helpers                                                      //
// ------------------------------------------------------------------------- //
__device__ __forceinline__ int stage_input_chunks(const PruneArgs& a, int stage, int r,
                                                  const Geo& geo) {
  if (stage == 0) return geo.n1;
  return a.cnt[r * kMaxStages + stage - 1] * (a.chunk[stage - 1] / a.chunk[stage]);
}

// First key position of chunk j of stage `stage` in row r.
__device__ __forceinline__ int chunk_start(const PruneArgs& a, int stage, int r, int j) {
  if (stage == 0) return a.n_sink + j * a.chunk[0];
  const int ratio = a.chunk[stage - 1] / a.chunk[stage];
  const int32_t* prev =
      a.starts + static_cast<size_t>((stage - 1) & 1) * a.R * a.maxK + static_cast<size_t>(r) * a.maxK;
  return prev[j / ratio] + (j % ratio) * a.chunk[stage];
}

// ------------------------------------------------------------------------- //
// decode scoring: one query per row                                         //
// ------------------------------------------------------------------------- //
// Workgroup = 16 lane groups of 16 lanes; a group owns one (chunk, kv head)
// and runs the G SelectRep tournaments of that kv head's query heads side by
// side, so each step issues G independent 16-lane row loads (256 B per row at
// bf16 d=128, fully coalesced). The first split's two representatives are
// shared by all heads. Group results are max-reduced per chunk in LDS.
template <typename T, int D, int G>
__global__ void __launch_bounds__(256) k_score_decode(PruneArgs a, int stage) {
  constexpr int EPL = D / 16;
  const KvLayout& kv = a.kv;
  const int r = blockIdx.y;
  int b, s, e;
  row_bounds(kv, r, b, s, e);
  const Geo geo = make_geo(s, e, a.n_sink, a.n_window, a.chunk[0]);
  const int nc = stage_input_chunks(a, stage, r, geo);
  const int l = a.chunk[stage];
  if (nc <= a.keep[stage] / l) return;          // stage keeps everything for this row
  const int cpw = 16 / kv.Hkv;                  // chunks per workgroup
  const int j0 = blockIdx.x * cpw;
  if (j0 >= nc) return;

  const int tid = threadIdx.x;
  const int gi = tid >> 4, li = tid & 15;
  const int cl = gi / kv.Hkv, g = gi - cl * kv.Hkv;
  const int j = j0 + cl;
  const bool active = (cl < cpw) && (j < nc);
  __shared__ float red[16];

  float best = -INFINITY;
  if (active) {
    const T* K = static_cast<const T*>(a.k);
    const T* Q = static_cast<const T*>(a.q);
    const int st = chunk_start(a, stage, r, j);
    float q[G][EPL];
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
      SliceLoad<T, EPL>::run(Q + (static_cast<size_t>(b) * kv.Hq + g * G + hh) * D + li * EPL, q[hh]);

    float sa[G];
    int lo[G], hi[G];
    unsigned long long nvis = 0;
    float k0[EPL];
    SliceLoad<T, EPL>::run(static_cast<const T*>(K) + kv_offset(kv, b, g, st) + li * EPL, k0);
    if (l == 1) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float acc = 0.f;
#pragma unroll
        for (int x = 0; x < EPL; ++x) acc = fmaf(q[hh][x], k0[x], acc);
        sa[hh] = group16_sum(acc);
      }
      nvis = 1;
    } else {
      const int mid0 = l >> 1;
      float k1[EPL];
      SliceLoad<T, EPL>::run(K + kv_offset(kv, b, g, st + mid0) + li * EPL, k1);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int x = 0; x < EPL; ++x) {
          a0 = fmaf(q[hh][x], k0[x], a0);
          a1 = fmaf(q[hh][x], k1[x], a1);
        }
        a0 = group16_sum(a0);
        a1 = group16_sum(a1);
        if (a1 > a0) { lo[hh] = mid0; hi[hh] = l - 1; sa[hh] = a1; }
        else         { lo[hh] = 0;    hi[hh] = mid0 - 1; sa[hh] = a0; }
      }
      nvis = 2;
      for (int w = l >> 2; w >= 1; w >>= 1) {   // remaining log2(l) - 1 splits
        float kk[G][EPL];
        int mid[G];
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          mid[hh] = (lo[hh] + hi[hh] + 1) >> 1;
          SliceLoad<T, EPL>::run(K + kv_offset(kv, b, g, st + mid[hh]) + li * EPL, kk[hh]);
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          float acc = 0.f;
#pragma unroll
          for (int x = 0; x < EPL; ++x) acc = fmaf(q[hh][x], kk[hh][x], acc);
          acc = group16_sum(acc);
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
  if (nc <= a.keep[stage] / l) return;
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
// top-K per row + index assembly                                            //
// ------------------------------------------------------------------------- //
template <int NT>
__device__ __forceinline__ int block_sum(int v, int* sh) {
  v = wave_sum_int(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) sh[w] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) t += sh[i];
  __syncthreads();
  return t;
}

template <int NT>
__device__ __forceinline__ uint32_t block_and(uint32_t v, uint32_t* sh) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v &= static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), o, 64));
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) sh[w] = v;
  __syncthreads();
  uint32_t t = 0xffffffffu;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) t &= sh[i];
  __syncthreads();
  return t;
}

template <int NT>
__device__ __forceinline__ uint32_t block_or(uint32_t v, uint32_t* sh) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), o, 64));
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) sh[w] = v;
  __syncthreads();
  uint32_t t = 0u;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) t |= sh[i];
  __syncthreads();
  return t;
}

// Exclusive prefix sum over threads in thread order; `total` gets the sum.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* sh, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[w] = x;
  __syncthreads();
  int base = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const int t = sh[i];
    base += (i < w) ? t : 0;
    total += t;
  }
  __syncthreads();
  return base + x - v;
}

constexpr int kSelCap = 8192;   // longest kept-chunk list held in LDS

// One workgroup per row. Keys live in registers: thread t owns the contiguous
// segment [t*E, t*E + E) so thread order is chunk-index order.
// The K-th largest key tau is found by a most-significant-first bit search
// restricted to the bits that vary across the row's keys; then every key >
// tau is kept plus the lowest-index keys == tau until K are kept.
template <int NT, int MAXE>
__global__ void __launch_bounds__(NT) k_topk(PruneArgs a, int stage) {
  const KvLayout& kv = a.kv;
  const int r = blockIdx.x;
  int b, s, e;
  row_bounds(kv, r, b, s, e);
  const Geo geo = make_geo(s, e, a.n_sink, a.n_window, a.chunk[0]);
  const int nc = stage_input_chunks(a, stage, r, geo);
  const int l = a.chunk[stage];
  const int kc = a.keep[stage] / l;
  const int tid = threadIdx.x;
  __shared__ int sh[NT / 64];
  __shared__ uint32_t shu[NT / 64];
  __shared__ int sel[kSelCap];
  int32_t* out = a.starts + static_cast<size_t>(stage & 1) * a.R * a.maxK + static_cast<size_t>(r) * a.maxK;
  int n_sel;
  if (nc <= kc) {
    for (int j = tid; j < nc; j += NT) {
      const int p = chunk_start(a, stage, r, j);
      out[j] = p;
      sel[j] = p;
    }
    n_sel = nc;
  } else {
    const int E = (nc + NT - 1) / NT;
    const int base = tid * E;
    uint32_t key[MAXE];
    uint32_t vand = 0xffffffffu, vor = 0u;
    const uint32_t* sc = a.scores + static_cast<size_t>(r) * a.maxNC;
#pragma unroll
    for (int x = 0; x < MAXE; ++x) {
      const int j = base + x;
      const bool ok = (x < E) && (j < nc);
      key[x] = ok ? sc[j] : 0u;
      if (ok) { vand &= key[x]; vor |= key[x]; }
    }
    vand = block_and<NT>(vand, shu);
    vor = block_or<NT>(vor, shu);
    const uint32_t varying = vand ^ vor;
    uint32_t tau = vand;
    for (int bit = 31; bit >= 0; --bit) {
      if (!((varying >> bit) & 1u)) continue;
      const uint32_t c = tau | (1u << bit);
      int n = 0;
#pragma unroll
      for (int x = 0; x < MAXE; ++x) n += (key[x] >= c) ? 1 : 0;
      if (block_sum<NT>(n, sh) >= kc) tau = c;
    }
    int ngt = 0, neq = 0;
#pragma unroll
    for (int x = 0; x < MAXE; ++x) {
      ngt += (key[x] > tau) ? 1 : 0;
      neq += (key[x] == tau) ? 1 : 0;
    }
    const int need = kc - block_sum<NT>(ngt, sh);
    int tot;
    int eq_before = block_excl_scan<NT>(neq, sh, tot);
    bool take[MAXE];
    int nt = 0;
#pragma unroll
    for (int x = 0; x < MAXE; ++x) {
      bool t = key[x] > tau;
      if (key[x] == tau) {
        t = eq_before < need;
        ++eq_before;
      }
      take[x] = t;
      nt += t ? 1 : 0;
    }
    int rank = block_excl_scan<NT>(nt, sh, tot);
#pragma unroll
    for (int x = 0; x < MAXE; ++x) {
      if (take[x]) {
        const int p = chunk_start(a, stage, r, base + x);
        out[rank] = p;
        sel[rank] = p;
        ++rank;
      }
    }
    n_sel = kc;
  }
  if (tid == 0) a.cnt[r * kMaxStages + stage] = n_sel;
  if (stage != a.n_stages - 1) return;

  // final stage: write the index row
  __syncthreads();
  int32_t* row = a.idx + static_cast<size_t>(r) * a.L;
  const int n_pr = n_sel * l;
  const int n_win = max(0, e - geo.mid_hi);
  for (int i = tid; i < a.L; i += NT) {
    int v;
    if (i < geo.sink_hi) {
      v = i;
    } else if (i < geo.sink_hi + n_pr) {
      const int k = i - geo.sink_hi;
      v = sel[k / l] + (k % l);
    } else if (i < geo.sink_hi + n_pr + n_win) {
      v = geo.mid_hi + (i - geo.sink_hi - n_pr);
    } else {
      v = -1;
    }
    row[i] = v;
  }
}

// ------------------------------------------------------------------------- //
// launcher                                                                  //
// ------------------------------------------------------------------------- //
static const char* const kScoreNames[kMaxStages] = {"prune_score_stage1", "prune_score_stage2",
                                                    "prune_score_stage3", "prune_score_stage4"};
static const char* const kTopkNames[kMaxStages] = {"prune_topk_stage1", "prune_topk_stage2",
                                                   "prune_topk_stage3", "prune_topk_stage4"};

template <typename T, int D, int G>
static void launch_decode_score(const PruneArgs& a, int stage, int max_chunks, hipStream_t st) {
  const int cpw = 16 / a.kv.Hkv;
  dim3 grid((max_chunks + cpw - 1) / cpw, a.R);
  DSA_LAUNCH(kScoreNames[stage], (k_score_decode<T, D, G>), grid, dim3(256), st, a, stage);
}

template <typename T, int D>
static hipError_t launch_typed(const PruneArgs& a, hipStream_t st) {
  const int G = a.kv.Hq / a.kv.Hkv;
  for (int stage = 0; stage < a.n_stages; ++stage) {
    // largest input list any row can present to this stage
    int max_chunks;
    if (stage == 0) {
      max_chunks = a.n1max;
    } else {
      max_chunks = a.keep[stage - 1] / a.chunk[stage];
    }
    if (max_chunks > 0) {
      if (a.kv.decode) {
        switch (G) {
          case 1: launch_decode_score<T, D, 1>(a, stage, max_chunks, st); break;
          case 2: launch_decode_score<T, D, 2>(a, stage, max_chunks, st); break;
          case 4: launch_decode_score<T, D, 4>(a, stage, max_chunks, st); break;
          case 8: launch_decode_score<T, D, 8>(a, stage, max_chunks, st); break;
          default: return hipErrorInvalidValue;
        }
      } else {
        dim3 grid((max_chunks + 15) / 16, a.R);
        DSA_LAUNCH(kScoreNames[stage], (k_score_prefill<T, D>), grid, dim3(256), st, a, stage);
      }
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int cap = a.maxNC;
    if (cap <= 1024 * 4) {
      DSA_LAUNCH(kTopkNames[stage], (k_topk<1024, 4>), dim3(a.R), dim3(1024), st, a, stage);
    } else if (cap <= 1024 * 16) {
      DSA_LAUNCH(kTopkNames[stage], (k_topk<1024, 16>), dim3(a.R), dim3(1024), st, a, stage);
    } else {
      DSA_LAUNCH(kTopkNames[stage], (k_topk<1024, 64>), dim3(a.R), dim3(1024), st, a, stage);
    }
    err = hipGetLastError();
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
