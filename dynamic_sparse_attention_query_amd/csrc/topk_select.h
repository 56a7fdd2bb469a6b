// Exact top-K of one row of uint32 keys held in the registers of a
// workgroup (larger key first, lower index first among equal keys), shared by
// the chunk selection of the hierarchical pruning (InfiniteHiP page, section
// 3.4, "Formal Mechanism of a Single Pruning Stage", step 6) and the block
// selection of the block-sparse estimation (MInference page, "Online Dynamic
// Index Estimation: Block-Sparse Heads (Algorithm 3)", step 3).
#pragma once

#include "dsa_internal.h"

namespace dsa {

constexpr int kTopkThreads = 256;
constexpr int kTopkWaves = kTopkThreads / 64;

__device__ __forceinline__ uint32_t wave_and_u32(uint32_t v) {
  return static_cast<uint32_t>(wave_reduce_int(static_cast<int>(v), [](int x, int y) { return x & y; }));
}
__device__ __forceinline__ uint32_t wave_or_u32(uint32_t v) {
  return static_cast<uint32_t>(wave_reduce_int(static_cast<int>(v), [](int x, int y) { return x | y; }));
}

// LDS of one row's top-K selection by NW waves
template <int NW = kTopkWaves>
struct SelectLds {
  uint32_t hist[2][NW][256];
  uint32_t sred[2][NW];
  uint32_t sscan[NW];
  int sdec[3];
  int wcand[NW];                                 // small boundary digit: per-wave counts,
  uint32_t ckey[NW][64];                         // keys and chunk ids (each wave's share is
  int cidx[NW][64];                              // below 64: the digit holds at most 64 keys)
  uint32_t sfin[2];
};

// Top-K of one row, run by all kTopkThreads threads of the workgroup. Thread
// t holds the keys of chunks j = t*E .. t*E+E-1 in registers (index order =
// thread order, so one block-wide scan ranks everything). The K-th largest
// key is found by radix selection over the bits that vary across the row:
// 8-bit digits from the most significant varying bit down, each pass a
// per-wave LDS histogram of the keys still tied with the prefix chosen so
// far, scanned by one wave. A pass stops the search as soon as the boundary
// digit's keys are all kept. Keys above the threshold are kept, plus the
// lowest-index keys equal to it until K are kept; emit(j, pos) is called for
// every kept chunk j with its output slot pos = the number of kept chunks of
// lower index. With nc <= kc every chunk j < nc is kept at slot j.
template <int E, int NT = kTopkThreads, typename Emit>
__device__ __forceinline__ void select_row(uint32_t (&key)[E], int j0, int nc, int kc, SelectLds<NT / 64>& L,
                                           Emit&& emit) {
  constexpr int kTopkThreads = NT;              // this selection's threads and waves
  constexpr int kTopkWaves = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // common bits of the row's keys (0 marks chunks beyond nc: real keys are
  // never 0); the histograms are cleared under the same barrier
  uint32_t vand = 0xffffffffu, vor = 0u;
#pragma unroll
  for (int x = 0; x < E; ++x) {
    if (j0 + x >= nc) key[x] = 0u;
    if (key[x] != 0u) { vand &= key[x]; vor |= key[x]; }
  }
  vand = wave_and_u32(vand);
  vor = wave_or_u32(vor);
  if (lane == 0) { L.sred[0][w] = vand; L.sred[1][w] = vor; }
  {
    uint32_t* h = &L.hist[0][0][0];
#pragma unroll
    for (int i = 0; i < 2 * kTopkWaves * 256 / kTopkThreads; ++i) h[i * kTopkThreads + tid] = 0u;
  }
  __syncthreads();                                 // also publishes the caller's LDS data
  if (nc <= kc) {                                  // every chunk is kept, in index order
    for (int j = j0; j < min(j0 + E, nc); ++j) emit(j, j);
  } else {
    vand = 0xffffffffu;
    vor = 0u;
#pragma unroll
    for (int i = 0; i < kTopkWaves; ++i) { vand &= L.sred[0][i]; vor |= L.sred[1][i]; }
    const uint32_t varying = vand ^ vor;

    // radix passes: bits [shift, 32) of the threshold are decided
    int shift = varying ? 32 - __clz(static_cast<int>(varying)) : 0;
    uint32_t prefix = shift >= 32 ? 0u : (vand & (~0u << shift));
    int need = kc;                                   // keys still to keep among the tied ones
    bool whole = false;                              // the boundary digit is kept whole
    for (int p = 0; shift > 0; ++p) {
      const int wd = min(8, shift);
      shift -= wd;
      const uint32_t himask = shift + wd >= 32 ? 0u : (~0u << (shift + wd));
      const uint32_t dmask = (1u << wd) - 1u;
      uint32_t (*H)[256] = L.hist[p & 1];
      {
        uint32_t* h = &L.hist[(p + 1) & 1][0][0];      // next pass's buffer, idle since the last scan
#pragma unroll
        for (int i = 0; i < kTopkWaves * 256 / kTopkThreads; ++i) h[i * kTopkThreads + tid] = 0u;
      }
#pragma unroll
      for (int x = 0; x < E; ++x) {
        const uint32_t k = key[x];
        if (k != 0u && ((k ^ prefix) & himask) == 0u) atomicAdd(&H[w][(k >> shift) & dmask], 1u);
      }
      __syncthreads();
      if (w == 0) {
        // lane handles bins 255-4*lane .. 252-4*lane, so lane order is digit
        // order from the top
        uint32_t c[4], tot = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int bin = 255 - (4 * lane + i);
          c[i] = 0;
#pragma unroll
          for (int ww = 0; ww < kTopkWaves; ++ww) c[i] += H[ww][bin];
          tot += c[i];
        }
        const uint32_t inc = wave_incl_scan_u32(tot);
        const unsigned long long m = __ballot(inc >= static_cast<uint32_t>(need));
        if (lane == __ffsll(static_cast<long long>(m)) - 1) {
          uint32_t run = inc - tot;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (run + c[i] >= static_cast<uint32_t>(need)) {
              L.sdec[0] = 255 - (4 * lane + i);
              L.sdec[1] = need - static_cast<int>(run);
              L.sdec[2] = static_cast<int>(c[i]);
              break;
            }
            run += c[i];
          }
        }
      }
      __syncthreads();
      prefix |= static_cast<uint32_t>(L.sdec[0]) << shift;
      need = L.sdec[1];
      const int cd = L.sdec[2];
      if (cd == need) { whole = true; break; }
      if (shift > 0 && cd <= 64) {
        // Few keys share the boundary digit: gather them and let one wave
        // rank them exactly (score descending, chunk index ascending). The
        // need-th of them is the threshold tau; keys above it are kept, and
        // of the keys equal to it the lowest-index ones up to need.
        const uint32_t hm = ~0u << shift;
        int run = 0;                               // this wave's candidates so far (uniform)
#pragma unroll
        for (int x = 0; x < E; ++x) {
          const uint32_t k = key[x];
          const bool c = k != 0u && ((k ^ prefix) & hm) == 0u;
          const unsigned long long cb = __ballot(c);
          if (c) {
            const int slot = run + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(cb >> 32),
                                                             __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(cb), 0));
            L.ckey[w][slot] = k;
            L.cidx[w][slot] = j0 + x;
          }
          run += __popcll(cb);
        }
        if (lane == 0) L.wcand[w] = run;
        __syncthreads();
        if (w == 0) {
          // lane l takes candidate l of the waves' shares in wave order
          int src_w = 0, src_i = lane;
#pragma unroll
          for (int ww = 0; ww < kTopkWaves - 1; ++ww)
            if (src_w == ww && src_i >= L.wcand[ww]) { src_i -= L.wcand[ww]; src_w = ww + 1; }
          const bool valid = lane < cd;
          const uint32_t kl = valid ? L.ckey[src_w][src_i] : 0u;
          const int il = valid ? L.cidx[src_w][src_i] : 0x7fffffff;
          int rank = 0;
          for (int m = 0; m < cd; ++m) {
            const uint32_t km = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(kl), m));
            const int im = __builtin_amdgcn_readlane(il, m);
            rank += (km > kl || (km == kl && im < il)) ? 1 : 0;
          }
          const unsigned long long bm = __ballot(valid && rank == need - 1);
          const uint32_t t = static_cast<uint32_t>(
              __builtin_amdgcn_readlane(static_cast<int>(kl), __ffsll(static_cast<long long>(bm)) - 1));
          const int ngt = __popcll(__ballot(valid && kl > t));
          if (lane == 0) { L.sfin[0] = t; L.sfin[1] = need - ngt; }
        }
        __syncthreads();
        prefix = L.sfin[0];                       // tau, every bit decided
        need = static_cast<int>(L.sfin[1]);       // keys equal to tau to keep
        break;
      }
    }

    // kept: key > tau, or key == tau among the first need_eq such keys; with a
    // whole boundary digit, every key >= prefix. Per-thread bit masks of the
    // two classes, then one packed (strict << 16 | equal) block-wide scan.
    const uint32_t tau = prefix;
    const int need_eq = whole ? 0 : need;
    constexpr int NM = (E + 31) / 32;
    uint32_t sm[NM], em[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) { sm[m] = 0u; em[m] = 0u; }
#pragma unroll
    for (int x = 0; x < E; ++x) {
      const uint32_t k = key[x];
      const bool strict = k != 0u && (whole ? k >= tau : k > tau);
      const bool eq = !whole && k == tau && k != 0u;
      sm[x >> 5] |= (strict ? 1u : 0u) << (x & 31);
      em[x >> 5] |= (eq ? 1u : 0u) << (x & 31);
    }
    uint32_t cnt = 0;
#pragma unroll
    for (int m = 0; m < NM; ++m) cnt += (static_cast<uint32_t>(__popc(sm[m])) << 16) + __popc(em[m]);
    const uint32_t inc = wave_incl_scan_u32(cnt);
    if (lane == 63) L.sscan[w] = inc;
    __syncthreads();
    uint32_t base = inc - cnt;
#pragma unroll
    for (int i = 0; i < kTopkWaves; ++i)
      if (i < w) base += L.sscan[i];
    int cs = static_cast<int>(base >> 16), ce = static_cast<int>(base & 0xffffu);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      for (uint32_t rest = sm[m] | em[m]; rest != 0u; rest &= rest - 1u) {
        const int bit = __ffs(static_cast<int>(rest)) - 1;
        const uint32_t below = (1u << bit) - 1u;
        const int ps = cs + __popc(sm[m] & below);       // strict keys of lower index
        const int pe = ce + __popc(em[m] & below);       // equal keys of lower index
        if ((sm[m] >> bit) & 1u) emit(j0 + 32 * m + bit, ps + min(need_eq, pe));
        else if (pe < need_eq) emit(j0 + 32 * m + bit, ps + pe);
      }
      cs += __popc(sm[m]);
      ce += __popc(em[m]);
    }
  }
}

}  // namespace dsa

namespace dsa {

// ------------------------------------------------------------------------- //
// Latency-oriented top-K of one row, keys in thread order                   //
// ------------------------------------------------------------------------- //
// The same selection as select_row (larger key first, lower index first among
// equal keys), written for the shortest instruction stream per wave: the
// decode kernels run it in every workgroup, on the critical path. Thread t
// holds the keys of indices j = t*E .. t*E+E-1, so thread order is index
// order and one block-wide scan ranks every key.
//   * Every key becomes its distance below the OR of the row's keys,
//     d = (vor - key) >> lsb, with lsb the lowest bit in which the keys differ:
//     vor >= every key and all keys share the bits below lsb, so d is exact
//     and ascending d is descending key.
//     Absent keys (index >= nc) take the value 0: they are below every real
//     key and above it in index, so while more than K real keys exist (the
//     only case that selects) they are never kept; the first pass clamps their
//     bin to the last one, where they cannot be the boundary.
//   * The K-th smallest d is found by histogramming d into 2048 bins of width
//     2^s (s just large enough for the row's varying bits) with LDS atomics,
//     one barrier per pass, after which every wave scans the histogram by
//     itself (lane l sums bins 32l .. 32l+31, then the boundary lane's 32
//     bins), so sharing the result takes no further barrier. A boundary bin
//     that is not kept whole is split again at a finer width until its width
//     is one; the exact-score keys of the decode workloads take two passes.
//   * Each thread counts its keys strictly inside the kept range and equal to
//     the threshold; one block-wide scan of the packed counts gives each
//     thread the number of kept keys before its own (ties at the threshold go
//     to the lowest indices), and the thread writes its kept indices in
//     order from there.
// kept[0 .. min(nc, kc)) receives the kept indices in ascending order; it is
// complete after the caller's next barrier. Keys are 0 for absent chunks
// (real keys are never 0). Returns the number kept.
constexpr int kHistBins = 2048;
// The histogram is stored as 64 blocks of 32 bins, each followed by 4 words of
// padding: a lane's block then starts 4 banks after its left neighbour's, so
// the wave's 16-byte reads of whole blocks (the scan) are free of bank
// conflicts (unpadded, every lane's block starts on the same bank).
constexpr int kHistBlock = 36;
constexpr int kHistWords = kHistBins / 32 * kHistBlock;
__device__ __forceinline__ uint32_t hist_slot(uint32_t bin) { return bin + ((bin >> 5) << 2); }

template <int NW>
struct SelectKeysLds {
  uint32_t hist[2][kHistWords + 64];             // + one spare bin per lane (second pass)
  uint32_t wred[2][NW];
  uint32_t wcnt[NW];
};

template <int E, int NT = kTopkThreads>
__device__ __forceinline__ int select_keys(const uint32_t (&key)[E], int nc, int kc, SelectKeysLds<NT / 64>& L,
                                           int* kept) {
  constexpr int NW = NT / 64;
  constexpr uint32_t kSpare = kHistWords;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int j0 = tid * E;                          // this thread's first index
  if (nc <= kc) {                                  // every chunk is kept, in index order
    __syncthreads();                               // publishes the caller's LDS data, as below
#pragma unroll
    for (int x = 0; x < E; ++x)
      if (j0 + x < nc) kept[j0 + x] = j0 + x;
    return nc;
  }
  uint32_t k[E];
  uint32_t vand = 0xffffffffu, vor = 0u;
#pragma unroll
  for (int x = 0; x < E; ++x) {
    k[x] = j0 + x < nc ? key[x] : 0u;
    vand &= k[x] ? k[x] : 0xffffffffu;
    vor |= k[x];
  }
  vand = wave_and_u32(vand);
  vor = wave_or_u32(vor);
  if (lane == 0) {
    L.wred[0][w] = vand;
    L.wred[1][w] = vor;
  }
  {
    constexpr int N4 = 2 * (kHistWords + 64) / 4;
    uint4* h4 = reinterpret_cast<uint4*>(&L.hist[0][0]);
#pragma unroll
    for (int i = 0; i < (N4 + NT - 1) / NT; ++i)
      if (i * NT + tid < N4) h4[i * NT + tid] = make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();                                 // also publishes the caller's LDS data
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    vand &= L.wred[0][i];
    vor |= L.wred[1][i];
  }
  const uint32_t varying = vand ^ vor;
  const int lsb = varying ? __ffs(static_cast<int>(varying)) - 1 : 0;
  const int bits = varying ? 32 - __clz(static_cast<int>(varying)) - lsb : 0;
  int s = max(0, bits - 11);
  uint32_t d[E];
#pragma unroll
  for (int x = 0; x < E; ++x) {
    d[x] = (vor - k[x]) >> lsb;
    atomicAdd(&L.hist[0][hist_slot(min(d[x] >> s, static_cast<uint32_t>(kHistBins - 1)))], 1u);
  }
  __syncthreads();
  uint32_t base = 0u;                              // lower edge (in d) of the boundary bin
  int need = kc;                                   // keys of the boundary bin still to keep
  bool whole = false;
  for (int p = 0;; ++p) {
    const uint32_t* H = L.hist[p & 1];
    const uint4* H4 = reinterpret_cast<const uint4*>(H + lane * kHistBlock);
    uint32_t sl = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint4 u = H4[i];
      sl += (u.x + u.y) + (u.z + u.w);
    }
    const uint32_t il = wave_incl_scan_u32(sl);
    const int bl = __ffsll(static_cast<long long>(__ballot(il >= static_cast<uint32_t>(need)))) - 1;
    const uint32_t above_l = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(il - sl), bl));
    const uint32_t c = lane < 32 ? H[bl * kHistBlock + lane] : 0u;
    const uint32_t ic = wave_incl_scan_u32(c);
    const int bi = __ffsll(static_cast<long long>(__ballot(above_l + ic >= static_cast<uint32_t>(need)))) - 1;
    const int cnt_in = __builtin_amdgcn_readlane(static_cast<int>(c), bi);
    need -= static_cast<int>(above_l) + __builtin_amdgcn_readlane(static_cast<int>(ic - c), bi);
    base += static_cast<uint32_t>(bl * 32 + bi) << s;
    if (cnt_in == need) { whole = true; break; }
    if (s == 0) break;                             // the bin is the threshold value d == base
    const uint32_t wprev = 1u << s;
    s = max(0, s - 11);
    uint32_t* Hn = L.hist[(p + 1) & 1];
    if (p >= 1) {                                  // a third pass reuses the first buffer
      __syncthreads();                             // every wave has scanned it
      for (int i = tid; i < kHistWords; i += NT) Hn[i] = 0u;
      __syncthreads();
    }
#pragma unroll
    for (int x = 0; x < E; ++x) {
      const uint32_t r = d[x] - base;              // wraps for keys above the bin
      atomicAdd(&Hn[r < wprev ? hist_slot(r >> s) : kSpare + lane], 1u);
    }
    __syncthreads();
  }

  // kept: d below the boundary bin (or inside it when it is kept whole), and
  // the lowest-index `need` keys equal to the threshold d == base otherwise.
  // (the counts below are the same in every lane; readfirstlane lets the
  // compiler keep them, and the branches on them, scalar)
  const int need_eq = __builtin_amdgcn_readfirstlane(whole ? 0 : need);
  const uint32_t wbin = whole ? (1u << s) : 0u;    // width of the boundary bin kept whole
  const uint32_t eqv = whole ? 0xffffffffu : base; // d of the ties (none when whole)
  uint32_t ms = 0u, me = 0u;                       // this thread's strict / equal keys, by x
#pragma unroll
  for (int x = 0; x < E; ++x) {
    ms |= static_cast<uint32_t>(d[x] < base || d[x] - base < wbin) << x;
    me |= static_cast<uint32_t>(d[x] == eqv) << x;
  }
  // counts packed (strict << 16 | equal): a workgroup holds at most 65,535
  // keys of each, so the halves never carry into each other
  const uint32_t cnt = (static_cast<uint32_t>(__popc(ms)) << 16) | static_cast<uint32_t>(__popc(me));
  const uint32_t inc = wave_incl_scan_u32(cnt);
  if (lane == 63) L.wcnt[w] = inc;
  __syncthreads();
  uint32_t before = inc - cnt;                     // keys of the threads before, this wave
#pragma unroll
  for (int i = 0; i < NW; ++i) before += i < w ? L.wcnt[i] : 0u;
  int erank = static_cast<int>(before & 0xffffu);  // ties at the threshold before this thread's
  int slot = static_cast<int>(before >> 16) + min(erank, need_eq);
  // this thread's kept keys: the strict ones and, in index order, its ties
  // while fewer than need_eq ties come before them; then one store per kept
  // key (a lane loops over its own kept keys only: few of them when K is a
  // small share of the row)
  uint32_t km = ms;
  if (need_eq > 0)
    for (uint32_t m = me; m != 0u && erank < need_eq; m &= m - 1u, ++erank) km |= m & (0u - m);
  for (; km != 0u; km &= km - 1u) kept[slot++] = j0 + __builtin_ctz(km);
  return kc;
}

}  // namespace dsa
