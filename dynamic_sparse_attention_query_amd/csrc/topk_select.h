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
