// Prefill SelectRep scoring on the bf16 matrix cores (InfiniteHiP page,
// 2502.08910, section 3.4, "The Representative Token Selection Algorithm
// (SelectRep)" and the chunk score of "Formal Mechanism of a Single Pruning
// Stage", step 5).
//
// For a query block of 64 queries, evaluating one candidate key k means
// sigma(k) = max_t q_t . k. A wave evaluates 32 chunks at once, one candidate
// key per chunk: S = Q K_sel^T with Q (64 x d) as the A operand and the 32
// gathered key rows as the B operand of v_mfma_f32_32x32x16_bf16, so lane l
// holds key column l % 32 and the max over queries is a max over the lane's
// own accumulators plus one exchange between the half-waves. The products
// and partial sums of grid-valued inputs are exact in fp32, so the MFMA
// result equals the scalar dot product bit for bit.
//
// Workgroup = 4 waves x kSlices slices of 32*T chunks of one row (query
// block) and one kv head; the waves split the query heads of that kv head's
// group, and a wave runs its head's tournaments slice after slice with the
// query fragments staged once (4 slices: 5% faster than one per workgroup at
// 128K, 8: slower). Consecutive workgroups on an XCD take 16 neighbouring rows
// for the same (kv head, slices): the rows' chunk lists coincide (stage 1) or
// overlap (later stages), so the key rows they gather are shared in L2. Each
// workgroup folds the max over its heads into the row's score list with an
// atomic max (the list is cleared first; max is order-independent, so the
// result is exact). For
// each of its heads a wave runs T groups of 32 tournaments side by side (the
// groups share the head's query fragments), so
// every dependent round of key-row loads has T independent row sets in
// flight. Rows reach the matrix-core operand layout through a per-wave LDS
// staging buffer: a wave-wide 16-byte load covers whole rows (PPR lanes per
// row, 4 rows per load at d = 128) instead of touching 32 rows at once, and
// the fragments are then read from LDS. The buffer holds one 32-row set
// (8.5 KB), so the query block of each head is staged in two halves and the
// first split's two representatives are fetched as two rounds: the rows in
// flight never exceed T sets per wave, the kernel stays under 168 registers
// and three waves share each SIMD, which hides more of each round's
// dependent gather latency than two waves with twice the rows each.
//
// With RT (relative RoPE in SelectRep, InfiniteHiP page, "Four RoPE Styles
// for Context Pruning"), the wave holds the fragments of the head's two
// rotated query blocks (left and right offsets, bf16 on the 1/128 grid) and
// scores every staged key against both; the tournament keeps the
// representative's left score and the score it last won with. The doubled
// fragments leave room for two waves per SIMD.
#include "prune_common.h"

namespace dsa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));   // 16-byte staging word

constexpr int kRowGroup = 16;           // neighbouring query blocks scheduled together
constexpr int kScoreGroups = 2;         // T: 32-chunk tournament groups per wave
constexpr int kScoreGroupsRt = 2;       // T of the relative-RoPE tournaments
constexpr int kSlices = 4;              // 32*T-chunk slices of a row per workgroup

template <int D, int T, bool RT>
__global__ void __launch_bounds__(256, RT ? 2 : 3)
k_score_prefill_mfma(PruneArgs a, int stage, int ngrp, const uint16_t* ql_all, const uint16_t* qr_all) {
  constexpr int NQ = RT ? 2 : 1;        // query sets: plain, or left and right
  constexpr int KS = D / 16;
  constexpr int CPB = 32 * T;           // chunks per workgroup
  constexpr int PPR = D / 8;            // 16-byte pieces per row
  constexpr int RPI = 64 / PPR;         // rows per wave-wide load
  constexpr int LPS = 32 / RPI;         // loads per 32-row set
  constexpr int KROW = D + 8;           // staging row stride (bf16): shifts banks by 4 words per row
  constexpr int NS = kSlices;
  __shared__ __align__(16) uint16_t sbuf[4][32 * KROW];
  __shared__ int spos[4][T][32];
  __shared__ int sst[NS * CPB];         // first key of each chunk of the workgroup's slices
  __shared__ float red[4][NS * CPB];    // per wave: max over its heads so far

  const KvLayout& kv = a.kv;
  const int x = blockIdx.x & 7, i = blockIdx.x >> 3;
  const int per_group = kv.Hkv * ngrp * kRowGroup;
  const int rbl = i / per_group, rem = i - rbl * per_group;
  const int r = ((rbl << 3) + x) * kRowGroup + rem % kRowGroup;
  const int gj = rem / kRowGroup;
  const int g = gj / ngrp;
  const int jg = (gj - g * ngrp) * (NS * CPB);
  if (r >= a.R) return;
  int b, s, e;
  row_bounds(kv, r, b, s, e);
  const Geo geo = make_geo(s, e, a.n_sink, a.n_window, a.chunk[0]);
  const int nc = stage_input_chunks(a, stage, r, geo);
  if (nc <= (a.keep[stage] >> a.lchunk[stage])) return;    // stage keeps everything
  if (jg >= nc) return;
  const int nsl = min(NS, (nc - jg + CPB - 1) / CPB);    // slices holding chunks

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int piece = lane % PPR, rsub = lane / PPR;          // loader view of the lane
  uint16_t* buf = sbuf[w];
  // The chunk starts do not depend on the head: looked up once for all
  // slices (idle columns score the first chunk of their slice).
  for (int c = tid; c < nsl * CPB; c += 256) {
    const int j = jg + c;
    sst[c] = chunk_start(a, stage, r, j < nc ? j : jg + c / CPB * CPB);
#pragma unroll
    for (int u = 0; u < 4; ++u) red[u][c] = -INFINITY;
  }
  __syncthreads();
  const int l = a.chunk[stage];
  const int G = kv.Hq / kv.Hkv;
  // the first two rounds shared by the waves (every wave has the same number
  // of heads, so the barriers inside are uniform)
  const bool share = !RT && T == 2 && (G & 3) == 0 && l >= 2;
  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* Kg = static_cast<const uint16_t*>(a.k) + (static_cast<size_t>(b) * kv.Hkv + g) * kv.T * D;

  // a set of 32 rows at the positions published in spos[w][set]
  auto fetch = [&](const uint16_t* base, int set, u32x4_t (&v)[LPS]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < LPS; ++u) {
      const int p_ = spos[w][set][u * RPI + rsub];
      v[u] = *reinterpret_cast<const u32x4_t*>(base + static_cast<size_t>(p_) * D + piece * 8);
    }
  };
  auto stage_set = [&](const u32x4_t (&v)[LPS]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < LPS; ++u)
      *reinterpret_cast<u32x4_t*>(buf + (u * RPI + rsub) * KROW + piece * 8) = v[u];
  };

  int st[T];                            // this slice's chunk starts (lane column)
  for (int h = g * G + w; h < (g + 1) * G; h += 4) {
    bf16x8_t qf[NQ][2][KS];
#pragma unroll
    for (int set = 0; set < NQ; ++set) {
      const uint16_t* qblk = RT ? (set ? qr_all : ql_all) + (static_cast<size_t>(r) * kv.Hq + h) * 64 * D
                                : Q + ((static_cast<size_t>(b) * kv.Hq + h) * kv.T + s) * D;
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        u32x4_t v[LPS];
#pragma unroll
        for (int u = 0; u < LPS; ++u)
          v[u] = *reinterpret_cast<const u32x4_t*>(qblk + (qt * 32 + u * RPI + rsub) * D + piece * 8);
        stage_set(v);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          qf[set][qt][ks] = *reinterpret_cast<const bf16x8_t*>(buf + l32 * KROW + ks * 16 + hi * 8);
      }
    }
    // sigma of the key staged in bb for this lane's chunk column, against
    // query set `set`
    auto sigma_in = [&](const uint16_t* bb, int set) __attribute__((always_inline)) {
      f32x16_t acc[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int i2 = 0; i2 < 16; ++i2) acc[qt][i2] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(bb + l32 * KROW + ks * 16 + hi * 8);
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
          acc[qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[set][qt][ks], kf, acc[qt], 0, 0, 0);
      }
      float m = acc[0][0];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int i2 = 0; i2 < 16; ++i2) m = fmaxf(m, acc[qt][i2]);
      // with the other half-wave's max (a lane swap, no LDS round trip)
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
      return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    };
    auto sigma_staged = [&](int set) __attribute__((always_inline)) { return sigma_in(buf, set); };
    // one round: the rows at offsets off[t] of every group, scored against
    // the first query set (sg) and, with RT and `right`, the right one (sr)
    auto round = [&](const int (&off)[T], float (&sg)[T], float (&sr)[T], bool right) __attribute__((always_inline)) {
      if (hi == 0) {
#pragma unroll
        for (int t = 0; t < T; ++t) spos[w][t][l32] = st[t] + off[t];
      }
      u32x4_t v[T][LPS];
#pragma unroll
      for (int t = 0; t < T; ++t) fetch(Kg, t, v[t]);
#pragma unroll
      for (int t = 0; t < T; ++t) {
        stage_set(v[t]);
        sg[t] = sigma_staged(0);
        if constexpr (RT) {
          if (right) sr[t] = sigma_staged(1);
        }
      }
    };

    // the head's query fragments serve every slice
    for (int sl = 0; sl < nsl; ++sl) {
#pragma unroll
      for (int t = 0; t < T; ++t) st[t] = sst[sl * CPB + 32 * t + l32];
      float sa[T], win[T], unused[T];
      int lo[T], hi_r[T];
      int wd0 = l >> 1;
      if (share) {
        // The first two rounds of every head score key 0 and key l/2 of each
        // chunk, so the four waves (the heads of one kv head's group) gather
        // them once: wave w stages round w / 2 of group w % 2 in its buffer,
        // and every wave scores its head against all four sets.
        const int tw = w & 1, offw = (w >> 1) ? (l >> 1) : 0;
        if (hi == 0) spos[w][0][l32] = (tw ? st[T - 1] : st[0]) + offw;
        {
          u32x4_t v[LPS];
          fetch(Kg, 0, v);
          stage_set(v);
        }
        __syncthreads();
        float s1[T];
#pragma unroll
        for (int t = 0; t < T; ++t) {
          sa[t] = sigma_in(sbuf[t], 0);
          s1[t] = sigma_in(sbuf[2 + t], 0);
        }
        __syncthreads();                          // the buffers are the waves' own again
#pragma unroll
        for (int t = 0; t < T; ++t) {
          lo[t] = 0;
          hi_r[t] = l - 1;
          const int mid = l >> 1;
          if (s1[t] > sa[t]) { lo[t] = mid; sa[t] = s1[t]; }
          else               { hi_r[t] = mid - 1; }
          win[t] = sa[t];
        }
        wd0 = l >> 2;
      } else {
        int off[T];
#pragma unroll
        for (int t = 0; t < T; ++t) off[t] = 0;
        round(off, sa, unused, false);            // key 0 is never a right candidate
#pragma unroll
        for (int t = 0; t < T; ++t) { lo[t] = 0; hi_r[t] = l - 1; win[t] = sa[t]; }
      }
      for (int wd = wd0; wd >= 1; wd >>= 1) {
        int mid[T];
        float sm[T], smr[T];
#pragma unroll
        for (int t = 0; t < T; ++t) mid[t] = (lo[t] + hi_r[t] + 1) >> 1;
        round(mid, sm, smr, true);
#pragma unroll
        for (int t = 0; t < T; ++t) {
          if constexpr (RT) {
            if (smr[t] > sa[t]) { lo[t] = mid[t]; win[t] = smr[t]; sa[t] = sm[t]; }
            else                { hi_r[t] = mid[t] - 1; win[t] = sa[t]; }
          } else {
            if (sm[t] > sa[t]) { lo[t] = mid[t]; sa[t] = sm[t]; }
            else               { hi_r[t] = mid[t] - 1; }
            win[t] = sa[t];
          }
        }
      }
      if (hi == 0) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
          float& rb = red[w][sl * CPB + 32 * t + l32];
          rb = fmaxf(rb, win[t]);
        }
      }
    }
  }
  __syncthreads();
  for (int c = tid; c < nsl * CPB; c += 256) {
    if (jg + c < nc) {
      const float m = fmaxf(fmaxf(red[0][c], red[1][c]), fmaxf(red[2][c], red[3][c]));
      atomicMax(stage_scores(a, stage, r) + jg + c, score_key(m));
    }
  }
}

// Clears n keys (key 0 is below every score's key).
__global__ void __launch_bounds__(256) k_clear_keys(uint32_t* p, long long n) {
  const long long i = (static_cast<long long>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i + 3 < n) {
    *reinterpret_cast<uint4*>(p + i) = make_uint4(0, 0, 0, 0);
  } else {
    for (long long k = i; k < n; ++k) p[k] = 0;
  }
}

// bf16 prefill with query blocks of 64: score stage `stage` on the matrix cores
// (with ql and qr, the relative-RoPE tournaments over those rotated queries).
bool launch_score_prefill_mfma(const PruneArgs& a, int stage, int max_chunks, hipStream_t st,
                               const char* name, const uint16_t* ql, const uint16_t* qr) {
  if (a.kv.decode || a.kv.bq != 64 || max_chunks <= 0) return false;
  const bool rt = ql != nullptr;
  const int T = rt ? kScoreGroupsRt : kScoreGroups;
  const int ncg = (max_chunks + 32 * T - 1) / (32 * T);
  const int ngrp = (ncg + kSlices - 1) / kSlices;
  const long long groups = (a.R + 8LL * kRowGroup - 1) / (8LL * kRowGroup);   // per XCD
  const dim3 grid(static_cast<unsigned>(groups * 8 * kRowGroup * ngrp * a.kv.Hkv));
  if (a.kv.D != 128 && a.kv.D != 64) return false;
  {
    // the stage's score lists (the workgroups fold their maxima into them)
    const long long n = static_cast<long long>(a.R) * a.maxNC;
    uint32_t* sc = a.scores + static_cast<size_t>(stage & 1) * a.R * a.maxNC;
    DSA_LAUNCH("prune_clear_scores", k_clear_keys, dim3(static_cast<unsigned>((n + 1023) / 1024)), dim3(256), st,
               sc, n);
  }
  if (a.kv.D == 128) {
    if (rt) DSA_LAUNCH(name, (k_score_prefill_mfma<128, kScoreGroupsRt, true>), grid, dim3(256), st, a, stage, ngrp, ql, qr);
    else    DSA_LAUNCH(name, (k_score_prefill_mfma<128, kScoreGroups, false>), grid, dim3(256), st, a, stage, ngrp, ql, qr);
    return true;
  }
  if (a.kv.D == 64) {
    if (rt) DSA_LAUNCH(name, (k_score_prefill_mfma<64, kScoreGroupsRt, true>), grid, dim3(256), st, a, stage, ngrp, ql, qr);
    else    DSA_LAUNCH(name, (k_score_prefill_mfma<64, kScoreGroups, false>), grid, dim3(256), st, a, stage, ngrp, ql, qr);
    return true;
  }
  return false;
}

}  // namespace dsa
