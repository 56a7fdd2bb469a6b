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
// Workgroup = 4 waves x 32 chunks of one row (query block); the waves split
// the query heads, each running its heads' tournaments for the 32 chunks; the
// chunk score (max over all heads) is reduced in LDS.
#include "prune_common.h"

namespace dsa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int D>
__global__ void __launch_bounds__(256) k_score_prefill_mfma(PruneArgs a, int stage) {
  constexpr int KS = D / 16;
  const KvLayout& kv = a.kv;
  // rows vary fastest, so concurrently running workgroups score the same
  // chunk positions for neighbouring query blocks (shared rows in L2)
  const int r = blockIdx.x, j0 = blockIdx.y * 32;
  int b, s, e;
  row_bounds(kv, r, b, s, e);
  const Geo geo = make_geo(s, e, a.n_sink, a.n_window, a.chunk[0]);
  const int nc = stage_input_chunks(a, stage, r, geo);
  if (nc <= (a.keep[stage] >> a.lchunk[stage])) return;    // stage keeps everything
  if (j0 >= nc) return;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int j = j0 + l32;
  const bool active = j < nc;
  const int st = chunk_start(a, stage, r, active ? j : j0);
  const int l = a.chunk[stage];
  const int G = kv.Hq / kv.Hkv;
  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* K = static_cast<const uint16_t*>(a.k);
  __shared__ float red[4][32];

  float best = -INFINITY;
  for (int h = w; h < kv.Hq; h += 4) {
    const int g = h / G;
    const size_t kvbase = (static_cast<size_t>(b) * kv.Hkv + g) * kv.T;
    bf16x8_t qf[2][KS];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const uint16_t* qrow = Q + ((static_cast<size_t>(b) * kv.Hq + h) * kv.T + s + qt * 32 + l32) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qf[qt][ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qrow + ks * 16 + hi * 8));
    }
    // sigma of the key at position `pos` for this lane's chunk
    auto sigma_of = [&](const bf16x8_t* kf) {
      f32x16_t acc[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[qt][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
          acc[qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[qt][ks], kf[ks], acc[qt], 0, 0, 0);
      float m = acc[0][0];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int i = 0; i < 16; ++i) m = fmaxf(m, acc[qt][i]);
      return fmaxf(m, __shfl_xor(m, 32, 64));
    };
    auto load_row = [&](int pos, bf16x8_t* kf) {
      const uint16_t* krow = K + (kvbase + pos) * D + hi * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kf[ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(krow + ks * 16));
    };

    float sa;
    if (l == 1) {
      bf16x8_t k0[KS];
      load_row(st, k0);
      sa = sigma_of(k0);
    } else {
      // first split: both representatives are loaded in one round
      const int mid0 = l >> 1;
      int lo, hi_r;
      {
        bf16x8_t k0[KS], k1[KS];
        load_row(st, k0);
        load_row(st + mid0, k1);
        const float s0 = sigma_of(k0), s1 = sigma_of(k1);
        if (s1 > s0) { lo = mid0; hi_r = l - 1; sa = s1; }
        else         { lo = 0;    hi_r = mid0 - 1; sa = s0; }
      }
      for (int wd = mid0 >> 1; wd >= 1; wd >>= 1) {
        const int mid = (lo + hi_r + 1) >> 1;
        bf16x8_t km[KS];
        load_row(st + mid, km);
        const float sm = sigma_of(km);
        if (sm > sa) { lo = mid; sa = sm; }
        else         { hi_r = mid - 1; }
      }
    }
    best = fmaxf(best, sa);
  }
  if (hi == 0) red[w][l32] = best;
  __syncthreads();
  if (tid < 32 && j0 + tid < nc) {
    const float m = fmaxf(fmaxf(red[0][tid], red[1][tid]), fmaxf(red[2][tid], red[3][tid]));
    a.scores[static_cast<size_t>(r) * a.maxNC + j0 + tid] = score_key(m);
  }
}

// bf16 prefill with query blocks of 64: score stage `stage` on the matrix cores.
bool launch_score_prefill_mfma(const PruneArgs& a, int stage, int max_chunks, hipStream_t st,
                               const char* name) {
  if (a.kv.decode || a.kv.bq != 64 || max_chunks <= 0) return false;
  dim3 grid(a.R, (max_chunks + 31) / 32);
  if (a.kv.D == 128) {
    DSA_LAUNCH(name, (k_score_prefill_mfma<128>), grid, dim3(256), st, a, stage);
    return true;
  }
  if (a.kv.D == 64) {
    DSA_LAUNCH(name, (k_score_prefill_mfma<64>), grid, dim3(256), st, a, stage);
    return true;
  }
  return false;
}

}  // namespace dsa
