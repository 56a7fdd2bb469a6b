// Prefill attention over gathered key tiles on the bf16 matrix cores (gfx950
// v_mfma_f32_32x32x16_bf16), "similar to FlashAttention" as the InfiniteHiP
// page describes its prefill kernel ("Block Sparse Attention Implementation").
// The key tiles are gathered through the index row as the MInference page's
// permutation-gather (PIT) idea does: non-contiguous keys are packed into a
// dense tile in LDS, then dense matrix products run on the tile.
//
// One workgroup per (sequence, query block of 64, kv head); one wave per query
// head of the GQA group, all sharing the group's K/V tiles in LDS.
//   S^T = K Q^T  (32x32 tiles: rows = keys, columns = queries), so each lane
//                owns whole query columns and the row softmax needs a single
//                exchange between the two half-waves;
//   O^T += V^T P^T, with P^T taken straight from the S^T accumulators: the
//                keys of a 16-key step are permuted identically in both
//                operands (V^T is staged transposed in LDS to allow it).
// Online softmax in base 2 (scale folded into log2 e); causal and padding
// masks are applied only on tiles that need them.
#include "dsa_internal.h"

namespace dsa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// two floats to packed bf16 (round to nearest even) in one conversion
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

template <int D, int NW>
__global__ void __launch_bounds__(64 * NW) k_prefill_mfma(AttnArgs a) {
  constexpr int KS = D / 16;          // 16-wide steps over d
  constexpr int DT = D / 32;          // 32-row tiles of O^T
  constexpr int KROW = D + 8;         // K tile row stride (bf16 elements)
  constexpr int VROW = 64 + 4;        // V^T tile row stride (bf16 elements), 34 dwords
  constexpr int COMBOS = 4 * DT;      // (16-key group, 4-chunk group) pairs per tile
  static_assert(COMBOS % NW == 0, "tile loads must split evenly over the waves");
  __shared__ __align__(16) uint16_t sq[NW * 64 * KROW];   // each wave's query block
  __shared__ __align__(16) uint16_t sk[64 * KROW];
  __shared__ __align__(16) uint16_t svt[D * VROW];
  __shared__ __align__(16) int spos[64];
  __shared__ int sneed[NW], sany[NW];

  const KvLayout& kv = a.kv;
  // XCD-aware order: consecutive workgroup ids go to different XCDs, so give
  // each XCD a contiguous run of work (adjacent query blocks of one kv head
  // share most window keys and sit in the same L2).
  const int G = kv.Hq / kv.Hkv;
  const int HG = G / NW;                          // workgroups per (block, kv head)
  const int nwork = kv.B * kv.Hkv * HG * kv.nblk;
  const int per_xcd = gridDim.x >> 3;
  const int work = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (work >= nwork) return;
  const int m = work % kv.nblk;
  const int hg = (work / kv.nblk) % (kv.Hkv * HG);
  const int b = work / (kv.nblk * kv.Hkv * HG);
  const int g = hg / HG;
  const int s = m * 64, e = s + 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int h = g * G + (hg % HG) * NW + w;
  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* K = static_cast<const uint16_t*>(a.k);
  const uint16_t* V = static_cast<const uint16_t*>(a.v);
  const size_t kvbase = (static_cast<size_t>(b) * kv.Hkv + g) * kv.T;

  // the wave's query block, row-major in LDS; B operand fragments of Q^T are
  // read from it per 16-wide d step (8 consecutive d of one query row)
  uint16_t* qs = sq + w * 64 * KROW;
  {
    const uint16_t* qblk = Q + ((static_cast<size_t>(b) * kv.Hq + h) * kv.T + s) * D;
#pragma unroll
    for (int it = 0; it < 64 * D / 8 / 64; ++it) {
      const int c = it * 64 + lane;            // 16-byte chunk of the 64 x D block
      const int qrow = c / (D / 8), qcol = (c % (D / 8)) * 8;
      *reinterpret_cast<uint4*>(qs + qrow * KROW + qcol) =
          *reinterpret_cast<const uint4*>(qblk + qrow * D + qcol);
    }
  }
  f32x16_t o[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][qt][i] = 0.f;
  float mrun[2] = {kNegBig, kNegBig}, lrun[2] = {0.f, 0.f};

  const int r = b * kv.nblk + m;
  const int32_t* row = a.idx ? a.idx + static_cast<size_t>(r) * a.L : nullptr;
  const int n_ent = row ? a.L : e;
  const int n_tiles = (n_ent + 63) / 64;
  const int kl = lane & 15, cl = lane >> 4;       // loader lane: key and 16-byte chunk
  constexpr int PER = COMBOS / NW;                // (key, chunk) loads per thread per tile

  // row entry i as a key position visible to some query of the block, else -1
  auto entry = [&](int i) {
    int p = -1;
    if (i < n_ent) {
      p = row ? row[i] : i;
      if (p < 0 || p >= e) p = -1;
    }
    return p;
  };
  // Software pipeline: while tile i is computed from LDS, the K/V rows of tile
  // i+1 are in flight into registers and the positions of tile i+2 are read.
  int pcur[PER], pnext[PER];
  uint4 kreg[PER], vreg[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int key = ((u * NW + w) & 3) * 16 + kl;
    const int chunk = ((u * NW + w) >> 2) * 4 + cl;
    pcur[u] = entry(key);
    pnext[u] = entry(64 + key);
    const size_t off = (kvbase + max(pcur[u], 0)) * D + chunk * 8;
    kreg[u] = *reinterpret_cast<const uint4*>(K + off);
    vreg[u] = *reinterpret_cast<const uint4*>(V + off);
  }

  for (int ti = 0; ti < n_tiles; ++ti) {
    __syncthreads();                               // the previous tile is consumed
    bool need = false, any = false;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int combo = u * NW + w;
      const int key = (combo & 3) * 16 + kl;
      const int chunk = (combo >> 2) * 4 + cl;
      const int p = pcur[u];
      need |= (p < 0 || p > s);
      any |= (p >= 0);
      if (cl == 0) spos[key] = p;
      const uint4 kv4 = p >= 0 ? kreg[u] : make_uint4(0, 0, 0, 0);
      const uint4 vv4 = p >= 0 ? vreg[u] : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(sk + key * KROW + chunk * 8) = kv4;
      const uint32_t vw[4] = {vv4.x, vv4.y, vv4.z, vv4.w};
#pragma unroll
      for (int j = 0; j < 8; ++j)
        svt[(chunk * 8 + j) * VROW + key] = static_cast<uint16_t>(vw[j >> 1] >> ((j & 1) * 16));
    }
    const unsigned long long nb = __ballot(need), ab = __ballot(any);
    if (lane == 0) { sneed[w] = nb != 0; sany[w] = ab != 0; }
    __syncthreads();
    int flag = 2;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      flag |= sneed[i] ? 1 : 0;
      if (sany[i]) flag &= ~2;
    }
    flag = __builtin_amdgcn_readfirstlane(flag);   // uniform: scalar branches below
    // start the next tile's loads and the positions of the one after
    if (ti + 1 < n_tiles) {
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int key = ((u * NW + w) & 3) * 16 + kl;
        const int chunk = ((u * NW + w) >> 2) * 4 + cl;
        pcur[u] = pnext[u];
        const size_t off = (kvbase + max(pcur[u], 0)) * D + chunk * 8;
        kreg[u] = *reinterpret_cast<const uint4*>(K + off);
        vreg[u] = *reinterpret_cast<const uint4*>(V + off);
        pnext[u] = entry((ti + 2) * 64 + key);
      }
    }
    if (flag & 2) continue;                        // nothing visible in this tile

    // S^T tiles: [key tile kt][query tile qt]
    f32x16_t sacc[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kt][qt][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8_t qf[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
        qf[qt] = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const uint4*>(qs + (qt * 32 + l32) * KROW + ks * 16 + hi * 8));
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8_t af = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const uint4*>(sk + (kt * 32 + l32) * KROW + ks * 16 + hi * 8));
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
          sacc[kt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[qt], sacc[kt][qt], 0, 0, 0);
      }
    }
    // causal / padding mask: this lane's keys are 4 runs of 4 per key tile
    if (flag & 1) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int rn = 0; rn < 4; ++rn) {
          const int4 p4 = *reinterpret_cast<const int4*>(spos + kt * 32 + rn * 8 + hi * 4);
          const int pp[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) {
            // padding (-1) compares as the largest unsigned value
            const unsigned t = static_cast<unsigned>(s + qt * 32 + l32);
#pragma unroll
            for (int c = 0; c < 4; ++c)
              if (static_cast<unsigned>(pp[c]) > t) sacc[kt][qt][rn * 4 + c] = -INFINITY;
          }
        }
    }
    // online softmax per query column, base 2. The running max is raised
    // only when a score exceeds it by more than 2^8 (p stays <= 256, exact
    // in the final normalisation).
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kt][qt][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * a.scale_log2;
      const bool raise = mx > mrun[qt] + 8.0f;
      const float m_use = raise ? mx : mrun[qt];
      const float alpha = __builtin_amdgcn_exp2f(mrun[qt] - m_use);
      float ps = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pz = __builtin_amdgcn_exp2f(fmaf(sacc[kt][qt][i], a.scale_log2, -m_use));
          sacc[kt][qt][i] = pz;
          ps += pz;
        }
      ps += __shfl_xor(ps, 32, 64);
      lrun[qt] = lrun[qt] * alpha + ps;
      mrun[qt] = m_use;
      if (__ballot(raise)) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[dt][qt][i] *= alpha;
      }
    }
    // O^T += V^T P^T over four 16-key steps
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kt = ks >> 1, half = ks & 1;
      bf16x8_t pb[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        uint4 u;
        u.x = pack_bf16x2(sacc[kt][qt][half * 8 + 0], sacc[kt][qt][half * 8 + 1]);
        u.y = pack_bf16x2(sacc[kt][qt][half * 8 + 2], sacc[kt][qt][half * 8 + 3]);
        u.z = pack_bf16x2(sacc[kt][qt][half * 8 + 4], sacc[kt][qt][half * 8 + 5]);
        u.w = pack_bf16x2(sacc[kt][qt][half * 8 + 6], sacc[kt][qt][half * 8 + 7]);
        pb[qt] = __builtin_bit_cast(bf16x8_t, u);
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint16_t* vr = svt + (dt * 32 + l32) * VROW + ks * 16 + hi * 4;
        const uint2 lo4 = *reinterpret_cast<const uint2*>(vr);
        const uint2 hi4 = *reinterpret_cast<const uint2*>(vr + 8);
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, make_uint4(lo4.x, lo4.y, hi4.x, hi4.y));
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
          o[dt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[qt], o[dt][qt], 0, 0, 0);
      }
    }
  }

  // out[b, h, t, d] = O^T[d, t] / l
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const float inv = 1.0f / lrun[qt];
    float* orow = a.out + ((static_cast<size_t>(b) * kv.Hq + h) * kv.T + s + qt * 32 + l32) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        float4 v;
        v.x = o[dt][qt][i4 * 4 + 0] * inv;
        v.y = o[dt][qt][i4 * 4 + 1] * inv;
        v.z = o[dt][qt][i4 * 4 + 2] * inv;
        v.w = o[dt][qt][i4 * 4 + 3] * inv;
        *reinterpret_cast<float4*>(orow + dt * 32 + i4 * 8 + hi * 4) = v;
      }
  }
}

template <int D, int NW>
static void launch_mfma(const AttnArgs& a, hipStream_t st) {
  const int G = a.kv.Hq / a.kv.Hkv;
  const int nwork = a.kv.B * a.kv.Hkv * (G / NW) * a.kv.nblk;
  const int grid = (nwork + 7) / 8 * 8;
  DSA_LAUNCH(a.idx ? "attn_prefill" : "dense_prefill", (k_prefill_mfma<D, NW>), dim3(grid), dim3(64 * NW),
             st, a);
}

// bf16 prefill with query blocks of 64 rows; a workgroup covers up to 4 query
// heads of one GQA group.
bool launch_prefill_mfma(const AttnArgs& a, hipStream_t st) {
  if (a.kv.decode || a.kv.bq != 64) return false;
  const int G = a.kv.Hq / a.kv.Hkv;
  const int nw = G >= 4 ? 4 : G;
  if (a.kv.D == 128) {
    switch (nw) {
      case 1: launch_mfma<128, 1>(a, st); return true;
      case 2: launch_mfma<128, 2>(a, st); return true;
      case 4: launch_mfma<128, 4>(a, st); return true;
    }
  } else if (a.kv.D == 64) {
    switch (nw) {
      case 1: launch_mfma<64, 1>(a, st); return true;
      case 2: launch_mfma<64, 2>(a, st); return true;
      case 4: launch_mfma<64, 4>(a, st); return true;
    }
  }
  return false;
}

}  // namespace dsa
