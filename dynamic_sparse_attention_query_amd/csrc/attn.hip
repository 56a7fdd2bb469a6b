// Attention over an index row (sparse) or over every causal key (dense).
//
// out[h, t] = sum_{p in row, p <= t} softmax_p(scale * q_{h,t} . k_p) v_p
// (InfLLM blog page, "Mathematical Formulation of Efficient Softmax
// Normalization"; MInference page, masked attention with in-kernel causal
// masking). Masked keys are excluded exactly. The softmax runs in the base-2
// domain with the scale folded into log2(e).
//
// Decode ("Flash Decoding", InfiniteHiP page, "Block Sparse Attention
// Implementation"): the row is cut into splits of `kps` entries; one
// workgroup per (split, kv head, sequence) produces an unnormalised partial
// (running max m, sum l, o[d]) for each query head of the group; a second
// kernel merges the partials.
// Prefill: one workgroup per (query block, query head) streams 64-key tiles of
// the row through LDS with an online softmax (generic FMA path).
#include "dsa_internal.h"

namespace dsa {


// ------------------------------------------------------------------------- //
// decode: split partials                                                    //
// ------------------------------------------------------------------------- //
template <typename T, int D, int G>
__global__ void __launch_bounds__(256) k_decode_partial(AttnArgs a) {
  constexpr int EPL = D / 16;
  constexpr int NO = (G * D + 255) / 256;
  const KvLayout& kv = a.kv;
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int Tb = seq_len_of(kv, b);
  const int tq = Tb - 1;
  const int tid = threadIdx.x, gi = tid >> 4, li = tid & 15, lane = tid & 63, w = tid >> 6;
  __shared__ float sv[64][D + 4];
  __shared__ float sp[G][64];
  __shared__ int spos[64];
  __shared__ float sm[G], sl[G], salpha[G];
  const T* Q = static_cast<const T*>(a.q);
  const T* K = static_cast<const T*>(a.k);
  const T* V = static_cast<const T*>(a.v);

  float q[G][EPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
    SliceLoad<T, EPL>::run(Q + (static_cast<size_t>(b) * kv.Hq + g * G + hh) * D + li * EPL, q[hh]);
  if (tid < G) {
    sm[tid] = kNegBig;
    sl[tid] = 0.f;
  }
  float acc[NO];
#pragma unroll
  for (int i = 0; i < NO; ++i) acc[i] = 0.f;

  const int n_total = a.idx ? a.L : Tb;
  const int k_begin = split * a.kps;
  const int k_end = min(n_total, k_begin + a.kps);
  const int32_t* row = a.idx ? a.idx + static_cast<size_t>(b) * a.L : nullptr;

  for (int kb = k_begin; kb < k_end; kb += 64) {
    __syncthreads();
    if (tid < 64) {
      const int i = kb + tid;
      int p = -1;
      if (i < k_end) {
        p = row ? row[i] : i;
        if (p < 0 || p > tq) p = -1;
      }
      spos[tid] = p;
    }
    __syncthreads();
    // issue every K/V row load of the sub-tile before any arithmetic; padding
    // entries read row 0 (always present) and are masked below
    float kr[4][EPL], vr[4][EPL];
    int pu[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      pu[u] = spos[gi + 16 * u];
      const size_t off = kv_offset(kv, b, g, max(pu[u], 0)) + li * EPL;
      SliceLoad<T, EPL>::run(K + off, kr[u]);
      SliceLoad<T, EPL>::run(V + off, vr[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kk = gi + 16 * u;
      const bool ok = pu[u] >= 0;
#pragma unroll
      for (int x = 0; x < EPL; ++x) sv[kk][li * EPL + x] = ok ? vr[u][x] : 0.f;
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float d = 0.f;
#pragma unroll
        for (int x = 0; x < EPL; ++x) d = fmaf(q[hh][x], kr[u][x], d);
        d = group16_sum(d);
        if (li == 0) sp[hh][kk] = ok ? d * a.scale_log2 : -INFINITY;
      }
    }
    __syncthreads();
    for (int hh = w; hh < G; hh += 4) {
      const float z = sp[hh][lane];
      const float m_old = sm[hh];
      const float m_new = fmaxf(m_old, wave_max_f(z));
      const float pz = (z == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(z - m_new);
      const float ls = wave_sum_f(pz);
      sp[hh][lane] = pz;
      if (lane == 0) {
        const float alpha = __builtin_amdgcn_exp2f(m_old - m_new);
        salpha[hh] = alpha;
        sl[hh] = sl[hh] * alpha + ls;
        sm[hh] = m_new;
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NO; ++i) {
      const int o = tid + 256 * i;
      if (o < G * D) {
        const int hh = o / D, dd = o - hh * D;
        float v = acc[i] * salpha[hh];
#pragma unroll 8
        for (int kk = 0; kk < 64; ++kk) v = fmaf(sp[hh][kk], sv[kk][dd], v);
        acc[i] = v;
      }
    }
  }
  __syncthreads();
  float* P = a.part;
#pragma unroll
  for (int i = 0; i < NO; ++i) {
    const int o = tid + 256 * i;
    if (o < G * D) {
      const int hh = o / D, dd = o - hh * D;
      P[((static_cast<size_t>(b) * kv.Hq + g * G + hh) * a.n_splits + split) * (D + 2) + dd] = acc[i];
    }
  }
  if (tid < G) {
    float* mlp = P + ((static_cast<size_t>(b) * kv.Hq + g * G + tid) * a.n_splits + split) * (D + 2) + D;
    mlp[0] = sm[tid];
    mlp[1] = sl[tid];
  }
}

// Merge split partials: M = max m_s, out = sum o_s 2^(m_s-M) / sum l_s 2^(m_s-M).
// (Exponentials of the decode kernels use the hardware 2^x: every argument is
// <= 0, and below -126 it returns 0 where the library routine would return a
// denormal.)
// 1024 threads: 1024/D groups of D threads each take a strided share of the
// splits. Every load a thread needs (its first kPrefetch shares of o, and
// m_s, l_s of split tid) is issued before the first barrier, so a merge of up
// to 1024 splits costs one memory round trip; longer rows (the dense path)
// loop over the rest.
constexpr int kCombineThreads = 1024;
constexpr int kMaxSplits = 4096;

template <int D>
__global__ void __launch_bounds__(kCombineThreads) k_decode_combine(AttnArgs a) {
  constexpr int kPrefetch = 8;
  constexpr int SG = kCombineThreads / D;
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  constexpr int NW = kCombineThreads / 64;
  const int ns = a.n_splits;
  const float* P = a.part + (static_cast<size_t>(b) * a.kv.Hq + h) * ns * (D + 2);
  __shared__ float wsh[kMaxSplits];
  __shared__ float red[NW];
  __shared__ float red2[NW];
  const int dd = tid % D, sg = tid / D;
  float v[kPrefetch];
#pragma unroll
  for (int u = 0; u < kPrefetch; ++u) {
    const int s = sg + u * SG;
    v[u] = s < ns ? P[static_cast<size_t>(s) * (D + 2) + dd] : 0.f;
  }
  float m0 = kNegBig, l0 = 0.f;
  if (tid < ns) {
    const float2 ml = *reinterpret_cast<const float2*>(P + static_cast<size_t>(tid) * (D + 2) + D);
    m0 = ml.x;
    l0 = ml.y;
  }
  float m = m0;
  for (int s = tid + kCombineThreads; s < ns; s += kCombineThreads) m = fmaxf(m, P[static_cast<size_t>(s) * (D + 2) + D]);
  m = wave_max_f(m);
  if (lane == 0) red[w] = m;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) M = fmaxf(M, red[i]);
  float lsum = 0.f;
  if (tid < ns) {
    const float f = __builtin_amdgcn_exp2f(m0 - M);
    wsh[tid] = f;
    lsum = l0 * f;
  }
  for (int s = tid + kCombineThreads; s < ns; s += kCombineThreads) {
    const float* ps = P + static_cast<size_t>(s) * (D + 2);
    const float f = __builtin_amdgcn_exp2f(ps[D] - M);
    wsh[s] = f;
    lsum = fmaf(ps[D + 1], f, lsum);
  }
  lsum = wave_sum_f(lsum);
  if (lane == 0) red2[w] = lsum;
  __syncthreads();
  float Ltot = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) Ltot += red2[i];
  float o = 0.f;
#pragma unroll
  for (int u = 0; u < kPrefetch; ++u) {
    const int s = sg + u * SG;
    if (s < ns) o = fmaf(v[u], wsh[s], o);
  }
  int s = sg + kPrefetch * SG;
  for (; s + 7 * SG < ns; s += 8 * SG) {
    float x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = P[static_cast<size_t>(s + u * SG) * (D + 2) + dd];
#pragma unroll
    for (int u = 0; u < 8; ++u) o = fmaf(x[u], wsh[s + u * SG], o);
  }
  for (; s < ns; s += SG) o = fmaf(P[static_cast<size_t>(s) * (D + 2) + dd], wsh[s], o);
  __shared__ float so[SG][D];
  so[sg][dd] = o;
  __syncthreads();
  if (sg == 0) {
    float ot = 0.f;
#pragma unroll
    for (int x = 0; x < SG; ++x) ot += so[x][dd];
    a.out[(static_cast<size_t>(b) * a.kv.Hq + h) * D + dd] = Ltot > 0.f ? ot / Ltot : 0.f;   // no visible key: 0
  }
}

// ------------------------------------------------------------------------- //
// prefill: generic FMA flash attention over gathered 64-key tiles           //
// ------------------------------------------------------------------------- //
template <typename T, int D>
__global__ void __launch_bounds__(256) k_prefill_generic(AttnArgs a) {
  const KvLayout& kv = a.kv;
  const int m = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int bq = kv.bq;
  const int s = m * bq, e = s + bq;
  const int G = kv.Hq / kv.Hkv;
  const int g = h / G;
  const int TPR = 256 / bq;           // threads per query row (4 .. 64)
  const int DPT = D / TPR;            // output dims per thread
  const int tid = threadIdx.x;
  const int q = tid / TPR, sub = tid - q * TPR;
  const int tq = s + q;
  __shared__ float qs[64][D + 1];
  __shared__ float ks[64][D + 1];
  __shared__ float vs[64][D + 1];
  __shared__ float ps[64][65];
  __shared__ int spos[64];
  const T* Q = static_cast<const T*>(a.q);
  const T* K = static_cast<const T*>(a.k);
  const T* V = static_cast<const T*>(a.v);

  for (int x = tid; x < bq * D; x += 256) {
    const int t = x / D, dd = x - t * D;
    qs[t][dd] = load_one<T>(Q + ((static_cast<size_t>(b) * kv.Hq + h) * kv.T + s + t) * D + dd);
  }
  const int r = a.row_heads ? (b * kv.Hq + h) * kv.nblk + m : b * kv.nblk + m;
  const int32_t* row = a.idx ? a.idx + static_cast<size_t>(r) * a.L : nullptr;
  const int n_ent = row ? a.L : e;
  float mrun = kNegBig, lrun = 0.f;
  float o[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) o[j] = 0.f;

  for (int kb = 0; kb < n_ent; kb += 64) {
    __syncthreads();
    if (tid < 64) {
      const int i = kb + tid;
      int p = -1;
      if (i < n_ent) {
        p = row ? row[i] : i;
        if (p < 0 || p >= e) p = -1;
      }
      spos[tid] = p;
    }
    __syncthreads();
    for (int x = tid; x < 64 * D; x += 256) {
      const int kk = x / D, dd = x - kk * D;
      const int p = spos[kk];
      float kvv = 0.f, vvv = 0.f;
      if (p >= 0) {
        const size_t off = kv_offset(kv, b, g, p) + dd;
        kvv = load_one<T>(K + off);
        vvv = load_one<T>(V + off);
      }
      ks[kk][dd] = kvv;
      vs[kk][dd] = vvv;
    }
    __syncthreads();
    float tmax = -INFINITY;
    for (int i = 0; i < 64 / TPR; ++i) {
      const int kk = sub + TPR * i;
      const int p = spos[kk];
      float d = 0.f;
#pragma unroll 8
      for (int x = 0; x < D; ++x) d = fmaf(qs[q][x], ks[kk][x], d);
      const float z = (p >= 0 && p <= tq) ? d * a.scale_log2 : -INFINITY;
      ps[q][kk] = z;
      tmax = fmaxf(tmax, z);
    }
    for (int off = TPR >> 1; off >= 1; off >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, off, TPR));
    const float m_new = fmaxf(mrun, tmax);
    const float alpha = exp2f(mrun - m_new);
    float psum = 0.f;
    for (int i = 0; i < 64 / TPR; ++i) {
      const int kk = sub + TPR * i;
      const float z = ps[q][kk];
      const float pz = (z == -INFINITY) ? 0.f : exp2f(z - m_new);
      ps[q][kk] = pz;
      psum += pz;
    }
    for (int off = TPR >> 1; off >= 1; off >>= 1) psum += __shfl_xor(psum, off, TPR);
    lrun = lrun * alpha + psum;
    mrun = m_new;
    __syncthreads();
    for (int j = 0; j < DPT; ++j) {
      const int dd = sub + TPR * j;
      float v = o[j] * alpha;
#pragma unroll 8
      for (int kk = 0; kk < 64; ++kk) v = fmaf(ps[q][kk], vs[kk][dd], v);
      o[j] = v;
    }
  }
  float* out = a.out + ((static_cast<size_t>(b) * kv.Hq + h) * kv.T + tq) * D;
  for (int j = 0; j < DPT; ++j) out[sub + TPR * j] = lrun > 0.f ? o[j] / lrun : 0.f;   // no visible key: 0
}

// ------------------------------------------------------------------------- //
// launcher                                                                  //
// ------------------------------------------------------------------------- //
template <typename T, int D, int G>
static void launch_decode(const AttnArgs& a, hipStream_t st) {
  dim3 grid(a.n_splits, a.kv.Hkv, a.kv.B);
  DSA_LAUNCH(a.idx ? "attn_decode_partial" : "dense_decode_partial", (k_decode_partial<T, D, G>), grid,
             dim3(256), st, a);
  DSA_LAUNCH(a.idx ? "attn_decode_combine" : "dense_decode_combine", (k_decode_combine<D>),
             dim3(a.kv.Hq, a.kv.B), dim3(kCombineThreads), st, a);
}

void launch_decode_combine(const AttnArgs& a, hipStream_t st) {
  if (a.kv.D == 128)
    DSA_LAUNCH("attn_decode_combine", (k_decode_combine<128>), dim3(a.kv.Hq, a.kv.B), dim3(kCombineThreads), st, a);
  else
    DSA_LAUNCH("attn_decode_combine", (k_decode_combine<64>), dim3(a.kv.Hq, a.kv.B), dim3(kCombineThreads), st, a);
}

template <typename T, int D>
static hipError_t launch_attn_typed(const AttnArgs& a, hipStream_t st) {
  if (a.kv.decode) {
    switch (a.kv.Hq / a.kv.Hkv) {
      case 1: launch_decode<T, D, 1>(a, st); break;
      case 2: launch_decode<T, D, 2>(a, st); break;
      case 4: launch_decode<T, D, 4>(a, st); break;
      case 8: launch_decode<T, D, 8>(a, st); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    if (sizeof(T) == 2 && launch_prefill_mfma(a, st)) return hipGetLastError();
    dim3 grid(a.kv.nblk, a.kv.Hq, a.kv.B);
    const char* name = a.row_heads ? "attn_prefill_heads" : a.idx ? "attn_prefill" : "dense_prefill";
    DSA_LAUNCH(name, (k_prefill_generic<T, D>), grid, dim3(256), st, a);
  }
  return hipGetLastError();
}

hipError_t launch_sparse_attn(const AttnArgs& a, int dtype, hipStream_t st) {
  if (dtype == 1) {
    if (a.kv.D == 128) return launch_attn_typed<uint16_t, 128>(a, st);
    if (a.kv.D == 64) return launch_attn_typed<uint16_t, 64>(a, st);
  } else {
    if (a.kv.D == 128) return launch_attn_typed<float, 128>(a, st);
    if (a.kv.D == 64) return launch_attn_typed<float, 64>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace dsa
