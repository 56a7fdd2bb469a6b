// Hierarchical pruning whose SelectRep tournaments use relative RoPE
// (InfiniteHiP page, 2502.08910, "Four RoPE Styles for Context Pruning":
// Relative; "Layer-Specific Strategy Assignment"): at every split the left
// branch's representative is scored as if it sat n_stream + 1 positions
// behind the query and the right branch's as n_stream behind (n_stream = the
// window), the right half winning only on a strictly greater score.
//
// The rotation is carried by the queries: each block's queries are rotated
// once to the two relative offsets (rotate-half pairing, theta_i =
// base^(-2i/d), fp64 without fused multiply-adds) and rounded to multiples of
// 1/128, which bf16 holds exactly; every score against grid-valued keys is
// then an exact fp32 number whatever the summation order. Each evaluated key
// is scored against both query sets in one pass: a right winner becomes the
// next split's left representative with its left score already at hand. A
// chunk's score is the one its representative won its last split with.
// The stage's top-K and the index row are those of the plain pruning.
#include "prune_common.h"

namespace dsa {

constexpr int kRopeQuant = 128;

// one rotated pair (x1, x2) -> (y1, y2) at position pos, rounded to the 1/128 grid
__device__ __forceinline__ void rope_pair(double x1, double x2, double theta, double pos, float& y1, float& y2) {
#pragma clang fp contract(off)
  const double ang = pos * theta;
  const double c = cos(ang), s = sin(ang);
  const double a = x1 * c - x2 * s;
  const double b = x2 * c + x1 * s;
  y1 = static_cast<float>(rint(a * kRopeQuant) / kRopeQuant);
  y2 = static_cast<float>(rint(b * kRopeQuant) / kRopeQuant);
}

__device__ __forceinline__ uint16_t exact_bf16(float f) { return static_cast<uint16_t>(__float_as_uint(f) >> 16); }

// Rotated query sets of row r, head h: [R, Hq, b_q, D] each.
template <typename T, int D>
__global__ void __launch_bounds__(256) k_rope_queries(PruneArgs a, uint16_t* ql, uint16_t* qr, double base) {
  const KvLayout& kv = a.kv;
  const int r = blockIdx.x, h = blockIdx.y;
  int b, s, e;
  row_bounds(kv, r, b, s, e);
  constexpr int half = D / 2;
  const int bq = kv.bq;
  const T* Q = static_cast<const T*>(a.q);
  for (int x = threadIdx.x; x < bq * half; x += blockDim.x) {
    const int t = x / half, i = x - t * half;
    const T* qrow = kv.decode ? Q + (static_cast<size_t>(b) * kv.Hq + h) * D
                              : Q + ((static_cast<size_t>(b) * kv.Hq + h) * kv.T + s + t) * D;
    const double x1 = load_one<T>(qrow + i), x2 = load_one<T>(qrow + i + half);
    const double theta = pow(base, (-2.0 * i) / D);
    const size_t o = ((static_cast<size_t>(r) * kv.Hq + h) * bq + t) * D;
    float y1, y2;
    rope_pair(x1, x2, theta, static_cast<double>(a.n_window + 1), y1, y2);
    ql[o + i] = exact_bf16(y1);
    ql[o + i + half] = exact_bf16(y2);
    rope_pair(x1, x2, theta, static_cast<double>(a.n_window), y1, y2);
    qr[o + i] = exact_bf16(y1);
    qr[o + i + half] = exact_bf16(y2);
  }
}

// Workgroup = 16 chunks of one row (a lane group of 16 per chunk), heads one
// after another with both query sets in LDS; the groups evaluate in lockstep.
template <typename T, int D>
__global__ void __launch_bounds__(256) k_score_rope(PruneArgs a, int stage, const uint16_t* ql, const uint16_t* qr) {
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
  __shared__ float qsl[64][D + 1];
  __shared__ float qsr[64][D + 1];
  __shared__ float ks[16][D + 4];
  const T* K = static_cast<const T*>(a.k);
  const int st = active ? chunk_start(a, stage, r, j) : 0;
  int n_iter = 0;
  while ((1 << n_iter) < l) ++n_iter;

  float best = -INFINITY;
  for (int h = 0; h < kv.Hq; ++h) {
    const int g = h / G;
    __syncthreads();
    const size_t qo = (static_cast<size_t>(r) * kv.Hq + h) * bq * D;
    for (int x = tid; x < bq * D; x += 256) {
      const int t = x / D, dd = x - t * D;
      qsl[t][dd] = bf16_to_f32(ql[qo + x]);
      qsr[t][dd] = bf16_to_f32(qr[qo + x]);
    }
    // left and right scores of the key at `pos` for this group's chunk
    auto eval = [&](int pos, float& sl, float& sr) {
      __syncthreads();
      if (active) {
        float kr[EPL];
        SliceLoad<T, EPL>::run(K + kv_offset(kv, b, g, pos) + li * EPL, kr);
#pragma unroll
        for (int x = 0; x < EPL; ++x) ks[gi][li * EPL + x] = kr[x];
      }
      __syncthreads();
      float ml = -INFINITY, mr = -INFINITY;
      if (active) {
        for (int t = li; t < bq; t += 16) {
          float al = 0.f, ar = 0.f;
#pragma unroll 8
          for (int x = 0; x < D; ++x) {
            al = fmaf(qsl[t][x], ks[gi][x], al);
            ar = fmaf(qsr[t][x], ks[gi][x], ar);
          }
          ml = fmaxf(ml, al);
          mr = fmaxf(mr, ar);
        }
      }
      sl = group16_max(ml);
      sr = group16_max(mr);
    };
    int lo = 0, hi = l - 1;
    float sl, sr;
    eval(st, sl, sr);
    float win = sl;
    for (int it = 0; it < n_iter; ++it) {
      const int mid = (lo + hi + 1) >> 1;
      float ml, mr;
      eval(st + mid, ml, mr);
      if (mr > sl) { lo = mid; win = mr; sl = ml; }
      else         { hi = mid - 1; win = sl; }
    }
    best = fmaxf(best, win);
  }
  if (active && li == 0) stage_scores(a, stage, r)[j] = score_key(best);
}

template <typename T, int D>
static hipError_t launch_rope_typed(const PruneArgs& a, uint16_t* ql, uint16_t* qr, double base, hipStream_t st) {
  DSA_LAUNCH("prune_rope_queries", (k_rope_queries<T, D>), dim3(a.R, a.kv.Hq), dim3(256), st, a, ql, qr, base);
  static const char* const names[kMaxStages] = {"prune_rope_score1", "prune_rope_score2", "prune_rope_score3",
                                                "prune_rope_score4"};
  for (int stage = 0; stage < a.n_stages; ++stage) {
    const int max_chunks = stage == 0 ? a.n1max : a.keep[stage - 1] / a.chunk[stage];
    if (max_chunks > 0) {
      DSA_LAUNCH(names[stage], (k_score_rope<T, D>), dim3((max_chunks + 15) / 16, a.R), dim3(256), st, a, stage,
                 ql, qr);
    }
    launch_topk(a, stage, max_chunks, st);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

hipError_t launch_prune_rope(const PruneArgs& a, int dtype, uint16_t* ql, uint16_t* qr, double base,
                             hipStream_t st) {
  if (dtype == 1) {
    if (a.kv.D == 128) return launch_rope_typed<uint16_t, 128>(a, ql, qr, base, st);
    if (a.kv.D == 64) return launch_rope_typed<uint16_t, 64>(a, ql, qr, base, st);
  } else {
    if (a.kv.D == 128) return launch_rope_typed<float, 128>(a, ql, qr, base, st);
    if (a.kv.D == 64) return launch_rope_typed<float, 64>(a, ql, qr, base, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace dsa
