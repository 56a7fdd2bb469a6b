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

// cos and sin of the angle pos * theta_i (fp64)
__device__ __forceinline__ void rope_angle(double theta, double pos, double& c, double& s) {
#pragma clang fp contract(off)
  const double ang = pos * theta;
  c = cos(ang);
  s = sin(ang);
}

// one pair (x1, x2) rotated by the angle with cosine c and sine s, each
// result rounded to the 1/128 grid (fp64, no fused multiply-adds)
__device__ __forceinline__ void rope_pair(double x1, double x2, double c, double s, float& y1, float& y2) {
#pragma clang fp contract(off)
  const double a = x1 * c - x2 * s;
  const double b = x2 * c + x1 * s;
  y1 = static_cast<float>(rint(a * kRopeQuant) / kRopeQuant);
  y2 = static_cast<float>(rint(b * kRopeQuant) / kRopeQuant);
}

__device__ __forceinline__ uint32_t exact_bf16(float f) { return __float_as_uint(f) >> 16; }

// Rotated query sets of row r, head h: [R, Hq, b_q, D] each. The angles
// depend only on the pair index and the two offsets, so their cosines and
// sines are computed once per workgroup; each thread then rotates 4
// consecutive pairs of one query (8-byte loads and stores at bf16).
template <typename T, int D>
__global__ void __launch_bounds__(256) k_rope_queries(PruneArgs a, uint16_t* ql, uint16_t* qr, double base) {
  constexpr int half = D / 2;
  __shared__ double cs[2][half][2];             // [left, right][pair][cos, sin]
  const KvLayout& kv = a.kv;
  const int r = blockIdx.x, h = blockIdx.y;
  int b, s, e;
  row_bounds(kv, r, b, s, e);
  const int bq = kv.bq;
  const T* Q = static_cast<const T*>(a.q);
  for (int x = threadIdx.x; x < 2 * half; x += blockDim.x) {
    const int side = x / half, i = x - side * half;
    const double theta = pow(base, (-2.0 * i) / D);
    rope_angle(theta, static_cast<double>(side ? a.n_window : a.n_window + 1), cs[side][i][0], cs[side][i][1]);
  }
  __syncthreads();
  constexpr int QG = half / 4;                  // groups of 4 pairs per query
  for (int x = threadIdx.x; x < bq * QG; x += blockDim.x) {
    const int t = x / QG, i0 = (x - t * QG) * 4;
    const T* qrow = kv.decode ? Q + (static_cast<size_t>(b) * kv.Hq + h) * D
                              : Q + ((static_cast<size_t>(b) * kv.Hq + h) * kv.T + s + t) * D;
    float x1[4], x2[4];
    SliceLoad<T, 4>::run(qrow + i0, x1);
    SliceLoad<T, 4>::run(qrow + i0 + half, x2);
    const size_t o = ((static_cast<size_t>(r) * kv.Hq + h) * bq + t) * D + i0;
#pragma unroll
    for (int side = 0; side < 2; ++side) {
      uint32_t lo[2] = {0, 0}, hi[2] = {0, 0};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float y1, y2;
        rope_pair(x1[k], x2[k], cs[side][i0 + k][0], cs[side][i0 + k][1], y1, y2);
        lo[k >> 1] |= exact_bf16(y1) << (16 * (k & 1));
        hi[k >> 1] |= exact_bf16(y2) << (16 * (k & 1));
      }
      uint16_t* out = side ? qr : ql;
      *reinterpret_cast<uint2*>(out + o) = make_uint2(lo[0], lo[1]);
      *reinterpret_cast<uint2*>(out + o + half) = make_uint2(hi[0], hi[1]);
    }
  }
}

// ------------------------------------------------------------------------- //
// decode: lane-group tournaments on rows held in registers                  //
// ------------------------------------------------------------------------- //
// A rotated query slice (bf16 on the 1/128 grid) in the key type's slice form.
template <typename T, int EPL>
__device__ __forceinline__ void load_rotated(RowSlice<T, EPL>& q, const uint16_t* p) {
  if constexpr (sizeof(T) == 2) q.load(p);
  else SliceLoad<uint16_t, EPL>::run(p, q.v);
}

// One lane group's relative-RoPE tournaments: the G query heads of kv head g
// over the chunk of l keys starting at st, side by side; every evaluated key
// is dotted with the head's left and right query slices. With SPEC, the SPEC
// keys that can represent the first log2(SPEC) splits (positions i*l/SPEC)
// are loaded and scored in one round and those splits are decided from them.
// Returns the best chunk score over the heads.
template <typename T, int D, int G, int SPEC, bool PAGED>
__device__ __forceinline__ float score_group_rt(const PruneArgs& a, int stage, int b, int g, int li, int st,
                                                const RowSlice<T, D / 16> (&ql)[G],
                                                const RowSlice<T, D / 16> (&qr)[G]) {
  using Row = RowSlice<T, D / 16>;
  const int l = a.chunk[stage];
  const ChunkRows<T, D, PAGED> rows(a, b, g, li, st, l);
  auto dl = [&](const Row& kr, int hh) { return group16_sum(kr.dot(ql[hh])); };
  auto dr = [&](const Row& kr, int hh) { return group16_sum(kr.dot(qr[hh])); };

  float sl[G], win[G];                         // left score of the representative, last winning score
  int lo[G], hi[G];
  int width;                                   // size of every head's remaining range
  if (l == 1) {
    const Row k0 = rows.at(st);
#pragma unroll
    for (int hh = 0; hh < G; ++hh) { sl[hh] = win[hh] = dl(k0, hh); lo[hh] = hi[hh] = 0; }
    width = 1;
  } else {
    bool spec = false;
    if constexpr (SPEC > 0) {
      if (l >= SPEC) {
        spec = true;
        const int u = l / SPEC;
        Row kr[SPEC];
#pragma unroll
        for (int i = 0; i < SPEC; ++i) kr[i] = rows.at(st + i * u);
        // scores are kept in named scalars: an indexed score array would be
        // selected from through memory
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          int A = 0;
          float s = dl(kr[0], hh), w = s;
          auto take = [&](int c, float r, float lf) __attribute__((always_inline)) {
            if (r > s) { A = c; w = r; s = lf; }
            else       { w = s; }
          };
          if constexpr (SPEC == 8) {
            take(4, dr(kr[4], hh), dl(kr[4], hh));
            {
              const bool b4 = A & 4;
              const float r2 = dr(kr[2], hh), r6 = dr(kr[6], hh), l2 = dl(kr[2], hh), l6 = dl(kr[6], hh);
              take(A + 2, b4 ? r6 : r2, b4 ? l6 : l2);
            }
            {
              const bool b2 = A & 2, b4 = A & 4;
              const float r1 = dr(kr[1], hh), r3 = dr(kr[3], hh), r5 = dr(kr[5], hh), r7 = dr(kr[7], hh);
              const float l1 = dl(kr[1], hh), l3 = dl(kr[3], hh), l5 = dl(kr[5], hh), l7 = dl(kr[7], hh);
              take(A + 1, b4 ? (b2 ? r7 : r5) : (b2 ? r3 : r1), b4 ? (b2 ? l7 : l5) : (b2 ? l3 : l1));
            }
          } else {
            static_assert(SPEC == 4, "speculative rounds of 4 or 8 keys");
            take(2, dr(kr[2], hh), dl(kr[2], hh));
            const bool b2 = A & 2;
            const float r1 = dr(kr[1], hh), r3 = dr(kr[3], hh), l1 = dl(kr[1], hh), l3 = dl(kr[3], hh);
            take(A + 1, b2 ? r3 : r1, b2 ? l3 : l1);
          }
          lo[hh] = A * u;
          hi[hh] = A * u + u - 1;
          sl[hh] = s;
          win[hh] = w;
        }
        width = u;
      }
    }
    if (!spec) {
      const int mid0 = l >> 1;
      const Row k0 = rows.at(st), k1 = rows.at(st + mid0);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float s0 = dl(k0, hh), r1 = dr(k1, hh), l1 = dl(k1, hh);
        if (r1 > s0) { lo[hh] = mid0; hi[hh] = l - 1;    win[hh] = r1; sl[hh] = l1; }
        else         { lo[hh] = 0;    hi[hh] = mid0 - 1; win[hh] = s0; sl[hh] = s0; }
      }
      width = mid0;
    }
  }
  for (int wdt = width >> 1; wdt >= 1; wdt >>= 1) {   // remaining splits
    Row kk[G];
    int mid[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      mid[hh] = (lo[hh] + hi[hh] + 1) >> 1;
      kk[hh] = rows.at(st + mid[hh]);
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float mr = dr(kk[hh], hh), ml = dl(kk[hh], hh);
      if (mr > sl[hh]) { lo[hh] = mid[hh]; win[hh] = mr; sl[hh] = ml; }
      else             { hi[hh] = mid[hh] - 1; win[hh] = sl[hh]; }
    }
  }
  float best = win[0];
#pragma unroll
  for (int hh = 1; hh < G; ++hh) best = fmaxf(best, win[hh]);
  return best;
}

// Decode scoring of one stage: workgroup = 16 lane groups; a group owns one
// (chunk, kv head) and runs that kv head's G tournaments side by side with
// the rotated query slices in registers; chunk results are max-reduced over
// the kv heads in LDS.
template <typename T, int D, int G, int SPEC, bool PAGED>
__global__ void __launch_bounds__(256, (G > 4 || (G == 4 && sizeof(T) == 4)) ? 2 : 4)
k_score_decode_rt(PruneArgs a, int stage, const uint16_t* ql_all, const uint16_t* qr_all) {
  constexpr int EPL = D / 16;
  using Row = RowSlice<T, EPL>;
  const KvLayout& kv = a.kv;
  const int r = blockIdx.y, b = r;              // one row per sequence
  const int cpw = 16 / kv.Hkv;                  // chunks per workgroup
  const int j0 = blockIdx.x * cpw;
  const int tid = threadIdx.x;
  const int gi = tid >> 4, li = tid & 15;
  const int cl = gi / kv.Hkv, g = gi - cl * kv.Hkv;
  const int j = j0 + cl;
  __shared__ float red[16];

  const int e = kv.seq_lens[r];
  int nc_prev = 0, st;
  if (stage == 0) {
    st = a.n_sink + (j << a.lchunk[0]);
  } else {
    const int sh = a.lchunk[stage - 1] - a.lchunk[stage];
    nc_prev = a.cnt[r * kMaxStages + stage - 1];
    const int32_t* prev = stage_starts(a, stage - 1, r);
    st = prev[min(j >> sh, a.maxK - 1)] + ((j & ((1 << sh) - 1)) << a.lchunk[stage]);
  }
  Row ql[G], qr[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const size_t o = (static_cast<size_t>(r) * kv.Hq + g * G + hh) * D + li * EPL;
    load_rotated(ql[hh], ql_all + o);
    load_rotated(qr[hh], qr_all + o);
  }

  const Geo geo = make_geo(e - 1, e, a.n_sink, a.n_window, a.chunk[0]);
  const int nc = stage == 0 ? geo.n1 : nc_prev << (a.lchunk[stage - 1] - a.lchunk[stage]);
  if (nc <= (a.keep[stage] >> a.lchunk[stage])) return;   // stage keeps everything for this row
  if (j0 >= nc) return;
  const bool active = j < nc;

  float best = -INFINITY;
  if (active) best = score_group_rt<T, D, G, SPEC, PAGED>(a, stage, b, g, li, st, ql, qr);
  if (li == 0) red[gi] = best;
  __syncthreads();
  if (tid < cpw) {
    const int jj = j0 + tid;
    if (jj < nc) {
      float m = red[tid * kv.Hkv];
      for (int x = 1; x < kv.Hkv; ++x) m = fmaxf(m, red[tid * kv.Hkv + x]);
      stage_scores(a, stage, r)[jj] = score_key(m);
    }
  }
}

// ------------------------------------------------------------------------- //
// prefill fallback (fp32, or query blocks other than 64)                    //
// ------------------------------------------------------------------------- //
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

static const char* const kRopeNames[kMaxStages] = {"prune_rope_score1", "prune_rope_score2", "prune_rope_score3",
                                                   "prune_rope_score4"};

// Speculative first round of a decode tournament: 8 keys for chunks of 8..64,
// 4 for longer chunks (register budget), none below 8.
static int rope_spec(int l) { return l >= 8 && l <= 64 ? 8 : l > 64 ? 4 : l >= 4 ? 4 : 0; }

template <typename T, int D, int G, bool PAGED>
static void launch_decode_rt(const PruneArgs& a, int stage, int max_chunks, const uint16_t* ql,
                             const uint16_t* qr, hipStream_t st) {
  const int cpw = 16 / a.kv.Hkv;
  const dim3 grid((max_chunks + cpw - 1) / cpw, a.R);
  const char* nm = kRopeNames[stage];
  switch (rope_spec(a.chunk[stage])) {
    case 8:  DSA_LAUNCH(nm, (k_score_decode_rt<T, D, G, 8, PAGED>), grid, dim3(256), st, a, stage, ql, qr); break;
    case 4:  DSA_LAUNCH(nm, (k_score_decode_rt<T, D, G, 4, PAGED>), grid, dim3(256), st, a, stage, ql, qr); break;
    default: DSA_LAUNCH(nm, (k_score_decode_rt<T, D, G, 0, PAGED>), grid, dim3(256), st, a, stage, ql, qr); break;
  }
}

template <typename T, int D, int G>
static void launch_decode_rt_g(const PruneArgs& a, int stage, int max_chunks, const uint16_t* ql,
                               const uint16_t* qr, hipStream_t st) {
  if (a.kv.block_table) launch_decode_rt<T, D, G, true>(a, stage, max_chunks, ql, qr, st);
  else                  launch_decode_rt<T, D, G, false>(a, stage, max_chunks, ql, qr, st);
}

// Rotation, then per stage: scoring (decode: lane-group tournaments; bf16
// prefill with 64-query blocks: the matrix-core tournaments; otherwise the
// generic kernel) and the plain top-K.
template <typename T, int D>
static hipError_t launch_rope_typed(const PruneArgs& a, uint16_t* ql, uint16_t* qr, double base, hipStream_t st) {
  DSA_LAUNCH("prune_rope_queries", (k_rope_queries<T, D>), dim3(a.R, a.kv.Hq), dim3(256), st, a, ql, qr, base);
  const int G = a.kv.Hq / a.kv.Hkv;
  for (int stage = 0; stage < a.n_stages; ++stage) {
    const int max_chunks = stage == 0 ? a.n1max : a.keep[stage - 1] / a.chunk[stage];
    if (max_chunks > 0) {
      if (a.kv.decode) {
        switch (G) {
          case 1: launch_decode_rt_g<T, D, 1>(a, stage, max_chunks, ql, qr, st); break;
          case 2: launch_decode_rt_g<T, D, 2>(a, stage, max_chunks, ql, qr, st); break;
          case 4: launch_decode_rt_g<T, D, 4>(a, stage, max_chunks, ql, qr, st); break;
          case 8: launch_decode_rt_g<T, D, 8>(a, stage, max_chunks, ql, qr, st); break;
          default: return hipErrorInvalidValue;
        }
      } else if (!(sizeof(T) == 2 && launch_score_prefill_mfma(a, stage, max_chunks, st, kRopeNames[stage], ql, qr))) {
        DSA_LAUNCH(kRopeNames[stage], (k_score_rope<T, D>), dim3((max_chunks + 15) / 16, a.R), dim3(256), st, a,
                   stage, ql, qr);
      }
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
