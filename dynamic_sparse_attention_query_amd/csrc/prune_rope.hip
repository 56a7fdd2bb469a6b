// Hierarchical pruning with RoPE inside the SelectRep tournaments
// (InfiniteHiP page, 2502.08910, "Four RoPE Styles for Context Pruning" and
// "Layer-Specific Strategy Assignment").
//
// Relative RoPE (the section's Relative style): at every split the left
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
//
// Chunk-indexed RoPE (same section, Chunk-indexed): within a stage of chunk
// length l a key sits at its chunk's index (position - n_sink) / l and every
// query n_stream after the stage's last chunk (capped at the query's own
// position); queries and keys are each rotated in fp64 and rounded to the
// 1/128 grid, and the plain tournaments run on the rotated rows. The queries
// are rotated once per stage; prefill rotates the keys once per stage into a
// bf16 copy that the plain scoring kernels read, decode rotates each row it
// evaluates in registers (the partner half of every pair comes from lane
// li ^ 8 of the lane group).
#include <algorithm>
#include <type_traits>

#include "prune_common.h"
#include "selectrep.h"

namespace dsa {

constexpr int kRopeQuant = 128;
constexpr int kRopeRelative = 1;        // the ABI's rope styles
constexpr int kRopeChunkIndexed = 2;

// theta_i = base^(-2i/d) (fp64)
__device__ __forceinline__ double rope_theta(double base, int i, int d) { return pow(base, (-2.0 * i) / d); }

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
    rope_angle(rope_theta(base, i, D), static_cast<double>(side ? a.n_window : a.n_window + 1), cs[side][i][0],
               cs[side][i][1]);
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
template <typename T, int D, int G, int SPEC, class Rows>
__device__ __forceinline__ float score_group_rt_rows(const PruneArgs& a, int stage, int li, int st, const Rows& rows,
                                                     const RowSlice<T, D / 16> (&ql)[G],
                                                     const RowSlice<T, D / 16> (&qr)[G]) {
  using Row = RowSlice<T, D / 16>;
  const int l = a.chunk[stage];
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

// The tournaments above on the chunk's rows: contiguous, or paged with the
// page ids in registers when they fit, else through the page table.
template <typename T, int D, int G, int SPEC, bool PAGED>
__device__ __forceinline__ float score_group_rt(const PruneArgs& a, int stage, int b, int g, int li, int st,
                                                const RowSlice<T, D / 16> (&ql)[G],
                                                const RowSlice<T, D / 16> (&qr)[G]) {
  return paged_rows<T, D, PAGED>(a, b, g, li, st, a.chunk[stage], nullptr, 0, [&](const auto& rows) {
    return score_group_rt_rows<T, D, G, SPEC>(a, stage, li, st, rows, ql, qr);
  });
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
  const int tid = threadIdx.x;
  const int gi = tid >> 4, li = tid & 15;
  const DecodeLane dl = decode_lane(a, blockIdx.x, gi);
  const int cpw = dl.cpw, j0 = dl.j0, g = dl.g;  // chunks per workgroup, first chunk, kv head
  const int j = j0 + dl.cl;
  __shared__ float red[16];

  const int e = seq_len_of(kv, r);
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
  const bool active = dl.used && j < nc;

  float best = -INFINITY;
  if (active) best = score_group_rt<T, D, G, SPEC, PAGED>(a, stage, b, g, li, st, ql, qr);
  if (li == 0) red[gi] = best;
  __syncthreads();
  if (tid < cpw) {
    const int jj = j0 + tid;
    if (jj < nc) {
      float m = red[tid * a.hpw];
      for (int x = 1; x < a.hpw; ++x) m = fmaxf(m, red[tid * a.hpw + x]);
      stage_scores(a, stage, r, dl.sl)[jj] = score_key(m);
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

// ------------------------------------------------------------------------- //
// chunk-indexed RoPE                                                        //
// ------------------------------------------------------------------------- //
constexpr int kDppRowRor8 = 0x128;      // lane i <- lane (i + 8) mod 16 of its row

template <int CTRL>
__device__ __forceinline__ double dpp_perm_d(double v) {
  const uint64_t u = __double_as_longlong(v);
  const uint32_t lo = static_cast<uint32_t>(dpp_perm<CTRL>(static_cast<int>(static_cast<uint32_t>(u))));
  const uint32_t hi = static_cast<uint32_t>(dpp_perm<CTRL>(static_cast<int>(static_cast<uint32_t>(u >> 32))));
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

// x * c + p * ss with ss = -s for the first half of a pair (x1 c - x2 s) and
// +s for the second (x2 c + x1 s), rounded to the 1/128 grid
__device__ __forceinline__ float rope_half(double x, double p, double c, double ss) {
#pragma clang fp contract(off)
  const double y = x * c + p * ss;
  return static_cast<float>(rint(y * kRopeQuant) / kRopeQuant);
}

// Query ID of a stage: n_stream after the last chunk of the stage's tiling of
// the middle [n_sink, mid_hi).
__device__ __forceinline__ int ci_query_id(const PruneArgs& a, int stage, const Geo& geo) {
  return ((geo.mid_hi - a.n_sink) >> a.lchunk[stage]) - 1 + a.n_window;
}

// Rotated queries of one stage, in the layout of q (bf16): workgroup = (row,
// head); the angles of the stage's query ID are tabled once, a query capped
// at its own position computes its own. blockIdx.z selects stage stage0 + z,
// written qstride elements after the previous stage's.
template <typename T, int D>
__global__ void __launch_bounds__(256) k_ci_queries(PruneArgs a, int stage0, uint16_t* qo, double base,
                                                    size_t qstride) {
  constexpr int half = D / 2;
  __shared__ double cs[half][2];
  const KvLayout& kv = a.kv;
  const int r = blockIdx.x, h = blockIdx.y;
  const int stage = stage0 + blockIdx.z;
  qo += blockIdx.z * qstride;
  int b, s, e;
  row_bounds(kv, r, b, s, e);
  const Geo geo = make_geo(s, e, a.n_sink, a.n_window, a.chunk[0]);
  const int qid = ci_query_id(a, stage, geo);
  for (int i = threadIdx.x; i < half; i += blockDim.x) rope_angle(rope_theta(base, i, D), qid, cs[i][0], cs[i][1]);
  __syncthreads();
  const int bq = kv.bq;
  const T* Q = static_cast<const T*>(a.q);
  constexpr int QG = half / 4;
  for (int x = threadIdx.x; x < bq * QG; x += blockDim.x) {
    const int t = x / QG, i0 = (x - t * QG) * 4;
    const size_t o = kv.decode ? (static_cast<size_t>(b) * kv.Hq + h) * D
                               : ((static_cast<size_t>(b) * kv.Hq + h) * kv.T + s + t) * D;
    float x1[4], x2[4];
    SliceLoad<T, 4>::run(Q + o + i0, x1);
    SliceLoad<T, 4>::run(Q + o + i0 + half, x2);
    const int i_orig = kv.decode ? e - 1 : s + t;
    uint32_t lo[2] = {0, 0}, hi[2] = {0, 0};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      double c = cs[i0 + k][0], sn = cs[i0 + k][1];
      if (i_orig < qid) rope_angle(rope_theta(base, i0 + k, D), i_orig, c, sn);
      float y1, y2;
      rope_pair(x1[k], x2[k], c, sn, y1, y2);
      lo[k >> 1] |= exact_bf16(y1) << (16 * (k & 1));
      hi[k >> 1] |= exact_bf16(y2) << (16 * (k & 1));
    }
    *reinterpret_cast<uint2*>(qo + o + i0) = make_uint2(lo[0], lo[1]);
    *reinterpret_cast<uint2*>(qo + o + i0 + half) = make_uint2(hi[0], hi[1]);
  }
}

// Rotated keys of one stage, in the layout of k (bf16): workgroup = 32
// positions of every (sequence, kv head) from p_lo, up to p_hi; the angles of
// the (at most 33) chunk indices the tile touches are tabled in LDS.
// Positions before n_sink are never candidates and are left as they are.
// blockIdx.y selects stage stage0 + y, written to out.ko[y]. A key's chunk
// index in a stage depends only on its position (the tiling is anchored at
// n_sink), so a rotated copy stays valid as the context grows.
constexpr int kCiTile = 32;
struct CiKeyOut {
  uint16_t* ko[kMaxStages];
};
template <typename T, int D>
__global__ void __launch_bounds__(256) k_ci_keys(PruneArgs a, int stage0, CiKeyOut out, double base, int p_lo,
                                                 int p_hi) {
  constexpr int half = D / 2;
  __shared__ double cs[kCiTile + 1][half][2];
  const KvLayout& kv = a.kv;
  const int stage = stage0 + blockIdx.y;
  uint16_t* ko = out.ko[blockIdx.y];
  const int p0 = max(p_lo + static_cast<int>(blockIdx.x) * kCiTile, a.n_sink);
  const int p1 = min(p_lo + static_cast<int>(blockIdx.x + 1) * kCiTile, p_hi);
  if (p0 >= p1) return;
  const int lc = a.lchunk[stage];
  const int c0 = (p0 - a.n_sink) >> lc, nch = ((p1 - 1 - a.n_sink) >> lc) - c0 + 1;
  for (int x = threadIdx.x; x < nch * half; x += blockDim.x) {
    const int cc = x / half, i = x - cc * half;
    rope_angle(rope_theta(base, i, D), static_cast<double>(c0 + cc), cs[cc][i][0], cs[cc][i][1]);
  }
  __syncthreads();
  const T* K = static_cast<const T*>(a.k);
  constexpr int QG = half / 4;
  const int np = p1 - p0;
  const int rows = kv.B * kv.Hkv;
  for (int x = threadIdx.x; x < rows * np * QG; x += blockDim.x) {
    const int i0 = (x % QG) * 4, rp = x / QG;
    const int pos = p0 + rp % np, bg = rp / np;
    const size_t o = (static_cast<size_t>(bg) * kv.T + pos) * D;
    float x1[4], x2[4];
    SliceLoad<T, 4>::run(K + o + i0, x1);
    SliceLoad<T, 4>::run(K + o + i0 + half, x2);
    const int cc = ((pos - a.n_sink) >> lc) - c0;
    uint32_t lo[2] = {0, 0}, hi[2] = {0, 0};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float y1, y2;
      rope_pair(x1[k], x2[k], cs[cc][i0 + k][0], cs[cc][i0 + k][1], y1, y2);
      lo[k >> 1] |= exact_bf16(y1) << (16 * (k & 1));
      hi[k >> 1] |= exact_bf16(y2) << (16 * (k & 1));
    }
    *reinterpret_cast<uint2*>(ko + o + i0) = make_uint2(lo[0], lo[1]);
    *reinterpret_cast<uint2*>(ko + o + i0 + half) = make_uint2(hi[0], hi[1]);
  }
}

// Key rows of one decode chunk rotated to the chunk's index: lane li holds
// elements li*EPL .. of a row, so its pair partners sit in lane li ^ 8 (one
// DPP rotation of the 16-lane row). The lane's EPL angles are computed once
// per chunk, split between the two lanes of each pair (each takes EPL/2 and
// receives the other half), from the workgroup's table of theta_i. The
// rotation runs in fp64 as in the oracle. (An fp32 evaluation with an fp64
// re-evaluation of the elements near a rounding half-step was slower: the
// re-evaluation reaches about one row in eight per wave.)
template <typename T, int D, bool PAGED, bool TABLE = false>
struct CiRows {
  static constexpr int EPL = D / 16;
  ChunkRows<T, D, PAGED, TABLE> raw;
  double c[EPL], ss[EPL];                       // cos, and sin signed for this lane's half

  __device__ __forceinline__ CiRows(const PruneArgs& a, int stage, int b, int g, int li, int st, const double* theta)
      : raw(a, b, g, li, st, a.chunk[stage]) {
    const double cid = static_cast<double>((st - a.n_sink) >> a.lchunk[stage]);
    const bool first = li < 8;
    const int k0 = first ? 0 : EPL / 2;         // the half of the angles computed here
    double mc[EPL / 2], ms[EPL / 2];
#pragma unroll
    for (int k = 0; k < EPL / 2; ++k) rope_angle(theta[(li & 7) * EPL + k0 + k], cid, mc[k], ms[k]);
#pragma unroll
    for (int k = 0; k < EPL / 2; ++k) {
      const double oc = dpp_perm_d<kDppRowRor8>(mc[k]), os = dpp_perm_d<kDppRowRor8>(ms[k]);
      const double c_lo = first ? mc[k] : oc, s_lo = first ? ms[k] : os;     // angle k
      const double c_hi = first ? oc : mc[k], s_hi = first ? os : ms[k];     // angle EPL/2 + k
      c[k] = c_lo;
      ss[k] = first ? -s_lo : s_lo;
      c[EPL / 2 + k] = c_hi;
      ss[EPL / 2 + k] = first ? -s_hi : s_hi;
    }
  }

  __device__ __forceinline__ RowSlice<T, EPL> at(int pos) const {
    RowSlice<T, EPL> x = raw.at(pos), y;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int w = 0; w < EPL / 2; ++w) {
        const uint32_t mine = x.w[w];
        const uint32_t other = static_cast<uint32_t>(dpp_perm<kDppRowRor8>(static_cast<int>(mine)));
        const float a0 = rope_half(__uint_as_float(mine << 16), __uint_as_float(other << 16), c[2 * w], ss[2 * w]);
        const float a1 = rope_half(__uint_as_float(mine & 0xffff0000u), __uint_as_float(other & 0xffff0000u),
                                   c[2 * w + 1], ss[2 * w + 1]);
        y.w[w] = exact_bf16(a0) | (exact_bf16(a1) << 16);
      }
    } else {
#pragma unroll
      for (int k = 0; k < EPL; ++k) {
        const float other = dpp_perm_f<kDppRowRor8>(x.v[k]);
        y.v[k] = rope_half(x.v[k], other, c[k], ss[k]);
      }
    }
    return y;
  }
};

// Decode scoring of one stage with chunk-indexed RoPE: the plain lane-group
// tournaments on rotated rows, against the stage's rotated queries.
template <typename T, int D, int G, int SPEC, bool PAGED>
__global__ void __launch_bounds__(256, (G > 4 || (G == 4 && sizeof(T) == 4)) ? 2 : 4)
k_score_decode_ci(PruneArgs a, int stage, const uint16_t* q_all, double base) {
  constexpr int EPL = D / 16;
  using Row = RowSlice<T, EPL>;
  __shared__ double theta[D / 2];
  for (int i = threadIdx.x; i < D / 2; i += blockDim.x) theta[i] = rope_theta(base, i, D);
  __syncthreads();
  const KvLayout& kv = a.kv;
  const int r = blockIdx.y, b = r;
  const int tid = threadIdx.x;
  const int gi = tid >> 4, li = tid & 15;
  const DecodeLane dl = decode_lane(a, blockIdx.x, gi);
  const int cpw = dl.cpw, j0 = dl.j0, g = dl.g;  // chunks per workgroup, first chunk, kv head
  const int j = j0 + dl.cl;
  __shared__ float red[16];

  const int e = seq_len_of(kv, r);
  int nc_prev = 0, st;
  if (stage == 0) {
    st = a.n_sink + (j << a.lchunk[0]);
  } else {
    const int sh = a.lchunk[stage - 1] - a.lchunk[stage];
    nc_prev = a.cnt[r * kMaxStages + stage - 1];
    const int32_t* prev = stage_starts(a, stage - 1, r);
    st = prev[min(j >> sh, a.maxK - 1)] + ((j & ((1 << sh) - 1)) << a.lchunk[stage]);
  }
  Row q[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
    load_rotated(q[hh], q_all + (static_cast<size_t>(r) * kv.Hq + g * G + hh) * D + li * EPL);

  const Geo geo = make_geo(e - 1, e, a.n_sink, a.n_window, a.chunk[0]);
  const int nc = stage == 0 ? geo.n1 : nc_prev << (a.lchunk[stage - 1] - a.lchunk[stage]);
  if (nc <= (a.keep[stage] >> a.lchunk[stage])) return;   // stage keeps everything for this row
  if (j0 >= nc) return;
  const bool active = dl.used && j < nc;

  float best = -INFINITY;
  if (active) {
    const CiRows<T, D, PAGED> rows(a, stage, b, g, li, st, theta);
    if (!PAGED || rows.raw.hoist) {
      best = selectrep_group<T, D, G, SPEC>(a, stage, li, st, rows, q);
    } else if constexpr (PAGED) {               // a chunk over more pages: rows through the page table
      const CiRows<T, D, true, true> trows(a, stage, b, g, li, st, theta);
      best = selectrep_group<T, D, G, SPEC>(a, stage, li, st, trows, q);
    }
  }
  if (li == 0) red[gi] = best;
  __syncthreads();
  if (tid < cpw) {
    const int jj = j0 + tid;
    if (jj < nc) {
      float m = red[tid * a.hpw];
      for (int x = 1; x < a.hpw; ++x) m = fmaxf(m, red[tid * a.hpw + x]);
      stage_scores(a, stage, r, dl.sl)[jj] = score_key(m);
    }
  }
}

// ------------------------------------------------------------------------- //
// decode: top-K of one stage fused with the RoPE scoring of the next        //
// ------------------------------------------------------------------------- //
// As k_topk_score_decode (bf16, contiguous K): every workgroup selects the
// row's kept chunks of stage `stage - 1` itself (workgroup 0 also writes the
// kept starts and their count), then scores its chunks of `stage` with the
// tournaments of k_score_decode_rt (KIND relative: qa, qb the rotated query
// sets) or k_score_decode_ci (KIND chunk-indexed: qa the stage's rotated
// queries).
template <int D, int G, int SPEC, int E, int KIND>
__global__ void __launch_bounds__(256, 2)
k_topk_score_decode_rope(PruneArgs a, int stage, const uint16_t* qa, const uint16_t* qb, double base) {
  using T = uint16_t;
  constexpr int EPL = D / 16;
  using Row = RowSlice<T, EPL>;
  __shared__ SelectLds<> L;
  __shared__ int sprev[kMaxKeptChunks];
  __shared__ int ssel[kMaxKeptChunks];
  __shared__ float red[16];
  __shared__ double theta[D / 2];
  const KvLayout& kv = a.kv;
  const int ps = stage - 1;                     // the stage selected here
  const int r = blockIdx.y, b = r;              // one row per sequence
  const int tid = threadIdx.x;
  const int gi = tid >> 4, li = tid & 15;
  const DecodeLane dl = decode_lane(a, blockIdx.x, gi);
  const int cpw = dl.cpw, j0 = dl.j0, g = dl.g;  // chunks per workgroup, first chunk, kv head

  const int e = seq_len_of(kv, r);
  const int nc_before = ps > 0 ? a.cnt[r * kMaxStages + ps - 1] : 0;
  const int js = tid * E;
  uint32_t key[E];
  load_keys<E>(a, ps, r, js, key);
  if (ps > 0) load_kept_starts(a, ps - 1, r, sprev);
  Row qx[G], qy[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const size_t o = (static_cast<size_t>(r) * kv.Hq + g * G + hh) * D + li * EPL;
    load_rotated(qx[hh], qa + o);
    if constexpr (KIND == kRopeRelative) load_rotated(qy[hh], qb + o);
  }
  if constexpr (KIND == kRopeChunkIndexed) {    // published by the selection's barriers
    for (int i = tid; i < D / 2; i += blockDim.x) theta[i] = rope_theta(base, i, D);
  }

  const Geo geo = make_geo(e - 1, e, a.n_sink, a.n_window, a.chunk[0]);
  const int lgp = a.lchunk[ps];
  const int shp = ps > 0 ? a.lchunk[ps - 1] - lgp : 0;
  const int nc_ps = ps == 0 ? geo.n1 : nc_before << shp;
  const int kc_ps = a.keep[ps] >> lgp;
  const int n_sel = nc_ps <= kc_ps ? nc_ps : kc_ps;
  const bool writer = blockIdx.x == 0;
  int32_t* out = stage_starts(a, ps, r);
  select_row<E>(key, js, nc_ps, kc_ps, L, [&](int j, int pos) {
    const int st = ps == 0 ? a.n_sink + (j << lgp) : sprev[j >> shp] + ((j & ((1 << shp) - 1)) << lgp);
    ssel[pos] = st;
    if (writer) out[pos] = st;
  });
  if (writer && tid == 0) record_stage(a, ps, r, n_sel, geo);
  __syncthreads();                              // the kept starts are in ssel

  const int sh = lgp - a.lchunk[stage];
  const int nc = n_sel << sh;
  if (nc <= (a.keep[stage] >> a.lchunk[stage])) return;   // stage keeps everything for this row
  if (j0 >= nc) return;
  const int j = j0 + dl.cl;
  const bool active = dl.used && j < nc;
  const int st = ssel[min(j >> sh, n_sel - 1)] + ((j & ((1 << sh) - 1)) << a.lchunk[stage]);
  float best = -INFINITY;
  if (active) {
    if constexpr (KIND == kRopeRelative) {
      best = score_group_rt<T, D, G, SPEC, false>(a, stage, b, g, li, st, qx, qy);
    } else {
      const CiRows<T, D, false> rows(a, stage, b, g, li, st, theta);
      best = selectrep_group<T, D, G, SPEC, CiRows<T, D, false>, true>(a, stage, li, st, rows, qx);
    }
  }
  if (li == 0) red[gi] = best;
  __syncthreads();
  if (tid < cpw) {
    const int jj = j0 + tid;
    if (jj < nc) {
      float m = red[tid * a.hpw];
      for (int x = 1; x < a.hpw; ++x) m = fmaxf(m, red[tid * a.hpw + x]);
      stage_scores(a, stage, r, dl.sl)[jj] = score_key(m);
    }
  }
}

static const char* const kRopeNames[kMaxStages] = {"prune_rope_score1", "prune_rope_score2", "prune_rope_score3",
                                                   "prune_rope_score4"};
static const char* const kCiQueryNames[kMaxStages] = {"prune_ci_queries1", "prune_ci_queries2", "prune_ci_queries3",
                                                      "prune_ci_queries4"};
static const char* const kRopeFusedNames[kMaxStages] = {"", "prune_topk1_rope_score2", "prune_topk2_rope_score3",
                                                        "prune_topk3_rope_score4"};
static const char* const kCiKeyNames[kMaxStages] = {"prune_ci_keys1", "prune_ci_keys2", "prune_ci_keys3",
                                                    "prune_ci_keys4"};

// Speculative first round of a decode tournament: 8 keys for chunks of 8..64,
// 4 for longer chunks (register budget), none below 8.
static int rope_spec(int l) { return l >= 8 && l <= 64 ? 8 : l > 64 ? 4 : l >= 4 ? 4 : 0; }

template <typename T, int D, int G, bool PAGED>
static void launch_decode_rt(const PruneArgs& a, int stage, int max_chunks, const uint16_t* ql,
                             const uint16_t* qr, hipStream_t st) {
  const int cpw = 16 / a.hpw;
  const dim3 grid((max_chunks + cpw - 1) / cpw * a.nsl, a.R);
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

template <typename T, int D, int G, bool PAGED>
static void launch_decode_ci(const PruneArgs& a, int stage, int max_chunks, const uint16_t* q, double base,
                             hipStream_t st) {
  const int cpw = 16 / a.hpw;
  const dim3 grid((max_chunks + cpw - 1) / cpw * a.nsl, a.R);
  const char* nm = kRopeNames[stage];
  switch (rope_spec(a.chunk[stage])) {
    case 8:  DSA_LAUNCH(nm, (k_score_decode_ci<T, D, G, 8, PAGED>), grid, dim3(256), st, a, stage, q, base); break;
    case 4:  DSA_LAUNCH(nm, (k_score_decode_ci<T, D, G, 4, PAGED>), grid, dim3(256), st, a, stage, q, base); break;
    default: DSA_LAUNCH(nm, (k_score_decode_ci<T, D, G, 0, PAGED>), grid, dim3(256), st, a, stage, q, base); break;
  }
}

template <typename T, int D, int G>
static void launch_decode_ci_g(const PruneArgs& a, int stage, int max_chunks, const uint16_t* q, double base,
                               hipStream_t st) {
  if (a.kv.block_table) launch_decode_ci<T, D, G, true>(a, stage, max_chunks, q, base, st);
  else                  launch_decode_ci<T, D, G, false>(a, stage, max_chunks, q, base, st);
}

constexpr long long kRopeFuseMaxWorkgroups = 2048;   // largest fused top-K + scoring launch

// Top-K of stage - 1 and RoPE scoring of `stage` in one launch (bf16 decode,
// contiguous K, one sequence's worth of workgroups); false if this shape takes
// the separate kernels.
template <typename T, int D, int G>
static bool launch_rope_fused(const PruneArgs& a, int style, int stage, int max_chunks, int sel_chunks,
                              const uint16_t* qa, const uint16_t* qb, double base, hipStream_t st) {
  if constexpr (sizeof(T) != 2) {
    return false;
  } else {
    const int cpw = 16 / a.hpw;
    const dim3 grid(std::max(1, (max_chunks + cpw - 1) / cpw) * a.nsl, a.R);
    if (static_cast<long long>(grid.x) * grid.y > kRopeFuseMaxWorkgroups || a.kv.block_table) return false;
    if (sel_chunks > kTopkThreads * 16) return false;
    const bool e4 = sel_chunks <= kTopkThreads * 4;
    const int spec = rope_spec(a.chunk[stage]);
    const char* nm = kRopeFusedNames[stage];
#define DSA_ROPE_FUSED(SP, EE)                                                                              \
  do {                                                                                                      \
    if (style == kRopeRelative)                                                                             \
      DSA_LAUNCH(nm, (k_topk_score_decode_rope<D, G, SP, EE, kRopeRelative>), grid, dim3(256), st, a, stage, \
                 qa, qb, base);                                                                             \
    else                                                                                                    \
      DSA_LAUNCH(nm, (k_topk_score_decode_rope<D, G, SP, EE, kRopeChunkIndexed>), grid, dim3(256), st, a,    \
                 stage, qa, qb, base);                                                                      \
  } while (0)
    if (spec == 8)      { if (e4) DSA_ROPE_FUSED(8, 4); else DSA_ROPE_FUSED(8, 16); }
    else if (spec == 4) { if (e4) DSA_ROPE_FUSED(4, 4); else DSA_ROPE_FUSED(4, 16); }
    else                { if (e4) DSA_ROPE_FUSED(0, 4); else DSA_ROPE_FUSED(0, 16); }
#undef DSA_ROPE_FUSED
    return true;
  }
}

// Decode: score stage 1; for every later stage, the previous stage's top-K and
// this stage's scoring (fused where possible); the last top-K writes idx. The
// chunk-indexed style rotates the queries to each stage's position ID first.
template <typename T, int D, int G>
static void launch_rope_decode(const PruneArgs& a, int style, uint16_t* qa, uint16_t* qb, double base,
                               hipStream_t st) {
  auto chunks_of = [&](int stage) { return stage == 0 ? a.n1max : a.keep[stage - 1] / a.chunk[stage]; };
  const bool rt = style == kRopeRelative;
  auto score = [&](int stage) {
    if (chunks_of(stage) <= 0) return;
    if (rt) launch_decode_rt_g<T, D, G>(a, stage, chunks_of(stage), qa, qb, st);
    else    launch_decode_ci_g<T, D, G>(a, stage, chunks_of(stage), qa, base, st);
  };
  auto rotate = [&](int stage) {
    if (!rt)
      DSA_LAUNCH(kCiQueryNames[stage], (k_ci_queries<T, D>), dim3(a.R, a.kv.Hq), dim3(256), st, a, stage, qa, base,
                 size_t{0});
  };
  rotate(0);
  score(0);
  for (int stage = 1; stage < a.n_stages; ++stage) {
    rotate(stage);
    if (!launch_rope_fused<T, D, G>(a, style, stage, chunks_of(stage), chunks_of(stage - 1), qa, qb, base, st)) {
      launch_topk(a, stage - 1, chunks_of(stage - 1), st);
      score(stage);
    }
  }
  launch_topk(a, a.n_stages - 1, chunks_of(a.n_stages - 1), st);
}

// Relative style: the queries are rotated once; chunk-indexed: per stage.
// Decode runs launch_rope_decode; prefill scores each stage (relative: the
// matrix-core tournaments for bf16 with 64-query blocks, else the generic
// kernel; chunk-indexed: the plain scoring on rotated copies of the queries
// and keys) and runs the plain top-K.
template <typename T, int D>
static hipError_t launch_rope_typed(const PruneArgs& a, int style, uint16_t* qa, uint16_t* qb, uint16_t* kb,
                                    double base, hipStream_t st) {
  const bool rt = style == kRopeRelative;
  if (rt) DSA_LAUNCH("prune_rope_queries", (k_rope_queries<T, D>), dim3(a.R, a.kv.Hq), dim3(256), st, a, qa, qb, base);
  const int G = a.kv.Hq / a.kv.Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return hipErrorInvalidValue;
  if (a.kv.decode) {
    switch (G) {
      case 1: launch_rope_decode<T, D, 1>(a, style, qa, qb, base, st); break;
      case 2: launch_rope_decode<T, D, 2>(a, style, qa, qb, base, st); break;
      case 4: launch_rope_decode<T, D, 4>(a, style, qa, qb, base, st); break;
      default: launch_rope_decode<T, D, 8>(a, style, qa, qb, base, st); break;
    }
    return hipGetLastError();
  }
  for (int stage = 0; stage < a.n_stages; ++stage) {
    const int max_chunks = stage == 0 ? a.n1max : a.keep[stage - 1] / a.chunk[stage];
    if (max_chunks > 0 && rt) {
      if (!(sizeof(T) == 2 && launch_score_prefill_mfma(a, stage, max_chunks, st, kRopeNames[stage], qa, qb))) {
        DSA_LAUNCH(kRopeNames[stage], (k_score_rope<T, D>), dim3((max_chunks + 15) / 16, a.R), dim3(256), st, a,
                   stage, qa, qb);
      }
    } else if (max_chunks > 0) {
      DSA_LAUNCH(kCiQueryNames[stage], (k_ci_queries<T, D>), dim3(a.R, a.kv.Hq), dim3(256), st, a, stage, qa, base,
                 size_t{0});
      CiKeyOut ko{};
      ko.ko[0] = kb;
      DSA_LAUNCH(kCiKeyNames[stage], (k_ci_keys<T, D>), dim3((a.kv.T + kCiTile - 1) / kCiTile), dim3(256), st, a,
                 stage, ko, base, 0, a.kv.T);
      PruneArgs ar = a;                         // the plain scoring, on the rotated copies
      ar.q = qa;
      ar.k = kb;
      launch_score_prefill_bf16(ar, stage, max_chunks, st, kRopeNames[stage]);
    }
    launch_topk(a, stage, max_chunks, st);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

// Chunk-indexed decode over rotated key copies: the query is rotated to every
// stage's position ID in one launch (stage s at qa + s * qstride), then the
// plain decode kernels run stage by stage on (rotated query, rotated keys of
// that stage).
hipError_t launch_prune_rope_keys(const PruneArgs& a, int dtype, uint16_t* qa, size_t qstride,
                                  uint16_t* const* k_rot, double base, hipStream_t st) {
  if (!a.kv.decode || a.kv.block_table) return hipErrorInvalidValue;
  const dim3 grid(a.R, a.kv.Hq, a.n_stages);
  if (dtype == 1) {
    if (a.kv.D == 128) DSA_LAUNCH("prune_ci_queries", (k_ci_queries<uint16_t, 128>), grid, dim3(256), st, a, 0, qa, base, qstride);
    else               DSA_LAUNCH("prune_ci_queries", (k_ci_queries<uint16_t, 64>), grid, dim3(256), st, a, 0, qa, base, qstride);
  } else {
    if (a.kv.D == 128) DSA_LAUNCH("prune_ci_queries", (k_ci_queries<float, 128>), grid, dim3(256), st, a, 0, qa, base, qstride);
    else               DSA_LAUNCH("prune_ci_queries", (k_ci_queries<float, 64>), grid, dim3(256), st, a, 0, qa, base, qstride);
  }
  PruneArgs as[kMaxStages];
  for (int s = 0; s < a.n_stages; ++s) {
    as[s] = a;
    as[s].q = qa + s * qstride;
    as[s].k = k_rot[s];
  }
  return launch_prune_decode_staged(as, st);
}

// Rotated copies of the keys at positions [p_lo, p_hi) for every stage (the
// chunk-indexed style), contiguous K of a decode shape.
hipError_t launch_rope_rotate_keys(const PruneArgs& a, int dtype, uint16_t* const* k_rot, double base, int p_lo,
                                   int p_hi, hipStream_t st) {
  if (p_hi <= p_lo) return hipSuccess;
  CiKeyOut ko{};
  for (int s = 0; s < a.n_stages; ++s) ko.ko[s] = k_rot[s];
  const dim3 grid((p_hi - p_lo + kCiTile - 1) / kCiTile, a.n_stages);
  if (dtype == 1) {
    if (a.kv.D == 128) DSA_LAUNCH("rope_rotate_keys", (k_ci_keys<uint16_t, 128>), grid, dim3(256), st, a, 0, ko, base, p_lo, p_hi);
    else               DSA_LAUNCH("rope_rotate_keys", (k_ci_keys<uint16_t, 64>), grid, dim3(256), st, a, 0, ko, base, p_lo, p_hi);
  } else {
    if (a.kv.D == 128) DSA_LAUNCH("rope_rotate_keys", (k_ci_keys<float, 128>), grid, dim3(256), st, a, 0, ko, base, p_lo, p_hi);
    else               DSA_LAUNCH("rope_rotate_keys", (k_ci_keys<float, 64>), grid, dim3(256), st, a, 0, ko, base, p_lo, p_hi);
  }
  return hipGetLastError();
}

hipError_t launch_prune_rope(const PruneArgs& a, int dtype, int style, uint16_t* qa, uint16_t* qb, uint16_t* kb,
                             double base, hipStream_t st) {
  if (style != kRopeRelative && style != kRopeChunkIndexed) return hipErrorInvalidValue;
  if (dtype == 1) {
    if (a.kv.D == 128) return launch_rope_typed<uint16_t, 128>(a, style, qa, qb, kb, base, st);
    if (a.kv.D == 64) return launch_rope_typed<uint16_t, 64>(a, style, qa, qb, kb, base, st);
  } else {
    if (a.kv.D == 128) return launch_rope_typed<float, 128>(a, style, qa, qb, kb, base, st);
    if (a.kv.D == 64) return launch_rope_typed<float, 64>(a, style, qa, qb, kb, base, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace dsa
