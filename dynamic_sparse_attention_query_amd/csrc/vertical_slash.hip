// Vertical-slash index estimation for prefill (MInference page, 2407.02490,
// "Online Dynamic Index Estimation: Vertical-Slash Heads (Algorithm 2)" and
// the index building of "Vertical-Slash Hybrid Kernel (Appendix C.4.2)"),
// bf16 inputs, one query head at a time (keys of kv head h / G):
//   stats : for the last 64 queries of the sequence (query i at position
//           T - 64 + i, causal), the row max and the sum of exp(z - max) of
//           z = q.k / sqrt(d) over key ranges, then combined per row;
//   sums  : A = exp(z - max) / sum for the 64 x T causal block, summed over
//           the queries per key column (vertical) and per offset d = query
//           position - key position (slash). A workgroup owns 128 columns
//           and the 128 offsets at the same distances from the last query,
//           holds the 64 x 191 block of A they need in LDS, and adds each sum
//           in query order: every sum comes from one workgroup, deterministic;
//   top-k : the k_v largest column sums and the k_s largest offset sums
//           (rounded once to fp32, ties to the lower index), by segments of
//           16,384 candidates whose survivors are selected again;
//   rows  : per query block m, every kept offset's key range [64m - d,
//           64m + 63 - d] is rounded out to the 64-aligned key blocks it
//           touches (attended whole), kept columns before the block's end
//           outside those blocks are attended singly; ascending, -1 padded.
// The dot products are bf16 matrix products accumulated in fp32 (exact on
// the input grid); everything after them is fp64.
#include "topk_select.h"
#include "vs_internal.h"

namespace dsa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kVsTopkE = 16;          // keys per thread of a selection segment
constexpr int kVsTopkThreads = 1024;
constexpr int kVsSeg = kVsTopkE * kVsTopkThreads;
constexpr int kVsMaxBlocks = 16384;   // query blocks per sequence (T <= 1,048,576)

// Q^T fragments (B operand) of estimation queries qt*32 .. qt*32+31 of head h.
template <int D>
__device__ __forceinline__ void vs_qfrag(const VsArgs& a, int b, int h, int qt, int lane, bf16x8_t (&qf)[D / 16]) {
  const KvLayout& kv = a.kv;
  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* qr = Q + ((static_cast<size_t>(b) * kv.Hq + h) * kv.T + kv.T - kVsLastQ + qt * 32 + (lane & 31)) * D +
                       (lane >> 5) * 8;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) qf[ks] = *reinterpret_cast<const bf16x8_t*>(qr + ks * 16);
}

// S^T tile of keys j0 .. j0+31 (rows) against 32 estimation queries
// (columns): lane l holds query column l % 32, accumulator 4rn + c is key
// j0 + 8rn + 4(l / 32) + c. Keys outside [0, T) read as zero.
template <int D>
__device__ __forceinline__ f32x16_t vs_tile(const uint16_t* Kg, int T, const bf16x8_t (&qf)[D / 16], int j0, int lane) {
  const int j = j0 + (lane & 31);
  const bool in = j >= 0 && j < T;
  const uint16_t* kr = Kg + static_cast<size_t>(in ? j : 0) * D + (lane >> 5) * 8;
  f32x16_t acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(kr + ks * 16);
    if (!in) af = bf16x8_t{};
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[ks], acc, 0, 0, 0);
  }
  return acc;
}

__device__ __forceinline__ int vs_tile_key(int j0, int lane, int e) {
  return j0 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
}

// Row max and exp sum of every estimation query over keys [r * 256, r * 256 + 256).
template <int D>
__global__ void __launch_bounds__(256) k_vs_stats(VsArgs a) {
  const KvLayout& kv = a.kv;
  const int r = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = kv.Hq / kv.Hkv;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int T = kv.T;
  const uint16_t* Kg = static_cast<const uint16_t*>(a.k) + (static_cast<size_t>(b) * kv.Hkv + g) * T * D;
  for (int u = w; u < 2 * G; u += 4) {            // (head, query tile) pairs
    const int h = g * G + (u >> 1), qt = u & 1;
    bf16x8_t qf[D / 16];
    vs_qfrag<D>(a, b, h, qt, lane, qf);
    const int i = qt * 32 + (lane & 31);
    const int ti = T - kVsLastQ + i;
    double m = -INFINITY, z = 0.0;
    for (int kt = 0; kt < kVsRange / 32; ++kt) {
      const int j0 = r * kVsRange + kt * 32;
      if (j0 >= T) break;
      const f32x16_t S = vs_tile<D>(Kg, T, qf, j0, lane);
      double tm = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (vs_tile_key(j0, lane, e) <= ti) tm = fmax(tm, static_cast<double>(S[e]) * a.scale);
      if (tm > m) {
        z *= exp(m - tm);
        m = tm;
      }
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (vs_tile_key(j0, lane, e) <= ti) z += exp(static_cast<double>(S[e]) * a.scale - m);
    }
    const double m2 = __shfl_xor(m, 32, 64), z2 = __shfl_xor(z, 32, 64);
    const double M = fmax(m, m2);
    double Z = 0.0;
    if (M > -INFINITY) Z = (m > -INFINITY ? z * exp(m - M) : 0.0) + (m2 > -INFINITY ? z2 * exp(m2 - M) : 0.0);
    if (lane < 32) {
      double* p = a.part + ((static_cast<size_t>(b * kv.Hq + h) * a.nr + r) * kVsLastQ + i) * 2;
      p[0] = M;
      p[1] = Z;
    }
  }
}

// Per (sequence, head, estimation query): the ranges' maxima and sums combined in range order.
__global__ void __launch_bounds__(64) k_vs_combine(VsArgs a) {
  const int bh = blockIdx.x, i = threadIdx.x;
  const double* p = a.part + (static_cast<size_t>(bh) * a.nr * kVsLastQ + i) * 2;
  double M = -INFINITY;
  for (int r = 0; r < a.nr; ++r) M = fmax(M, p[static_cast<size_t>(r) * kVsLastQ * 2]);
  double Z = 0.0;
  for (int r = 0; r < a.nr; ++r) {
    const double mr = p[static_cast<size_t>(r) * kVsLastQ * 2];
    if (mr > -INFINITY) Z += p[static_cast<size_t>(r) * kVsLastQ * 2 + 1] * exp(mr - M);
  }
  double* s = a.stat + (static_cast<size_t>(bh) * kVsLastQ + i) * 2;
  s[0] = M;
  s[1] = Z;
}

// Column sums of keys [T - d0 - 128, T - d0) and offset sums of d in [d0, d0 + 128).
template <int D>
__global__ void __launch_bounds__(256) k_vs_sums(VsArgs a) {
  constexpr int WK = kVsWin + 64;                 // window keys (191 used)
  constexpr int NKT = WK / 32;
  __shared__ double A[kVsLastQ][WK + 1];
  const KvLayout& kv = a.kv;
  const int wi = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = kv.Hq / kv.Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = kv.T;
  const int d0 = wi * kVsWin;
  const int ws = T - (kVsLastQ - 1) - d0 - kVsWin;   // first window key
  const uint16_t* Kg = static_cast<const uint16_t*>(a.k) + (static_cast<size_t>(b) * kv.Hkv + g) * T * D;
  for (int hh = 0; hh < G; ++hh) {
    const int h = g * G + hh;
    const int bh = b * kv.Hq + h;
    for (int u = w; u < 2 * NKT; u += 4) {        // (key tile, query tile) pairs
      const int kt = u >> 1, qt = u & 1;
      bf16x8_t qf[D / 16];
      vs_qfrag<D>(a, b, h, qt, lane, qf);
      const int j0 = ws + kt * 32;
      const f32x16_t S = vs_tile<D>(Kg, T, qf, j0, lane);
      const int i = qt * 32 + (lane & 31);
      const int ti = T - kVsLastQ + i;
      const double M = a.stat[(static_cast<size_t>(bh) * kVsLastQ + i) * 2];
      const double Z = a.stat[(static_cast<size_t>(bh) * kVsLastQ + i) * 2 + 1];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int j = vs_tile_key(j0, lane, e);
        A[i][j - ws] = (j >= 0 && j <= ti) ? exp(static_cast<double>(S[e]) * a.scale - M) / Z : 0.0;
      }
    }
    __syncthreads();
    if (tid < kVsWin) {                           // column j, query order
      const int j = T - d0 - kVsWin + tid;
      if (j >= 0) {
        double s = 0.0;
        for (int i = 0; i < kVsLastQ; ++i) s += A[i][j - ws];
        a.sums[(static_cast<size_t>(bh) * 2) * T + j] = score_key(static_cast<float>(s));
      }
    } else {                                      // offset d, query order
      const int dd = tid - kVsWin, d = d0 + dd;
      if (d < T) {
        double s = 0.0;
        for (int i = 0; i < kVsLastQ; ++i)
          if (T - kVsLastQ + i - d >= 0) s += A[i][kVsWin - 1 - dd + i];
        a.sums[(static_cast<size_t>(bh) * 2 + 1) * T + d] = score_key(static_cast<float>(s));
      }
    }
    __syncthreads();
  }
}

// One selection level: segment blockIdx.x of the column (which = 0) or
// offset (which = 1) candidates of head bh = blockIdx.y / 2 keeps its top
// keep[which]; survivors are written compactly in index order (every segment
// but the last holds exactly min(keep, segment) of them), or, at the last
// level, their indices go to sel[which].
__global__ void __launch_bounds__(kVsTopkThreads) k_vs_topk(VsArgs a, int from_sums, int sb, int db, int n0, int n1,
                                                          int last) {
  __shared__ SelectLds<kVsTopkThreads / 64> L;
  const KvLayout& kv = a.kv;
  const int sel = blockIdx.y, which = sel & 1, bh = sel >> 1;
  const int n = which ? n1 : n0;
  const int k = a.keep[which];
  const int seg = blockIdx.x;
  if (k <= 0 || seg * kVsSeg >= n) return;
  const int seg_n = min(kVsSeg, n - seg * kVsSeg);
  const size_t base = static_cast<size_t>(sel) * kv.T + static_cast<size_t>(seg) * kVsSeg;
  const uint32_t* skey = from_sums ? a.sums + base : a.ckey[sb] + base;
  const int32_t* sidx = from_sums ? nullptr : a.cidx[sb] + base;
  const int j0 = threadIdx.x * kVsTopkE;
  uint32_t key[kVsTopkE];
#pragma unroll
  for (int v = 0; v < kVsTopkE / 4; ++v) {
    const int j = j0 + 4 * v;
    uint4 u = make_uint4(0u, 0u, 0u, 0u);
    if (j + 4 <= seg_n) {
      u = *reinterpret_cast<const uint4*>(skey + j);
    } else {
      if (j + 0 < seg_n) u.x = skey[j + 0];
      if (j + 1 < seg_n) u.y = skey[j + 1];
      if (j + 2 < seg_n) u.z = skey[j + 2];
    }
    key[4 * v + 0] = u.x; key[4 * v + 1] = u.y; key[4 * v + 2] = u.z; key[4 * v + 3] = u.w;
  }
  const size_t obase = static_cast<size_t>(sel) * kv.T + static_cast<size_t>(seg) * min(k, kVsSeg);
  select_row<kVsTopkE, kVsTopkThreads>(key, j0, seg_n, k, L, [&](int j, int pos) {
    const int id = from_sums ? seg * kVsSeg + j : sidx[j];
    if (last) {
      a.sel[which][static_cast<size_t>(bh) * k + pos] = id;
    } else {
      a.ckey[db][obase + pos] = skey[j];
      a.cidx[db][obase + pos] = id;
    }
  });
}

// Exclusive prefix sum over the 256 threads of a workgroup; *total gets the sum.
__device__ __forceinline__ int block_excl_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int inc = static_cast<int>(wave_incl_scan_u32(static_cast<uint32_t>(v)));
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < w) before += wsum[i];
    all += wsum[i];
  }
  *total = all;
  __syncthreads();
  return before + inc - v;
}

// The index row of (sequence, head, query block m).
__global__ void __launch_bounds__(256) k_vs_rows(VsArgs a) {
  __shared__ uint32_t bits[kVsMaxBlocks / 32];
  __shared__ int wpre[kVsMaxBlocks / 32 + 1];
  __shared__ int kept[kVsMaxKeep];
  __shared__ int wsum[4];
  const KvLayout& kv = a.kv;
  const int m = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int bh = b * kv.Hq + h;
  const int tid = threadIdx.x;
  const int s = 64 * m, e = s + 64;
  const int nw = (m + 1 + 31) / 32;               // bitmap words of key blocks 0..m
  for (int x = tid; x < nw; x += 256) bits[x] = 0u;
  __syncthreads();
  const int ks = a.keep[1], kvn = a.keep[0];
  const int32_t* offs = a.sel[1] + static_cast<size_t>(bh) * ks;
  for (int x = tid; x < ks; x += 256) {
    const int d = offs[x];
    const int lo = max(0, s - d), hi = e - 1 - d;
    if (hi >= 0) {
      atomicOr(&bits[(lo >> 6) >> 5], 1u << ((lo >> 6) & 31));
      atomicOr(&bits[(hi >> 6) >> 5], 1u << ((hi >> 6) & 31));
    }
  }
  __syncthreads();
  auto marked = [&](int blk) { return (bits[blk >> 5] >> (blk & 31)) & 1u; };
  // kept columns: before the block's end and in no attended block, in order
  const int32_t* cols = a.sel[0] + static_cast<size_t>(bh) * kvn;
  const int per = (kvn + 255) / 256;
  const int c0 = tid * per;
  int cnt = 0;
  for (int x = c0; x < min(c0 + per, kvn); ++x) {
    const int v = cols[x];
    cnt += (v < e && !marked(v >> 6)) ? 1 : 0;
  }
  int nc;
  int pos = block_excl_scan(cnt, wsum, &nc);
  for (int x = c0; x < min(c0 + per, kvn); ++x) {
    const int v = cols[x];
    if (v < e && !marked(v >> 6)) kept[pos++] = v;
  }
  // attended blocks before each bitmap word
  const int wpt = (nw + 255) / 256;
  int pc = 0;
  for (int x = tid * wpt; x < min(tid * wpt + wpt, nw); ++x) pc += __popc(bits[x]);
  int nb;
  int wp = block_excl_scan(pc, wsum, &nb);
  for (int x = tid * wpt; x < min(tid * wpt + wpt, nw); ++x) {
    wpre[x] = wp;
    wp += __popc(bits[x]);
  }
  __syncthreads();
  if (a.lblk) {
    // the hybrid kernel's two lists: the marked blocks ascending (each
    // thread its bitmap words, from the block count before them), then the
    // kept columns, each -1 padded
    const size_t rr = static_cast<size_t>(bh) * kv.nblk + m;
    int32_t* lb = a.lblk + rr * a.wb;
    for (int x = tid * wpt; x < min(tid * wpt + wpt, nw); ++x) {
      int r = wpre[x];
      for (uint32_t word = bits[x]; word != 0u; word &= word - 1u) lb[r++] = 32 * x + __ffs(static_cast<int>(word)) - 1;
    }
    for (int i = nb + tid; i < a.wb; i += 256) lb[i] = -1;
    int32_t* lc = a.lcol + rr * a.wc;
    for (int c = tid; c < nc; c += 256) lc[c] = kept[c];
    for (int i = nc + tid; i < a.wc; i += 256) lc[i] = -1;
    if (tid == 0) {
      a.lcnt[2 * rr] = nb;
      a.lcnt[2 * rr + 1] = nc;
    }
    return;
  }
  auto rank = [&](int blk) { return wpre[blk >> 5] + __popc(bits[blk >> 5] & ((1u << (blk & 31)) - 1u)); };
  int32_t* row = a.idx + (static_cast<size_t>(bh) * kv.nblk + m) * a.L;
  // each attended block is written by one wave, one entry per lane; a wave
  // walks every fourth bitmap word and visits only its set bits
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int x = w; x < nw; x += 4) {
    const uint32_t word = bits[x];
    if (word == 0u) continue;
    // lane l < 32 finds the kept columns before block 32x + l (all at once)
    int lo = 0;
    if (lane < 32 && ((word >> lane) & 1u)) {
      int hi = nc;
      const int key = 64 * (32 * x + lane);
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (kept[mid] < key) lo = mid + 1; else hi = mid;
      }
    }
    int r = wpre[x];
    for (uint32_t rest = word; rest != 0u; rest &= rest - 1u) {
      const int l = __ffs(static_cast<int>(rest)) - 1;
      const int blk = 32 * x + l;
      const int before = __builtin_amdgcn_readlane(lo, l);
      row[64 * r + before + lane] = 64 * blk + lane;
      ++r;
    }
  }
  for (int c = tid; c < nc; c += 256) {
    const int v = kept[c];
    row[64 * rank(v >> 6) + c] = v;
  }
  // padding: single entries up to a multiple of 4, then 16-byte stores (L is a multiple of 64)
  const int n_ent = 64 * nb + nc;
  const int a4 = min((n_ent + 3) & ~3, a.L);
  if (tid < a4 - n_ent) row[n_ent + tid] = -1;
  int4* row4 = reinterpret_cast<int4*>(row);
  for (int x = (a4 >> 2) + tid; x < (a.L >> 2); x += 256) row4[x] = make_int4(-1, -1, -1, -1);
}

template <int D>
static void launch_vs_typed(const VsArgs& a, hipStream_t st) {
  const KvLayout& kv = a.kv;
  DSA_LAUNCH("vs_stats", (k_vs_stats<D>), dim3(a.nr, kv.Hkv, kv.B), dim3(256), st, a);
  DSA_LAUNCH("vs_combine", k_vs_combine, dim3(kv.B * kv.Hq), dim3(kVsLastQ), st, a);
  DSA_LAUNCH("vs_sums", (k_vs_sums<D>), dim3((kv.T + kVsWin - 1) / kVsWin, kv.Hkv, kv.B), dim3(256), st, a);
  // selection levels until every candidate list fits one segment
  int n[2] = {kv.T, kv.T};
  int src = -1, dst = 0;
  for (;;) {
    const bool last = n[0] <= kVsSeg && n[1] <= kVsSeg;
    const int nseg = (max(n[0], n[1]) + kVsSeg - 1) / kVsSeg;
    DSA_LAUNCH("vs_topk", k_vs_topk, dim3(nseg, 2 * kv.B * kv.Hq), dim3(kVsTopkThreads), st, a, src < 0 ? 1 : 0,
               src < 0 ? 0 : src, dst, n[0], n[1], last ? 1 : 0);
    if (last) break;
    for (int w = 0; w < 2; ++w) {
      const int k = a.keep[w];
      const int full = n[w] / kVsSeg, rest = n[w] - full * kVsSeg;
      n[w] = full * min(k, kVsSeg) + min(k, rest);
    }
    src = dst;
    dst ^= 1;
  }
  DSA_LAUNCH(a.lblk ? "vs_lists" : "vs_rows", k_vs_rows, dim3(kv.nblk, kv.Hq, kv.B), dim3(256), st, a);
}

// bf16, d in {64, 128}, T a multiple of 64 up to 64 * 16384; keep[] <= 8192
// (validated by the caller).
hipError_t launch_vertical_slash(const VsArgs& a, hipStream_t st) {
  if (a.kv.D == 128) launch_vs_typed<128>(a, st);
  else launch_vs_typed<64>(a, st);
  return hipGetLastError();
}

}  // namespace dsa
