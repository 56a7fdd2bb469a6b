// Block-sparse index estimation for prefill (MInference page, 2407.02490,
// "Online Dynamic Index Estimation: Block-Sparse Heads (Algorithm 3)"):
//   1. pool : every 64 consecutive query rows and key rows of a head are
//             averaged into one pooled row (fp64);
//   2. score: pooled logits q~_m . k~_j of every query block m against the key
//             blocks j <= m (later key blocks are masked out; the diagonal
//             block stays), in fp64 on the matrix cores, rounded once to fp32.
//             The row softmax and the 1/sqrt(d) scale of the page's block
//             attention are monotone and do not change the ranking, so they
//             are not applied;
//   3. top-k: per (q head, query block) the k_b key blocks with the highest
//             logits (ties to the lower block);
//   4. rows : the kept blocks, ascending, as runs of 64 key positions, then
//             -1 padding. The per-head gathered attention consumes them
//             ("Block-Sparse FlashAttention Kernel (Appendix C.4.1)").
// On grid-valued inputs (multiples of 1/8 in [-1, 1]) the pooled rows are
// multiples of 1/512 and every product and partial sum of the logits is an
// exact fp64 number, so the logits do not depend on the summation order.
#include "topk_select.h"

namespace dsa {

typedef double f64x4_t __attribute__((ext_vector_type(4)));

constexpr int kBsBlock = 64;             // pooling block (the page's block_size)

// ------------------------------------------------------------------------- //
// step 1: mean pooling                                                      //
// ------------------------------------------------------------------------- //
// Workgroup = one 64-row block of one head: blockIdx.x = block, blockIdx.y =
// head over the Hq query heads then the Hkv key heads, blockIdx.z = sequence.
// Each thread sums one 16-byte piece of NP rows in fp64, the partial rows meet
// in LDS and are added in a fixed order.
template <typename T, int D>
__global__ void __launch_bounds__(256) k_bs_pool(BsArgs a) {
  constexpr int EPP = 16 / static_cast<int>(sizeof(T));   // elements per 16-byte piece
  constexpr int PPR = D / EPP;                            // pieces per row
  constexpr int RPI = 256 / PPR;                          // rows per pass
  constexpr int NP = kBsBlock / RPI;                      // passes
  static_assert(RPI * PPR == 256 && NP * RPI == kBsBlock, "pieces must tile the block");
  __shared__ double part[RPI][D + 1];

  const KvLayout& kv = a.kv;
  const int m = blockIdx.x, hh = blockIdx.y, b = blockIdx.z;
  const bool is_q = hh < kv.Hq;
  const int h = is_q ? hh : hh - kv.Hq;
  const int H = is_q ? kv.Hq : kv.Hkv;
  const T* X = static_cast<const T*>(is_q ? a.q : a.k) +
               ((static_cast<size_t>(b) * H + h) * kv.T + static_cast<size_t>(m) * kBsBlock) * D;
  const int tid = threadIdx.x, piece = tid % PPR, rsub = tid / PPR;

  uint4 u[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p)
    u[p] = *reinterpret_cast<const uint4*>(X + static_cast<size_t>(p * RPI + rsub) * D + piece * EPP);
  double acc[EPP];
#pragma unroll
  for (int e = 0; e < EPP; ++e) acc[e] = 0.0;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const uint32_t w[4] = {u[p].x, u[p].y, u[p].z, u[p].w};
#pragma unroll
    for (int e = 0; e < EPP; ++e) {
      float f;
      if constexpr (sizeof(T) == 2) {
        f = __uint_as_float((e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16));
      } else {
        f = __uint_as_float(w[e]);
      }
      acc[e] += static_cast<double>(f);
    }
  }
#pragma unroll
  for (int e = 0; e < EPP; ++e) part[rsub][piece * EPP + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    double s = 0.0;
#pragma unroll
    for (int r = 0; r < RPI; ++r) s += part[r][tid];
    double* out = (is_q ? a.qp : a.kp) + ((static_cast<size_t>(b) * H + h) * kv.nblk + m) * D;
    out[tid] = s * (1.0 / kBsBlock);
  }
}

// ------------------------------------------------------------------------- //
// step 2: block-causal pooled logits on the fp64 matrix cores               //
// ------------------------------------------------------------------------- //
// v_mfma_f64_16x16x4f64: lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16] and receives D[4 * r + l / 16][l % 16] in accumulator r.
// A wave owns 16 query blocks (rows) of one head and sweeps the key blocks 16
// at a time up to the diagonal. The reduction over d is split by lane group:
// lane group kk (= l / 16) feeds d-indices kk * D/4 .. kk * D/4 + D/4 - 1 of
// its row in D/4 successive products, so every lane reads its operands as
// contiguous 16-byte loads. Each wave of a workgroup takes a different query
// head of the same 16 query blocks (heads of one kv group share their key
// operand loads), and workgroups are issued from the last query blocks (the
// longest sweeps) to the first.
template <int D>
__global__ void __launch_bounds__(256) k_bs_scores(BsArgs a, int nmt) {
  constexpr int KQ = D / 4;                      // d-indices per lane group
  const KvLayout& kv = a.kv;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long long unit = static_cast<long long>(blockIdx.x) * 4 + w;
  const int h = static_cast<int>(unit % kv.Hq);
  const long long rest = unit / kv.Hq;
  const int mtr = static_cast<int>(rest % nmt);
  const int b = static_cast<int>(rest / nmt);
  if (b >= kv.B) return;
  const int mt = nmt - 1 - mtr;
  const int g = h / (kv.Hq / kv.Hkv);
  const int nblk = kv.nblk;
  const int i = lane & 15, kk = lane >> 4;

  double av[KQ];
  {
    const int mA = min(16 * mt + i, nblk - 1);   // rows past the last block are computed and dropped
    const double2* src = reinterpret_cast<const double2*>(
        a.qp + ((static_cast<size_t>(b) * kv.Hq + h) * nblk + mA) * D + kk * KQ);
#pragma unroll
    for (int x = 0; x < KQ / 2; ++x) {
      const double2 v = src[x];
      av[2 * x] = v.x;
      av[2 * x + 1] = v.y;
    }
  }
  const double* kbase = a.kp + (static_cast<size_t>(b) * kv.Hkv + g) * nblk * D + kk * KQ;
  uint32_t* krow = a.keys + (static_cast<size_t>(b) * kv.Hq + h) * nblk * static_cast<size_t>(a.nblkp);

  auto load_b = [&](int jt, double (&dst)[KQ]) __attribute__((always_inline)) {
    const int jB = min(16 * jt + i, nblk - 1);
    const double2* src = reinterpret_cast<const double2*>(kbase + static_cast<size_t>(jB) * D);
#pragma unroll
    for (int x = 0; x < KQ / 2; ++x) {
      const double2 v = src[x];
      dst[2 * x] = v.x;
      dst[2 * x + 1] = v.y;
    }
  };
  auto tile = [&](int jt, const double (&bv)[KQ]) __attribute__((always_inline)) {
    f64x4_t acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int s = 0; s < KQ; ++s) acc = __builtin_amdgcn_mfma_f64_16x16x4f64(av[s], bv[s], acc, 0, 0, 0);
    const int j = 16 * jt + i;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 16 * mt + 4 * r + kk;
      if (m < nblk && j <= m) krow[static_cast<size_t>(m) * a.nblkp + j] = score_key(static_cast<float>(acc[r]));
    }
  };
  // two operand buffers in turn: the next key tile loads under this one's products
  double b0[KQ], b1[KQ];
  load_b(0, b0);
  int jt = 0;
  for (; jt + 1 <= mt; jt += 2) {
    load_b(jt + 1, b1);
    tile(jt, b0);
    if (jt + 2 <= mt) load_b(jt + 2, b0);
    tile(jt + 1, b1);
  }
  if (jt == mt) tile(jt, b0);
}

// ------------------------------------------------------------------------- //
// steps 3-4: top-k_b blocks of a row and the index row                      //
// ------------------------------------------------------------------------- //
// One workgroup per row r = (b * Hq + h) * nblk + m; thread t holds the keys
// of blocks t*E .. t*E+E-1. Each kept block writes its own 64 entries.
template <int E>
__global__ void __launch_bounds__(kTopkThreads) k_bs_topk(BsArgs a) {
  __shared__ SelectLds<kTopkWaves> L;
  const int r = blockIdx.x;
  const int m = r % a.kv.nblk;
  const int nc = m + 1, kc = a.k_blocks;
  const int tid = threadIdx.x;
  const int j0 = tid * E;
  uint32_t key[E];
  {
    const uint4* src = reinterpret_cast<const uint4*>(a.keys + static_cast<size_t>(r) * a.nblkp);
    const int nv = (nc + 3) >> 2;                // written groups of four (the rest is masked)
#pragma unroll
    for (int v = 0; v < E / 4; ++v) {
      const uint4 u = src[min((j0 >> 2) + v, nv - 1)];
      key[4 * v + 0] = u.x; key[4 * v + 1] = u.y; key[4 * v + 2] = u.z; key[4 * v + 3] = u.w;
    }
  }
  if (a.lblk) {                                  // block lists: the ids, then -1
    int32_t* lb = a.lblk + static_cast<size_t>(r) * a.wb;
    select_row<E>(key, j0, nc, kc, L, [&](int j, int pos) { lb[pos] = j; });
    const int n_sel = min(nc, kc);
    for (int x = n_sel + tid; x < a.wb; x += kTopkThreads) lb[x] = -1;
    if (tid == 0) {
      a.lcnt[2 * static_cast<size_t>(r)] = n_sel;
      a.lcnt[2 * static_cast<size_t>(r) + 1] = 0;
    }
    return;
  }
  int32_t* row = a.idx + static_cast<size_t>(r) * a.L;
  select_row<E>(key, j0, nc, kc, L, [&](int j, int pos) {
    int4* dst = reinterpret_cast<int4*>(row + pos * kBsBlock);
    const int p0 = j * kBsBlock;
#pragma unroll
    for (int x = 0; x < kBsBlock / 4; ++x) dst[x] = make_int4(p0 + 4 * x, p0 + 4 * x + 1, p0 + 4 * x + 2, p0 + 4 * x + 3);
  });
  const int n_sel = min(nc, kc);
  int4* pad = reinterpret_cast<int4*>(row);
  for (int x = n_sel * (kBsBlock / 4) + tid; x < a.L / 4; x += kTopkThreads) pad[x] = make_int4(-1, -1, -1, -1);
}

// ------------------------------------------------------------------------- //
// launcher                                                                  //
// ------------------------------------------------------------------------- //
template <typename T, int D>
static void launch_bs_typed(const BsArgs& a, hipStream_t st) {
  const KvLayout& kv = a.kv;
  DSA_LAUNCH("bs_pool", (k_bs_pool<T, D>), dim3(kv.nblk, kv.Hq + kv.Hkv, kv.B), dim3(256), st, a);
  const int nmt = (kv.nblk + 15) / 16;
  const long long units = static_cast<long long>(kv.B) * nmt * kv.Hq;
  DSA_LAUNCH("bs_scores", (k_bs_scores<D>), dim3(static_cast<unsigned>((units + 3) / 4)), dim3(256), st, a, nmt);
  const dim3 grid(static_cast<unsigned>(static_cast<long long>(kv.B) * kv.Hq * kv.nblk));
  const int per = (kv.nblk + kTopkThreads - 1) / kTopkThreads;
  const char* nm = a.lblk ? "bs_topk_lists" : "bs_topk";
  if (per <= 4)       DSA_LAUNCH(nm, (k_bs_topk<4>), grid, dim3(kTopkThreads), st, a);
  else if (per <= 8)  DSA_LAUNCH(nm, (k_bs_topk<8>), grid, dim3(kTopkThreads), st, a);
  else if (per <= 16) DSA_LAUNCH(nm, (k_bs_topk<16>), grid, dim3(kTopkThreads), st, a);
  else if (per <= 32) DSA_LAUNCH(nm, (k_bs_topk<32>), grid, dim3(kTopkThreads), st, a);
  else                DSA_LAUNCH(nm, (k_bs_topk<64>), grid, dim3(kTopkThreads), st, a);
}

// Blocks per row are validated by the caller (at most 64 * kTopkThreads).
hipError_t launch_block_sparse(const BsArgs& a, int dtype, hipStream_t st) {
  if (dtype == 1) {
    if (a.kv.D == 128) launch_bs_typed<uint16_t, 128>(a, st);
    else               launch_bs_typed<uint16_t, 64>(a, st);
  } else {
    if (a.kv.D == 128) launch_bs_typed<float, 128>(a, st);
    else               launch_bs_typed<float, 64>(a, st);
  }
  return hipGetLastError();
}

}  // namespace dsa
