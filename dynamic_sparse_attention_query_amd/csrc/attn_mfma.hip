// Prefill attention over gathered key tiles on the bf16 matrix cores (gfx950
// v_mfma_f32_32x32x16_bf16), "similar to FlashAttention" as the InfiniteHiP
// page describes its prefill kernel ("Block Sparse Attention Implementation").
// The key tiles are gathered through the index row as the MInference page's
// permutation-gather (PIT) idea does: non-contiguous keys are packed into a
// dense tile in LDS, then dense matrix products run on the tile.
//
// A workgroup owns one query block of 64 (or half of it) and the query heads
// of one GQA group; each wave computes 32 queries of one head, and the waves
// share the group's K/V tiles in LDS.
//   S^T = K Q^T  (32x32 tiles: rows = keys, columns = queries), so each lane
//                owns whole query columns and the row softmax needs a single
//                exchange between the two half-waves;
//   O^T += V^T P^T, with P^T taken straight from the S^T accumulators: the
//                keys of a 16-key step are permuted identically in both
//                operands (V^T is staged transposed in LDS to allow it).
// Online softmax in base 2 (scale folded into log2 e); causal and padding
// masks are applied only on tiles that need them.
#include "dsa_internal.h"

#include <type_traits>

namespace dsa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef i16x4_t __attribute__((address_space(3))) lds_i16x4_t;

// ds_read_b64_tr_b16: within each 16-lane group, lane 4a+c receives element c
// of the 64-bit words addressed by lanes a, a+4, a+8, a+12 (in that order).
// With lane s addressing row (s >> 2) at column 4 * (s & 3) of a row-major
// 16-bit tile, lane i of the group therefore receives column i of 4
// consecutive rows: a transposed read.
__device__ __forceinline__ i16x4_t lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));
}

// two floats to packed bf16 (round to nearest even) in one conversion
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// the sum of the two bf16 values of a packed pair, in fp32. Plain adds: the
// bf16 dot-product instruction waits for the matrix core while another wave
// of the SIMD issues products, the adds run beside them.
__device__ __forceinline__ float bf16_pair_sum(uint32_t pw) {
  return __uint_as_float(pw << 16) + __uint_as_float(pw & 0xffff0000u);
}

// Workgroup = NH heads of one GQA group x QH query halves (32 queries each),
// one wave per (head, half): 4 waves for every group size. Each wave keeps its
// 32 queries' fragments and its O^T accumulators in registers, so a workgroup
// needs only the two key tiles in LDS and two workgroups share a CU; their
// independent barriers let one workgroup's matrix products overlap the
// other's softmax. K and V rows are fetched whole-row per load (coalesced)
// and staged row-major; the V^T operand is read with LDS transpose reads. The
// two tiles in flight use alternating LDS buffers.
template <int D, int NH, int QH>
__global__ void __launch_bounds__(64 * NH * QH) k_prefill_mfma(AttnArgs a) {
  constexpr int NWV = NH * QH;        // waves
  constexpr int NT = 64 * NWV;        // threads
  constexpr int KS = D / 16;          // 16-wide steps over d
  constexpr int DT = D / 32;          // 32-row tiles of O^T
  constexpr int PPR = D / 8;          // 16-byte pieces per key row
  constexpr int KROW = D + 8;         // K tile row stride (bf16 elements)
  constexpr int VROW = D + 32;        // V tile row stride: the 4 rows x 2 groups of a transpose read hit 64 distinct banks
  constexpr int KPER = 64 * PPR / NT; // K (and V) pieces per thread per tile
  static_assert(KPER >= 1 && (64 * PPR) % NT == 0, "tile loads must split evenly");
  // two tile buffers: tile i is computed from one while tile i+1 is written
  // to the other, so one barrier per tile separates the phases
  __shared__ __align__(16) uint16_t sk[2][64 * KROW];
  __shared__ __align__(16) uint16_t sv[2][64 * VROW];
  __shared__ __align__(16) int spos[2][64];
  __shared__ int sneed[2][NWV], sany[2][NWV];

  const KvLayout& kv = a.kv;
  // XCD-aware order: consecutive workgroup ids go to different XCDs, so give
  // each XCD a contiguous run of work (both halves of a query block and the
  // neighbouring blocks of one kv head share most window keys in that L2).
  const int G = kv.Hq / kv.Hkv;
  const int HG = G / NH;                          // head groups per kv head
  constexpr int NQS = 2 / QH;                     // query-half splits across workgroups
  const int nwork = kv.B * kv.Hkv * HG * kv.nblk * NQS;
  int qsplit, m, hg, b;
  if (a.row_heads) {
    // Per-head rows gather different keys for every head, so reuse comes from
    // the last-level cache: the whole grid walks one kv head at a time (its
    // K and V stay resident there) and deals neighbouring work to all XCDs.
    int work = blockIdx.x;
    if (work >= nwork) return;
    const int hw = work % HG;
    work /= HG;
    m = work % kv.nblk;
    work /= kv.nblk;
    hg = (work % kv.Hkv) * HG + hw;
    b = work / kv.Hkv;
    qsplit = 0;
  } else {
    const int per_xcd = gridDim.x >> 3;
    int work = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (work >= nwork) return;
    qsplit = work % NQS;
    work /= NQS;
    m = work % kv.nblk;
    work /= kv.nblk;
    hg = work % (kv.Hkv * HG);
    b = work / (kv.Hkv * HG);
  }
  const int g = hg / HG;
  const int s = m * 64, e = s + 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  // transpose-read addressing of this lane: row (lane & 15) >> 2, column
  // 4 * (lane & 3) within its 16-lane group, groups 1 and 3 on d-rows 16..31
  const int tr_row = (lane & 15) >> 2, tr_col = ((lane >> 4) & 1) * 16 + 4 * (lane & 3);
  const int hw = w % NH, qg = w / NH;
  const int h = g * G + (hg % HG) * NH + hw;
  const int q0 = s + (qsplit * QH + qg) * 32;     // this wave's first query
  const int wq_lo = s + qsplit * QH * 32;         // the workgroup's query range
  const int wq_hi = wq_lo + QH * 32 - 1;
  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* K = static_cast<const uint16_t*>(a.k);
  const uint16_t* V = static_cast<const uint16_t*>(a.v);
  const size_t kvbase = (static_cast<size_t>(b) * kv.Hkv + g) * kv.T;

  // B operand fragments of Q^T: lane holds 8 consecutive d of one query row
  bf16x8_t qf[KS];
  {
    const uint16_t* qrow = Q + ((static_cast<size_t>(b) * kv.Hq + h) * kv.T + q0 + l32) * D + hi * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8_t*>(qrow + ks * 16);
  }
  f32x16_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
  float mrun = kNegBig, lrun = 0.f;

  // with per-head rows the workgroup holds a single head (NH == 1)
  const int r = a.row_heads ? (b * kv.Hq + h) * kv.nblk + m : b * kv.nblk + m;
  const int32_t* row = a.idx ? a.idx + static_cast<size_t>(r) * a.L : nullptr;
  const int n_ent = row ? a.L : e;
  const int n_tiles = (n_ent + 63) / 64;

  // row entry i as a key position visible to some query of the workgroup,
  // else -1
  auto entry = [&](int i) {
    int p = -1;
    if (i < n_ent) {
      p = row ? row[i] : i;
      if (p < 0 || p > wq_hi) p = -1;
    }
    return p;
  };
  // loader view: piece u covers (row, 16-byte piece), PPR lanes per row
  auto krow_of = [&](int u) { return (u * NT + tid) / PPR; };
  auto kpiece_of = [&](int u) { return (u * NT + tid) % PPR; };

  int pk[KPER], pkn[KPER];
  u32x4_t kreg[KPER], vreg[KPER];
  // registers -> tile buffer `bi`, with the tile's mask / visibility flags
#define DSA_STAGE_TILE(bi)                                                                          \
  do {                                                                                              \
    bool need_ = false, any_ = false;                                                               \
    _Pragma("unroll") for (int u = 0; u < KPER; ++u) {                                              \
      const int p_ = pk[u];                                                                         \
      need_ |= (p_ < 0 || p_ > wq_lo);                                                              \
      any_ |= (p_ >= 0);                                                                            \
      if (kpiece_of(u) == 0) spos[bi][krow_of(u)] = p_;                                             \
      const u32x4_t zero_ = {0u, 0u, 0u, 0u};                                                       \
      *reinterpret_cast<u32x4_t*>(sk[bi] + krow_of(u) * KROW + kpiece_of(u) * 8) =                  \
          p_ >= 0 ? kreg[u] : zero_;                                                                \
      *reinterpret_cast<u32x4_t*>(sv[bi] + krow_of(u) * VROW + kpiece_of(u) * 8) =                  \
          p_ >= 0 ? vreg[u] : zero_;                                                                \
    }                                                                                               \
    const unsigned long long nb_ = __ballot(need_), ab_ = __ballot(any_);                           \
    if (lane == 0) { sneed[bi][w] = nb_ != 0; sany[bi][w] = ab_ != 0; }                             \
  } while (0)
  // issue the loads of the tile whose positions are in pk / pv
#define DSA_LOAD_TILE()                                                                             \
  do {                                                                                              \
    _Pragma("unroll") for (int u = 0; u < KPER; ++u) {                                              \
      const size_t off_ = (kvbase + max(pk[u], 0)) * D + kpiece_of(u) * 8;                          \
      kreg[u] = *reinterpret_cast<const u32x4_t*>(K + off_);                                        \
      vreg[u] = *reinterpret_cast<const u32x4_t*>(V + off_);                                        \
    }                                                                                               \
  } while (0)

  // prologue: tile 0 staged in buffer 0, tile 1 in flight, positions of tile 2
#pragma unroll
  for (int u = 0; u < KPER; ++u) { pk[u] = entry(krow_of(u)); pkn[u] = entry(64 + krow_of(u)); }
  DSA_LOAD_TILE();
  DSA_STAGE_TILE(0);
#pragma unroll
  for (int u = 0; u < KPER; ++u) { pk[u] = pkn[u]; pkn[u] = entry(128 + krow_of(u)); }
  if (n_tiles > 1) DSA_LOAD_TILE();
  __syncthreads();

  for (int ti = 0; ti < n_tiles; ++ti) {
    const int cur = ti & 1;
    int flag = 2;
#pragma unroll
    for (int i = 0; i < NWV; ++i) {
      flag |= sneed[cur][i] ? 1 : 0;
      if (sany[cur][i]) flag &= ~2;
    }
    flag = __builtin_amdgcn_readfirstlane(flag);   // uniform: scalar branches below
    if (!(flag & 2)) {
      const uint16_t* skc = sk[cur];
      const uint16_t* svc = sv[cur];
      // S^T tiles [key tile kt]: 32 keys x this wave's 32 queries
      f32x16_t sacc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kt][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const bf16x8_t af =
              *reinterpret_cast<const bf16x8_t*>(skc + (kt * 32 + l32) * KROW + ks * 16 + hi * 8);
          sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[ks], sacc[kt], 0, 0, 0);
        }
      }
      // causal / padding mask: this lane's keys are 4 runs of 4 per key tile
      if (flag & 1) {
        const unsigned t = static_cast<unsigned>(q0 + l32);   // padding (-1) compares as the largest
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int rn = 0; rn < 4; ++rn) {
            const int4 p4 = *reinterpret_cast<const int4*>(spos[cur] + kt * 32 + rn * 8 + hi * 4);
            const int pp[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
            for (int c = 0; c < 4; ++c)
              if (static_cast<unsigned>(pp[c]) > t) sacc[kt][rn * 4 + c] = -INFINITY;
          }
      }
      // online softmax per query column, base 2. The running max is raised
      // only when a score exceeds it by more than 2^8 (p stays <= 256, exact
      // in the final normalisation).
      {
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kt][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * a.scale_log2;
        const bool raise = mx > mrun + 8.0f;
        const float m_use = raise ? mx : mrun;
        const float alpha = __builtin_amdgcn_exp2f(mrun - m_use);
        float ps = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float pz = __builtin_amdgcn_exp2f(fmaf(sacc[kt][i], a.scale_log2, -m_use));
            sacc[kt][i] = pz;
            ps += pz;
          }
        ps += __shfl_xor(ps, 32, 64);
        lrun = lrun * alpha + ps;
        mrun = m_use;
        if (__ballot(raise)) {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
        }
      }
      // O^T += V^T P^T over four 16-key steps
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int kt = ks >> 1, half = ks & 1;
        u32x4_t u;
        u[0] = pack_bf16x2(sacc[kt][half * 8 + 0], sacc[kt][half * 8 + 1]);
        u[1] = pack_bf16x2(sacc[kt][half * 8 + 2], sacc[kt][half * 8 + 3]);
        u[2] = pack_bf16x2(sacc[kt][half * 8 + 4], sacc[kt][half * 8 + 5]);
        u[3] = pack_bf16x2(sacc[kt][half * 8 + 6], sacc[kt][half * 8 + 7]);
        const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, u);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          // A operand V^T: lane (hi, n) takes d-row dt*32+n at keys
          // ks*16 + hi*4 + 0..3 and ks*16 + 8 + hi*4 + 0..3, matching P^T
          const uint16_t* vr = svc + (ks * 16 + hi * 4 + tr_row) * VROW + dt * 32 + tr_col;
          const i16x4_t lo4 = lds_read_tr16(vr);
          const i16x4_t hi4 = lds_read_tr16(vr + 8 * VROW);
          const bf16x8_t av = __builtin_bit_cast(
              bf16x8_t, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb, o[dt], 0, 0, 0);
        }
      }
    }
    // stage tile ti+1 (its loads were issued a whole tile ago) into the other
    // buffer, whose last reader was tile ti-1, then start tile ti+2
    if (ti + 1 < n_tiles) {
      DSA_STAGE_TILE(cur ^ 1);
      if (ti + 2 < n_tiles) {
#pragma unroll
        for (int u = 0; u < KPER; ++u) { pk[u] = pkn[u]; pkn[u] = entry((ti + 3) * 64 + krow_of(u)); }
        DSA_LOAD_TILE();
      }
    }
    __syncthreads();
  }
#undef DSA_STAGE_TILE
#undef DSA_LOAD_TILE

  // out[b, h, t, d] = O^T[d, t] / l
  const float inv = lrun > 0.f ? 1.0f / lrun : 0.f;   // no visible key: output 0
  float* orow = a.out + ((static_cast<size_t>(b) * kv.Hq + h) * kv.T + q0 + l32) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      float4 v;
      v.x = o[dt][i4 * 4 + 0] * inv;
      v.y = o[dt][i4 * 4 + 1] * inv;
      v.z = o[dt][i4 * 4 + 2] * inv;
      v.w = o[dt][i4 * 4 + 3] * inv;
      *reinterpret_cast<float4*>(orow + dt * 32 + i4 * 8 + hi * 4) = v;
    }
}

// XOR swizzle of an unpadded 256-byte tile row: LDS slot s of row r holds the
// row's 16-byte piece s ^ swz(r). Sixteen consecutive rows read at one piece
// (the K fragments) and four consecutive rows read at four consecutive
// pieces (the V^T transpose reads) both land in 16 distinct slots, i.e. all
// 64 banks once.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// A buffer resource over `bytes` bytes at `base` (raw dword loads; offsets at
// or beyond `bytes` read as zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

typedef __attribute__((address_space(3))) void lds_void_t;

// d = 128 variant of k_prefill_mfma whose K/V tiles go straight from global
// memory into LDS (buffer_load_dwordx4 ... lds: a wave-wide load fills 1 KB of
// LDS in lane order, here 4 swizzled rows), so no registers stage the tiles and
// no LDS stores copy them. The loads of tile i+1 are issued after the barrier
// that retires tile i-1 and run under tile i's products.
//
// Tile entry e (0..63) lives in LDS row 16 * (e % 4) + e / 4: the 16 lanes of
// lane group g = 4 * wave + lane / 16 take entries 4g .. 4g+3 (one 16-byte
// load of the index row) and their four row loads land in rows 16u + g. Keys
// in any order give the same result (softmax and P.V are sums over keys), so
// the permutation only has to be the same for K, V and the positions used by
// the mask. Addresses are 32-bit offsets into buffer resources of this kv
// head's K and V; invisible entries load key 0 (or, beyond the tensor, zeros
// through the resource's range check) and are removed by the mask.
template <int NH, int QH>
__global__ void __launch_bounds__(64 * NH * QH, 2) k_prefill_mfma_lds(AttnArgs a) {
  constexpr int D = 128;
  constexpr int NWV = NH * QH;        // waves
  constexpr int KS = D / 16;          // 16-wide steps over d
  constexpr int DT = D / 32;          // 32-row tiles of O^T
  static_assert(NWV == 4, "each of 16 lane groups loads four entries of a 64-entry tile");
  // Two tile buffers as distinct objects, used alternately by the unrolled
  // loop below: the compiler can then tell the reads of one buffer from the
  // loads landing in the other and need not wait for those loads.
  __shared__ __align__(16) uint16_t sk0[64 * D], sk1[64 * D];
  __shared__ __align__(16) uint16_t sv0[64 * D], sv1[64 * D];
  __shared__ __align__(16) int spos0[64], spos1[64];     // positions by LDS row
  __shared__ __align__(16) int sflag0[NWV], sflag1[NWV];   // per wave: 1 = needs the mask, 2 = visible keys
  // the buffers are written only by the loads below: make that visible
  asm volatile("" ::"r"(sk0), "r"(sk1), "r"(sv0), "r"(sv1) : "memory");

  const KvLayout& kv = a.kv;
  // XCD-aware order, as in k_prefill_mfma
  const int G = kv.Hq / kv.Hkv;
  const int HG = G / NH;
  constexpr int NQS = 2 / QH;
  const int nwork = kv.B * kv.Hkv * HG * kv.nblk * NQS;
  const int per_xcd = gridDim.x >> 3;
  int work = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (work >= nwork) return;
  const int qsplit = work % NQS;
  work /= NQS;
  const int m = work % kv.nblk;
  work /= kv.nblk;
  const int hg = work % (kv.Hkv * HG);
  const int b = work / (kv.Hkv * HG);
  const int g = hg / HG;
  const int s = m * 64, e = s + 64;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  // transpose-read addressing of this lane (see lds_read_tr16): row
  // (lane & 15) >> 2 of four, column 4 * (lane & 3), groups 1 and 3 on d-rows 16..31
  const int tr_row = (lane & 15) >> 2, tr_col = ((lane >> 4) & 1) * 16 + 4 * (lane & 3);
  const int hw = w % NH, qg = w / NH;
  const int h = g * G + (hg % HG) * NH + hw;
  const int q0 = s + (qsplit * QH + qg) * 32;     // this wave's first query
  const int wq_lo = s + qsplit * QH * 32;         // the workgroup's query range
  const int wq_hi = wq_lo + QH * 32 - 1;
  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  const size_t kvbase = (static_cast<size_t>(b) * kv.Hkv + g) * kv.T;
  const uint32_t kv_bytes = static_cast<uint32_t>(kv.T) * D * 2;
  const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(static_cast<const uint16_t*>(a.k) + kvbase * D, kv_bytes);
  const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(static_cast<const uint16_t*>(a.v) + kvbase * D, kv_bytes);

  bf16x8_t qf[KS];
  {
    const uint16_t* qrow = Q + ((static_cast<size_t>(b) * kv.Hq + h) * kv.T + q0 + l32) * D + hi * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8_t*>(qrow + ks * 16);
  }
  f32x16_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
  float mrun = kNegBig, lrun = 0.f;

  const int r = b * kv.nblk + m;
  const int32_t* row = a.idx ? a.idx + static_cast<size_t>(r) * a.L : nullptr;
  const int n_ent = row ? a.L : e;                // a multiple of 64 (index width, or e)
  const int n_tiles = (n_ent + 63) / 64;
  const int lg = 4 * w + (lane >> 4);             // this lane's group: entries 4lg .. 4lg+3
  const int lslot = lane & 15;                    // and its 16-byte piece of each row
  // raw entries of tile ti (fetched two tiles ahead; judged only when issued)
  auto raw_entries = [&](int ti) {
    int4 v = make_int4(-1, -1, -1, -1);
    if (ti < n_tiles) {
      if (row) {
        v = *reinterpret_cast<const int4*>(row + ti * 64 + 4 * lg);
      } else {
        const int p0 = ti * 64 + 4 * lg;
        v = make_int4(p0, p0 + 1, p0 + 2, p0 + 3);
      }
    }
    return v;
  };
  int4 pr, prn;                                   // entries of the next two tiles
  // tile with entries pr -> buffers: the row loads, the positions for the
  // mask and the tile's mask / visibility flags
  auto issue = [&](uint16_t* skb, uint16_t* svb, int* sposb, int* sflagb) __attribute__((always_inline)) {
    const int pp[4] = {pr.x, pr.y, pr.z, pr.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int rr = 16 * u + lg;                 // LDS row of entry 4lg + u
      const int off = max(pp[u], 0) * (D * 2) + ((lslot ^ swz(rr)) << 4);
      const int lbase = (16 * u + 4 * w) * D;     // the wave's 4 rows of this load
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void_t*)(skb + lbase), 16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void_t*)(svb + lbase), 16, off, 0, 0, 0);
    }
    int pv = pr.x;                                // lanes 0..3 of the group store entries 0..3
    pv = lslot == 1 ? pr.y : pv;
    pv = lslot == 2 ? pr.z : pv;
    pv = lslot == 3 ? pr.w : pv;
    if (lslot < 4) sposb[16 * lslot + lg] = pv;
    // unsigned: padding (-1) is the largest
    const unsigned umax = max(max(static_cast<unsigned>(pr.x), static_cast<unsigned>(pr.y)),
                              max(static_cast<unsigned>(pr.z), static_cast<unsigned>(pr.w)));
    const unsigned umin = min(min(static_cast<unsigned>(pr.x), static_cast<unsigned>(pr.y)),
                              min(static_cast<unsigned>(pr.z), static_cast<unsigned>(pr.w)));
    const unsigned long long nb = __ballot(umax > static_cast<unsigned>(wq_lo));
    const unsigned long long ab = __ballot(umin <= static_cast<unsigned>(wq_hi));
    if (lane == 0) sflagb[w] = (nb != 0 ? 1 : 0) | (ab != 0 ? 2 : 0);
  };
  // one tile: products from buffers c, loads of the next tile into buffers n
  auto step = [&](int ti, const uint16_t* skc, const uint16_t* svc, const int* sposc, const int* sflagc,
                  uint16_t* skn, uint16_t* svn, int* sposn, int* sflagn) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0);                // this wave's loads of tile ti are in LDS
    __syncthreads();                              // everyone's; and tile ti-1 is retired
    if (ti + 1 < n_tiles) {
      issue(skn, svn, sposn, sflagn);
      pr = prn;
      prn = raw_entries(ti + 3);
    }
    const int4 f4 = *reinterpret_cast<const int4*>(sflagc);
    const int flag = __builtin_amdgcn_readfirstlane(f4.x | f4.y | f4.z | f4.w);
    if (!(flag & 2)) return;                      // nothing visible in this tile
    // S^T tiles [key tile kt]: 32 keys x this wave's 32 queries
    f32x16_t sacc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kt][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int rr = kt * 32 + l32;
        const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(skc + rr * D + ((2 * ks + hi) ^ swz(rr)) * 8);
        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[ks], sacc[kt], 0, 0, 0);
      }
    }
    if (flag & 1) {
      // accumulator element 4rn + c of key tile kt is LDS row 32kt + 8rn + 4hi + c
      const unsigned t = static_cast<unsigned>(q0 + l32);   // padding (-1) compares as the largest
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int rn = 0; rn < 4; ++rn) {
          const int4 p4 = *reinterpret_cast<const int4*>(sposc + kt * 32 + rn * 8 + hi * 4);
          const int pp[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
          for (int c = 0; c < 4; ++c)
            if (static_cast<unsigned>(pp[c]) > t) sacc[kt][rn * 4 + c] = -INFINITY;
        }
    }
    // online softmax per query column, base 2. The running max is raised
    // only when a score exceeds it by more than 2^8 (p stays <= 256, exact in
    // the final normalisation). The row sum adds the bf16-rounded p that the
    // P.V product uses, two at a time.
    {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kt][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * a.scale_log2;
      const bool raise = mx > mrun + 8.0f;
      const float m_use = raise ? mx : mrun;
      const float alpha = __builtin_amdgcn_exp2f(mrun - m_use);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kt][i] = __builtin_amdgcn_exp2f(fmaf(sacc[kt][i], a.scale_log2, -m_use));
      mrun = m_use;
      if (__ballot(raise)) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
      }
      lrun *= alpha;
    }
    float ps = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kt = ks >> 1, half = ks & 1;
      u32x4_t u;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        // the packed pair feeds the sum from its own register (reading it
        // back out of the vector has been compiled to the wrong element)
        const uint32_t pw = pack_bf16x2(sacc[kt][half * 8 + 2 * x], sacc[kt][half * 8 + 2 * x + 1]);
        ps += bf16_pair_sum(pw);
        u[x] = pw;
      }
      const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, u);
      const int r0 = ks * 16 + hi * 4 + tr_row, r1 = r0 + 8;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int c = dt * 32 + tr_col;           // 4 consecutive d inside one 16-byte piece
        const i16x4_t lo4 = lds_read_tr16(svc + r0 * D + (((c >> 3) ^ swz(r0)) << 3) + (c & 7));
        const i16x4_t hi4 = lds_read_tr16(svc + r1 * D + (((c >> 3) ^ swz(r1)) << 3) + (c & 7));
        const bf16x8_t av = __builtin_bit_cast(
            bf16x8_t, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb, o[dt], 0, 0, 0);
      }
    }
    lrun += ps + __shfl_xor(ps, 32, 64);
  };

  // prologue: tile 0 into buffers 0, entries of tiles 1 and 2 in hand
  pr = raw_entries(0);
  prn = raw_entries(1);
  issue(sk0, sv0, spos0, sflag0);
  pr = prn;
  prn = raw_entries(2);
  for (int ti = 0; ti < n_tiles; ti += 2) {
    step(ti, sk0, sv0, spos0, sflag0, sk1, sv1, spos1, sflag1);
    if (ti + 1 < n_tiles) step(ti + 1, sk1, sv1, spos1, sflag1, sk0, sv0, spos0, sflag0);
  }

  const float inv = lrun > 0.f ? 1.0f / lrun : 0.f;   // no visible key: output 0
  float* orow = a.out + ((static_cast<size_t>(b) * kv.Hq + h) * kv.T + q0 + l32) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      float4 v;
      v.x = o[dt][i4 * 4 + 0] * inv;
      v.y = o[dt][i4 * 4 + 1] * inv;
      v.z = o[dt][i4 * 4 + 2] * inv;
      v.w = o[dt][i4 * 4 + 3] * inv;
      *reinterpret_cast<float4*>(orow + dt * 32 + i4 * 8 + hi * 4) = v;
    }
}

// Per-head index rows (one row per sequence, query head and query block, as
// the block-sparse heads of the MInference page produce: "Block-Sparse
// FlashAttention Kernel (Appendix C.4.1)"), d = 128. No two heads share a key
// tile, so a workgroup owns one head's 64-query block: two waves of 32
// queries. K and V have one LDS tile each (33 KB in all, four workgroups per
// CU) and are refilled as soon as their readers are done, straight from
// global memory (buffer_load_dwordx4 ... lds):
//   wait K_i, barrier | issue V_i | S = K_i Q^T, mask | barrier | issue K_i+1
//   | softmax | wait V_i, barrier | O^T += V_i^T P^T
// so V_i loads under the QK product and the softmax, K_i+1 under the softmax
// and the PV product. Tile entry e (0..63) lives in LDS row 8 * (e % 8) + e / 8:
// lane group g = 4 * wave + lane / 16 (0..7) takes entries 8g .. 8g+7 and its
// eight row loads land in rows 8u + g. Entries that are padding (or tiles past
// the row) load through an out-of-range offset: zeros, no memory traffic.
// Workgroup barrier that leaves this wave's loads into LDS in flight: LDS
// reads and writes are complete (lgkmcnt 0), vector memory is not waited.
// (The compiler's own barrier waits for every load into LDS still pending.)
__device__ __forceinline__ void barrier_keep_loads() {
  __builtin_amdgcn_s_waitcnt(0xC07F);           // lgkmcnt(0); vmcnt, expcnt not waited
  asm volatile("s_barrier" ::: "memory");
}

//
// With LISTS, a (head, query block) gives a block list and a column list
// instead of a row (the MInference page's "Vertical-Slash Hybrid Kernel
// (Appendix C.4.2, Algorithms 4 and 5)"; the block-sparse heads have blocks
// only): its tiles are the listed 64-key blocks, whose positions follow from
// the block id, then the columns, 64 to a tile, gathered like row entries.
// A block tile's index fetch reads the aligned quad of ids holding its own,
// twice, so every tile still issues exactly two index loads.
template <bool LISTS>
__global__ void __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2, 2))) k_prefill_heads(AttnArgs a) {
  constexpr int D = 128;
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  __shared__ __align__(16) uint16_t skb[64 * D];
  __shared__ __align__(16) uint16_t svb[64 * D];
  __shared__ __align__(16) int spos0[64], spos1[64];     // positions by LDS row
  __shared__ __align__(16) int sflag0[2], sflag1[2];     // per wave: 1 = needs the mask, 2 = visible keys
  asm volatile("" ::"r"(skb), "r"(svb) : "memory");

  const KvLayout& kv = a.kv;
  const int G = kv.Hq / kv.Hkv;
  // the grid walks one kv head at a time (its K and V stay in the
  // last-level cache), the heads of a group next to each other
  int work = blockIdx.x;
  if (work >= kv.B * kv.Hq * kv.nblk) return;
  const int hw = work % G;
  work /= G;
  const int m = work % kv.nblk;
  work /= kv.nblk;
  const int g = work % kv.Hkv;
  const int b = work / kv.Hkv;
  const int h = g * G + hw;
  const int s = m * 64;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int tr_row = (lane & 15) >> 2, tr_col = ((lane >> 4) & 1) * 16 + 4 * (lane & 3);
  const int q0 = s + w * 32;                      // this wave's first query
  const int wq_lo = s, wq_hi = s + 63;
  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  const size_t kvbase = (static_cast<size_t>(b) * kv.Hkv + g) * kv.T;
  const uint32_t kv_bytes = static_cast<uint32_t>(kv.T) * D * 2;
  const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(static_cast<const uint16_t*>(a.k) + kvbase * D, kv_bytes);
  const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(static_cast<const uint16_t*>(a.v) + kvbase * D, kv_bytes);

  bf16x8_t qf[KS];
  {
    const uint16_t* qrow = Q + ((static_cast<size_t>(b) * kv.Hq + h) * kv.T + q0 + l32) * D + hi * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8_t*>(qrow + ks * 16);
  }
  f32x16_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
  float mrun = kNegBig, lrun = 0.f;

  const size_t rowid = static_cast<size_t>(b * kv.Hq + h) * kv.nblk + m;
  const int32_t* row = LISTS ? nullptr : a.idx + rowid * a.L;
  const int32_t* lb = LISTS ? a.lblk + rowid * a.wb : nullptr;
  const int32_t* lc = LISTS && a.lcol ? a.lcol + rowid * a.wc : lb;   // (no columns: never read)
  const int wcl = LISTS && a.lcol ? a.wc : 4;
  int nbl = 0, ncl = 0;                           // listed blocks, listed columns
  if constexpr (LISTS) {
    const int2 c2 = *reinterpret_cast<const int2*>(a.lcnt + 2 * rowid);
    nbl = min(max(c2.x, 0), a.wb);                // (counts never send a list read past its width)
    ncl = min(max(c2.y, 0), a.wc);
  }
  const int n_tiles = LISTS ? nbl + (ncl + 63) / 64 : (a.L + 63) / 64;
  const int lg = 4 * w + (lane >> 4);             // entries 8lg .. 8lg+7 of a tile
  const int lslot = lane & 15;
  // Entries 8lg .. 8lg+7 of a tile: two 16-byte loads at clamped addresses
  // inside the row (L is a multiple of 4), issued a step before their use and
  // decoded only then (-1 for padding, beyond the row, or past the last
  // tile), so each step issues exactly two such loads and never waits on them
  // early: the waits below count them.
  auto load_raw = [&](int ti, int4& v0, int4& v1) __attribute__((always_inline)) {
    if constexpr (LISTS) {
      const int tt = max(0, min(ti, n_tiles - 1));
      if (tt < nbl) {                               // the quad holding the block id (wb is a multiple of 4)
        v0 = *reinterpret_cast<const int4*>(lb + (tt & ~3));
        v1 = *reinterpret_cast<const int4*>(lb + (tt & ~3));
      } else {
        const int i0 = (tt - nbl) * 64 + 8 * lg;
        v0 = *reinterpret_cast<const int4*>(lc + min(i0, wcl - 4));
        v1 = *reinterpret_cast<const int4*>(lc + min(i0 + 4, wcl - 4));
      }
    } else {
      const int i0 = min(ti, n_tiles - 1) * 64 + 8 * lg;
      v0 = *reinterpret_cast<const int4*>(row + min(i0, a.L - 4));
      v1 = *reinterpret_cast<const int4*>(row + min(i0 + 4, a.L - 4));
    }
  };
  auto decode = [&](int ti, const int4& v0, const int4& v1, int (&p)[8]) __attribute__((always_inline)) {
    const bool live = ti < n_tiles;
    if constexpr (LISTS) {
      const int tt = max(0, min(ti, n_tiles - 1));
      if (tt < nbl) {
        const int q4 = tt & 3;
        const int blk = q4 == 0 ? v0.x : q4 == 1 ? v0.y : q4 == 2 ? v0.z : v0.w;
#pragma unroll
        for (int x = 0; x < 8; ++x) p[x] = live ? 64 * blk + 8 * lg + x : -1;
      } else {
        const int i0 = (tt - nbl) * 64 + 8 * lg;
        const int raw[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int x = 0; x < 8; ++x) p[x] = (live && i0 + x < ncl) ? raw[x] : -1;
      }
    } else {
      const int i0 = min(ti, n_tiles - 1) * 64 + 8 * lg;
      const int raw[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int x = 0; x < 8; ++x) p[x] = (live && i0 + x < a.L) ? raw[x] : -1;
    }
  };
  auto issue = [&](const __amdgpu_buffer_rsrc_t& rs, uint16_t* dst, const int (&p)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int rr = 8 * u + lg;                  // LDS row of entry 8lg + u
      const int off = p[u] < 0 ? static_cast<int>(kv_bytes) : p[u] * (D * 2) + ((lslot ^ swz(rr)) << 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(dst + (8 * u + 4 * w) * D), 16, off, 0, 0, 0);
    }
  };
  auto publish = [&](const int (&p)[8], int* sposb, int* sflagb) __attribute__((always_inline)) {
    int pv = p[0];
#pragma unroll
    for (int x = 1; x < 8; ++x) pv = lslot == x ? p[x] : pv;
    if (lslot < 8) sposb[8 * lslot + lg] = pv;
    unsigned umax = 0u, umin = 0xffffffffu;       // unsigned: padding (-1) is the largest
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      umax = max(umax, static_cast<unsigned>(p[x]));
      umin = min(umin, static_cast<unsigned>(p[x]));
    }
    const unsigned long long nb = __ballot(umax > static_cast<unsigned>(wq_lo));
    const unsigned long long ab = __ballot(umin <= static_cast<unsigned>(wq_hi));
    if (lane == 0) sflagb[w] = (nb != 0 ? 1 : 0) | (ab != 0 ? 2 : 0);
  };

  int cur[8];                                     // decoded entries of the tile in hand
  int4 r0, r1;                                    // raw entries of the next tile
  load_raw(0, r0, r1);
  decode(0, r0, r1, cur);
  load_raw(1, r0, r1);
  issue(krs, skb, cur);
  publish(cur, spos0, sflag0);

  auto step = [&](int ti, const int* sposc, const int* sflagc, int* sposn, int* sflagn) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0);                // this wave's K_i rows are in LDS
    barrier_keep_loads();                         // everyone's; V is free again
    issue(vrs, svb, cur);
    asm volatile("" ::: "memory");
    decode(ti + 1, r0, r1, cur);
    load_raw(ti + 2, r0, r1);
    asm volatile("" ::: "memory");
    const int2 f2 = *reinterpret_cast<const int2*>(sflagc);
    const int flag = __builtin_amdgcn_readfirstlane(f2.x | f2.y);
    f32x16_t sacc[2];
    if (flag & 2) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kt][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const int rr = kt * 32 + l32;
          const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(skb + rr * D + ((2 * ks + hi) ^ swz(rr)) * 8);
          sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[ks], sacc[kt], 0, 0, 0);
        }
      }
      if (flag & 1) {
        // accumulator element 4rn + c of key tile kt is LDS row 32kt + 8rn + 4hi + c
        const unsigned t = static_cast<unsigned>(q0 + l32);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int rn = 0; rn < 4; ++rn) {
            const int4 p4 = *reinterpret_cast<const int4*>(sposc + kt * 32 + rn * 8 + hi * 4);
            const int pp[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
            for (int c = 0; c < 4; ++c)
              if (static_cast<unsigned>(pp[c]) > t) sacc[kt][rn * 4 + c] = -INFINITY;
          }
      }
    }
    barrier_keep_loads();                         // K is free: refill it with tile i + 1
    issue(krs, skb, cur);
    publish(cur, sposn, sflagn);
    asm volatile("" ::: "memory");
    if (flag & 2) {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kt][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * a.scale_log2;
      const bool raise = mx > mrun + 8.0f;
      const float m_use = raise ? mx : mrun;
      const float alpha = __builtin_amdgcn_exp2f(mrun - m_use);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kt][i] = __builtin_amdgcn_exp2f(fmaf(sacc[kt][i], a.scale_log2, -m_use));
      mrun = m_use;
      if (__ballot(raise)) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
      }
      lrun *= alpha;
    }
    // V_i was issued before the entries of tile i + 2 and K_i+1 (2 + 8 loads)
    __builtin_amdgcn_s_waitcnt(0x0F7A);           // vmcnt(10); expcnt, lgkmcnt not waited
    barrier_keep_loads();
    if (flag & 2) {
      float ps = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int kt = ks >> 1, half = ks & 1;
        u32x4_t u;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const uint32_t pw = pack_bf16x2(sacc[kt][half * 8 + 2 * x], sacc[kt][half * 8 + 2 * x + 1]);
          ps += bf16_pair_sum(pw);
          u[x] = pw;
        }
        const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, u);
        const int r0 = ks * 16 + hi * 4 + tr_row, r1 = r0 + 8;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int c = dt * 32 + tr_col;
          const i16x4_t lo4 = lds_read_tr16(svb + r0 * D + (((c >> 3) ^ swz(r0)) << 3) + (c & 7));
          const i16x4_t hi4 = lds_read_tr16(svb + r1 * D + (((c >> 3) ^ swz(r1)) << 3) + (c & 7));
          const bf16x8_t av = __builtin_bit_cast(
              bf16x8_t, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb, o[dt], 0, 0, 0);
        }
      }
      lrun += ps + __shfl_xor(ps, 32, 64);
    }
  };
  for (int ti = 0; ti < n_tiles; ti += 2) {
    step(ti, spos0, sflag0, spos1, sflag1);
    if (ti + 1 < n_tiles) step(ti + 1, spos1, sflag1, spos0, sflag0);
  }
  __builtin_amdgcn_s_waitcnt(0);                  // no load into LDS outlives the workgroup

  const float inv = lrun > 0.f ? 1.0f / lrun : 0.f;   // no visible key: output 0
  float* orow = a.out + ((static_cast<size_t>(b) * kv.Hq + h) * kv.T + q0 + l32) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      float4 v;
      v.x = o[dt][i4 * 4 + 0] * inv;
      v.y = o[dt][i4 * 4 + 1] * inv;
      v.z = o[dt][i4 * 4 + 2] * inv;
      v.w = o[dt][i4 * 4 + 3] * inv;
      *reinterpret_cast<float4*>(orow + dt * 32 + i4 * 8 + hi * 4) = v;
    }
}

// Shared rows, d = 128, groups of at least 4 query heads: one workgroup per
// (query block, 4 heads of a kv group) with all 64 queries, eight waves
// (4 heads x 2 query halves), so each K/V tile is loaded into LDS once for 256
// (query, head) rows. Tile entry e lives in LDS row 32 * (e % 2) + e / 2: lane
// group g = 4 * wave + lane / 16 (0..31) takes entries 2g, 2g+1 (one 8-byte
// load of the index row) and its two row loads land in rows 32u + g. Padding
// and tiles past the row load through an out-of-range offset (zeros, no
// traffic).
//
// The two waves of each SIMD run a phase apart ("ping-pong"). A tile's work
// per wave is S = K Q^T (16 matrix products), the online softmax (vector ALU
// only) and O += V^T P^T (16 products, plus 4 that give the row sums of P).
// Waves 0-3 (query half 0) and 4-7 (query half 1) share the four SIMDs in
// pairs, and the half-1 waves run one phase behind: in every phase one wave
// of each SIMD issues the products of P_i V_i and S_i+1 while the other
// computes a softmax, so the matrix core is fed while its partner runs the
// exponentials. Phases end at workgroup barriers, and each wave passes the
// same number of them. Measured on gfx950: the bf16 dot-product instruction
// waits for the matrix core of its SIMD (about one product per use), so the
// softmax keeps none; every value that crosses lanes or waves in the loop
// stays out of LDS (the tile flags come from a ballot over one index entry
// per lane, the half-wave max from a lane swap), since an LDS round trip
// costs several hundred cycles while the tile loads stream into LDS.
//
// Tile buffers rotate over three slots per operand. In phase 2m every wave
// issues its rows of V_m+1 and K_m+2 and the index entries of tile m+3;
// K_m+2 lands in the slot K_m-1 left at the end of phase 2m-1, V_m+1 in the
// slot of V_m-2, so each load has two phases (one tile) to arrive before the
// wait at the end of phase 2m+1 (vmcnt 6: the six loads of phase 2m stay in
// flight) and the barrier after it.
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) k_prefill_gqa8(AttnArgs a) {
  constexpr int D = 128;
  constexpr int NH = 4;
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  __shared__ __align__(16) uint16_t sk0[64 * D], sk1[64 * D], sk2[64 * D], sk3[64 * D];
  __shared__ __align__(16) uint16_t sv0[64 * D], sv1[64 * D], sv2[64 * D], sv3[64 * D];
  __shared__ __align__(16) int spos0[64], spos1[64], spos2[64], spos3[64];
  asm volatile("" ::"r"(sk0), "r"(sk1), "r"(sk2), "r"(sk3), "r"(sv0), "r"(sv1), "r"(sv2), "r"(sv3) : "memory");

  const KvLayout& kv = a.kv;
  const int G = kv.Hq / kv.Hkv;
  const int HG = G / NH;
  const int nwork = kv.B * kv.Hkv * HG * kv.nblk;
  const int per_xcd = gridDim.x >> 3;
  int work = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (work >= nwork) return;
  const int m = work % kv.nblk;
  work /= kv.nblk;
  const int hg = work % (kv.Hkv * HG);
  const int b = work / (kv.Hkv * HG);
  const int g = hg / HG;
  const int s = m * 64;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int tr_row = (lane & 15) >> 2, tr_col = ((lane >> 4) & 1) * 16 + 4 * (lane & 3);
  const int hw = w % NH, qg = w / NH;
  const int h = g * G + (hg % HG) * NH + hw;
  const int q0 = s + qg * 32;
  const int wq_lo = s, wq_hi = s + 63;
  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  const size_t kvbase = (static_cast<size_t>(b) * kv.Hkv + g) * kv.T;
  const uint32_t kv_bytes = static_cast<uint32_t>(kv.T) * D * 2;
  const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(static_cast<const uint16_t*>(a.k) + kvbase * D, kv_bytes);
  const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(static_cast<const uint16_t*>(a.v) + kvbase * D, kv_bytes);

  bf16x8_t qf[KS];
  {
    const uint16_t* qrow = Q + ((static_cast<size_t>(b) * kv.Hq + h) * kv.T + q0 + l32) * D + hi * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8_t*>(qrow + ks * 16);
  }
  f32x16_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
  // row sums of P by the matrix cores: O_sum^T += 1 P^T (every row of the
  // product holds the sum over the tile's keys for the lane's query)
  f32x16_t osum = {};
  float mrun = kNegBig;
  f32x16_t sacc[2];
  bf16x8_t pb[4] = {};

  const int32_t* row = a.idx + static_cast<size_t>(b * kv.nblk + m) * a.L;
  const int n_tiles = a.L / 64;                   // whole tiles (checked by the launcher)
  const int lg = 4 * w + (lane >> 4);
  const int lslot = lane & 15;
  auto load_raw = [&](int ti) __attribute__((always_inline)) {
    return *reinterpret_cast<const int2*>(row + min(ti, n_tiles - 1) * 64 + 2 * lg);
  };
  // entry `lane` of tile ti, for the tile's flags
  auto load_ent = [&](int ti) __attribute__((always_inline)) { return row[min(ti, n_tiles - 1) * 64 + lane]; };
  // this wave's two rows of tile ti (entries 2 lg, 2 lg + 1) into sb
  auto issue_rows = [&](int ti, int2 raw, __amdgpu_buffer_rsrc_t rs, uint16_t* sb) __attribute__((always_inline)) {
    const bool live = ti < n_tiles;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int p = live ? (u ? raw.y : raw.x) : -1;
      const int rr = 32 * u + lg;
      const int off = p < 0 ? static_cast<int>(kv_bytes) : p * (D * 2) + ((lslot ^ swz(rr)) << 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(sb + (32 * u + 4 * w) * D), 16, off, 0, 0, 0);
    }
  };
  // positions of tile ti in LDS row order, for the causal mask
  auto publish = [&](int ti, int2 raw, int* sposb) __attribute__((always_inline)) {
    const bool live = ti < n_tiles;
    if (lslot < 2) sposb[32 * lslot + lg] = live ? (lslot == 0 ? raw.x : raw.y) : -1;
  };
  // flags of tile ti from its entries (one per lane): bit 0 some entry may
  // follow a query of the block (masking needed), bit 1 some key is visible
  auto flag_of = [&](int ti, int e) __attribute__((always_inline)) {
    const bool live = ti < n_tiles;
    const unsigned u = static_cast<unsigned>(e);
    const unsigned long long nb = __ballot(live && u > static_cast<unsigned>(wq_lo));
    const unsigned long long ab = __ballot(live && u <= static_cast<unsigned>(wq_hi));
    return (nb != 0 ? 1 : 0) | (ab != 0 ? 2 : 0);
  };

  int2 r1 = load_raw(0), r2 = load_raw(1);
  int e1 = load_ent(0), e2 = load_ent(1);
  // phase 2m's loads: index entries of tile m+3, rows of V_m+1 and K_m+2;
  // returns the flags of tile m+1
  auto issue_block = [&](int mm, uint16_t* svd, int* sposd, uint16_t* skd) __attribute__((always_inline)) {
    const int2 r3 = load_raw(mm + 3);
    const int e3 = load_ent(mm + 3);
    asm volatile("" ::: "memory");
    issue_rows(mm + 1, r1, vrs, svd);
    publish(mm + 1, r1, sposd);
    issue_rows(mm + 2, r2, krs, skd);
    asm volatile("" ::: "memory");
    const int f1 = flag_of(mm + 1, e1);
    r1 = r2;
    r2 = r3;
    e1 = e2;
    e2 = e3;
    return f1;
  };
  // the max of x over lanes l and l ^ 32 (both halves get the same bits)
  auto halves_max = [&](float x) __attribute__((always_inline)) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  };

  // operand fragments of one stream step: the K rows of key step ks (both
  // 32-row halves) for S, or the V^T rows of two d-tiles for O
  struct Frag {
    u32x4_t r[2];
  };
  // per-lane byte offsets inside a tile: K rows of step ks (the second
  // 32-row half adds 32 rows), V^T rows of step 0 for d-tile dt (row r0 and
  // r0 + 8; step ks adds 16 rows). The swizzle of a V row depends only on
  // the lane, since steps move by 16 rows.
  int kofs[KS], vofs[2 * DT];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) kofs[ks] = (l32 * D + (((2 * ks + hi) ^ swz(l32)) << 3)) * 2;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const int r0 = hi * 4 + tr_row, c = dt * 32 + tr_col;
    vofs[2 * dt] = (r0 * D + (((c >> 3) ^ swz(r0)) << 3) + (c & 7)) * 2;
    vofs[2 * dt + 1] = ((r0 + 8) * D + (((c >> 3) ^ swz(r0 + 8)) << 3) + (c & 7)) * 2;
  }
  auto load_k = [&](Frag& f, const uint16_t* skc, int ks) __attribute__((always_inline)) {
    const char* base = reinterpret_cast<const char*>(skc) + kofs[ks];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) f.r[kt] = *reinterpret_cast<const u32x4_t*>(base + kt * 32 * D * 2);
  };
  auto load_v = [&](Frag& f, const uint16_t* svc, int ks, int dt0) __attribute__((always_inline)) {
    const char* base = reinterpret_cast<const char*>(svc) + ks * 16 * D * 2;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const i16x4_t lo4 = lds_read_tr16(reinterpret_cast<const uint16_t*>(base + vofs[2 * (dt0 + j)]));
      const i16x4_t hi4 = lds_read_tr16(reinterpret_cast<const uint16_t*>(base + vofs[2 * (dt0 + j) + 1]));
      f.r[j] = __builtin_bit_cast(u32x4_t, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  // S accumulates from zero at key step 0, so it holds no value before
  auto use_k = [&](const Frag& f, int ks) __attribute__((always_inline)) {
    const f32x16_t zero = {};
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
      sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, f.r[kt]), qf[ks],
                                                         ks == 0 ? zero : sacc[kt], 0, 0, 0);
  };
  auto use_v = [&](const Frag& f, int ks, int dt0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      o[dt0 + j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, f.r[j]), pb[ks], o[dt0 + j],
                                                           0, 0, 0);
    if (dt0 == 2) {
      const bf16x8_t ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f),
                             static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f),
                             static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
      osum = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, pb[ks], osum, 0, 0, 0);
    }
  };
  // The matrix phase is a stream of up to 16 steps of two products each:
  // steps 0-7 O += V_i^T P_i^T (key step st / 2, d-tiles 2 (st % 2) and
  // 2 (st % 2) + 1), steps 8-15 S_i+1 (key step st - 8). The fragments of a
  // step are read NF - 1 steps ahead of its products, so the LDS latency
  // stays hidden while one wave of the SIMD issues all its products.
  constexpr int NF = 4;
  auto stream = [&](const uint16_t* svc, const uint16_t* skn, auto s0c, auto s1c) __attribute__((always_inline)) {
    constexpr int S0 = decltype(s0c)::value, S1 = decltype(s1c)::value;
    Frag F[NF];
    auto load_step = [&](int st) __attribute__((always_inline)) {
      if (st < 8) load_v(F[st % NF], svc, st >> 1, 2 * (st & 1));
      else load_k(F[st % NF], skn, st - 8);
    };
#pragma unroll
    for (int st = S0; st < S0 + NF - 1 && st < S1; ++st) load_step(st);
#pragma unroll
    for (int st = S0; st < S1; ++st) {
      if (st + NF - 1 < S1) load_step(st + NF - 1);
      __builtin_amdgcn_sched_barrier(0);
      if (st < 8) use_v(F[st % NF], st >> 1, 2 * (st & 1));
      else use_k(F[st % NF], st - 8);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // the matrix phase: O += V_i^T P_i^T, then S_i+1, unless neither tile has
  // a visible key (a tile without one has P = 0, its S is not used)
  auto mfma_phase = [&](const uint16_t* svc, int fp, const uint16_t* skn, int fq) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(3);                // the products first when both waves of a SIMD are ready
    if ((fp | fq) & 2) stream(svc, skn, std::integral_constant<int, 0>{}, std::integral_constant<int, 16>{});
    __builtin_amdgcn_s_setprio(0);
  };
  // online softmax of S_i (flag f): P_i in bf16 (pb), running max and sum
  auto softmax = [&](const int* sposc, int f) __attribute__((always_inline)) {
    if (!(f & 2)) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) pb[ks] = bf16x8_t{};
      return;
    }
    if (f & 1) {
      const unsigned t = static_cast<unsigned>(q0 + l32);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int rn = 0; rn < 4; ++rn) {
          const int4 p4 = *reinterpret_cast<const int4*>(sposc + kt * 32 + rn * 8 + hi * 4);
          const int pp[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
          for (int c = 0; c < 4; ++c)
            if (static_cast<unsigned>(pp[c]) > t) sacc[kt][rn * 4 + c] = -INFINITY;
        }
    }
    // four independent max chains, then their max
    float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) m4[(kt * 16 + i) & 3] = fmaxf(m4[(kt * 16 + i) & 3], sacc[kt][i]);
    float mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
    mx = halves_max(mx) * a.scale_log2;
    const bool raise = mx > mrun + 8.0f;
    const float m_use = raise ? mx : mrun;
    const float alpha = __builtin_amdgcn_exp2f(mrun - m_use);
    mrun = m_use;
    if (__ballot(raise)) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
#pragma unroll
      for (int i = 0; i < 16; ++i) osum[i] *= alpha;
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kt = ks >> 1, half = ks & 1;
      u32x4_t u;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kt][half * 8 + 2 * x], a.scale_log2, -m_use));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kt][half * 8 + 2 * x + 1], a.scale_log2, -m_use));
        u[x] = pack_bf16x2(p0, p1);
      }
      pb[ks] = __builtin_bit_cast(bf16x8_t, u);
    }
  };
  // waits for the rows of all but the last one (half 1) or two (half 0) load
  // blocks this wave issued
  auto wait_rows1 = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0F76);           // vmcnt(6); expcnt, lgkmcnt not waited
  };
  auto wait_rows0 = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0F7C);           // vmcnt(12); expcnt, lgkmcnt not waited
  };

  // prologue: K_0, then the loads a phase 2m = -2 would issue (index
  // entries of tile 2, V_0, K_1); half 0 also issues the next block now
  issue_rows(0, r1, krs, sk0);
  int f = issue_block(-1, sv0, spos0, sk1);      // tile 0's flags
  int fn = 0;
  if (qg == 0) {
    fn = issue_block(0, sv1, spos1, sk2);
    wait_rows0();
  } else {
    wait_rows1();
  }
  barrier_keep_loads();

  // tile i of a wave that is in phase 2i+1 (half 0) or 2i+2 (half 1) for its
  // softmax, with the flags fc of tile i and fn of tile i+1. Slots of tile
  // i: A, of i+1: B, of i+2: C, of i+3: D. The load block of the softmax
  // phase writes V_i+2 (slot C) and K_i+3 (slot D); for half 0 that is
  // phase 2i+1, when the half-1 waves still read V_i-1 and K_i (slots D and
  // A), which four slots keep apart.
  auto tile0 = [&](int i, int& fc, int& fn, const int* sposA, uint16_t* svA, const uint16_t* skB,
                   uint16_t* svC, int* sposC, uint16_t* skD) __attribute__((always_inline)) {
    const int fnn = issue_block(i + 1, svC, sposC, skD);
    softmax(sposA, fc);
    wait_rows0();
    barrier_keep_loads();
    mfma_phase(svA, fc, skB, fn);
    barrier_keep_loads();
    fc = fn;
    fn = fnn;
  };
  auto tile1 = [&](int i, int& fc, int& fn, const int* sposA, uint16_t* svA, const uint16_t* skB,
                   uint16_t* svC, int* sposC, uint16_t* skD) __attribute__((always_inline)) {
    const int fnn = issue_block(i + 1, svC, sposC, skD);
    softmax(sposA, fc);
    barrier_keep_loads();
    mfma_phase(svA, fc, skB, fn);
    wait_rows1();
    barrier_keep_loads();
    fc = fn;
    fn = fnn;
  };

  if (qg == 0) {
    // phase 0: S_0
    if (f & 2) stream(sv0, sk0, std::integral_constant<int, 8>{}, std::integral_constant<int, 16>{});
    barrier_keep_loads();
    int i = 0;
    for (; i + 4 <= n_tiles; i += 4) {
      tile0(i, f, fn, spos0, sv0, sk1, sv2, spos2, sk3);
      tile0(i + 1, f, fn, spos1, sv1, sk2, sv3, spos3, sk0);
      tile0(i + 2, f, fn, spos2, sv2, sk3, sv0, spos0, sk1);
      tile0(i + 3, f, fn, spos3, sv3, sk0, sv1, spos1, sk2);
    }
    if (i < n_tiles) tile0(i, f, fn, spos0, sv0, sk1, sv2, spos2, sk3);
    if (i + 1 < n_tiles) tile0(i + 1, f, fn, spos1, sv1, sk2, sv3, spos3, sk0);
    if (i + 2 < n_tiles) tile0(i + 2, f, fn, spos2, sv2, sk3, sv0, spos0, sk1);
    barrier_keep_loads();                         // the half-1 waves' last phase
  } else {
    // phase 0: loads; phase 1: S_0
    fn = issue_block(0, sv1, spos1, sk2);
    barrier_keep_loads();
    if (f & 2) stream(sv0, sk0, std::integral_constant<int, 8>{}, std::integral_constant<int, 16>{});
    wait_rows1();
    barrier_keep_loads();
    int i = 0;
    for (; i + 4 <= n_tiles; i += 4) {
      tile1(i, f, fn, spos0, sv0, sk1, sv2, spos2, sk3);
      tile1(i + 1, f, fn, spos1, sv1, sk2, sv3, spos3, sk0);
      tile1(i + 2, f, fn, spos2, sv2, sk3, sv0, spos0, sk1);
      tile1(i + 3, f, fn, spos3, sv3, sk0, sv1, spos1, sk2);
    }
    if (i < n_tiles) tile1(i, f, fn, spos0, sv0, sk1, sv2, spos2, sk3);
    if (i + 1 < n_tiles) tile1(i + 1, f, fn, spos1, sv1, sk2, sv3, spos3, sk0);
    if (i + 2 < n_tiles) tile1(i + 2, f, fn, spos2, sv2, sk3, sv0, spos0, sk1);
  }
  __builtin_amdgcn_s_waitcnt(0);                  // no load into LDS outlives the workgroup

  const float lrun = osum[0];
  const float inv = lrun > 0.f ? 1.0f / lrun : 0.f;   // no visible key: output 0
  float* orow = a.out + ((static_cast<size_t>(b) * kv.Hq + h) * kv.T + q0 + l32) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      float4 v;
      v.x = o[dt][i4 * 4 + 0] * inv;
      v.y = o[dt][i4 * 4 + 1] * inv;
      v.z = o[dt][i4 * 4 + 2] * inv;
      v.w = o[dt][i4 * 4 + 3] * inv;
      *reinterpret_cast<float4*>(orow + dt * 32 + i4 * 8 + hi * 4) = v;
    }
}

template <int NH, int QH>
static void launch_mfma_lds(const AttnArgs& a, hipStream_t st) {
  const int G = a.kv.Hq / a.kv.Hkv;
  const int nwork = a.kv.B * a.kv.Hkv * (G / NH) * a.kv.nblk * (2 / QH);
  const int grid = (nwork + 7) / 8 * 8;
  DSA_LAUNCH(a.idx ? "attn_prefill" : "dense_prefill", (k_prefill_mfma_lds<NH, QH>), dim3(grid),
             dim3(64 * NH * QH), st, a);
}

template <int D, int NH, int QH>
static void launch_mfma(const AttnArgs& a, hipStream_t st) {
  const int G = a.kv.Hq / a.kv.Hkv;
  const int nwork = a.kv.B * a.kv.Hkv * (G / NH) * a.kv.nblk * (2 / QH);
  const int grid = (nwork + 7) / 8 * 8;
  const char* name = a.row_heads ? "attn_prefill_heads" : a.idx ? "attn_prefill" : "dense_prefill";
  DSA_LAUNCH(name, (k_prefill_mfma<D, NH, QH>), dim3(grid), dim3(64 * NH * QH), st, a);
}

// bf16 prefill over per-head block and column lists (d = 128, kv rows
// addressable with 32-bit byte offsets, lists 16-byte aligned with widths
// that are multiples of 4: checked by the caller).
void launch_prefill_lists(const AttnArgs& a, hipStream_t st) {
  const int nwork = a.kv.B * a.kv.Hq * a.kv.nblk;
  DSA_LAUNCH("attn_prefill_lists", k_prefill_heads<true>, dim3(nwork), dim3(128), st, a);
}

// bf16 prefill with query blocks of 64 rows; 4 waves per workgroup: the 4
// heads of a GQA group for one query half, or 2 heads / 1 head for both.
bool launch_prefill_mfma(const AttnArgs& a, hipStream_t st) {
  if (a.kv.decode || a.kv.bq != 64) return false;
  const int G = a.kv.Hq / a.kv.Hkv;
  // the LDS-direct kernels address a kv head's rows with 32-bit offsets and
  // read index rows 16 bytes at a time, whole 64-entry tiles for the shared
  // rows (the per-head kernel checks the end of its rows)
  const bool lds_ok = static_cast<long long>(a.kv.T) * 256 <= 0x7fffffffLL &&
                      (reinterpret_cast<uintptr_t>(a.idx) & 15) == 0 && (a.L & 3) == 0;
  const bool whole_tiles = a.idx == nullptr || (a.L & 63) == 0;
  if (a.row_heads) {                              // one head per workgroup
    if (a.kv.D == 128 && lds_ok) {
      const int nwork = a.kv.B * a.kv.Hq * a.kv.nblk;
      DSA_LAUNCH("attn_prefill_heads", k_prefill_heads<false>, dim3(nwork), dim3(128), st, a);
      return true;
    }
    if (a.kv.D == 128) { launch_mfma<128, 1, 2>(a, st); return true; }
    if (a.kv.D == 64) { launch_mfma<64, 1, 2>(a, st); return true; }
    return false;
  }
  if (a.kv.D == 128 && lds_ok && whole_tiles) {
    if (G >= 4 && a.idx) {
      const int nwork = a.kv.B * a.kv.Hkv * (G / 4) * a.kv.nblk;
      DSA_LAUNCH("attn_prefill", k_prefill_gqa8, dim3((nwork + 7) / 8 * 8), dim3(512), st, a);
      return true;
    }
    if (G >= 4) { launch_mfma_lds<4, 1>(a, st); return true; }
    if (G == 2) { launch_mfma_lds<2, 2>(a, st); return true; }
    if (G == 1) { launch_mfma<128, 1, 2>(a, st); return true; }
  } else if (a.kv.D == 64) {
    if (G >= 4) { launch_mfma<64, 4, 1>(a, st); return true; }
    if (G == 2) { launch_mfma<64, 2, 2>(a, st); return true; }
    if (G == 1) { launch_mfma<64, 1, 2>(a, st); return true; }
  }
  return false;
}

}  // namespace dsa
