// Internal declarations shared by the libdsa translation units: argument
// blocks passed by value to kernels, device helpers, and host launchers.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

constexpr int kMaxStages = 4;
constexpr float kNegBig = -1.0e30f;   // finite "no key yet" running max

// ------------------------------------------------------------------------- //
// argument blocks                                                           //
// ------------------------------------------------------------------------- //
// Paged decode: page ids kept per selected chunk (a chunk spanning more pages
// is left to the page table).
constexpr int kKeptPages = 8;

struct KvLayout {
  int B, Hq, Hkv, D;
  int T;                     // prefill length, or decode token stride / capacity
  int decode;                // 0 prefill, 1 decode
  int nblk, bq;              // query blocks per sequence and their size (decode: 1, 1)
  const int32_t* seq_lens;   // decode only
  const int32_t* block_table;// decode paged, else nullptr
  int page_size, page_shift, max_pages;
};

struct PruneArgs {
  KvLayout kv;
  const void* q;
  const void* k;
  int n_stages;
  int chunk[kMaxStages];
  int lchunk[kMaxStages];    // log2 of chunk[]
  int keep[kMaxStages];
  int n_sink, n_window;
  int32_t* idx;              // [R, L]
  int L;
  int R;                     // rows = B * nblk
  int maxK;                  // longest chunk-start list of any stage
  int maxNC;                 // longest chunk-score list of any stage
  int n1max;                 // most stage-1 chunks of any row
  int32_t* cnt;              // [R, kMaxStages] chunks kept by each stage
  int32_t* starts;           // [slots, R, maxK] kept chunk starts; stage i uses slot[i]
  int slot[kMaxStages];      // one call: slots alternate by stage parity; with remembered
                             // stages (mask caching) every stage owns its slot
  int32_t* mid_end;          // mask caching: [R, kMaxStages] end of the stage-1 middle each
                             // stage's record descends from; nullptr otherwise
  int32_t* row_status;       // mask caching: [R] 1 if the last row did not fit in L; or nullptr
  uint32_t* scores;          // [2, nsl, R, maxNC] orderable chunk-score keys, by stage parity
  unsigned long long* visited;  // [n_stages] or nullptr
  // Decode scoring: a workgroup holds the kv heads [s * hpw, (s + 1) * hpw) of
  // 16 / hpw chunks, hpw the largest divisor of Hkv up to 16; with more kv heads
  // than that (nsl = Hkv / hpw > 1) each slice s of workgroups writes its own
  // score list (the chunk maxima over its heads) and the readers take the max
  // over the nsl lists. Prefill and the generic paths: hpw = Hkv, nsl = 1.
  int hpw;
  int nsl;
  // Paged decode (or nullptr): the per-row top-K resolves the pages once for
  // the kernels after it. kpages [slots, R, maxK, kKeptPages]: the page ids of
  // every kept chunk's pages (first page first, -1 past the last or when the
  // chunk spans more than kKeptPages pages); prow [R, L]: the last stage's
  // index row with each position p turned into (page id << page_shift) |
  // (p mod page_size), -1 for padding.
  int32_t* kpages;
  int32_t* prow;
};

struct AttnArgs {
  KvLayout kv;
  const void* q;
  const void* k;
  const void* v;
  const int32_t* idx;        // nullptr => dense causal rows [0, e)
  const int32_t* prow;       // paged decode: idx with pages resolved (PruneArgs::prow), or nullptr
  int L;                     // idx row width
  float* out;
  float* part;               // decode split partials [B, Hq, n_splits, D + 2]
  int n_splits;
  int kps;                   // decode keys per split (multiple of 64)
  float scale_log2;          // softmax scale * log2(e)
  int row_heads;             // prefill: 0 = one idx row per (b, block) shared by the heads,
                             // 1 = one row per (b, q head, block): row (b * Hq + h) * nblk + m
  // per-head block and column lists instead of rows (row (b * Hq + h) * nblk + m)
  const int32_t* lblk;       // [.., wb] key-block ids, ascending
  const int32_t* lcol;       // [.., wc] single key positions, ascending (nullptr: none)
  const int32_t* lcnt;       // [.., 2] number of blocks, of columns
  int wb, wc;
};

// One fused decode step (decode_fused.hip): the pruning state of the call,
// V, the split partials and the output.
struct StepArgs {
  PruneArgs p;               // pruning state; p.idx receives the index rows
  const void* v;
  float* part;               // [B, Hq, nsp, D + 2] split partials (o[D], m, l)
  float* out;                // [B, Hq, D]
  float scale_log2;
  int nsp;                   // splits per row
  int sh0;                   // split sp holds row entries [sp * kStepSplitKeys - sh0, + kStepSplitKeys)
  int ks0, ks1;              // splits [ks0, ks1) may hold kept chunks (scheduled first)
};

// Block-sparse index estimation (MInference page, "Online Dynamic Index
// Estimation: Block-Sparse Heads (Algorithm 3)"): prefill, blocks of 64.
struct BsArgs {
  KvLayout kv;               // prefill layout; kv.nblk = T / 64
  const void* q;
  const void* k;
  int k_blocks;              // k_b: key blocks kept per (q head, query block)
  int nblkp;                 // score row stride (nblk rounded up to 4)
  double* qp;                // [B, Hq, nblk, D] pooled queries (fp64)
  double* kp;                // [B, Hkv, nblk, D] pooled keys (fp64)
  uint32_t* keys;            // [B, Hq, nblk, nblkp] orderable pooled-logit keys
  int32_t* idx;              // [B, Hq, nblk, L] index rows
  int L;                     // row width: 64 * k_blocks
  int32_t* lblk;             // block lists instead of rows (when set): [B, Hq, nblk, wb]
  int32_t* lcnt;             // [B, Hq, nblk, 2] number of blocks, 0 columns
  int wb;
};

// ------------------------------------------------------------------------- //
// device helpers                                                            //
// ------------------------------------------------------------------------- //
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Monotone map float -> uint32 (larger float => larger key) with -0 == +0.
__device__ __forceinline__ uint32_t score_key(float x) {
  if (x == 0.0f) x = 0.0f;
  uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct Geo {
  int s, e;        // query block [s, e)
  int sink_hi;     // sinks [0, sink_hi)
  int mid_hi;      // prunable middle [n_sink, mid_hi), window [mid_hi, e)
  int n1;          // whole stage-1 chunks
};

__device__ __forceinline__ Geo make_geo(int s, int e, int n_sink, int n_window, int l1) {
  Geo g;
  g.s = s;
  g.e = e;
  g.sink_hi = min(n_sink, e);
  int mid = max(0, e - n_window - n_sink);
  g.n1 = mid / l1;
  g.mid_hi = n_sink + g.n1 * l1;
  return g;
}

// Context length of decode sequence b, clamped to [0, T]: a length above the
// capacity the launch was sized for would index past the K/V rows (or the
// block table) and past the chunk lists; 0 makes an empty row (every index
// entry -1, output 0). Out-of-range lengths are caller errors that the
// checked mode (dsa_check_decode_inputs) reports; the clamp keeps them in
// bounds.
__device__ __forceinline__ int seq_len_of(const KvLayout& kv, int b) {
  return min(max(kv.seq_lens[b], 0), kv.T);
}

// Query block bounds of row r (decode: the last position of sequence r).
__device__ __forceinline__ void row_bounds(const KvLayout& kv, int r, int& b, int& s, int& e) {
  if (kv.decode) {
    b = r;
    e = seq_len_of(kv, r);
    s = e - 1;
  } else {
    b = r / kv.nblk;
    s = (r % kv.nblk) * kv.bq;
    e = s + kv.bq;
  }
}

// Element offset of key/value row (b, g, p).
__device__ __forceinline__ size_t kv_offset(const KvLayout& kv, int b, int g, int p) {
  if (kv.block_table) {
    int page = kv.block_table[static_cast<size_t>(b) * kv.max_pages + (p >> kv.page_shift)];
    return ((static_cast<size_t>(page) * kv.Hkv + g) * kv.page_size + (p & (kv.page_size - 1))) *
           kv.D;
  }
  return ((static_cast<size_t>(b) * kv.Hkv + g) * kv.T + p) * kv.D;
}

// Load N consecutive elements starting at ptr into fp32 registers.
template <typename T, int N>
struct SliceLoad;

template <int N>
struct SliceLoad<uint16_t, N> {
  static __device__ __forceinline__ void run(const uint16_t* ptr, float* out) {
    static_assert(N % 4 == 0, "bf16 slices are loaded 4 at a time");
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      uint2 w = *reinterpret_cast<const uint2*>(ptr + i);
      out[i + 0] = __uint_as_float(w.x << 16);
      out[i + 1] = __uint_as_float(w.x & 0xffff0000u);
      out[i + 2] = __uint_as_float(w.y << 16);
      out[i + 3] = __uint_as_float(w.y & 0xffff0000u);
    }
  }
};

template <int N>
struct SliceLoad<float, N> {
  static __device__ __forceinline__ void run(const float* ptr, float* out) {
    static_assert(N % 4 == 0, "fp32 slices are loaded 4 at a time");
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      float4 w = *reinterpret_cast<const float4*>(ptr + i);
      out[i + 0] = w.x;
      out[i + 1] = w.y;
      out[i + 2] = w.z;
      out[i + 3] = w.w;
    }
  }
};

// A lane's slice of one row, kept in its storage format: bf16 stays packed in
// pairs and dot products use the packed bf16 dot instruction (exact on the
// input grid: every product and partial sum is representable in fp32).
template <typename T, int N>
struct RowSlice;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int N>
struct RowSlice<uint16_t, N> {
  static_assert(N == 4 || N == 8, "bf16 slices hold 4 or 8 values");
  uint32_t w[N / 2];
  __device__ __forceinline__ void load(const uint16_t* p) {
    if constexpr (N == 8) {
      const uint4 x = *reinterpret_cast<const uint4*>(p);
      w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
    } else {
      const uint2 x = *reinterpret_cast<const uint2*>(p);
      w[0] = x.x; w[1] = x.y;
    }
  }
  __device__ __forceinline__ float dot(const RowSlice& o) const {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < N / 2; ++i)
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[i]),
                                            __builtin_bit_cast(bf16x2_t, o.w[i]), acc, false);
    return acc;
  }
};

template <int N>
struct RowSlice<float, N> {
  float v[N];
  __device__ __forceinline__ void load(const float* p) { SliceLoad<float, N>::run(p, v); }
  __device__ __forceinline__ float dot(const RowSlice& o) const {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < N; ++i) acc = fmaf(v[i], o.v[i], acc);
    return acc;
  }
};

template <typename T>
__device__ __forceinline__ float load_one(const T* p);
template <>
__device__ __forceinline__ float load_one<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }
template <>
__device__ __forceinline__ float load_one<float>(const float* p) { return *p; }

// ------------------------------------------------------------------------- //
// cross-lane primitives on DPP operand routing (VALU latency, no LDS round  //
// trip): a wave is 4 rows of 16 lanes                                       //
// ------------------------------------------------------------------------- //
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppRowMirror = 0x140;    // lane i <- 15 - i within the row
constexpr int kDppHalfMirror = 0x141;   // lane i <- 7 - i within each 8 lanes
constexpr int kDppRowShr = 0x110;       // + n: lane i <- i - n within the row
constexpr int kDppBcast15 = 0x142;      // lane 15 of a row -> the next row
constexpr int kDppBcast31 = 0x143;      // lane 31 -> rows 2 and 3

template <int CTRL>
__device__ __forceinline__ int dpp_perm(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}
// src routed by CTRL into the enabled rows; 0 where the row is masked off or
// the source lane lies outside the row
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_or0(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_perm_f(float v) {
  return __int_as_float(dpp_perm<CTRL>(__float_as_int(v)));
}

// Sum / max over the 16 lanes of a row (all lanes get the same bits: every
// lane combines the same partial results, in commuted order at most).
__device__ __forceinline__ float group16_sum(float v) {
  v += dpp_perm_f<kDppXor1>(v);
  v += dpp_perm_f<kDppXor2>(v);
  v += dpp_perm_f<kDppHalfMirror>(v);
  v += dpp_perm_f<kDppRowMirror>(v);
  return v;
}
__device__ __forceinline__ float group16_max(float v) {
  v = fmaxf(v, dpp_perm_f<kDppXor1>(v));
  v = fmaxf(v, dpp_perm_f<kDppXor2>(v));
  v = fmaxf(v, dpp_perm_f<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_perm_f<kDppRowMirror>(v));
  return v;
}

// Whole-wave reductions: rows first, then the four row results through
// scalar registers (the result is wave-uniform).
template <typename Op>
__device__ __forceinline__ int wave_reduce_int(int v, Op op) {
  v = op(v, dpp_perm<kDppXor1>(v));
  v = op(v, dpp_perm<kDppXor2>(v));
  v = op(v, dpp_perm<kDppHalfMirror>(v));
  v = op(v, dpp_perm<kDppRowMirror>(v));
  return op(op(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
            op(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
__device__ __forceinline__ int wave_sum_int(int v) {
  return wave_reduce_int(v, [](int x, int y) { return x + y; });
}
__device__ __forceinline__ float wave_max_f(float v) {
  return __int_as_float(wave_reduce_int(__float_as_int(v), [](int x, int y) {
    return __float_as_int(fmaxf(__int_as_float(x), __int_as_float(y)));
  }));
}
__device__ __forceinline__ float wave_sum_f(float v) {
  return __int_as_float(wave_reduce_int(__float_as_int(v), [](int x, int y) {
    return __float_as_int(__int_as_float(x) + __int_as_float(y));
  }));
}

// Inclusive prefix sum over the 64 lanes (lane order).
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  int x = static_cast<int>(v);
  x += dpp_or0<kDppRowShr + 1, 0xF>(x);
  x += dpp_or0<kDppRowShr + 2, 0xF>(x);
  x += dpp_or0<kDppRowShr + 4, 0xF>(x);
  x += dpp_or0<kDppRowShr + 8, 0xF>(x);
  x += dpp_or0<kDppBcast15, 0xA>(x);    // rows 1, 3 += last lane of rows 0, 2
  x += dpp_or0<kDppBcast31, 0xC>(x);    // rows 2, 3 += last lane of row 1
  return static_cast<uint32_t>(x);
}

// ------------------------------------------------------------------------- //
// launch with optional per-kernel timing (profile.hip)                      //
// ------------------------------------------------------------------------- //
// While profiling is on, prof_slot() hands out a start/stop event pair that the
// launch records at the kernel's own start and end (hipExtLaunchKernelGGL).
struct ProfSlot {
  hipEvent_t start = nullptr, stop = nullptr;
};
ProfSlot prof_slot(const char* name);

#define DSA_LAUNCH(NAME, KERNEL, GRID, BLOCK, STREAM, ...)                                  \
  do {                                                                                      \
    const ::dsa::ProfSlot dsa_ps_ = ::dsa::prof_slot(NAME);                                 \
    if (dsa_ps_.start)                                                                      \
      hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, 0, STREAM, dsa_ps_.start, dsa_ps_.stop, 0, \
                            __VA_ARGS__);                                                   \
    else                                                                                    \
      hipLaunchKernelGGL(KERNEL, GRID, BLOCK, 0, STREAM, __VA_ARGS__);                      \
  } while (0)

// ------------------------------------------------------------------------- //
// host launchers (defined in prune.hip / attn.hip)                          //
// ------------------------------------------------------------------------- //
hipError_t launch_prune(const PruneArgs& a, int dtype, hipStream_t stream);
// decode: every stage up to the last stage's scoring; the last top-K is left to
// the caller (the fused decode step).
hipError_t launch_prune_decode_stages(const PruneArgs& a, int dtype, hipStream_t stream);
// chunks the last stage's selection may see in one row
int last_stage_chunks(const PruneArgs& a);
// the fused tail of a decode step (last top-K + attention + merge); false if
// the shape takes the separate kernels (nothing launched then)
bool launch_decode_attend(const StepArgs& s, int sel_chunks, hipStream_t stream);
// bf16 decode split partials over index rows (d = 128, 2-8 query heads per kv head)
// and their merge; false for other shapes. a.n_splits = ceil(a.L / kStepSplitKeys).
bool launch_decode_rows(const AttnArgs& a, hipStream_t stream);
// bf16 decode split partials over spans of a.kps entries (dense when a.idx is
// null, else index rows; d = 128, 2-8 query heads per kv head) and their merge;
// false for other shapes.
bool launch_decode_span(const AttnArgs& a, hipStream_t stream);
constexpr int kStepSplitKeys = 128;   // index-row entries per workgroup of the fused tail
// Offset of the fused tail's split grid: the splits start at the end of the
// sinks, so the kept entries fill whole splits (with 64 sinks, 4,096 kept
// keys take 32 splits, not 33: one workgroup per CU for the 8 kv heads).
inline int step_split_shift(int n_sink) { return (kStepSplitKeys - n_sink % kStepSplitKeys) % kStepSplitKeys; }
// decode with remembered stages: only the stages flagged in due[] are recomputed
hipError_t launch_prune_cached(const PruneArgs& a, const bool* due, int dtype, hipStream_t stream);
hipError_t launch_sparse_attn(const AttnArgs& a, int dtype, hipStream_t stream);
// merge of decode split partials a.part [B, Hq, a.n_splits, D + 2] into a.out
void launch_decode_combine(const AttnArgs& a, hipStream_t stream);
hipError_t launch_block_sparse(const BsArgs& a, int dtype, hipStream_t stream);
bool launch_prefill_mfma(const AttnArgs& a, hipStream_t stream);   // bf16, b_q = 64
void launch_prefill_lists(const AttnArgs& a, hipStream_t stream);  // bf16, d = 128, per-head lists
struct PruneArgs;
// top-K of one stage over every row (prune.hip)
void launch_topk(const PruneArgs& a, int stage, int max_chunks, hipStream_t stream);
// pruning with RoPE inside SelectRep (prune_rope.hip). Relative style: qa, qb
// receive the two rotated query sets, [R, Hq, b_q, D] bf16 each. Chunk-indexed
// style: qa receives each stage's rotated queries in the layout of q (bf16),
// kb (prefill) each stage's rotated keys in the layout of k (bf16).
hipError_t launch_prune_rope(const PruneArgs& a, int dtype, int style, uint16_t* qa, uint16_t* qb, uint16_t* kb,
                             double base, hipStream_t stream);
// Chunk-indexed decode over per-stage rotated key copies (bf16, layout of k):
// the queries rotated for every stage into qa (stage s at qa + s * qstride),
// then the plain decode stages on the rotated vectors.
hipError_t launch_prune_rope_keys(const PruneArgs& a, int dtype, uint16_t* qa, size_t qstride,
                                  uint16_t* const* k_rot, double base, hipStream_t stream);
// Rotated copies (bf16) of the keys at positions [p_lo, p_hi) for every stage.
hipError_t launch_rope_rotate_keys(const PruneArgs& a, int dtype, uint16_t* const* k_rot, double base, int p_lo,
                                   int p_hi, hipStream_t stream);
// Decode stages with per-stage arguments (bf16 rows), as[0 .. n_stages).
hipError_t launch_prune_decode_staged(const PruneArgs* as, hipStream_t stream);
// plain scoring of a prefill stage on bf16 rows (prune.hip)
void launch_score_prefill_bf16(const PruneArgs& a, int stage, int max_chunks, hipStream_t stream, const char* name);
// bf16, b_q = 64; ql and qr (the rotated query sets) select the relative-RoPE
// tournaments, nullptr the plain ones
bool launch_score_prefill_mfma(const PruneArgs& a, int stage, int max_chunks, hipStream_t stream,
                               const char* name, const uint16_t* ql = nullptr, const uint16_t* qr = nullptr);

}  // namespace dsa
