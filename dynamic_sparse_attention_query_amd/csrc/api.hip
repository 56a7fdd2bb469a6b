// C ABI of libdsa: argument validation, workspace layout and launch order.
// The rules checked here are the ones documented in include/dsa.h.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "dsa.h"
#include "dsa_internal.h"
#include "vs_internal.h"

// Scratch memory of dsa_prune_attend_static (see below): a file-scope device
// array, one copy per GPU.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

thread_local char g_err[512] = "";

dsa_status fail(dsa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

bool is_pow2(long long x) { return x > 0 && (x & (x - 1)) == 0; }

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

dsa_status check_shape(const dsa_shape* s) {
  if (!s) return fail(DSA_ERR_INVALID_ARG, "shape is NULL");
  if (s->mode != DSA_PREFILL && s->mode != DSA_DECODE)
    return fail(DSA_ERR_INVALID_ARG, "mode %d is not DSA_PREFILL or DSA_DECODE", s->mode);
  if (s->dtype != DSA_F32 && s->dtype != DSA_BF16)
    return fail(DSA_ERR_INVALID_ARG, "dtype %d is not DSA_F32 or DSA_BF16", s->dtype);
  if (s->batch < 1 || s->hq < 1 || s->hkv < 1 || s->t < 1)
    return fail(DSA_ERR_INVALID_ARG, "batch, hq, hkv and t must be >= 1");
  if (s->hq % s->hkv != 0) return fail(DSA_ERR_INVALID_ARG, "hq %% hkv != 0");
  const int G = s->hq / s->hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(DSA_ERR_UNSUPPORTED, "hq / hkv = %d; supported group sizes are 1, 2, 4, 8", G);
  if (s->d != 64 && s->d != 128) return fail(DSA_ERR_UNSUPPORTED, "d = %d; supported: 64, 128", s->d);
  if (s->mode == DSA_DECODE) {
    if (!s->seq_lens) return fail(DSA_ERR_INVALID_ARG, "decode needs seq_lens");
    if (s->block_table) {
      if (!is_pow2(s->page_size)) return fail(DSA_ERR_INVALID_ARG, "page_size must be a power of two");
      if (s->max_pages < 1 || static_cast<long long>(s->max_pages) * s->page_size < s->t)
        return fail(DSA_ERR_INVALID_ARG, "max_pages * page_size must be >= t");
    }
  }
  return DSA_OK;
}

dsa_status check_params(const dsa_shape* s, const dsa_params* p) {
  if (!p) return fail(DSA_ERR_INVALID_ARG, "params is NULL");
  if (p->n_stages < 1 || p->n_stages > DSA_MAX_STAGES)
    return fail(DSA_ERR_INVALID_ARG, "n_stages = %d not in [1, %d]", p->n_stages, DSA_MAX_STAGES);
  for (int i = 0; i < p->n_stages; ++i) {
    if (!is_pow2(p->chunk[i])) return fail(DSA_ERR_INVALID_ARG, "chunk[%d] = %d is not a power of two", i, p->chunk[i]);
    if (p->keep[i] < 0 || p->keep[i] % p->chunk[i] != 0)
      return fail(DSA_ERR_INVALID_ARG, "keep[%d] = %d is not a non-negative multiple of chunk[%d]", i, p->keep[i], i);
    if (i > 0) {
      if (p->chunk[i - 1] % p->chunk[i] != 0)
        return fail(DSA_ERR_INVALID_ARG, "chunk[%d] does not divide chunk[%d]", i, i - 1);
      if (p->keep[i] > p->keep[i - 1]) return fail(DSA_ERR_INVALID_ARG, "keep[%d] > keep[%d]", i, i - 1);
    }
    if (p->keep[i] / p->chunk[i] > 8192)
      return fail(DSA_ERR_UNSUPPORTED, "keep[%d] / chunk[%d] > 8192 kept chunks", i, i);
  }
  if (p->n_sink < 0 || p->n_window < 0) return fail(DSA_ERR_INVALID_ARG, "n_sink and n_window must be >= 0");
  if (s) {
    if (s->mode == DSA_DECODE) {
      if (p->block_q != 1) return fail(DSA_ERR_INVALID_ARG, "decode requires block_q == 1");
    } else {
      if (p->block_q < 4 || p->block_q > 64 || !is_pow2(p->block_q))
        return fail(DSA_ERR_UNSUPPORTED, "prefill block_q = %d; supported: 4, 8, 16, 32, 64", p->block_q);
      if (s->t % p->block_q != 0) return fail(DSA_ERR_INVALID_ARG, "t %% block_q != 0");
    }
  }
  return DSA_OK;
}

long long index_width_ll(const dsa_params* p) {
  long long n = static_cast<long long>(p->n_sink) + p->keep[p->n_stages - 1] + p->n_window + p->chunk[0] - 1;
  return (n + 63) / 64 * 64;
}

struct PruneLayout {
  long long R, maxK, maxNC, n1max;
  int hpw, nsl;                       // decode scoring: kv heads per workgroup, score slices
  size_t off_cnt, off_starts, off_scores, bytes;
  size_t off_kpages, off_prow;        // paged decode: resolved pages (0: not laid out)
};

// Decode scoring holds the kv heads of a chunk in one workgroup of 16 lane
// groups when they fit: hpw = the largest divisor of hkv up to 16, and the
// hkv / hpw slices of heads write score lists of their own (maxed by the
// readers). Prefill scoring keeps every head of a row in one workgroup.
void head_slices(const dsa_shape* s, int& hpw, int& nsl) {
  hpw = s->hkv;
  nsl = 1;
  if (s->mode != DSA_DECODE) return;
  hpw = 1;
  for (int x = 1; x <= 16; ++x)
    if (s->hkv % x == 0) hpw = x;
  nsl = s->hkv / hpw;
}

PruneLayout prune_layout(const dsa_shape* s, const dsa_params* p) {
  PruneLayout L{};
  const long long nblk = s->mode == DSA_DECODE ? 1 : s->t / p->block_q;
  L.R = static_cast<long long>(s->batch) * nblk;
  long long maxK = 1, maxNC = 1;
  for (int i = 0; i < p->n_stages; ++i) maxK = std::max<long long>(maxK, p->keep[i] / p->chunk[i]);
  const long long mid = std::max<long long>(0, static_cast<long long>(s->t) - p->n_window - p->n_sink);
  L.n1max = mid / p->chunk[0];
  maxNC = std::max<long long>(maxNC, L.n1max);
  for (int i = 1; i < p->n_stages; ++i) maxNC = std::max<long long>(maxNC, p->keep[i - 1] / p->chunk[i]);
  L.maxK = maxK;
  L.maxNC = (maxNC + 63) / 64 * 64;   // rows of whole 16-byte key groups
  head_slices(s, L.hpw, L.nsl);
  L.off_cnt = 0;
  L.off_starts = align256(L.off_cnt + static_cast<size_t>(L.R) * dsa::kMaxStages * 4);
  L.off_scores = align256(L.off_starts + 2 * static_cast<size_t>(L.R) * maxK * 4);
  // two sets of score lists (stage parity), one list per head slice
  L.bytes = align256(L.off_scores + 2 * static_cast<size_t>(L.nsl) * L.R * L.maxNC * 4);
  if (s->mode == DSA_DECODE && s->block_table) {
    // paged: the kept chunks' page ids (two slots) and the page-resolved row
    L.off_kpages = L.bytes;
    L.off_prow = align256(L.off_kpages + 2 * static_cast<size_t>(L.R) * maxK * dsa::kKeptPages * 4);
    L.bytes = align256(L.off_prow + static_cast<size_t>(L.R) * index_width_ll(p) * 4);
  }
  return L;
}

// decode split geometry: 64-key sub-tiles, at most ~512 splits per (sequence, kv head)
int keys_per_split(long long n_total) {
  const long long per = (n_total + 64LL * 512 - 1) / (64LL * 512);
  return static_cast<int>(64 * std::max<long long>(1, per));
}

size_t attn_bytes(const dsa_shape* s, long long n_total) {
  if (s->mode != DSA_DECODE) return 0;
  const int kps = keys_per_split(n_total);
  const long long n_splits = (n_total + kps - 1) / kps;
  return align256(static_cast<size_t>(s->batch) * s->hq * n_splits * (s->d + 2) * 4);
}

// Workspace of dsa_prune_attend: the pruning state and the attention partials
// (split partials of the fused decode tail or of the separate kernels).
struct StepLayout {
  PruneLayout pl;
  long long nsp;
  size_t off_part, bytes;
};

StepLayout step_layout(const dsa_shape* s, const dsa_params* p) {
  StepLayout L{};
  L.pl = prune_layout(s, p);
  const long long width = index_width_ll(p);
  L.nsp = (width + dsa::step_split_shift(p->n_sink) + dsa::kStepSplitKeys - 1) / dsa::kStepSplitKeys;
  const size_t fused = s->mode == DSA_DECODE
                           ? static_cast<size_t>(s->batch) * s->hq * L.nsp * (s->d + 2) * 4 : 0;
  L.off_part = align256(L.pl.bytes);
  L.bytes = L.off_part + align256(std::max(fused, attn_bytes(s, width)));
  return L;
}

dsa::KvLayout make_kv(const dsa_shape* s, int bq) {
  dsa::KvLayout kv{};
  kv.B = s->batch;
  kv.Hq = s->hq;
  kv.Hkv = s->hkv;
  kv.D = s->d;
  kv.T = s->t;
  kv.decode = s->mode == DSA_DECODE;
  kv.bq = kv.decode ? 1 : bq;
  kv.nblk = kv.decode ? 1 : s->t / bq;
  kv.seq_lens = kv.decode ? s->seq_lens : nullptr;
  kv.block_table = kv.decode ? s->block_table : nullptr;
  kv.page_size = kv.block_table ? s->page_size : 1;
  int shift = 0;
  while ((1 << shift) < kv.page_size) ++shift;
  kv.page_shift = shift;
  kv.max_pages = kv.block_table ? s->max_pages : 0;
  return kv;
}

// prow (paged decode, or nullptr): idx with its pages resolved, written by the
// same call's pruning.
dsa_status run_attn(const dsa_shape* s, const void* q, const void* k, const void* v, const int32_t* idx,
                    int32_t L, int bq, float scale, float* out, void* ws, size_t ws_bytes, void* stream,
                    const int32_t* prow = nullptr) {
  const long long n_total = idx ? L : s->t;
  const size_t need = attn_bytes(s, n_total);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes, need);
  dsa::AttnArgs a{};
  a.kv = make_kv(s, bq);
  a.q = q;
  a.k = k;
  a.v = v;
  a.idx = idx;
  a.prow = prow;
  a.L = L;
  a.out = out;
  a.part = static_cast<float*>(ws);
  a.kps = keys_per_split(n_total);
  a.n_splits = static_cast<int>((n_total + a.kps - 1) / a.kps);
  const float sc = scale > 0.f ? scale : 1.0f / std::sqrt(static_cast<float>(s->d));
  a.scale_log2 = sc * 1.4426950408889634f;
  // bf16 decode over index rows: the fused step's split kernel (splits of
  // kStepSplitKeys entries, which the workspace holds while they are no fewer
  // entries than keys_per_split's)
  if (s->mode == DSA_DECODE && s->dtype == DSA_BF16 && idx && a.kps <= dsa::kStepSplitKeys) {
    dsa::AttnArgs r = a;
    r.kps = dsa::kStepSplitKeys;
    r.n_splits = static_cast<int>((n_total + r.kps - 1) / r.kps);
    if (dsa::launch_decode_rows(r, static_cast<hipStream_t>(stream))) {
      const hipError_t e2 = hipGetLastError();
      if (e2 != hipSuccess) return fail(DSA_ERR_HIP, "attention launch failed: %s", hipGetErrorString(e2));
      return DSA_OK;
    }
  }
  // other bf16 decode (the dense path, longer rows): spans of a.kps entries
  if (s->mode == DSA_DECODE && s->dtype == DSA_BF16 && dsa::launch_decode_span(a, static_cast<hipStream_t>(stream))) {
    const hipError_t e2 = hipGetLastError();
    if (e2 != hipSuccess) return fail(DSA_ERR_HIP, "attention launch failed: %s", hipGetErrorString(e2));
    return DSA_OK;
  }
  hipError_t err = dsa::launch_sparse_attn(a, s->dtype, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(DSA_ERR_HIP, "attention launch failed: %s", hipGetErrorString(err));
  return DSA_OK;
}


// Scratch memory of dsa_prune_attend_static, for callers that cannot allocate:
// one array per GPU in the library's device code, held until the process
// ends. Host code never uses the array's name as an address (on the host it
// is only a handle): the device address comes from hipGetSymbolAddress, once
// per device with that device current, and is kept per device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

dsa_status static_scratch(void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return fail(DSA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(err));
  if (dev < 0 || dev >= kMaxDevices) return fail(DSA_ERR_UNSUPPORTED, "device %d beyond the static scratch table", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err != hipSuccess || !ptr)
      return fail(DSA_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(err));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}

}  // namespace

extern "C" {

const char* dsa_status_str(dsa_status s) {
  switch (s) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_ARG: return "DSA_ERR_INVALID_ARG";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE";
    case DSA_ERR_HIP: return "DSA_ERR_HIP";
  }
  return "DSA_ERR_UNKNOWN";
}

const char* dsa_last_error(void) { return g_err; }

int32_t dsa_index_width(const dsa_params* p) {
  if (check_params(nullptr, p) != DSA_OK) return -1;
  const long long w = index_width_ll(p);
  if (w > (1LL << 30)) return -1;
  return static_cast<int32_t>(w);
}

dsa_status dsa_workspace_bytes(const dsa_shape* s, const dsa_params* p, size_t* out_bytes) {
  g_err[0] = 0;
  if (!out_bytes) return fail(DSA_ERR_INVALID_ARG, "out_bytes is NULL");
  dsa_status st = check_shape(s);
  if (st != DSA_OK) return st;
  size_t bytes = attn_bytes(s, s->t);
  if (p) {
    st = check_params(s, p);
    if (st != DSA_OK) return st;
    bytes = std::max(bytes, prune_layout(s, p).bytes);
    bytes = std::max(bytes, attn_bytes(s, index_width_ll(p)));
    bytes = std::max(bytes, step_layout(s, p).bytes);
  }
  *out_bytes = bytes;
  return DSA_OK;
}

}  // extern "C"

namespace {

// Argument block of a pruning call (validated by the caller); the kept-start
// lists and counts live in the workspace unless a mask cache supplies them.
dsa::PruneArgs prune_args(const dsa_shape* s, const void* q, const void* k, const dsa_params* p,
                          int32_t* idx, long long L, const PruneLayout& lay, void* ws,
                          uint64_t* visited) {
  dsa::PruneArgs a{};
  a.kv = make_kv(s, p->block_q);
  a.q = q;
  a.k = k;
  a.n_stages = p->n_stages;
  for (int i = 0; i < DSA_MAX_STAGES; ++i) {
    a.chunk[i] = i < p->n_stages ? p->chunk[i] : 1;
    a.lchunk[i] = 0;
    while ((1 << a.lchunk[i]) < a.chunk[i]) ++a.lchunk[i];
    a.keep[i] = i < p->n_stages ? p->keep[i] : 0;
  }
  a.n_sink = p->n_sink;
  a.n_window = p->n_window;
  a.idx = idx;
  a.L = static_cast<int>(L);
  a.R = static_cast<int>(lay.R);
  a.maxK = static_cast<int>(lay.maxK);
  a.maxNC = static_cast<int>(lay.maxNC);
  a.n1max = static_cast<int>(lay.n1max);
  a.hpw = lay.hpw;
  a.nsl = lay.nsl;
  for (int i = 0; i < DSA_MAX_STAGES; ++i) a.slot[i] = i & 1;
  if (ws) {                                       // no workspace: the call reads none of it
    char* w = static_cast<char*>(ws);
    a.cnt = reinterpret_cast<int32_t*>(w + lay.off_cnt);
    a.starts = reinterpret_cast<int32_t*>(w + lay.off_starts);
    a.scores = reinterpret_cast<uint32_t*>(w + lay.off_scores);
  }
  a.visited = reinterpret_cast<unsigned long long*>(visited);
  a.kpages = nullptr;
  a.prow = nullptr;
  return a;
}

// Plain paged decode (no remembered stages, no RoPE): the per-row top-K
// resolves the kept chunks' pages for the next stage, and with `row` the last
// stage's index row too.
// (Pages of at least 8 positions: the row writer resolves four consecutive
// positions with two table reads.)
void attach_pages(dsa::PruneArgs& a, const dsa_shape* s, const PruneLayout& lay, void* ws, bool row) {
  if (s->mode != DSA_DECODE || !s->block_table || !ws || lay.off_kpages == 0 || s->page_size < 8) return;
  char* w = static_cast<char*>(ws);
  a.kpages = reinterpret_cast<int32_t*>(w + lay.off_kpages);
  if (row) a.prow = reinterpret_cast<int32_t*>(w + lay.off_prow);
}

// Mask cache layout: status [B], then per-sequence stage records (kept counts,
// middle ends) and the kept-start lists, one slot per stage.
struct CacheLayout {
  size_t off_cnt, off_mid, off_starts, bytes;
};

CacheLayout cache_layout(const dsa_shape* s, const dsa_params* p, const PruneLayout& lay) {
  CacheLayout c{};
  const size_t B = static_cast<size_t>(s->batch);
  c.off_cnt = align256(B * 4);
  c.off_mid = c.off_cnt + align256(B * dsa::kMaxStages * 4);
  c.off_starts = c.off_mid + align256(B * dsa::kMaxStages * 4);
  c.bytes = align256(c.off_starts + static_cast<size_t>(p->n_stages) * B * lay.maxK * 4);
  return c;
}

long long cached_width_ll(const dsa_params* p, long long max_growth) {
  const long long n = static_cast<long long>(p->n_sink) + p->keep[p->n_stages - 1] + p->n_window +
                      p->chunk[0] - 1 + max_growth;
  return (n + 63) / 64 * 64;
}

// Validation shared by dsa_prune_attend and dsa_prune_attend_static; fills
// the workspace layout of the call.
dsa_status check_prune_attend(const dsa_shape* s, const void* q, const void* k, const void* v,
                              const dsa_params* p, const int32_t* idx, const float* out, StepLayout* lay) {
  dsa_status st = check_shape(s);
  if (st != DSA_OK) return st;
  st = check_params(s, p);
  if (st != DSA_OK) return st;
  if (!q || !k || !v || !idx || !out) return fail(DSA_ERR_INVALID_ARG, "q, k, v, idx and out must be non-NULL");
  if (index_width_ll(p) > (1LL << 30)) return fail(DSA_ERR_INVALID_ARG, "index width overflows");
  *lay = step_layout(s, p);
  if (lay->pl.maxNC > 32768)
    return fail(DSA_ERR_UNSUPPORTED, "a stage would score %lld chunks per row (limit 32768)", lay->pl.maxNC);
  return DSA_OK;
}

// The launches of one prune-and-attend call on a validated shape and a
// workspace of at least lay.bytes bytes.
dsa_status run_prune_attend(const dsa_shape* s, const void* q, const void* k, const void* v, const dsa_params* p,
                            float scale, int32_t* idx, float* out, void* ws, const StepLayout& lay,
                            uint64_t* visited, void* stream) {
  const long long L = index_width_ll(p);
  char* wsc = static_cast<char*>(ws);
  dsa::PruneArgs a = prune_args(s, q, k, p, idx, L, lay.pl, ws, visited);
  attach_pages(a, s, lay.pl, ws, true);
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const float sc = scale > 0.f ? scale : 1.0f / std::sqrt(static_cast<float>(s->d));
  hipError_t err = hipSuccess;
  bool fused = false;
  if (s->mode == DSA_DECODE && s->dtype == DSA_BF16) {
    err = dsa::launch_prune_decode_stages(a, s->dtype, hs);
    if (err != hipSuccess) return fail(DSA_ERR_HIP, "prune launch failed: %s", hipGetErrorString(err));
    dsa::StepArgs sa{};
    sa.p = a;
    sa.v = v;
    sa.part = reinterpret_cast<float*>(wsc + lay.off_part);
    sa.out = out;
    sa.scale_log2 = sc * 1.4426950408889634f;
    sa.nsp = static_cast<int>(lay.nsp);
    {
      const int ls = p->n_stages - 1;
      const long long kept_hi = static_cast<long long>(p->n_sink) + p->keep[ls];   // most kept entries
      sa.sh0 = dsa::step_split_shift(p->n_sink);
      sa.ks0 = std::min<int>(sa.nsp, (p->n_sink + sa.sh0) / dsa::kStepSplitKeys);
      sa.ks1 = static_cast<int>(
          std::min<long long>(sa.nsp, (kept_hi + sa.sh0 + dsa::kStepSplitKeys - 1) / dsa::kStepSplitKeys));
      sa.ks1 = std::max(sa.ks1, sa.ks0);
    }
    fused = dsa::launch_decode_attend(sa, dsa::last_stage_chunks(a), hs);
    if (!fused) dsa::launch_topk(a, p->n_stages - 1, dsa::last_stage_chunks(a), hs);
    err = hipGetLastError();
  } else {
    err = dsa::launch_prune(a, s->dtype, hs);
  }
  if (err != hipSuccess) return fail(DSA_ERR_HIP, "prune launch failed: %s", hipGetErrorString(err));
  if (fused) return DSA_OK;
  return run_attn(s, q, k, v, idx, static_cast<int32_t>(L), p->block_q, scale, out, wsc + lay.off_part,
                  lay.bytes - lay.off_part, stream, a.prow);
}


}  // namespace

extern "C" {

dsa_status dsa_prune_select(const dsa_shape* s, const void* q, const void* k, const dsa_params* p,
                            int32_t* idx, void* ws, size_t ws_bytes, uint64_t* visited, void* stream) {
  g_err[0] = 0;
  dsa_status st = check_shape(s);
  if (st != DSA_OK) return st;
  st = check_params(s, p);
  if (st != DSA_OK) return st;
  if (!q || !k || !idx) return fail(DSA_ERR_INVALID_ARG, "q, k and idx must be non-NULL");
  const long long L = index_width_ll(p);
  if (L > (1LL << 30)) return fail(DSA_ERR_INVALID_ARG, "index width overflows");
  const PruneLayout lay = prune_layout(s, p);
  if (lay.maxNC > 32768)
    return fail(DSA_ERR_UNSUPPORTED, "a stage would score %lld chunks per row (limit 32768)", lay.maxNC);
  if (!ws || ws_bytes < lay.bytes)
    return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes, lay.bytes);
  dsa::PruneArgs a = prune_args(s, q, k, p, idx, L, lay, ws, visited);
  attach_pages(a, s, lay, ws, false);
  hipError_t err = dsa::launch_prune(a, s->dtype, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(DSA_ERR_HIP, "prune launch failed: %s", hipGetErrorString(err));
  return DSA_OK;
}

int32_t dsa_cached_index_width(const dsa_params* p, int32_t max_growth) {
  if (check_params(nullptr, p) != DSA_OK || max_growth < 0) return -1;
  const long long w = cached_width_ll(p, max_growth);
  if (w > (1LL << 30)) return -1;
  return static_cast<int32_t>(w);
}

dsa_status dsa_mask_cache_bytes(const dsa_shape* s, const dsa_params* p, size_t* out_bytes) {
  g_err[0] = 0;
  if (!out_bytes) return fail(DSA_ERR_INVALID_ARG, "out_bytes is NULL");
  dsa_status st = check_shape(s);
  if (st != DSA_OK) return st;
  if (s->mode != DSA_DECODE) return fail(DSA_ERR_INVALID_ARG, "mask caching is a decode feature");
  st = check_params(s, p);
  if (st != DSA_OK) return st;
  *out_bytes = cache_layout(s, p, prune_layout(s, p)).bytes;
  return DSA_OK;
}

dsa_status dsa_prune_select_cached(const dsa_shape* s, const void* q, const void* k, const dsa_params* p,
                                   const int32_t* refresh, int64_t step, void* cache, size_t cache_bytes,
                                   int32_t* idx, int32_t idx_width, void* ws, size_t ws_bytes,
                                   uint64_t* visited, void* stream) {
  g_err[0] = 0;
  dsa_status st = check_shape(s);
  if (st != DSA_OK) return st;
  if (s->mode != DSA_DECODE) return fail(DSA_ERR_INVALID_ARG, "mask caching is a decode feature");
  st = check_params(s, p);
  if (st != DSA_OK) return st;
  if (!q || !k || !idx || !cache) return fail(DSA_ERR_INVALID_ARG, "q, k, idx and cache must be non-NULL");
  if (!refresh) return fail(DSA_ERR_INVALID_ARG, "refresh is NULL");
  if (step < 0) return fail(DSA_ERR_INVALID_ARG, "step must be >= 0");
  bool due[DSA_MAX_STAGES] = {false, false, false, false};
  for (int i = 0; i < p->n_stages; ++i) {
    if (refresh[i] < 1) return fail(DSA_ERR_INVALID_ARG, "refresh[%d] = %d must be >= 1", i, refresh[i]);
    due[i] = step % refresh[i] == 0;
  }
  if (idx_width < index_width_ll(p) || idx_width % 64 != 0)
    return fail(DSA_ERR_INVALID_ARG, "idx_width %d must be a multiple of 64 and >= dsa_index_width (%lld)",
                idx_width, index_width_ll(p));
  if (reinterpret_cast<uintptr_t>(idx) % 16 != 0 || reinterpret_cast<uintptr_t>(cache) % 16 != 0)
    return fail(DSA_ERR_INVALID_ARG, "idx and cache must be 16-byte aligned");
  const PruneLayout lay = prune_layout(s, p);
  if (lay.maxNC > 32768)
    return fail(DSA_ERR_UNSUPPORTED, "a stage would score %lld chunks per row (limit 32768)", lay.maxNC);
  if (!ws || ws_bytes < lay.bytes)
    return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes, lay.bytes);
  const CacheLayout cl = cache_layout(s, p, lay);
  if (cache_bytes < cl.bytes)
    return fail(DSA_ERR_INVALID_ARG, "mask cache of %zu bytes is smaller than the %zu needed", cache_bytes, cl.bytes);
  dsa::PruneArgs a = prune_args(s, q, k, p, idx, idx_width, lay, ws, visited);
  char* c = static_cast<char*>(cache);
  a.row_status = reinterpret_cast<int32_t*>(c);
  a.cnt = reinterpret_cast<int32_t*>(c + cl.off_cnt);
  a.mid_end = reinterpret_cast<int32_t*>(c + cl.off_mid);
  a.starts = reinterpret_cast<int32_t*>(c + cl.off_starts);
  for (int i = 0; i < DSA_MAX_STAGES; ++i) a.slot[i] = i < p->n_stages ? i : 0;
  hipError_t err = dsa::launch_prune_cached(a, due, s->dtype, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(DSA_ERR_HIP, "prune launch failed: %s", hipGetErrorString(err));
  return DSA_OK;
}

dsa_status dsa_sparse_attn(const dsa_shape* s, const void* q, const void* k, const void* v,
                           const int32_t* idx, int32_t idx_width, int32_t block_q, float scale,
                           float* out, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  dsa_status st = check_shape(s);
  if (st != DSA_OK) return st;
  if (!q || !k || !v || !idx || !out) return fail(DSA_ERR_INVALID_ARG, "q, k, v, idx and out must be non-NULL");
  if (idx_width < 1) return fail(DSA_ERR_INVALID_ARG, "idx_width must be >= 1");
  if (s->mode == DSA_DECODE) {
    if (block_q != 1) return fail(DSA_ERR_INVALID_ARG, "decode requires block_q == 1");
  } else {
    if (block_q < 4 || block_q > 64 || !is_pow2(block_q))
      return fail(DSA_ERR_UNSUPPORTED, "prefill block_q = %d; supported: 4, 8, 16, 32, 64", block_q);
    if (s->t % block_q != 0) return fail(DSA_ERR_INVALID_ARG, "t %% block_q != 0");
  }
  return run_attn(s, q, k, v, idx, idx_width, block_q, scale, out, ws, ws_bytes, stream);
}

dsa_status dsa_prune_attend(const dsa_shape* s, const void* q, const void* k, const void* v,
                            const dsa_params* p, float scale, int32_t* idx, float* out, void* ws,
                            size_t ws_bytes, uint64_t* visited, void* stream) {
  g_err[0] = 0;
  StepLayout lay{};
  dsa_status st = check_prune_attend(s, q, k, v, p, idx, out, &lay);
  if (st != DSA_OK) return st;
  if (!ws || ws_bytes < lay.bytes)
    return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes, lay.bytes);
  return run_prune_attend(s, q, k, v, p, scale, idx, out, ws, lay, visited, stream);
}

dsa_status dsa_prune_attend_static(const dsa_shape* s, const void* q, const void* k, const void* v,
                                   const dsa_params* p, float scale, int32_t* idx, float* out,
                                   uint64_t* visited, void* stream) {
  g_err[0] = 0;
  StepLayout lay{};
  dsa_status st = check_prune_attend(s, q, k, v, p, idx, out, &lay);
  if (st != DSA_OK) return st;
  if (lay.bytes > kStaticScratchBytes)
    return fail(DSA_ERR_UNSUPPORTED, "this shape needs %zu bytes of scratch; the static scratch holds %zu",
                lay.bytes, kStaticScratchBytes);
  void* ws = nullptr;
  st = static_scratch(&ws);
  if (st != DSA_OK) return st;
  return run_prune_attend(s, q, k, v, p, scale, idx, out, ws, lay, visited, stream);
}

dsa_status dsa_check_decode_inputs(const dsa_shape* s, const int32_t* seq_lens, const int32_t* block_table,
                                   int64_t n_pages) {
  g_err[0] = 0;
  dsa_status st = check_shape(s);
  if (st != DSA_OK) return st;
  if (s->mode != DSA_DECODE) return fail(DSA_ERR_INVALID_ARG, "checked mode covers decode shapes");
  if (!seq_lens) return fail(DSA_ERR_INVALID_ARG, "seq_lens (host copy) is NULL");
  for (int b = 0; b < s->batch; ++b)
    if (seq_lens[b] < 1 || seq_lens[b] > s->t)
      return fail(DSA_ERR_INVALID_ARG, "seq_lens[%d] = %d is not in [1, t = %d]", b, seq_lens[b], s->t);
  if (s->block_table) {
    if (!block_table) return fail(DSA_ERR_INVALID_ARG, "a paged shape needs the block table (host copy)");
    if (n_pages < 1) return fail(DSA_ERR_INVALID_ARG, "n_pages = %lld must be >= 1", static_cast<long long>(n_pages));
    for (int b = 0; b < s->batch; ++b) {
      const long long used = (static_cast<long long>(seq_lens[b]) + s->page_size - 1) / s->page_size;
      for (long long i = 0; i < used; ++i) {
        const int32_t id = block_table[static_cast<size_t>(b) * s->max_pages + i];
        if (id < 0 || id >= n_pages)
          return fail(DSA_ERR_INVALID_ARG, "block_table[%d][%lld] = %d is not a page of the pool [0, %lld)", b, i, id,
                      static_cast<long long>(n_pages));
      }
    }
  }
  return DSA_OK;
}

dsa_status dsa_dense_attn(const dsa_shape* s, const void* q, const void* k, const void* v, float scale,
                          float* out, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  dsa_status st = check_shape(s);
  if (st != DSA_OK) return st;
  if (!q || !k || !v || !out) return fail(DSA_ERR_INVALID_ARG, "q, k, v and out must be non-NULL");
  int bq = 64;
  if (s->mode == DSA_PREFILL) {
    while (bq > 4 && s->t % bq != 0) bq >>= 1;
    if (s->t % bq != 0) return fail(DSA_ERR_UNSUPPORTED, "dense prefill needs t to be a multiple of 4");
  }
  return run_attn(s, q, k, v, nullptr, 0, bq, scale, out, ws, ws_bytes, stream);
}


}  // extern "C"

namespace {

constexpr int kBsBlock = 64;
constexpr long long kBsMaxBlocks = 16384;          // query blocks per sequence the top-K holds

dsa_status check_block_sparse(const dsa_shape* s, int32_t k_blocks) {
  dsa_status st = check_shape(s);
  if (st != DSA_OK) return st;
  if (s->mode != DSA_PREFILL) return fail(DSA_ERR_INVALID_ARG, "block-sparse estimation is a prefill call");
  if (s->t % kBsBlock != 0) return fail(DSA_ERR_INVALID_ARG, "t = %d is not a multiple of 64", s->t);
  if (s->t / kBsBlock > kBsMaxBlocks)
    return fail(DSA_ERR_UNSUPPORTED, "t = %d; block-sparse estimation supports up to %lld tokens", s->t,
                kBsMaxBlocks * kBsBlock);
  if (k_blocks < 1 || k_blocks > kBsMaxBlocks)
    return fail(DSA_ERR_INVALID_ARG, "k_blocks = %d not in [1, %lld]", k_blocks, kBsMaxBlocks);
  return DSA_OK;
}

struct BsLayout {
  long long nblk, nblkp;
  size_t off_qp, off_kp, off_keys, bytes;
};

BsLayout bs_layout(const dsa_shape* s) {
  BsLayout L{};
  L.nblk = s->t / kBsBlock;
  L.nblkp = (L.nblk + 3) / 4 * 4;
  const size_t rows_q = static_cast<size_t>(s->batch) * s->hq * L.nblk;
  const size_t rows_k = static_cast<size_t>(s->batch) * s->hkv * L.nblk;
  L.off_qp = 0;
  L.off_kp = align256(L.off_qp + rows_q * s->d * sizeof(double));
  L.off_keys = align256(L.off_kp + rows_k * s->d * sizeof(double));
  L.bytes = align256(L.off_keys + rows_q * L.nblkp * 4);
  return L;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

extern "C" {

int32_t dsa_block_sparse_index_width(int32_t k_blocks) {
  if (k_blocks < 1 || k_blocks > kBsMaxBlocks) return -1;
  return k_blocks * kBsBlock;
}

dsa_status dsa_block_sparse_workspace_bytes(const dsa_shape* s, int32_t k_blocks, size_t* out_bytes) {
  g_err[0] = 0;
  if (!out_bytes) return fail(DSA_ERR_INVALID_ARG, "out_bytes is NULL");
  dsa_status st = check_block_sparse(s, k_blocks);
  if (st != DSA_OK) return st;
  *out_bytes = bs_layout(s).bytes;
  return DSA_OK;
}

dsa_status dsa_block_sparse_select(const dsa_shape* s, const void* q, const void* k, int32_t k_blocks,
                                   int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  dsa_status st = check_block_sparse(s, k_blocks);
  if (st != DSA_OK) return st;
  if (!q || !k || !idx) return fail(DSA_ERR_INVALID_ARG, "q, k and idx must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(idx))
    return fail(DSA_ERR_INVALID_ARG, "q, k and idx must be 16-byte aligned");
  const BsLayout lay = bs_layout(s);
  if (!ws || ws_bytes < lay.bytes)
    return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes, lay.bytes);
  if (!aligned16(ws)) return fail(DSA_ERR_INVALID_ARG, "ws must be 16-byte aligned");
  dsa::BsArgs a{};
  a.kv = make_kv(s, kBsBlock);
  a.q = q;
  a.k = k;
  a.k_blocks = k_blocks;
  a.nblkp = static_cast<int>(lay.nblkp);
  char* w = static_cast<char*>(ws);
  a.qp = reinterpret_cast<double*>(w + lay.off_qp);
  a.kp = reinterpret_cast<double*>(w + lay.off_kp);
  a.keys = reinterpret_cast<uint32_t*>(w + lay.off_keys);
  a.idx = idx;
  a.L = k_blocks * kBsBlock;
  hipError_t err = dsa::launch_block_sparse(a, s->dtype, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(DSA_ERR_HIP, "block-sparse launch failed: %s", hipGetErrorString(err));
  return DSA_OK;
}

dsa_status dsa_sparse_attn_heads(const dsa_shape* s, const void* q, const void* k, const void* v,
                                 const int32_t* idx, int32_t idx_width, float scale, float* out,
                                 void* stream) {
  g_err[0] = 0;
  dsa_status st = check_shape(s);
  if (st != DSA_OK) return st;
  if (s->mode != DSA_PREFILL) return fail(DSA_ERR_INVALID_ARG, "per-head rows are a prefill layout");
  if (s->t % kBsBlock != 0) return fail(DSA_ERR_INVALID_ARG, "t = %d is not a multiple of 64", s->t);
  if (!q || !k || !v || !idx || !out) return fail(DSA_ERR_INVALID_ARG, "q, k, v, idx and out must be non-NULL");
  if (idx_width < 1) return fail(DSA_ERR_INVALID_ARG, "idx_width must be >= 1");
  dsa::AttnArgs a{};
  a.kv = make_kv(s, kBsBlock);
  a.q = q;
  a.k = k;
  a.v = v;
  a.idx = idx;
  a.L = idx_width;
  a.out = out;
  a.row_heads = 1;
  const float sc = scale > 0.f ? scale : 1.0f / std::sqrt(static_cast<float>(s->d));
  a.scale_log2 = sc * 1.4426950408889634f;
  hipError_t err = dsa::launch_sparse_attn(a, s->dtype, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(DSA_ERR_HIP, "attention launch failed: %s", hipGetErrorString(err));
  return DSA_OK;
}

int32_t dsa_block_sparse_list_width(int32_t k_blocks) {
  if (k_blocks < 1 || k_blocks > kBsMaxBlocks) return -1;
  return (k_blocks + 3) / 4 * 4;
}

dsa_status dsa_block_sparse_select_lists(const dsa_shape* s, const void* q, const void* k, int32_t k_blocks,
                                         int32_t* blocks, int32_t* counts, void* ws, size_t ws_bytes,
                                         void* stream) {
  g_err[0] = 0;
  dsa_status st = check_block_sparse(s, k_blocks);
  if (st != DSA_OK) return st;
  if (!q || !k || !blocks || !counts) return fail(DSA_ERR_INVALID_ARG, "q, k, blocks and counts must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(blocks))
    return fail(DSA_ERR_INVALID_ARG, "q, k and blocks must be 16-byte aligned");
  const BsLayout lay = bs_layout(s);
  if (!ws || ws_bytes < lay.bytes)
    return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes, lay.bytes);
  if (!aligned16(ws)) return fail(DSA_ERR_INVALID_ARG, "ws must be 16-byte aligned");
  dsa::BsArgs a{};
  a.kv = make_kv(s, kBsBlock);
  a.q = q;
  a.k = k;
  a.k_blocks = k_blocks;
  a.nblkp = static_cast<int>(lay.nblkp);
  char* w = static_cast<char*>(ws);
  a.qp = reinterpret_cast<double*>(w + lay.off_qp);
  a.kp = reinterpret_cast<double*>(w + lay.off_kp);
  a.keys = reinterpret_cast<uint32_t*>(w + lay.off_keys);
  a.lblk = blocks;
  a.lcnt = counts;
  a.wb = dsa_block_sparse_list_width(k_blocks);
  hipError_t err = dsa::launch_block_sparse(a, s->dtype, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(DSA_ERR_HIP, "block-sparse launch failed: %s", hipGetErrorString(err));
  return DSA_OK;
}

dsa_status dsa_sparse_attn_lists(const dsa_shape* s, const void* q, const void* k, const void* v,
                                 const int32_t* blocks, int32_t wb, const int32_t* cols, int32_t wc,
                                 const int32_t* counts, float scale, float* out, void* stream) {
  g_err[0] = 0;
  dsa_status st = check_shape(s);
  if (st != DSA_OK) return st;
  if (s->mode != DSA_PREFILL) return fail(DSA_ERR_INVALID_ARG, "block and column lists are a prefill layout");
  if (s->dtype != DSA_BF16 || s->d != 128)
    return fail(DSA_ERR_UNSUPPORTED, "attention over lists takes bf16 inputs with d = 128");
  if (s->t % kBsBlock != 0) return fail(DSA_ERR_INVALID_ARG, "t = %d is not a multiple of 64", s->t);
  if (static_cast<long long>(s->t) * s->d * 2 > 0x7fffffffLL)
    return fail(DSA_ERR_UNSUPPORTED, "t = %d: a kv head's rows must fit 2^31 bytes", s->t);
  if (!q || !k || !v || !blocks || !counts || !out)
    return fail(DSA_ERR_INVALID_ARG, "q, k, v, blocks, counts and out must be non-NULL");
  if (wb < 4 || wb % 4 != 0) return fail(DSA_ERR_INVALID_ARG, "wb = %d is not a positive multiple of 4", wb);
  if (cols && (wc < 4 || wc % 4 != 0))
    return fail(DSA_ERR_INVALID_ARG, "wc = %d is not a positive multiple of 4", wc);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(blocks) || (cols && !aligned16(cols)) ||
      (reinterpret_cast<uintptr_t>(counts) & 7) != 0)
    return fail(DSA_ERR_INVALID_ARG, "q, k, v, blocks and cols must be 16-byte aligned, counts 8-byte aligned");
  dsa::AttnArgs a{};
  a.kv = make_kv(s, kBsBlock);
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.row_heads = 1;
  a.lblk = blocks;
  a.lcol = cols;
  a.lcnt = counts;
  a.wb = wb;
  a.wc = cols ? wc : 0;
  const float sc = scale > 0.f ? scale : 1.0f / std::sqrt(static_cast<float>(s->d));
  a.scale_log2 = sc * 1.4426950408889634f;
  dsa::launch_prefill_lists(a, static_cast<hipStream_t>(stream));
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(DSA_ERR_HIP, "attention launch failed: %s", hipGetErrorString(err));
  return DSA_OK;
}


}  // extern "C"

namespace {

dsa_status check_vertical_slash(const dsa_shape* s, int32_t k_v, int32_t k_s) {
  dsa_status st = check_shape(s);
  if (st != DSA_OK) return st;
  if (s->mode != DSA_PREFILL) return fail(DSA_ERR_INVALID_ARG, "vertical-slash estimation is a prefill call");
  if (s->dtype != DSA_BF16) return fail(DSA_ERR_UNSUPPORTED, "vertical-slash estimation takes bf16 inputs");
  if (s->t % kBsBlock != 0) return fail(DSA_ERR_INVALID_ARG, "t = %d is not a multiple of 64", s->t);
  if (s->t / kBsBlock > kBsMaxBlocks)
    return fail(DSA_ERR_UNSUPPORTED, "t = %d; vertical-slash estimation supports up to %lld tokens", s->t,
                kBsMaxBlocks * kBsBlock);
  const int cap = std::min(dsa::kVsMaxKeep, s->t);
  if (k_v < 0 || k_v > cap) return fail(DSA_ERR_INVALID_ARG, "k_v = %d not in [0, %d]", k_v, cap);
  if (k_s < 1 || k_s > cap) return fail(DSA_ERR_INVALID_ARG, "k_s = %d not in [1, %d]", k_s, cap);
  return DSA_OK;
}

long long vs_width_ll(long long t, long long k_v, long long k_s) {
  const long long n = 64 * std::min(t / 64, 2 * k_s) + k_v;
  return std::min(t, (n + 63) / 64 * 64);
}

struct VsLayout {
  int nr;
  size_t off_part, off_stat, off_sums, off_ckey[2], off_cidx[2], off_sel[2], bytes;
};

VsLayout vs_layout(const dsa_shape* s, int32_t k_v, int32_t k_s) {
  VsLayout L{};
  const size_t bh = static_cast<size_t>(s->batch) * s->hq;
  L.nr = (s->t + dsa::kVsRange - 1) / dsa::kVsRange;
  size_t o = 0;
  L.off_part = o; o = align256(o + bh * L.nr * dsa::kVsLastQ * 2 * sizeof(double));
  L.off_stat = o; o = align256(o + bh * dsa::kVsLastQ * 2 * sizeof(double));
  L.off_sums = o; o = align256(o + bh * 2 * s->t * 4);
  for (int i = 0; i < 2; ++i) { L.off_ckey[i] = o; o = align256(o + bh * 2 * s->t * 4); }
  for (int i = 0; i < 2; ++i) { L.off_cidx[i] = o; o = align256(o + bh * 2 * s->t * 4); }
  L.off_sel[0] = o; o = align256(o + bh * std::max(k_v, 1) * 4);
  L.off_sel[1] = o; o = align256(o + bh * std::max(k_s, 1) * 4);
  L.bytes = o;
  return L;
}

}  // namespace

extern "C" {

int32_t dsa_vertical_slash_index_width(int32_t t, int32_t k_v, int32_t k_s) {
  if (t < 64 || t % 64 != 0 || k_v < 0 || k_s < 1 || k_v > t || k_s > t) return -1;
  return static_cast<int32_t>(vs_width_ll(t, k_v, k_s));
}

dsa_status dsa_vertical_slash_workspace_bytes(const dsa_shape* s, int32_t k_v, int32_t k_s, size_t* out_bytes) {
  g_err[0] = 0;
  if (!out_bytes) return fail(DSA_ERR_INVALID_ARG, "out_bytes is NULL");
  dsa_status st = check_vertical_slash(s, k_v, k_s);
  if (st != DSA_OK) return st;
  *out_bytes = vs_layout(s, k_v, k_s).bytes;
  return DSA_OK;
}

dsa_status dsa_vertical_slash_select(const dsa_shape* s, const void* q, const void* k, int32_t k_v, int32_t k_s,
                                     int32_t* idx, int32_t* cols, int32_t* offsets, void* ws, size_t ws_bytes,
                                     void* stream) {
  g_err[0] = 0;
  dsa_status st = check_vertical_slash(s, k_v, k_s);
  if (st != DSA_OK) return st;
  if (!q || !k || !idx) return fail(DSA_ERR_INVALID_ARG, "q, k and idx must be non-NULL");
  if (!aligned16(q) || !aligned16(k)) return fail(DSA_ERR_INVALID_ARG, "q and k must be 16-byte aligned");
  const VsLayout lay = vs_layout(s, k_v, k_s);
  if (!ws || ws_bytes < lay.bytes)
    return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes, lay.bytes);
  if (!aligned16(ws)) return fail(DSA_ERR_INVALID_ARG, "ws must be 16-byte aligned");
  dsa::VsArgs a{};
  a.kv = make_kv(s, kBsBlock);
  a.q = q;
  a.k = k;
  a.keep[0] = k_v;
  a.keep[1] = k_s;
  a.scale = 1.0 / std::sqrt(static_cast<double>(s->d));
  a.nr = lay.nr;
  char* w = static_cast<char*>(ws);
  a.part = reinterpret_cast<double*>(w + lay.off_part);
  a.stat = reinterpret_cast<double*>(w + lay.off_stat);
  a.sums = reinterpret_cast<uint32_t*>(w + lay.off_sums);
  for (int i = 0; i < 2; ++i) {
    a.ckey[i] = reinterpret_cast<uint32_t*>(w + lay.off_ckey[i]);
    a.cidx[i] = reinterpret_cast<int32_t*>(w + lay.off_cidx[i]);
  }
  a.sel[0] = cols ? cols : reinterpret_cast<int32_t*>(w + lay.off_sel[0]);
  a.sel[1] = offsets ? offsets : reinterpret_cast<int32_t*>(w + lay.off_sel[1]);
  a.idx = idx;
  a.L = static_cast<int>(vs_width_ll(s->t, k_v, k_s));
  hipError_t err = dsa::launch_vertical_slash(a, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(DSA_ERR_HIP, "vertical-slash launch failed: %s", hipGetErrorString(err));
  return DSA_OK;
}

dsa_status dsa_vertical_slash_list_widths(int32_t t, int32_t k_v, int32_t k_s, int32_t* wb, int32_t* wc) {
  g_err[0] = 0;
  if (!wb || !wc) return fail(DSA_ERR_INVALID_ARG, "wb and wc must be non-NULL");
  if (t < 64 || t % 64 != 0 || k_v < 0 || k_s < 1 || k_v > t || k_s > t)
    return fail(DSA_ERR_INVALID_ARG, "t = %d, k_v = %d, k_s = %d out of range", t, k_v, k_s);
  const long long nb = std::min(static_cast<long long>(t) / 64, 2LL * k_s);
  *wb = static_cast<int32_t>((nb + 3) / 4 * 4);
  *wc = static_cast<int32_t>((std::max(k_v, 1) + 3) / 4 * 4);
  return DSA_OK;
}

dsa_status dsa_vertical_slash_select_lists(const dsa_shape* s, const void* q, const void* k, int32_t k_v,
                                           int32_t k_s, int32_t* blocks, int32_t* cols, int32_t* counts,
                                           int32_t* kept_cols, int32_t* kept_offsets, void* ws, size_t ws_bytes,
                                           void* stream) {
  g_err[0] = 0;
  dsa_status st = check_vertical_slash(s, k_v, k_s);
  if (st != DSA_OK) return st;
  if (!q || !k || !blocks || !cols || !counts)
    return fail(DSA_ERR_INVALID_ARG, "q, k, blocks, cols and counts must be non-NULL");
  if (!aligned16(q) || !aligned16(k)) return fail(DSA_ERR_INVALID_ARG, "q and k must be 16-byte aligned");
  const VsLayout lay = vs_layout(s, k_v, k_s);
  if (!ws || ws_bytes < lay.bytes)
    return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes, lay.bytes);
  if (!aligned16(ws)) return fail(DSA_ERR_INVALID_ARG, "ws must be 16-byte aligned");
  int32_t wb = 0, wc = 0;
  dsa_vertical_slash_list_widths(s->t, k_v, k_s, &wb, &wc);
  dsa::VsArgs a{};
  a.kv = make_kv(s, kBsBlock);
  a.q = q;
  a.k = k;
  a.keep[0] = k_v;
  a.keep[1] = k_s;
  a.scale = 1.0 / std::sqrt(static_cast<double>(s->d));
  a.nr = lay.nr;
  char* w = static_cast<char*>(ws);
  a.part = reinterpret_cast<double*>(w + lay.off_part);
  a.stat = reinterpret_cast<double*>(w + lay.off_stat);
  a.sums = reinterpret_cast<uint32_t*>(w + lay.off_sums);
  for (int i = 0; i < 2; ++i) {
    a.ckey[i] = reinterpret_cast<uint32_t*>(w + lay.off_ckey[i]);
    a.cidx[i] = reinterpret_cast<int32_t*>(w + lay.off_cidx[i]);
  }
  a.sel[0] = kept_cols ? kept_cols : reinterpret_cast<int32_t*>(w + lay.off_sel[0]);
  a.sel[1] = kept_offsets ? kept_offsets : reinterpret_cast<int32_t*>(w + lay.off_sel[1]);
  a.lblk = blocks;
  a.lcol = cols;
  a.lcnt = counts;
  a.wb = wb;
  a.wc = wc;
  hipError_t err = dsa::launch_vertical_slash(a, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(DSA_ERR_HIP, "vertical-slash launch failed: %s", hipGetErrorString(err));
  return DSA_OK;
}


}  // extern "C"

namespace {

dsa_status check_rope(const dsa_rope* r) {
  if (!r) return fail(DSA_ERR_INVALID_ARG, "rope is NULL");
  if (r->style != DSA_ROPE_RELATIVE && r->style != DSA_ROPE_CHUNK_INDEXED)
    return fail(DSA_ERR_UNSUPPORTED, "rope style %d; supported: DSA_ROPE_RELATIVE, DSA_ROPE_CHUNK_INDEXED", r->style);
  if (!(r->base > 1.0) || !std::isfinite(r->base)) return fail(DSA_ERR_INVALID_ARG, "rope base must be a finite value > 1");
  return DSA_OK;
}

// the plain pruning workspace, then the rotated query sets (bf16), then (the
// chunk-indexed style in prefill) the rotated keys
size_t rope_query_bytes(const dsa_shape* s, const dsa_params* p, const PruneLayout& lay) {
  const long long bq = s->mode == DSA_DECODE ? 1 : p->block_q;
  return align256(static_cast<size_t>(lay.R) * s->hq * bq * s->d * 2);
}
size_t rope_key_bytes(const dsa_shape* s, const dsa_rope* r) {
  if (r->style != DSA_ROPE_CHUNK_INDEXED || s->mode == DSA_DECODE) return 0;
  return align256(static_cast<size_t>(s->batch) * s->hkv * s->t * s->d * 2);
}
size_t rope_bytes(const dsa_shape* s, const dsa_params* p, const dsa_rope* r, const PruneLayout& lay) {
  // relative: two query sets; chunk-indexed decode: one per stage (the
  // rotated-key call rotates every stage's query at once); else one
  const int sets = r->style == DSA_ROPE_RELATIVE ? 2 : s->mode == DSA_DECODE ? p->n_stages : 1;
  return lay.bytes + sets * rope_query_bytes(s, p, lay) + rope_key_bytes(s, r);
}

// The rotated-key calls: a chunk-indexed decode shape with contiguous K and n
// non-NULL rotated copies.
dsa_status check_rope_keys(const dsa_shape* s, const dsa_params* p, const dsa_rope* r, const void* const* k_rot) {
  if (r->style != DSA_ROPE_CHUNK_INDEXED)
    return fail(DSA_ERR_UNSUPPORTED, "rotated key copies are for the chunk-indexed style only");
  if (s->mode != DSA_DECODE) return fail(DSA_ERR_INVALID_ARG, "rotated key copies are a decode layout");
  if (s->block_table) return fail(DSA_ERR_UNSUPPORTED, "rotated key copies need contiguous K (block_table NULL)");
  if (!k_rot) return fail(DSA_ERR_INVALID_ARG, "k_rot is NULL");
  for (int i = 0; i < p->n_stages; ++i)
    if (!k_rot[i]) return fail(DSA_ERR_INVALID_ARG, "k_rot[%d] is NULL", i);
  return DSA_OK;
}

}  // namespace

extern "C" {

dsa_status dsa_prune_rope_workspace_bytes(const dsa_shape* s, const dsa_params* p, const dsa_rope* rope,
                                          size_t* out_bytes) {
  g_err[0] = 0;
  if (!out_bytes) return fail(DSA_ERR_INVALID_ARG, "out_bytes is NULL");
  dsa_status st = check_shape(s);
  if (st != DSA_OK) return st;
  st = check_params(s, p);
  if (st != DSA_OK) return st;
  st = check_rope(rope);
  if (st != DSA_OK) return st;
  *out_bytes = rope_bytes(s, p, rope, prune_layout(s, p));
  return DSA_OK;
}

dsa_status dsa_prune_select_rope(const dsa_shape* s, const void* q, const void* k, const dsa_params* p,
                                 const dsa_rope* rope, int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  dsa_status st = check_shape(s);
  if (st != DSA_OK) return st;
  st = check_params(s, p);
  if (st != DSA_OK) return st;
  st = check_rope(rope);
  if (st != DSA_OK) return st;
  if (!q || !k || !idx) return fail(DSA_ERR_INVALID_ARG, "q, k and idx must be non-NULL");
  const long long L = index_width_ll(p);
  if (L > (1LL << 30)) return fail(DSA_ERR_INVALID_ARG, "index width overflows");
  const PruneLayout lay = prune_layout(s, p);
  if (lay.maxNC > 32768)
    return fail(DSA_ERR_UNSUPPORTED, "a stage would score %lld chunks per row (limit 32768)", lay.maxNC);
  const size_t qb = rope_query_bytes(s, p, lay);
  const size_t need = rope_bytes(s, p, rope, lay);
  if (!ws || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes, need);
  const dsa::PruneArgs a = prune_args(s, q, k, p, idx, L, lay, ws, nullptr);
  char* w = static_cast<char*>(ws);
  uint16_t* qa = reinterpret_cast<uint16_t*>(w + lay.bytes);
  uint16_t* qb2 = rope->style == DSA_ROPE_RELATIVE ? reinterpret_cast<uint16_t*>(w + lay.bytes + qb) : nullptr;
  uint16_t* kb = rope_key_bytes(s, rope) ? reinterpret_cast<uint16_t*>(w + lay.bytes + qb) : nullptr;
  hipError_t err = dsa::launch_prune_rope(a, s->dtype, rope->style, qa, qb2, kb, rope->base,
                                          static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(DSA_ERR_HIP, "prune launch failed: %s", hipGetErrorString(err));
  return DSA_OK;
}

dsa_status dsa_rope_rotate_keys(const dsa_shape* s, const void* k, const dsa_params* p, const dsa_rope* rope,
                                int32_t pos_begin, int32_t pos_end, void* const* k_rot, void* stream) {
  g_err[0] = 0;
  dsa_status st = check_shape(s);
  if (st != DSA_OK) return st;
  st = check_params(s, p);
  if (st != DSA_OK) return st;
  st = check_rope(rope);
  if (st != DSA_OK) return st;
  st = check_rope_keys(s, p, rope, k_rot);
  if (st != DSA_OK) return st;
  if (!k) return fail(DSA_ERR_INVALID_ARG, "k is NULL");
  if (pos_begin < 0 || pos_end < pos_begin || pos_end > s->t)
    return fail(DSA_ERR_INVALID_ARG, "positions [%d, %d) are not inside [0, t = %d]", pos_begin, pos_end, s->t);
  const PruneLayout lay = prune_layout(s, p);
  const dsa::PruneArgs a = prune_args(s, nullptr, k, p, nullptr, 0, lay, nullptr, nullptr);
  uint16_t* kr[dsa::kMaxStages] = {};
  for (int i = 0; i < p->n_stages; ++i) kr[i] = static_cast<uint16_t*>(const_cast<void*>(k_rot[i]));
  hipError_t err = dsa::launch_rope_rotate_keys(a, s->dtype, kr, rope->base, pos_begin, pos_end,
                                                static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(DSA_ERR_HIP, "key rotation launch failed: %s", hipGetErrorString(err));
  return DSA_OK;
}

dsa_status dsa_prune_select_rope_keys(const dsa_shape* s, const void* q, const void* const* k_rot,
                                      const dsa_params* p, const dsa_rope* rope, int32_t* idx, void* ws,
                                      size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  dsa_status st = check_shape(s);
  if (st != DSA_OK) return st;
  st = check_params(s, p);
  if (st != DSA_OK) return st;
  st = check_rope(rope);
  if (st != DSA_OK) return st;
  st = check_rope_keys(s, p, rope, k_rot);
  if (st != DSA_OK) return st;
  if (!q || !idx) return fail(DSA_ERR_INVALID_ARG, "q and idx must be non-NULL");
  const long long L = index_width_ll(p);
  if (L > (1LL << 30)) return fail(DSA_ERR_INVALID_ARG, "index width overflows");
  const PruneLayout lay = prune_layout(s, p);
  if (lay.maxNC > 32768)
    return fail(DSA_ERR_UNSUPPORTED, "a stage would score %lld chunks per row (limit 32768)", lay.maxNC);
  const size_t need = rope_bytes(s, p, rope, lay);
  if (!ws || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes, need);
  const dsa::PruneArgs a = prune_args(s, q, k_rot[0], p, idx, L, lay, ws, nullptr);
  uint16_t* qa = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + lay.bytes);
  const size_t qstride = rope_query_bytes(s, p, lay) / 2;     // elements between the stages' query sets
  uint16_t* kr[dsa::kMaxStages] = {};
  for (int i = 0; i < p->n_stages; ++i) kr[i] = static_cast<uint16_t*>(const_cast<void*>(k_rot[i]));
  hipError_t err = dsa::launch_prune_rope_keys(a, s->dtype, qa, qstride, kr, rope->base,
                                               static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(DSA_ERR_HIP, "prune launch failed: %s", hipGetErrorString(err));
  return DSA_OK;
}

}  // extern "C"

