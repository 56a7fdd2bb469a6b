/*
 * dsa.h -- C ABI of libdsa: dynamic, per-input block-sparse attention on
 * AMD MI355X (gfx950).
 *
 * Two steps, each a stream-ordered call on caller-owned device memory:
 *
 *   dsa_prune_select  Hierarchical context pruning: for every query block,
 *                     N stages each score the current key chunks through one
 *                     SelectRep representative per (chunk, query head), take the
 *                     max over heads and block queries, and keep the top-K
 *                     chunks. The surviving keys plus the attention-sink and
 *                     local-window keys form one ascending index row per block.
 *                     (InfiniteHiP page, 2502.08910, section 3.4: "Formal
 *                     Mechanism of a Single Pruning Stage", steps 1-8;
 *                     "The Representative Token Selection Algorithm
 *                     (SelectRep)"; "Important: Sink and Streaming Tokens Are
 *                     Never Pruned".)
 *   dsa_sparse_attn   Causal softmax attention of each block's queries over the
 *                     keys of its index row: a gathered FlashAttention pass for
 *                     prefill, a split-key Flash-Decoding pass for decode.
 *                     (InfiniteHiP page, "Block Sparse Attention
 *                     Implementation"; InfLLM blog page, "Mathematical
 *                     Formulation of Efficient Softmax Normalization";
 *                     MInference page, masked-attention formulation and
 *                     in-kernel causal masking.)
 *   dsa_block_sparse_select, dsa_sparse_attn_heads
 *                     The MInference page's Block-Sparse heads: per-head block
 *                     index estimation from mean-pooled queries and keys, and
 *                     attention over per-head index rows (see below); the
 *                     ..._lists calls give and take block lists instead.
 *   dsa_vertical_slash_select
 *                     The MInference page's Vertical-Slash heads: per-head
 *                     column and offset estimation from the last 64 queries,
 *                     rendered as index rows for dsa_sparse_attn_heads, or
 *                     (..._select_lists) as the hybrid kernel's block and
 *                     column lists for dsa_sparse_attn_lists.
 *   dsa_dense_attn    Exact causal attention over all keys: the comparison
 *                     point (InfiniteHiP page, "Dense Attention Optimizations"
 *                     and "Formal Background: Standard Multi-Head Attention").
 *
 * Conventions
 *   - Every pointer argument named q, k, v, idx, out, seq_lens, block_table,
 *     ws or visited is DEVICE memory owned by the caller; dsa_shape and
 *     dsa_params are HOST structs read only during the call.
 *   - The library never allocates, frees or synchronises. Scratch memory is
 *     the caller's workspace `ws` of at least dsa_workspace_bytes() bytes; one
 *     workspace must not be shared by calls that may run concurrently.
 *   - `stream` is a hipStream_t (NULL = the default stream). Calls only
 *     enqueue kernels; errors detected on the host are returned before any
 *     launch, launch failures return DSA_ERR_HIP, device faults surface at the
 *     caller's next synchronisation. Nothing throws across the ABI.
 *   - Results are bitwise deterministic run to run.
 *
 * Layouts (row-major, contiguous unless stated)
 *   PREFILL  q [B, Hq, T, d]; k, v [B, Hkv, T, d]; out [B, Hq, T, d] fp32;
 *            idx [B, T / block_q, L] int32.
 *   DECODE   q [B, Hq, d] (the query at position seq_lens[b]-1);
 *            k, v either contiguous [B, Hkv, t, d] (sequence b uses its first
 *            seq_lens[b] positions) or, when block_table != NULL, page pools
 *            [n_pages, Hkv, page_size, d] with position p of sequence b in page
 *            block_table[b * max_pages + p / page_size] at slot p % page_size;
 *            out [B, Hq, d] fp32; idx [B, L] int32.
 *   Query head h reads kv head h / (Hq / Hkv).
 *   q, k, v share one dtype (fp32 or bf16); out is always fp32.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1,   /* a parameter, shape or pointer violates a rule below */
  DSA_ERR_UNSUPPORTED = 2,   /* valid but not implemented (e.g. d not in {64,128}) */
  DSA_ERR_WORKSPACE = 3,     /* ws NULL or ws_bytes < dsa_workspace_bytes() */
  DSA_ERR_HIP = 4            /* a HIP launch failed; see dsa_last_error() */
} dsa_status;

typedef enum { DSA_F32 = 0, DSA_BF16 = 1 } dsa_dtype;
typedef enum { DSA_PREFILL = 0, DSA_DECODE = 1 } dsa_mode;

#define DSA_MAX_STAGES 4

/* One pruning configuration: the stage tuples (l_c, k) with a single query
 * block size b_q (InfiniteHiP page, "Stage Configuration"), plus the
 * always-kept sink and window counts.
 *   n_stages   1..DSA_MAX_STAGES
 *   block_q    b_q: PREFILL requires T % block_q == 0 and block_q <= 64;
 *              DECODE requires block_q == 1
 *   chunk[i]   l_c of stage i: a power of two; chunk[i+1] divides chunk[i]
 *   keep[i]    k of stage i: a multiple of chunk[i], >= 0; keep[i+1] <= keep[i]
 *   n_sink     keys [0, n_sink) are always kept (>= 0)
 *   n_window   the n_window most recent keys of a block, [e - n_window, e)
 *              with e one past the block's last query, are always kept (>= 0)
 * The prunable middle of block [s, e) is [n_sink, e - n_window); stage 1
 * partitions it into whole chunks of chunk[0] keys starting at n_sink, and the
 * tail that does not fill a chunk is kept with the window. */
typedef struct {
  int32_t n_stages;
  int32_t block_q;
  int32_t chunk[DSA_MAX_STAGES];
  int32_t keep[DSA_MAX_STAGES];
  int32_t n_sink;
  int32_t n_window;
} dsa_params;

/* Problem shape.
 *   mode, dtype   dsa_mode / dsa_dtype values
 *   batch, hq, hkv, d   B >= 1; hq % hkv == 0, hq / hkv in {1, 2, 4, 8}; d in {64, 128}
 *   t             PREFILL: tokens per sequence. DECODE: the largest context
 *                 length any sequence may have, and the token stride of
 *                 contiguous k / v
 *   seq_lens      DECODE: device int32 [B], each in [1, t]; ignored for PREFILL
 *   block_table   DECODE: device int32 [B, max_pages] or NULL (contiguous)
 *   page_size, max_pages   paged DECODE only: page_size a power of two;
 *                 max_pages * page_size >= t */
typedef struct {
  int32_t mode;
  int32_t dtype;
  int32_t batch, hq, hkv, d;
  int32_t t;
  const int32_t* seq_lens;
  const int32_t* block_table;
  int32_t page_size, max_pages;
} dsa_shape;

/* Width L of an index row: n_sink + keep[n_stages-1] + n_window + chunk[0] - 1
 * rounded up to a multiple of 64; -1 if p is NULL or invalid. */
int32_t dsa_index_width(const dsa_params* p);

/* Workspace bytes for any of dsa_prune_select, dsa_sparse_attn,
 * dsa_prune_attend and dsa_dense_attn on this shape (p may be NULL when only
 * dsa_dense_attn is used). Returns DSA_ERR_INVALID_ARG for an invalid
 * shape or params. */
dsa_status dsa_workspace_bytes(const dsa_shape* shape, const dsa_params* p, size_t* out_bytes);

/* Hierarchical pruning (see above). Writes idx: every row fully, with the
 * kept key positions strictly ascending followed by -1 padding to L =
 * dsa_index_width(p). Stage scores are unscaled dot products; the right half of
 * a SelectRep split wins only on a strictly greater score; top-K breaks score
 * ties towards the lower chunk index; a stage with no more chunks than it keeps
 * keeps them all.
 * visited: NULL, or device uint64 [n_stages] that is INCREMENTED by the number
 * of distinct (kv head, key position) rows SelectRep reads in each stage (a
 * traffic diagnostic; costs extra atomics). */
dsa_status dsa_prune_select(const dsa_shape* shape, const void* q, const void* k,
                            const dsa_params* p, int32_t* idx,
                            void* ws, size_t ws_bytes, uint64_t* visited, void* stream);

/* ---- Decoding with remembered stage outputs ("mask caching") -------------
 * InfiniteHiP page, section 3.4 "Sparse Attention Mask Caching": stage i of
 * the pruning recomputes its output only at decode steps where
 * step mod refresh[i] == 0 (the page's presets: (16, 8, 4) default,
 * (32, 16, 8) fast, (96, 24, 8) flash) and otherwise reuses the output it
 * remembered. A due stage scores the current output of the stage before it
 * (remembered or just recomputed; the whole middle of the current context for
 * stage 1) with the newest query. The index row of every step is the sinks,
 * the last stage's remembered keys, and every position from the end of the
 * stage-1 middle those keys descend from up to the newest token (keys that
 * left the window since that stage-1 refresh were never scored and stay).
 *
 * The mask cache is caller-owned DEVICE memory of dsa_mask_cache_bytes()
 * bytes, 16-byte aligned, one per (layer, batch) stream of decode steps. It
 * begins with int32 status[B]: after each call, status[b] is 1 if the row of
 * sequence b did not fit in idx_width (the row then holds its first idx_width
 * keys), else 0. The rest is opaque. The first call on a cache must be at a
 * step where every stage is due (e.g. step 0); the library cannot check this.
 * Calls on one cache must not overlap. */

/* Bytes of the mask cache for this decode shape and params. */
dsa_status dsa_mask_cache_bytes(const dsa_shape* shape, const dsa_params* p, size_t* out_bytes);

/* Row width for cached decoding: n_sink + keep[n_stages-1] + n_window +
 * chunk[0] - 1 + max_growth rounded up to 64, where max_growth is the most
 * tokens a sequence gains between stage-1 refreshes (refresh[0] - 1 when each
 * step appends one token); -1 if p is invalid or max_growth < 0. */
int32_t dsa_cached_index_width(const dsa_params* p, int32_t max_growth);

/* One decode step of hierarchical pruning with remembered stages (see above).
 * shape.mode must be DSA_DECODE; refresh is a HOST array [n_stages] of
 * intervals >= 1; step >= 0 is the decode step counter shared by the batch;
 * idx [B, idx_width] with idx_width a multiple of 64 and >= dsa_index_width(p),
 * 16-byte aligned; ws, visited, stream as for dsa_prune_select. Rows are
 * written as by dsa_prune_select (ascending, -1 padded). */
dsa_status dsa_prune_select_cached(const dsa_shape* shape, const void* q, const void* k,
                                   const dsa_params* p, const int32_t* refresh, int64_t step,
                                   void* cache, size_t cache_bytes, int32_t* idx, int32_t idx_width,
                                   void* ws, size_t ws_bytes, uint64_t* visited, void* stream);

/* out[h, t] = sum over p in row, p <= t, of softmax_p(scale * q_{h,t} . k_p) v_p,
 * for every query t of each block (row = idx row of the block; negative
 * entries are ignored, as are entries beyond the block's last query).
 * block_q is the query block size the rows were built with (PREFILL: a power
 * of two in [4, 64] dividing t; DECODE: 1). idx_width is the row width (>= 1).
 * scale <= 0 selects 1/sqrt(d). */
dsa_status dsa_sparse_attn(const dsa_shape* shape, const void* q, const void* k, const void* v,
                           const int32_t* idx, int32_t idx_width, int32_t block_q, float scale,
                           float* out, void* ws, size_t ws_bytes, void* stream);

/* One pass of the whole path: dsa_prune_select followed by dsa_sparse_attn
 * over the rows it writes, in one call (same arguments and outputs: idx as
 * written by dsa_prune_select, out as written by dsa_sparse_attn with
 * block_q = p->block_q). For bf16 decode the last stage's top-K, the gathered
 * attention and the merge of its split partials run as one kernel (every
 * attention workgroup re-derives the kept chunks from the stage's scores),
 * which removes two kernel boundaries from the step; the results are those of
 * the two calls (idx bit for bit, out within rounding of the partial merge).
 * ws: at least dsa_workspace_bytes() bytes (which covers this call). */
dsa_status dsa_prune_attend(const dsa_shape* shape, const void* q, const void* k, const void* v,
                            const dsa_params* p, float scale, int32_t* idx, float* out, void* ws,
                            size_t ws_bytes, uint64_t* visited, void* stream);

/* dsa_prune_attend for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. It takes no
 * workspace; its scratch memory is a 64 MiB array in the library's device
 * code (one per GPU, held until the process ends), so it calls no hipMalloc,
 * hipFree or allocating routine. Shapes whose scratch for this call exceeds
 * 64 MiB are rejected with DSA_ERR_UNSUPPORTED before any launch (the 1M and
 * 3M decode steps need about 1.5 MB, a batch of 32 ragged sequences of up to
 * 256K tokens about 46 MB, a 128K prefill about 42 MB). Every call on one GPU
 * shares that
 * GPU's array: calls that may overlap on one GPU (several streams, several
 * host threads) race and must not be issued; calls on different GPUs are
 * independent. Nothing in the array needs to start at zero (every call writes
 * what it reads). Arguments and results are those of dsa_prune_attend. */
dsa_status dsa_prune_attend_static(const dsa_shape* shape, const void* q, const void* k, const void* v,
                                   const dsa_params* p, float scale, int32_t* idx, float* out,
                                   uint64_t* visited, void* stream);

/* Exact causal attention over keys [0, t] for every query t. */
dsa_status dsa_dense_attn(const dsa_shape* shape, const void* q, const void* k, const void* v,
                          float scale, float* out, void* ws, size_t ws_bytes, void* stream);

/* ---- RoPE inside SelectRep ------------------------------------------------
 * InfiniteHiP page, "Four RoPE Styles for Context Pruning" (Relative,
 * Chunk-indexed) and "Layer-Specific Strategy Assignment": q and k are taken
 * before any rotary embedding (rotate-half pairing, theta_i = base^(-2i/d),
 * n_stream = p->n_window). Rotated vectors are computed in fp64 and rounded
 * to multiples of 1/128, so scores between them and grid-valued vectors are
 * exact. Everything else is dsa_prune_select (rows, top-K ties, sinks and
 * window).
 *
 * DSA_ROPE_RELATIVE: at every SelectRep split the left branch's
 * representative is scored as sitting n_stream + 1 positions behind the query
 * and the right branch's n_stream behind. The rotation is applied to the
 * queries (equal, in exact arithmetic, to rotating the query to n_stream + 1
 * and the keys to 0 and 1). A representative that wins from the right is
 * scored again as the next split's left one; a chunk's score is the score its
 * representative won its last split with.
 *
 * DSA_ROPE_CHUNK_INDEXED: in a stage of chunk length l, a key at position j
 * is rotated to its chunk's index (j - n_sink) / l, and every query to
 * min(its position, c_last + n_stream), c_last = (mid_end - n_sink) / l - 1
 * being the stage's last chunk of the middle (the query sits n_stream after
 * it); the plain SelectRep, chunk score and top-K run on the rotated vectors.
 * The page assigns this style to a model's first three layers and the
 * relative one to the rest. */
typedef enum { DSA_ROPE_RELATIVE = 1, DSA_ROPE_CHUNK_INDEXED = 2 } dsa_rope_style;

typedef struct {
  int32_t style;     /* DSA_ROPE_RELATIVE or DSA_ROPE_CHUNK_INDEXED */
  double base;       /* rotary base (e.g. 10000 or 500000), > 1 */
} dsa_rope;

/* Workspace bytes of dsa_prune_select_rope (and, for a chunk-indexed decode
 * shape, of dsa_prune_select_rope_keys) for this rope style: the pruning
 * workspace plus rotated copies in bf16 (relative: two of the queries;
 * chunk-indexed: one of the queries per stage in decode, one of the queries
 * and one of the keys in prefill). */
dsa_status dsa_prune_rope_workspace_bytes(const dsa_shape* shape, const dsa_params* p, const dsa_rope* rope,
                                          size_t* out_bytes);

/* Hierarchical pruning with RoPE inside SelectRep; arguments and idx as for
 * dsa_prune_select (prefill or decode, contiguous or paged). Returns
 * DSA_ERR_UNSUPPORTED for an unknown style, DSA_ERR_INVALID_ARG for a base
 * that is not a finite value > 1, DSA_ERR_WORKSPACE when ws_bytes is below
 * dsa_prune_rope_workspace_bytes. */
dsa_status dsa_prune_select_rope(const dsa_shape* shape, const void* q, const void* k, const dsa_params* p,
                                 const dsa_rope* rope, int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/* Chunk-indexed decode with the keys rotated once. In a stage of chunk length
 * l a key's chunk index (j - n_sink) / l depends only on its position, so its
 * rotated row in that stage never changes as the context grows; only the
 * query's position does. dsa_rope_rotate_keys writes, for every stage i, the
 * rotated rows (bf16, the values dsa_prune_select_rope computes) of the keys
 * at positions [pos_begin, pos_end) of every sequence and kv head into
 * k_rot[i]; call it over [0, t) once and then for each appended range. Rows
 * before n_sink are never candidates and are not written.
 *   shape      DECODE, contiguous K (block_table NULL): k [B, Hkv, t, d]
 *   k_rot      HOST array of p->n_stages DEVICE pointers, each a caller-owned
 *              bf16 buffer [B, Hkv, t, d] (the layout of k)
 *   pos_begin, pos_end   0 <= pos_begin <= pos_end <= t
 *   rope       style DSA_ROPE_CHUNK_INDEXED (else DSA_ERR_UNSUPPORTED)
 * dsa_prune_select_rope_keys then prunes as dsa_prune_select_rope does for the
 * chunk-indexed style, reading the rotated copies instead of k (every
 * position a sequence's stages can score must have been rotated: [n_sink,
 * seq_len - n_window)); idx is identical to dsa_prune_select_rope's. Each
 * step rotates only the query (one launch for all stages), then runs the
 * plain decode kernels. ws: at least dsa_prune_rope_workspace_bytes() bytes. */
dsa_status dsa_rope_rotate_keys(const dsa_shape* shape, const void* k, const dsa_params* p, const dsa_rope* rope,
                                int32_t pos_begin, int32_t pos_end, void* const* k_rot, void* stream);
dsa_status dsa_prune_select_rope_keys(const dsa_shape* shape, const void* q, const void* const* k_rot,
                                      const dsa_params* p, const dsa_rope* rope, int32_t* idx, void* ws,
                                      size_t ws_bytes, void* stream);

/* ---- Block-sparse heads --------------------------------------------------
 * MInference page, "Online Dynamic Index Estimation: Block-Sparse Heads
 * (Algorithm 3)" and "Block-Sparse FlashAttention Kernel (Appendix C.4.1)".
 * Prefill only, blocks of 64 tokens (the page's block size): for every query
 * head h and query block m, the queries of the block and the keys of kv head
 * h / (Hq / Hkv) are mean-pooled per 64 rows; the pooled logits q~_m . k~_j of
 * the key blocks j <= m (later blocks are masked; the diagonal block stays) are
 * evaluated in fp64 and rounded once to fp32; the k_blocks blocks with the
 * highest logits (ties to the lower block) are kept. Softmax and the 1/sqrt(d)
 * scale are monotone and do not change the selection. Each query head has its
 * own index rows.
 *
 * Layout: idx [B, Hq, T / 64, L] int32 with L = dsa_block_sparse_index_width();
 * row (b, h, m) holds the kept blocks in ascending order as runs of 64
 * positions (64 j .. 64 j + 63), min(m + 1, k_blocks) runs, then -1 padding.
 * Requires t a multiple of 64 with t / 64 <= 16384. */

/* Row width 64 * k_blocks; -1 if k_blocks is not in [1, 16384]. */
int32_t dsa_block_sparse_index_width(int32_t k_blocks);

/* Workspace bytes of dsa_block_sparse_select for this shape: the pooled
 * queries and keys in fp64 and one orderable logit key per (q head, query
 * block, key block), i.e. 8 d (B Hq + B Hkv) T/64 + 4 B Hq (T/64) ceil4(T/64)
 * bytes plus alignment. */
dsa_status dsa_block_sparse_workspace_bytes(const dsa_shape* shape, int32_t k_blocks, size_t* out_bytes);

/* Writes every index row of idx (see above). shape.mode must be DSA_PREFILL;
 * q [B, Hq, T, d], k [B, Hkv, T, d] (fp32 or bf16); q, k, idx and ws 16-byte
 * aligned; ws of at least dsa_block_sparse_workspace_bytes() bytes. */
dsa_status dsa_block_sparse_select(const dsa_shape* shape, const void* q, const void* k, int32_t k_blocks,
                                   int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/* dsa_sparse_attn with one index row per query head: out[h, t] = sum over p in
 * the row of (h, t / 64), p <= t, of softmax_p(scale * q_{h,t} . k_p) v_p.
 * shape.mode must be DSA_PREFILL with t a multiple of 64; idx [B, Hq, T / 64,
 * idx_width] (negative entries are ignored); scale <= 0 selects 1/sqrt(d).
 * Needs no workspace. */
dsa_status dsa_sparse_attn_heads(const dsa_shape* shape, const void* q, const void* k, const void* v,
                                 const int32_t* idx, int32_t idx_width, float scale, float* out,
                                 void* stream);

/* Block-sparse selection written as block lists (the form the page's
 * block-sparse kernel takes: block ids, not positions) for
 * dsa_sparse_attn_lists: blocks [B, Hq, T / 64, wb] int32, wb =
 * dsa_block_sparse_list_width(k_blocks), row (b, h, m) = the kept block ids
 * ascending, then -1; counts [B, Hq, T / 64, 2] int32 = (number of blocks, 0).
 * Same selection, shapes, alignment and workspace as dsa_block_sparse_select;
 * blocks 16-byte aligned. */
int32_t dsa_block_sparse_list_width(int32_t k_blocks);   /* k_blocks rounded up to 4; -1 if out of range */
dsa_status dsa_block_sparse_select_lists(const dsa_shape* shape, const void* q, const void* k, int32_t k_blocks,
                                         int32_t* blocks, int32_t* counts, void* ws, size_t ws_bytes,
                                         void* stream);

/* Attention over per-head block and column lists (MInference page,
 * "Vertical-Slash Hybrid Kernel (Appendix C.4.2, Algorithms 4 and 5)": the
 * listed 64-key blocks are loaded whole as contiguous tiles, the columns
 * gathered; block-sparse heads list blocks only). For query head h and query
 * block m (row r = (b * Hq + h) * (T / 64) + m): the keys are every position
 * of blocks[r][0 .. counts[r][0]) and the columns cols[r][0 .. counts[r][1]);
 * out[h, t] = sum over those keys p <= t of softmax_p(scale * q_{h,t} . k_p)
 * v_p, 0 for a query that sees none. The lists must be disjoint, ascending
 * and inside [0, t) (as the list selections write them). shape.mode
 * DSA_PREFILL, dtype DSA_BF16, d = 128, t a multiple of 64 with
 * t * 256 < 2^31; blocks [B, Hq, T / 64, wb], cols [B, Hq, T / 64, wc] or
 * NULL when every column count is 0, counts [B, Hq, T / 64, 2]; wb, wc
 * positive multiples of 4; q, k, v, blocks, cols 16-byte aligned, counts
 * 8-byte aligned; scale <= 0 selects 1/sqrt(d). Other shapes return
 * DSA_ERR_UNSUPPORTED. Needs no workspace. */
dsa_status dsa_sparse_attn_lists(const dsa_shape* shape, const void* q, const void* k, const void* v,
                                 const int32_t* blocks, int32_t wb, const int32_t* cols, int32_t wc,
                                 const int32_t* counts, float scale, float* out, void* stream);

/* ---- Vertical-slash heads ------------------------------------------------
 * MInference page, "Online Dynamic Index Estimation: Vertical-Slash Heads
 * (Algorithm 2)" and "Vertical-Slash Hybrid Kernel (Appendix C.4.2)".
 * Prefill only, bf16. For every query head h (keys of kv head h / (Hq / Hkv)):
 * the causal softmax of the last 64 queries (scale 1/sqrt(d)) is summed over
 * those queries per key column and per offset d = query position - key
 * position; the k_v columns and the k_s offsets with the largest sums (sums
 * rounded once to fp32, ties to the lower index) are kept. Each query block m
 * (queries 64m .. 64m+63) attends, whole, every 64-aligned key block that a
 * kept offset's key range [64m - d, 64m + 63 - d] touches, and singly every
 * kept column before the block's end that lies in none of those blocks.
 *
 * Layout: idx [B, Hq, T / 64, L] int32, L = dsa_vertical_slash_index_width();
 * each row holds its key positions ascending, then -1 padding; the causal
 * mask inside a block is applied by dsa_sparse_attn_heads, which consumes the
 * rows. A query that sees no key of its row gets output 0.
 * Requires t a multiple of 64 with t / 64 <= 16384, 0 <= k_v <= min(t, 8192),
 * 1 <= k_s <= min(t, 8192). */

/* Row width min(t, 64 * min(t / 64, 2 k_s) + k_v rounded up to 64); -1 if the
 * arguments are out of range. */
int32_t dsa_vertical_slash_index_width(int32_t t, int32_t k_v, int32_t k_s);

/* Workspace bytes of dsa_vertical_slash_select for this shape. */
dsa_status dsa_vertical_slash_workspace_bytes(const dsa_shape* shape, int32_t k_v, int32_t k_s,
                                              size_t* out_bytes);

/* Writes every index row of idx (see above). shape.mode DSA_PREFILL, dtype
 * DSA_BF16; q [B, Hq, T, d], k [B, Hkv, T, d]; q, k and ws 16-byte aligned.
 * cols (NULL or device int32 [B, Hq, k_v]) and offsets (NULL or device int32
 * [B, Hq, k_s]) receive the kept columns and offsets of every head, ascending. */
dsa_status dsa_vertical_slash_select(const dsa_shape* shape, const void* q, const void* k, int32_t k_v,
                                     int32_t k_s, int32_t* idx, int32_t* cols, int32_t* offsets, void* ws,
                                     size_t ws_bytes, void* stream);

/* The same index as the hybrid kernel's two lists (Appendix C.4.2), for
 * dsa_sparse_attn_lists: blocks [B, Hq, T / 64, wb] = the ascending ids of
 * the 64-key blocks that row attends whole, then -1; cols [B, Hq, T / 64, wc]
 * = its single columns (kept columns before the block's end in none of those
 * blocks), ascending, then -1; counts [B, Hq, T / 64, 2] = (blocks, columns).
 * The widths come from dsa_vertical_slash_list_widths (wb = min(T / 64,
 * 2 k_s), wc = max(k_v, 1), each rounded up to 4): about 2 k_s + k_v entries
 * per row instead of the row width L. kept_cols / kept_offsets as cols /
 * offsets of dsa_vertical_slash_select. Same shapes, alignment and workspace
 * as dsa_vertical_slash_select. */
dsa_status dsa_vertical_slash_list_widths(int32_t t, int32_t k_v, int32_t k_s, int32_t* wb, int32_t* wc);
dsa_status dsa_vertical_slash_select_lists(const dsa_shape* shape, const void* q, const void* k, int32_t k_v,
                                           int32_t k_s, int32_t* blocks, int32_t* cols, int32_t* counts,
                                           int32_t* kept_cols, int32_t* kept_offsets, void* ws, size_t ws_bytes,
                                           void* stream);

/* Per-kernel timing, a diagnostic for latency breakdowns. Between
 * dsa_profile_begin() and dsa_profile_end(), every kernel the library launches
 * records a pair of HIP events at its own start and end on its stream (do not
 * profile inside graph capture). dsa_profile_end() waits for those events, stops recording
 * and writes up to `capacity` aggregates (kernel name, launches, total
 * milliseconds) to `out` (host memory); *n_out receives the number of kernels
 * seen. */
typedef struct {
  char name[48];
  int64_t launches;
  double total_ms;
} dsa_kernel_time;

dsa_status dsa_profile_begin(void);
dsa_status dsa_profile_end(dsa_kernel_time* out, int32_t capacity, int32_t* n_out);

/* Checked mode for decode inputs (a caller aid; the pages define no such
 * step). The kernels read seq_lens and block_table from device memory and
 * cannot report a bad value: a length above t is clamped to t and a length
 * below 1 gives an empty row (every index entry -1, output 0), but a page id
 * outside the pool makes the gathers read outside it. This call checks HOST
 * copies of both arrays before the caller launches: every seq_lens[b] in
 * [1, shape->t], and for a paged shape every page id that a sequence's
 * length reaches (block_table[b][i], i < ceil(seq_lens[b] / page_size)) in
 * [0, n_pages). seq_lens: host int32 [B]; block_table: host int32
 * [B, max_pages] (ignored for contiguous K/V); n_pages: pages in the K/V
 * pools. Returns DSA_OK, or DSA_ERR_INVALID_ARG with dsa_last_error() naming
 * the first bad entry. Reads no device memory and launches nothing. */
dsa_status dsa_check_decode_inputs(const dsa_shape* shape, const int32_t* seq_lens, const int32_t* block_table,
                                   int64_t n_pages);

/* Static description of a status code. */
const char* dsa_status_str(dsa_status s);

/* Message of the last error returned on the calling host thread ("" if none). */
const char* dsa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H */
