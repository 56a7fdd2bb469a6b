"""CPU oracle for dynamic block-sparse attention (TEST INFRASTRUCTURE ONLY).

This module is the plain, slow, obviously-correct statement of what the GPU
library computes. Only the tests, the package's smoke check and the benchmark's
CPU-baseline leg may import it; the product path never does. It shares no code
with the HIP library and imports nothing from the package.

It follows the InfiniteHiP page (2502.08910), section 3.4:
  * "Formal Mechanism of a Single Pruning Stage", steps 1-8 (query blocking,
    chunk partitioning, per-head representative, chunk score, top-K chunks,
    index assembly, query-block propagation);
  * "The Representative Token Selection Algorithm (SelectRep)" (Algorithm 3);
  * "Important: Sink and Streaming Tokens Are Never Pruned" (Algorithm 1,
    initial candidate set) and "The Sink/Streaming Token Special Handling";
and the attention over the active key set as written on the InfLLM blog page
("Mathematical Formulation of Efficient Softmax Normalization") and as the
masked softmax of the MInference page (section on the sparse-attention
problem formulation), with causal masking inside the kernel; for decoding
with remembered masks, the InfiniteHiP page's "Sparse Attention Mask Caching"
(per-stage refresh intervals, stage 1 refreshed with the newest query); and
the MInference page's Block-Sparse head estimation ("Online Dynamic Index
Estimation: Block-Sparse Heads (Algorithm 3)": mean pooling, block-causal
pooled logits, top-k_b blocks per query head and block); and its Vertical-Slash
head estimation ("Online Dynamic Index Estimation: Vertical-Slash Heads
(Algorithm 2)": last 64 queries, column and offset sums of their causal
softmax, top-k_v columns and top-k_s offsets) with the index building of
"Vertical-Slash Hybrid Kernel (Appendix C.4.2)"; and SelectRep with relative
and chunk-indexed RoPE (InfiniteHiP page, "Four RoPE Styles for Context
Pruning", Relative and Chunk-indexed; "Layer-Specific Strategy Assignment").

Readings taken where the pages are silent or garbled (each is listed with its
reason in the project's design notes):
  * scores are unscaled fp32 dot products; the softmax scale is applied only in
    attention (the pages omit the constant scale "for brevity");
  * chunk score = max over ALL query heads and all queries of the block, each
    head using its own representative; GQA head h reads kv head h // (Hq/Hkv);
  * SelectRep midpoint = (a + z + 1) // 2 on a 0-based inclusive range [a, z];
    the right branch wins only if its score is strictly greater;
  * top-K orders chunks by (score descending, chunk index ascending); a stage
    with no more chunks than it keeps keeps them all;
  * the prunable middle of query block [s, e) is [n_sink, e - n_window); the
    window is the n_window most recent keys [e - n_window, e) (it contains the
    block itself); the stage-1 chunk grid is anchored at n_sink and the tail
    that does not fill a whole chunk joins the window;
  * masked keys are excluded exactly (the additive -c(1-M) form with c=1e5
    underflows to the same result), key p is visible to query t iff p <= t;
  * softmax and the P.V product are evaluated in fp64 and cast to fp32;
  * mask caching: one step counter per call for the whole batch; a due stage
    reads the current output of the stage before it (fresh or remembered);
    keys that slid out of the window since the stage-1 refresh a row descends
    from were never scored and are kept with the window;
  * block-sparse estimation: a key block is masked for query block m when it
    lies strictly after it (j > m; the diagonal block stays); blocks are ranked
    by the pooled logits in fp64 rounded to fp32 (the softmax and the scale are
    monotone), ties to the lower block; each query head has its own rows;
  * vertical-slash estimation: the last 64 queries of the sequence, each with
    its causal mask; a slash offset d is query position minus key position
    (d >= 0) and its sum runs over the estimation queries that reach key >= 0;
    sums in fp64, ranked after one rounding to fp32, ties to the lower index;
    per query block, each offset's key range is rounded out to the 64-aligned
    blocks it touches (attended whole) and vertical columns outside those
    blocks are attended singly;
  * relative RoPE in SelectRep: rotate-half pairing, theta_i = base^(-2i/d);
    the rotation is carried by the queries (offsets n_stream + 1 left and
    n_stream right, n_stream = the window), rounded to multiples of 1/128; a
    representative that won from the right is scored again as the next left
    one; a chunk's score is the one its representative won its last split with;
  * chunk-indexed RoPE in SelectRep: within a stage of chunk length l a key at
    position j sits at its chunk's index (j - n_sink) / l in the stage's tiling
    of the middle, and every query at min(i_orig, c_last + n_stream), so the
    last chunk c_last is n_stream behind it (the page's prose; its formula is
    garbled); queries and keys are both rotated in fp64 and rounded to the
    1/128 grid; the tournament is the plain SelectRep on the rotated vectors.

Every function here is pinned by tests/test_oracle.py against what the pages
and the mathematics fix (closed forms, brute force, special cases reducing to
textbook attention, invariants). The one part with no pin is the recall of
SelectRep against exact top-k on real attention (the pages only give
model-based recall): that quality figure is reported, never graded.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, List, Optional, Sequence, Tuple

import numpy as np


@dataclass(frozen=True)
class Params:
    """One pruning configuration: the stage tuples (l_c, k) of the InfiniteHiP
    page ("Stage Configuration") with a single query block size b_q, plus the
    always-kept sink and window counts."""
    block_q: int
    chunk: Tuple[int, ...]
    keep: Tuple[int, ...]
    n_sink: int
    n_window: int


def index_width(p: Params) -> int:
    """Row width of the index output: the largest possible row (sinks, the last
    stage's keep, window plus the chunk-grid tail), rounded up to 64."""
    n = p.n_sink + p.keep[-1] + p.n_window + p.chunk[0] - 1
    return (n + 63) // 64 * 64


# --------------------------------------------------------------------------- #
# geometry of one query block (Algorithm 1 initial set; step 3 chunk grid)     #
# --------------------------------------------------------------------------- #
@dataclass(frozen=True)
class Geometry:
    s: int          # first query of the block
    e: int          # one past the last query
    sink_hi: int    # sinks are [0, sink_hi)
    mid_lo: int     # prunable middle [mid_lo, mid_hi)
    mid_hi: int
    n1: int         # whole stage-1 chunks in the middle


def geometry(s: int, e: int, p: Params) -> Geometry:
    w0 = e - p.n_window                       # window = [w0, e)
    m = max(0, w0 - p.n_sink)                 # size of the prunable middle
    n1 = m // p.chunk[0]
    mid_hi = p.n_sink + n1 * p.chunk[0]       # the tail [mid_hi, w0) joins the window
    return Geometry(s, e, min(p.n_sink, e), p.n_sink, max(mid_hi, p.n_sink), n1)


# --------------------------------------------------------------------------- #
# scores                                                                      #
# --------------------------------------------------------------------------- #
def rep_score(qh: np.ndarray, krows: np.ndarray) -> np.ndarray:
    """sigma(k) = max_t q_t . k for each key row, fp32 dot products.

    qh: [b_q, d] float32, krows: [n, d] float32 -> [n] float32.
    """
    qh = np.asarray(qh, dtype=np.float32)
    krows = np.asarray(krows, dtype=np.float32)
    if krows.shape[0] == 0:
        return np.zeros(0, dtype=np.float32)
    return (qh @ krows.T).max(axis=0).astype(np.float32)


def select_rep(qh: np.ndarray, K, g: int, chunk: np.ndarray,
               visit: Optional[Callable[[int], None]] = None) -> int:
    """SelectRep (Algorithm 3) for one head and one chunk of key positions.

    Halves the range ceil(log2 l) times; each time the first key of each half
    represents it, and the half whose representative scores strictly higher
    wins (ties go left). Returns the chosen key position.
    """
    l = len(chunk)
    a, z = 0, l - 1
    n_iter = int(np.ceil(np.log2(l))) if l > 1 else 0
    for _ in range(n_iter):
        mid = (a + z + 1) // 2
        rows = K[g, np.array([chunk[a], chunk[mid]])]
        sig = rep_score(qh, rows)
        if visit is not None:
            visit(int(chunk[a]))
            visit(int(chunk[mid]))
        if sig[1] > sig[0]:
            a = mid
        else:
            z = mid - 1
    assert a == z or l == 1
    return int(chunk[a])


def select_rep_all(qh: np.ndarray, K, g: int, P2: np.ndarray,
                   visited: Optional[list] = None) -> np.ndarray:
    """select_rep applied to every row of P2 ([n_chunks, l]) at once: the same
    per-chunk steps, with the dot products of all chunks batched. If
    ``visited`` is a list, the arrays of key positions read are appended."""
    nc, l = P2.shape
    a = np.zeros(nc, dtype=np.int64)
    z = np.full(nc, l - 1, dtype=np.int64)
    n_iter = int(np.ceil(np.log2(l))) if l > 1 else 0
    rows = np.arange(nc)
    for _ in range(n_iter):
        mid = (a + z + 1) // 2
        sl = rep_score(qh, K[g, P2[rows, a]])
        sr = rep_score(qh, K[g, P2[rows, mid]])
        if visited is not None:
            visited.append(P2[rows, a])
            visited.append(P2[rows, mid])
        right = sr > sl
        a = np.where(right, mid, a)
        z = np.where(right, z, mid - 1)
    assert np.all(a == z) or l == 1
    return P2[rows, a]


def chunk_scores(Q: np.ndarray, K, P: np.ndarray, l: int,
                 visited: Optional[list] = None) -> np.ndarray:
    """Step 4-5: s_j = max over heads h and block queries t of q_{h,t} . k_{r_{h,j}}.

    Q: [Hq, b_q, d]; K indexable as K[g, positions] -> [n, d]; P: the ascending
    candidate positions, partitioned into contiguous groups of l entries.
    If ``visited`` is a list, (kv head, positions read) pairs are appended.
    """
    Hq = Q.shape[0]
    Hkv = K.shape[0]
    G = Hq // Hkv
    nc = len(P) // l
    P2 = np.asarray(P).reshape(nc, l)
    s = np.full(nc, -np.inf, dtype=np.float32)
    for h in range(Hq):
        g = h // G
        vis = [] if visited is not None else None
        r = select_rep_all(Q[h], K, g, P2, vis)
        if visited is not None:
            visited.extend((g, v) for v in vis)
        s = np.maximum(s, rep_score(Q[h], K[g, r]))
    return s


# --------------------------------------------------------------------------- #
# SelectRep with relative RoPE (InfiniteHiP page, "Four RoPE Styles for       #
# Context Pruning": Relative (RT); "Layer-Specific Strategy Assignment")      #
# --------------------------------------------------------------------------- #
ROPE_QUANT = 128        # rotated queries are rounded to multiples of 1/128


def rope_rotate(x: np.ndarray, pos: float, base: float) -> np.ndarray:
    """Rotary embedding of x ([..., d]) at position pos, in fp64, with the
    rotate-half pairing (element i with element i + d/2) and frequencies
    theta_i = base^(-2i/d): x * cos(pos theta) + rotate(x) * sin(pos theta)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    theta = np.power(np.float64(base), -2.0 * np.arange(half, dtype=np.float64) / d)
    ang = np.float64(pos) * theta
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rt_queries(q: np.ndarray, n_stream: int, base: float) -> Tuple[np.ndarray, np.ndarray]:
    """The two query sets of relative-RoPE SelectRep: the left-branch
    representative sits n_stream + 1 positions behind the query, the right one
    n_stream (keys unrotated; equal in exact arithmetic to rotating the query by
    n_stream + 1 and the keys by 0 and 1). Rounded to multiples of 1/128, so
    every score against grid keys is exact in fp32."""
    ql = np.rint(rope_rotate(q, n_stream + 1, base) * ROPE_QUANT) / ROPE_QUANT
    qr = np.rint(rope_rotate(q, n_stream, base) * ROPE_QUANT) / ROPE_QUANT
    return ql.astype(np.float32), qr.astype(np.float32)


def select_rep_rt_all(ql: np.ndarray, qr: np.ndarray, K, g: int, P2: np.ndarray,
                      visited: Optional[list] = None) -> Tuple[np.ndarray, np.ndarray]:
    """SelectRep with relative RoPE for every chunk (row of P2): at each split
    the left half's representative is scored with the left queries and the
    right half's with the right queries; the right half wins only on a
    strictly greater score; a representative that won from the right is scored
    again as the left one of the next split. Returns (representatives, chunk
    scores), the score being the one the representative won its last split
    with (its left score when the chunk has a single key)."""
    nc, l = P2.shape
    rows = np.arange(nc)
    a = np.zeros(nc, dtype=np.int64)
    z = np.full(nc, l - 1, dtype=np.int64)
    sl = rep_score(ql, K[g, P2[rows, a]])
    if visited is not None:
        visited.append(P2[rows, a])
    win = sl.copy()
    n_iter = int(np.ceil(np.log2(l))) if l > 1 else 0
    for _ in range(n_iter):
        mid = (a + z + 1) // 2
        sr = rep_score(qr, K[g, P2[rows, mid]])
        if visited is not None:
            visited.append(P2[rows, mid])
        right = sr > sl
        win = np.where(right, sr, sl)
        a = np.where(right, mid, a)
        z = np.where(right, z, mid - 1)
        sl = np.where(right, rep_score(ql, K[g, P2[rows, mid]]), sl)
    return P2[rows, a], win


def chunk_scores_rt(Q: np.ndarray, K, P: np.ndarray, l: int, n_stream: int, base: float) -> np.ndarray:
    """Step 5 with relative-RoPE SelectRep: the max over heads of each head's
    chunk score."""
    Hq = Q.shape[0]
    G = Hq // K.shape[0]
    nc = len(P) // l
    P2 = np.asarray(P).reshape(nc, l)
    s = np.full(nc, -np.inf, dtype=np.float32)
    for h in range(Hq):
        ql, qr = rt_queries(Q[h], n_stream, base)
        _, win = select_rep_rt_all(ql, qr, K, h // G, P2)
        s = np.maximum(s, win)
    return s


def prune_block_rt(Q: np.ndarray, K, s: int, e: int, p: Params, base: float) -> np.ndarray:
    """prune_block with relative-RoPE SelectRep (n_stream = the window)."""
    geo = geometry(s, e, p)
    P = np.arange(geo.mid_lo, geo.mid_hi, dtype=np.int64)
    for l, k in zip(p.chunk, p.keep):
        nc, kc = len(P) // l, k // l
        if nc <= kc:
            continue
        sel = top_k(chunk_scores_rt(Q, K, P, l, p.n_window, base), kc)
        P = np.asarray(P).reshape(nc, l)[sel].reshape(-1)
    return np.concatenate([np.arange(0, geo.sink_hi, dtype=np.int64), P,
                           np.arange(geo.mid_hi, e, dtype=np.int64)])


# --------------------------------------------------------------------------- #
# chunk-indexed RoPE in SelectRep (InfiniteHiP page, "Four RoPE Styles for    #
# Context Pruning": Chunk-indexed; "Layer-Specific Strategy Assignment")      #
# --------------------------------------------------------------------------- #
def rope_round(x: np.ndarray) -> np.ndarray:
    """Round rotated values to multiples of 1/128 (bf16-exact below 2)."""
    return (np.rint(np.asarray(x, dtype=np.float64) * ROPE_QUANT) / ROPE_QUANT).astype(np.float32)


def rope_rotate_rows(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """rope_rotate with its own position for each row: x [n, d], pos [n]."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    theta = np.power(np.float64(base), -2.0 * np.arange(half, dtype=np.float64) / d)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * theta[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def ci_chunk_index(pos, n_sink: int, l: int):
    """Position ID of a key: the index of its chunk of length l in the tiling
    of the middle that starts at n_sink."""
    return (np.asarray(pos) - n_sink) // l


def ci_query_positions(i_orig: np.ndarray, mid_hi: int, n_sink: int, n_stream: int, l: int) -> np.ndarray:
    """Position ID of each query: the last chunk of the stage's tiling of
    [n_sink, mid_hi) sits n_stream behind it, capped at the query's own
    position."""
    c_last = (mid_hi - n_sink) // l - 1
    return np.minimum(np.asarray(i_orig), c_last + n_stream)


class CiKeys:
    """K seen through chunk-indexed RoPE: K[g, positions] returns the rows
    rotated to their chunk index and rounded to the 1/128 grid."""

    def __init__(self, K, n_sink: int, l: int, base: float):
        self.K, self.n_sink, self.l, self.base = K, n_sink, l, base
        self.shape = K.shape

    def __getitem__(self, idx):
        g, pos = idx
        pos = np.asarray(pos)
        rows = np.asarray(self.K[g, pos], dtype=np.float64).reshape(len(pos), -1)
        return rope_round(rope_rotate_rows(rows, ci_chunk_index(pos, self.n_sink, self.l), self.base))


def prune_block_ci(Q: np.ndarray, K, s: int, e: int, p: Params, base: float) -> np.ndarray:
    """prune_block with chunk-indexed RoPE (n_stream = the window): in every
    stage the queries and the keys are rotated to their position IDs and the
    plain SelectRep, chunk score and top-K run on the rotated vectors."""
    geo = geometry(s, e, p)
    P = np.arange(geo.mid_lo, geo.mid_hi, dtype=np.int64)
    i_orig = np.arange(s, e)
    for l, k in zip(p.chunk, p.keep):
        nc, kc = len(P) // l, k // l
        if nc <= kc:
            continue
        qpos = ci_query_positions(i_orig, geo.mid_hi, p.n_sink, p.n_window, l)
        Qr = np.stack([rope_round(rope_rotate_rows(Q[h], qpos, base)) for h in range(Q.shape[0])])
        sel = top_k(chunk_scores(Qr, CiKeys(K, p.n_sink, l, base), P, l), kc)
        P = np.asarray(P).reshape(nc, l)[sel].reshape(-1)
    return np.concatenate([np.arange(0, geo.sink_hi, dtype=np.int64), P,
                           np.arange(geo.mid_hi, e, dtype=np.int64)])


def top_k(s: np.ndarray, k: int) -> np.ndarray:
    """Step 6: indices of the k highest scores, ties to the lower index; a full
    sort by (score descending, index ascending). Returned in ascending order."""
    n = len(s)
    if n <= k:
        return np.arange(n)
    order = np.lexsort((np.arange(n), -np.asarray(s, dtype=np.float64)))
    return np.sort(order[:k])


# --------------------------------------------------------------------------- #
# pruning of one query block                                                  #
# --------------------------------------------------------------------------- #
def prune_block(Q: np.ndarray, K, s: int, e: int, p: Params,
                trace: Optional[list] = None) -> np.ndarray:
    """The index row of query block [s, e): sinks, pruned middle, window.

    Q: [Hq, e-s, d] float32 (the block's queries); K: [Hkv, >=e, d] indexable.
    Returns the ascending int64 array of key positions (no padding).
    If ``trace`` is a list, one entry per executed stage is appended:
    (stage, n_chunks, kept chunk ids, representative positions per head).
    """
    geo = geometry(s, e, p)
    P = np.arange(geo.mid_lo, geo.mid_hi, dtype=np.int64)
    for i, (l, k) in enumerate(zip(p.chunk, p.keep)):
        nc = len(P) // l
        kc = k // l
        if nc <= kc:
            continue
        sc = chunk_scores(Q, K, P, l)
        sel = top_k(sc, kc)
        if trace is not None:
            trace.append((i, nc, sel, sc))
        P = np.asarray(P).reshape(nc, l)[sel].reshape(-1)
    row = np.concatenate([np.arange(0, geo.sink_hi, dtype=np.int64), P,
                          np.arange(geo.mid_hi, e, dtype=np.int64)])
    return row


def visited_rows(Q: np.ndarray, K, s: int, e: int, p: Params) -> List[int]:
    """Per stage, the number of distinct (kv head, key position) rows SelectRep
    reads for block [s, e) (0 for a stage that keeps everything): the
    algorithmic K traffic of the stage."""
    geo = geometry(s, e, p)
    P = np.arange(geo.mid_lo, geo.mid_hi, dtype=np.int64)
    out = []
    for l, k in zip(p.chunk, p.keep):
        nc = len(P) // l
        kc = k // l
        if nc <= kc:
            out.append(0)
            continue
        vis: list = []
        sc = chunk_scores(Q, K, P, l, visited=vis)
        keys = np.unique(np.concatenate([g * (1 << 40) + v for g, v in vis]))
        out.append(int(keys.size))
        P = P.reshape(nc, l)[top_k(sc, kc)].reshape(-1)
    return out


# --------------------------------------------------------------------------- #
# mask caching across decode steps ("Sparse Attention Mask Caching")          #
# --------------------------------------------------------------------------- #
@dataclass
class StageRecord:
    """The remembered output of one pruning stage for one sequence: the
    ascending key positions it kept (whole chunks of the stage's size) and the
    end of the stage-1 middle those positions were drawn from."""
    kept: np.ndarray
    mid_end: int


def stages_due(step: int, refresh: Sequence[int]) -> List[bool]:
    """Stage i recomputes its output at decode step ``step`` exactly when
    step mod n_refresh^(i) == 0; otherwise its remembered output is reused."""
    if step < 0 or any(n < 1 for n in refresh):
        raise ValueError("step must be >= 0 and every refresh interval >= 1")
    return [step % n == 0 for n in refresh]


def prune_decode_cached(q: np.ndarray, K, e: int, p: Params, refresh: Sequence[int],
                        step: int, cache: List[Optional[StageRecord]],
                        trace: Optional[list] = None) -> np.ndarray:
    """Index row of the decode query at position e-1 with per-stage mask caching.

    q: [Hq, d] float32, the newest query; K: [Hkv, >=e, d] indexable; cache: a
    list of n_stages records (None before the first refresh), updated in place.
    A stage that is due takes the current output of the stage before it (the
    one just recomputed if that stage was due too, its remembered one
    otherwise; for stage 1 the whole middle of the current context), scores it
    with the newest query exactly as an uncached stage does, and remembers what
    it keeps. The row is the current sinks, the last stage's remembered keys,
    and every position from the end of the middle those keys came from up to
    the newest token: keys that left the window since the last stage-1 refresh
    were never scored, so they stay with the window until the next one.
    If ``trace`` is a list, the indices of the recomputed stages are appended.
    """
    if len(cache) != len(p.chunk) or len(refresh) != len(p.chunk):
        raise ValueError("one cache record and one refresh interval per stage")
    geo = geometry(e - 1, e, p)
    due = stages_due(step, refresh)
    for i, (l, k) in enumerate(zip(p.chunk, p.keep)):
        if not due[i]:
            if cache[i] is None:
                raise ValueError(f"stage {i + 1} is not due at step {step} and has no record")
            continue
        if i == 0:
            P = np.arange(geo.mid_lo, geo.mid_hi, dtype=np.int64)
            mid_end = geo.mid_hi
        else:
            P = cache[i - 1].kept
            mid_end = cache[i - 1].mid_end
        nc = len(P) // l
        kc = k // l
        if nc > kc:
            sel = top_k(chunk_scores(q[:, None, :], K, P, l), kc)
            P = np.asarray(P).reshape(nc, l)[sel].reshape(-1)
        cache[i] = StageRecord(np.array(P, dtype=np.int64), int(mid_end))
        if trace is not None:
            trace.append(i)
    last = cache[-1]
    if last.mid_end > e:
        raise ValueError("the context is shorter than when its stage-1 record was made")
    return np.concatenate([np.arange(0, geo.sink_hi, dtype=np.int64), last.kept,
                           np.arange(last.mid_end, e, dtype=np.int64)])


def cached_row_bound(p: Params, growth: int) -> int:
    """Most entries a cached decode row can hold when the context has grown by
    ``growth`` tokens since the stage-1 refresh its keys descend from."""
    return p.n_sink + p.keep[-1] + p.n_window + p.chunk[0] - 1 + growth


def block_bounds(m: int, T: int, p: Params, decode: bool) -> Tuple[int, int]:
    """Step 1 query blocking: block m is [m*b_q, (m+1)*b_q); a decode step is the
    single query T-1."""
    if decode:
        return T - 1, T
    return m * p.block_q, (m + 1) * p.block_q


def pad_row(row: np.ndarray, width: int) -> np.ndarray:
    out = np.full(width, -1, dtype=np.int32)
    out[:len(row)] = row
    return out


# --------------------------------------------------------------------------- #
# MInference Block-Sparse heads: per-input block index estimation             #
# ("Online Dynamic Index Estimation: Block-Sparse Heads (Algorithm 3)")       #
# --------------------------------------------------------------------------- #
def bs_pool(X: np.ndarray, block: int) -> np.ndarray:
    """Step 1: the mean of every `block` consecutive token rows, per head.

    X: [H, T, d] (T a multiple of block) -> [H, T/block, d] float64."""
    X = np.asarray(X, dtype=np.float64)
    H, T, d = X.shape
    return X.reshape(H, T // block, block, d).mean(axis=2)


def bs_block_scores(Qp: np.ndarray, Kp: np.ndarray, h: int, m: int) -> np.ndarray:
    """Steps 2-3 ranking key of query block m for query head h: the pooled
    logits q~_m . k~_j of key blocks j = 0..m (strictly later key blocks are
    masked out), evaluated in fp64 and rounded once to fp32. The row softmax
    of step 2 and the 1/sqrt(d) scale are monotone, so they do not change which
    blocks score highest and are not applied.

    Qp: [Hq, nblk, d], Kp: [Hkv, nblk, d] pooled; kv head of h is h // (Hq/Hkv)."""
    G = Qp.shape[0] // Kp.shape[0]
    return (Kp[h // G, :m + 1] @ Qp[h, m]).astype(np.float32)


def bs_select(scores: np.ndarray, k_blocks: int) -> np.ndarray:
    """Step 3: the k_b key blocks with the highest scores (ties to the lower
    block index), ascending; every block when there are no more than k_b."""
    return top_k(scores, k_blocks)


def bs_rows(Q: np.ndarray, K, block: int, k_blocks: int) -> List[List[np.ndarray]]:
    """Step 4's block index lists as index rows: for every query head h and
    query block m, the ascending key positions of its selected blocks.

    Q: [Hq, T, d], K: [Hkv, T, d] (one sequence). Returns rows[h][m]."""
    Qp = bs_pool(Q, block)
    Kp = bs_pool(np.asarray(K[:, :Q.shape[1]]), block)
    Hq, nblk = Qp.shape[0], Qp.shape[1]
    rows = []
    for h in range(Hq):
        rh = []
        for m in range(nblk):
            sel = bs_select(bs_block_scores(Qp, Kp, h, m), k_blocks)
            rh.append((sel[:, None] * block + np.arange(block)[None, :]).reshape(-1).astype(np.int64))
        rows.append(rh)
    return rows


def bs_lists(Q: np.ndarray, K, block: int, k_blocks: int) -> List[List[np.ndarray]]:
    """Step 4's block index lists as lists: lists[h][m] = the ascending ids of
    the key blocks kept for query head h and query block m (the page's
    block-sparse kernel takes these ids, not positions)."""
    Qp = bs_pool(Q, block)
    Kp = bs_pool(np.asarray(K[:, :Q.shape[1]]), block)
    Hq, nblk = Qp.shape[0], Qp.shape[1]
    return [[bs_select(bs_block_scores(Qp, Kp, h, m), k_blocks).astype(np.int64) for m in range(nblk)]
            for h in range(Hq)]


def bs_index_width(block: int, k_blocks: int) -> int:
    """Width of a block-sparse index row: k_b blocks of `block` positions,
    rounded up to 64."""
    return (block * k_blocks + 63) // 64 * 64


# --------------------------------------------------------------------------- #
# MInference Vertical-Slash heads: per-input vertical and slash estimation    #
# ("Online Dynamic Index Estimation: Vertical-Slash Heads (Algorithm 2)";     #
# index building of "Vertical-Slash Hybrid Kernel (Appendix C.4.2)")          #
# --------------------------------------------------------------------------- #
VS_LAST_Q = 64          # estimation queries: the last 64 of the sequence
VS_BLOCK = 64           # query blocks and key blocks of the index rows


def vs_sums(Q: np.ndarray, K, h: int) -> Tuple[np.ndarray, np.ndarray]:
    """Steps 1-3 for query head h of one sequence: the causal softmax of the
    last 64 queries against every key (scale 1/sqrt(d), fp64 after exact fp32
    dot products), summed over the queries for every key column (vertical) and
    over the queries for every offset d = query position - key position >= 0
    (slash). Q: [Hq, T, d], K: [Hkv, T, d]. Returns (sum_v [T], sum_s [T])."""
    Hq, T, d = Q.shape
    G = Hq // K.shape[0]
    nq = min(VS_LAST_Q, T)
    t = np.arange(T - nq, T)
    q = np.asarray(Q[h, T - nq:], dtype=np.float32)
    k = np.asarray(K[h // G, :T], dtype=np.float32)
    z = (q @ k.T).astype(np.float64) * (1.0 / np.sqrt(np.float64(d)))
    z = np.where(np.arange(T)[None, :] <= t[:, None], z, -np.inf)
    a = np.exp(z - z.max(axis=1, keepdims=True))
    a /= a.sum(axis=1, keepdims=True)
    sum_v = a.sum(axis=0)
    sum_s = np.zeros(T)
    for i in range(nq):
        sum_s[:t[i] + 1] += a[i, t[i]::-1]          # offset d pairs query t[i] with key t[i] - d
    return sum_v, sum_s


def vs_select(sums: np.ndarray, k: int) -> np.ndarray:
    """Steps 2-3: the k highest sums, ranked in fp32 (the sums rounded once),
    ties to the lower index; ascending."""
    return top_k(np.asarray(sums).astype(np.float32), k)


def vs_row(i_v: np.ndarray, i_s: np.ndarray, m: int) -> np.ndarray:
    """Step 4 for query block m (queries [64m, 64m+64)): every slash offset d
    covers keys [64m - d, 64m + 63 - d] in this block's rows; those ranges,
    clipped to keys >= 0 and rounded out to the 64-aligned key blocks they
    touch, are attended whole; vertical columns before the block's end that
    lie in none of those blocks are attended as single columns. Returns the
    ascending key positions (the causal mask inside the block is applied by
    the attention)."""
    s, e = VS_BLOCK * m, VS_BLOCK * (m + 1)
    blocks = set()
    for d in np.asarray(i_s, dtype=np.int64):
        lo, hi = max(0, s - int(d)), e - 1 - int(d)
        if hi >= 0:
            blocks.update(range(lo // VS_BLOCK, hi // VS_BLOCK + 1))
    cols = [int(v) for v in i_v if v < e and int(v) // VS_BLOCK not in blocks]
    pos = [VS_BLOCK * b + x for b in sorted(blocks) for x in range(VS_BLOCK)] + cols
    return np.array(sorted(pos), dtype=np.int64)


def vs_lists(i_v: np.ndarray, i_s: np.ndarray, m: int) -> Tuple[np.ndarray, np.ndarray]:
    """Step 4 for query block m in the two lists of the hybrid kernel
    (MInference page, "Vertical-Slash Hybrid Kernel (Appendix C.4.2,
    Algorithms 4 and 5)": a block index list for the slash part, attended in
    whole 64-key blocks, and a column index list for the vertical part,
    gathered). Blocks: the ascending ids of the 64-aligned key blocks that
    the kept offsets' key ranges [64m - d, 64m + 63 - d] (clipped at key 0)
    touch. Columns: the kept columns before the block's end in none of those
    blocks, ascending. The positions of the blocks and the columns together
    are the row of vs_row."""
    s, e = VS_BLOCK * m, VS_BLOCK * (m + 1)
    touched = np.zeros(m + 1, dtype=bool)          # key blocks 0..m (later ones hold no key < e)
    for d in np.asarray(i_s, dtype=np.int64):
        lo, hi = max(0, s - int(d)), e - 1 - int(d)
        if hi >= 0:
            touched[lo // VS_BLOCK:hi // VS_BLOCK + 1] = True
    iv = np.sort(np.asarray(i_v, dtype=np.int64))
    iv = iv[iv < e]
    cols = iv[~touched[iv // VS_BLOCK]]
    return np.nonzero(touched)[0].astype(np.int64), cols


def vs_lists_all(Q: np.ndarray, K, k_v: int, k_s: int) -> List[List[Tuple[np.ndarray, np.ndarray]]]:
    """lists[h][m] = vs_lists(...) of one sequence (estimation and selection as
    in vs_rows)."""
    Hq, T, _ = Q.shape
    out = []
    for h in range(Hq):
        sv, ss = vs_sums(Q, K, h)
        iv, is_ = vs_select(sv, k_v), vs_select(ss, k_s)
        out.append([vs_lists(iv, is_, m) for m in range(T // VS_BLOCK)])
    return out


def list_positions(blocks: np.ndarray, cols: np.ndarray, block: int = VS_BLOCK) -> np.ndarray:
    """The key positions of a block list and a column list: every key of each
    listed block and every listed column, ascending (the two are disjoint)."""
    b = np.asarray(blocks, dtype=np.int64)
    pos = (b[:, None] * block + np.arange(block)[None, :]).reshape(-1)
    return np.sort(np.concatenate([pos, np.asarray(cols, dtype=np.int64)]))


def vs_index_width(T: int, k_v: int, k_s: int) -> int:
    """Row width: at most 2 key blocks per slash offset (and no more than the
    sequence's blocks) plus k_v columns, rounded up to 64 and at most T."""
    n = VS_BLOCK * min(T // VS_BLOCK, 2 * k_s) + k_v
    return min(T, (n + 63) // 64 * 64)


def vs_rows(Q: np.ndarray, K, k_v: int, k_s: int) -> List[List[np.ndarray]]:
    """rows[h][m] of one sequence: estimation, selection and index building."""
    Hq, T, _ = Q.shape
    rows = []
    for h in range(Hq):
        sv, ss = vs_sums(Q, K, h)
        iv, is_ = vs_select(sv, k_v), vs_select(ss, k_s)
        rows.append([vs_row(iv, is_, m) for m in range(T // VS_BLOCK)])
    return rows


# --------------------------------------------------------------------------- #
# attention over an index row                                                 #
# --------------------------------------------------------------------------- #
def attend_block(Q: np.ndarray, K, V, row: np.ndarray, s: int, scale: float) -> np.ndarray:
    """out[h, t] = sum_{p in row, p <= s+t} softmax_p(scale * q_{h,s+t} . k_p) v_p.

    Q: [Hq, n_q, d] float32; K, V: [Hkv, >=T, d] indexable; row: key positions
    (entries < 0 are padding and ignored). Dot products are fp32 (exact on the
    input grid), softmax and P.V are fp64, the result is cast to fp32.

    A query that sees no key of its row (possible for per-head rows such as
    the vertical-slash ones) attends to nothing: its output is 0, the empty
    sum (the pages define the softmax only over a non-empty key set).
    """
    row = np.asarray(row, dtype=np.int64)
    row = row[row >= 0]
    Hq, nq, d = Q.shape
    Hkv = K.shape[0]
    G = Hq // Hkv
    out = np.zeros((Hq, nq, d), dtype=np.float32)
    tpos = s + np.arange(nq)
    visible = row[None, :] <= tpos[:, None]               # causal mask [nq, n]
    for g in range(Hkv):
        kr = np.asarray(K[g, row], dtype=np.float32)
        vr = np.asarray(V[g, row], dtype=np.float64)
        for h in range(g * G, (g + 1) * G):
            z = (np.asarray(Q[h], dtype=np.float32) @ kr.T).astype(np.float64) * scale
            z = np.where(visible, z, -np.inf)
            seen = visible.any(axis=1, keepdims=True)
            zmax = np.where(seen, z.max(axis=1, keepdims=True, initial=-np.inf), 0.0)
            w = np.exp(z - zmax)
            den = w.sum(axis=1, keepdims=True)
            out[h] = np.where(seen, (w @ vr) / np.where(seen, den, 1.0), 0.0).astype(np.float32)
    return out


def dense_block(Q: np.ndarray, K, V, s: int, e: int, scale: float) -> np.ndarray:
    """Exact causal attention of queries [s, e) over keys [0, e)."""
    return attend_block(Q, K, V, np.arange(e, dtype=np.int64), s, scale)


def default_scale(d: int) -> float:
    return 1.0 / np.sqrt(d)
