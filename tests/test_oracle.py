"""Pins for the CPU oracle: what the pages and the mathematics fix.

None of these tests touches the GPU or the HIP library. Each checks the oracle
against something other than itself: values printed on the pages (fixtures in
tests/golden/), closed forms, brute force on tiny inputs, and special cases that
reduce to textbook attention computed by a library routine.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

from dynamic_sparse_attention_query_amd import gen
from oracle import ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def grid(rng, shape):
    return rng.integers(-8, 9, size=shape).astype(np.float32) / np.float32(8)


# --------------------------------------------------------------------------- #
# exactness of scores on the input grid                                       #
# --------------------------------------------------------------------------- #
def test_grid_dot_products_are_exact_in_any_order():
    rng = np.random.default_rng(0)
    q = rng.integers(-8, 9, size=(16, 128))
    k = rng.integers(-8, 9, size=(300, 128))
    exact = (q @ k.T).astype(np.float64) / 64.0               # integer arithmetic
    blas = ref.rep_score(q.astype(np.float32) / 8, k.astype(np.float32) / 8)
    assert np.array_equal(blas.astype(np.float64), exact.max(axis=0))
    qf, kf = q.astype(np.float32) / 8, k.astype(np.float32) / 8
    for trial in range(3):
        perm = rng.permutation(128)
        acc = np.zeros((16, 300), dtype=np.float32)
        for i in perm:                                         # shuffled fp32 summation
            acc = (acc + qf[:, i:i + 1] * kf[None, :, i]).astype(np.float32)
        assert np.array_equal(acc.astype(np.float64), exact)


# --------------------------------------------------------------------------- #
# a1: candidate set, sinks, window -- the pages' worked counts                #
# --------------------------------------------------------------------------- #
def test_page_counts_at_one_million_tokens():
    g = _load("p1_counts.json")
    p = ref.Params(1, tuple(g["stage_chunk"]), tuple(g["stage_keep"]), g["n_sink"], g["n_stream"])
    T = g["T"]
    s, e = ref.block_bounds(0, T, p, decode=True)
    geo = ref.geometry(s, e, p)
    always = geo.sink_hi + (e - (geo.mid_lo + (e - p.n_window - geo.mid_lo)))  # sinks + window
    middle = (e - p.n_window) - geo.mid_lo
    assert middle == g["pruned_middle"]
    assert geo.sink_hi + p.n_window == g["always_kept"] == always
    assert abs(geo.n1 - g["stage1_chunks_approx"]) / g["stage1_chunks_approx"] < 0.01
    assert abs(p.keep[0] // p.chunk[1] - g["stage2_chunks_approx"]) / 1000 < 0.03
    assert abs(p.keep[1] // p.chunk[2] - g["stage3_chunks_approx"]) / 1000 < 0.03


def test_infllm_active_length():
    g = _load("p2_active.json")
    S, Kc, C, W = g["S"], g["K"], g["C"], g["W"]
    p = ref.Params(1, (C,), (Kc * C,), S, W)
    T = S + W + 20 * C                       # middle is a whole number of chunks
    rng = np.random.default_rng(1)
    K = grid(rng, (1, T, 16))
    q = grid(rng, (1, 1, 16))
    s, e = ref.block_bounds(0, T, p, decode=True)
    row = ref.prune_block(q, K, s, e, p)
    assert len(row) == g["L_active"]


# --------------------------------------------------------------------------- #
# a2: SelectRep                                                               #
# --------------------------------------------------------------------------- #
def select_rep_recursive(qh, K, g, chunk):
    """The tournament as a recursion: a range is represented by its first key;
    split at the round-half-up midpoint; the right half wins only on a strictly
    greater representative score."""
    def sig(pos):
        return float((qh @ K[g, pos]).max())

    def go(lo, hi):                          # inclusive range of chunk offsets
        if lo == hi:
            return lo
        mid = (lo + hi + 1) // 2
        if sig(chunk[mid]) > sig(chunk[lo]):
            return go(mid, hi)
        return go(lo, mid - 1)
    return int(chunk[go(0, len(chunk) - 1)])


@pytest.mark.parametrize("l", [1, 2, 4, 8, 16, 32, 64, 256])
def test_selectrep_iterative_matches_recursive(l):
    rng = np.random.default_rng(l)
    d, bq = 16, 4
    K = grid(rng, (2, 2048, d))
    for trial in range(20):
        qh = grid(rng, (bq, d))
        g = int(rng.integers(0, 2))
        st = int(rng.integers(0, 2048 - l))
        chunk = np.arange(st, st + l)
        r_rec = select_rep_recursive(qh, K, g, chunk)
        r_it = ref.select_rep(qh, K, g, chunk)
        r_vec = ref.select_rep_all(qh, K, g, chunk[None, :])[0]
        assert r_rec == r_it == r_vec


def test_selectrep_evaluation_count():
    g = _load("p1_counts.json")["selectrep_evaluations"]
    rng = np.random.default_rng(3)
    K = grid(rng, (1, 4096, 8))
    qh = grid(rng, (2, 8))
    for l_str, n_eval in g.items():
        l = int(l_str)
        seen = []
        ref.select_rep(qh, K, 0, np.arange(100, 100 + l), visit=seen.append)
        assert len(seen) == n_eval == 2 * math.ceil(math.log2(l))
        assert len(set(seen)) == 1 + int(math.log2(l))


def test_selectrep_monotone_chunks_reach_true_argmax():
    d = 8
    q = np.zeros((1, d), dtype=np.float32)
    q[0, 0] = 1.0
    for l in (4, 16, 64):
        K = np.zeros((1, l, d), dtype=np.float32)
        K[0, :, 0] = np.arange(l) / 64.0                # score strictly increasing
        assert ref.select_rep(q, K, 0, np.arange(l)) == l - 1
        K[0, :, 0] = -np.arange(l) / 64.0               # strictly decreasing
        assert ref.select_rep(q, K, 0, np.arange(l)) == 0


def test_selectrep_score_dominates_first_and_visited():
    rng = np.random.default_rng(5)
    K = grid(rng, (1, 1024, 16))
    for trial in range(50):
        qh = grid(rng, (3, 16))
        chunk = np.arange(64 * trial % 960, 64 * trial % 960 + 32)
        seen = []
        r = ref.select_rep(qh, K, 0, chunk, visit=seen.append)
        sig = lambda p: (qh @ K[0, p]).max()
        assert sig(r) >= sig(chunk[0])
        assert sig(r) == max(sig(p) for p in seen)


# --------------------------------------------------------------------------- #
# a3 + a4 + a5: chunk score, top-K, assembly                                  #
# --------------------------------------------------------------------------- #
def _token_scores(Q, K, G):
    """max over heads and block queries of q.k for every key (library matmul)."""
    Hq = Q.shape[0]
    S = np.stack([Q[h] @ K[h // G].T for h in range(Hq)])   # [Hq, bq, T]
    return S.max(axis=(0, 1))


def test_chunk_size_one_is_token_topk():
    """l_c = 1: SelectRep is the token itself, so a stage is plain token-level
    top-k of max_{h,t} q.k, ties to the lower position."""
    rng = np.random.default_rng(7)
    Hq, Hkv, d, bq, T = 4, 2, 16, 8, 512
    Q = grid(rng, (Hq, T, d))
    K = grid(rng, (Hkv, T, d))
    p = ref.Params(bq, (1,), (40,), 8, 32)
    for m in (20, 45, 63):
        s, e = ref.block_bounds(m, T, p, decode=False)
        row = ref.prune_block(Q[:, s:e], K, s, e, p)
        geo = ref.geometry(s, e, p)
        sc = _token_scores(Q[:, s:e], K, Hq // Hkv)[geo.mid_lo:geo.mid_hi]
        order = np.argsort(-sc.astype(np.float64), kind="stable")[:40]
        expect = np.sort(order + geo.mid_lo)
        mid = row[(row >= geo.mid_lo) & (row < geo.mid_hi)]
        assert np.array_equal(mid, expect)


def test_constant_chunks_rank_by_max_over_heads_and_queries():
    """Keys constant inside each stage-1 chunk (per kv head): every
    representative has the chunk's exact score, so the two-stage result is the
    top (k2) tokens by max over ALL heads and queries, ties to the lower
    position (a mean over heads, or one head only, fails this)."""
    rng = np.random.default_rng(11)
    Hq, Hkv, d, bq = 8, 2, 16, 4
    l1, l2 = 16, 4
    T = 16 * 80
    K = np.repeat(grid(rng, (Hkv, T // l1, d)), l1, axis=1)
    Q = grid(rng, (Hq, T, d))
    p = ref.Params(bq, (l1, l2), (160, 48), 16, 64)
    for m in (100, 250, 319):
        s, e = ref.block_bounds(m, T, p, decode=False)
        row = ref.prune_block(Q[:, s:e], K, s, e, p)
        geo = ref.geometry(s, e, p)
        sc = _token_scores(Q[:, s:e], K, Hq // Hkv)[geo.mid_lo:geo.mid_hi]
        expect = np.sort(np.argsort(-sc.astype(np.float64), kind="stable")[:48] + geo.mid_lo)
        mid = row[(row >= geo.mid_lo) & (row < geo.mid_hi)]
        assert np.array_equal(mid, expect)


def test_topk_matches_brute_force_with_ties():
    rng = np.random.default_rng(13)
    for trial in range(200):
        n = int(rng.integers(1, 13))
        k = int(rng.integers(0, n + 2))
        s = rng.integers(-3, 4, size=n).astype(np.float32)   # heavy ties
        got = ref.top_k(s, k)
        if n <= k:
            assert np.array_equal(got, np.arange(n))
            continue
        valid = []
        for S in itertools.combinations(range(n), k):
            Sset = set(S)
            ok = all(s[j] > s[o] or (s[j] == s[o] and j < o)
                     for j in Sset for o in range(n) if o not in Sset)
            if ok:
                valid.append(S)
        assert len(valid) == 1
        assert tuple(got.tolist()) == valid[0]


def _small_case(seed, Hq=4, Hkv=2, d=16, T=1024):
    rng = np.random.default_rng(seed)
    Q = grid(rng, (Hq, T, d))
    K = grid(rng, (Hkv, T, d))
    V = rng.standard_normal((Hkv, T, d)).astype(np.float32)
    return Q, K, V


def test_row_invariants_and_count():
    Q, K, V = _small_case(17)
    T = Q.shape[1]
    p = ref.Params(16, (32, 8), (256, 64), 16, 64)
    for m in range(T // 16):
        s, e = ref.block_bounds(m, T, p, decode=False)
        row = ref.prune_block(Q[:, s:e], K, s, e, p)
        geo = ref.geometry(s, e, p)
        assert np.all(np.diff(row) > 0) and row[-1] == e - 1 and row[0] == 0
        assert set(range(min(16, e))) <= set(row.tolist())                  # sinks
        assert set(range(max(0, e - 64), e)) <= set(row.tolist())           # window
        n_mid = geo.mid_hi - geo.mid_lo
        assert len(row) == geo.sink_hi + min(64, n_mid) + (e - geo.mid_hi)
        assert len(row) <= ref.index_width(p)
        if n_mid >= 64:
            rem = (e - 64 - 16) % 32
            assert len(row) == 16 + 64 + 64 + rem


# --------------------------------------------------------------------------- #
# a6-a8: attention                                                            #
# --------------------------------------------------------------------------- #
def _sdpa(Q, K, V, scale, mask=None, causal=False):
    torch = pytest.importorskip("torch")
    Hq, Hkv = Q.shape[0], K.shape[0]
    G = Hq // Hkv
    q = torch.from_numpy(Q.astype(np.float64))[None]
    k = torch.from_numpy(np.repeat(K, G, axis=0).astype(np.float64))[None]
    v = torch.from_numpy(np.repeat(V, G, axis=0).astype(np.float64))[None]
    if mask is not None:
        mask = torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask,
                                                         is_causal=causal, scale=scale)
    return o[0].numpy()


def test_dense_matches_library_causal_attention():
    Q, K, V = _small_case(19, T=256)
    scale = ref.default_scale(16)
    out = np.concatenate([ref.dense_block(Q[:, s:s + 32], K, V, s, s + 32, scale)
                          for s in range(0, 256, 32)], axis=1)
    expect = _sdpa(Q, K, V, scale, causal=True)
    np.testing.assert_allclose(out, expect, rtol=2e-6, atol=2e-6)


def test_full_budget_is_dense_attention_bitwise():
    Q, K, V = _small_case(23)
    T = Q.shape[1]
    p = ref.Params(32, (32, 8), (T, T), 16, 64)
    scale = ref.default_scale(16)
    for m in (0, 5, 17, 31):
        s, e = ref.block_bounds(m, T, p, decode=False)
        row = ref.prune_block(Q[:, s:e], K, s, e, p)
        assert np.array_equal(row, np.arange(e))
        a = ref.attend_block(Q[:, s:e], K, V, row, s, scale)
        b = ref.dense_block(Q[:, s:e], K, V, s, e, scale)
        assert np.array_equal(a, b)


def test_zero_budget_is_sink_plus_window_attention():
    """keep = 0: only sinks and the local window remain (the A-shape /
    StreamingLLM pattern), checked against a library attention with that mask.
    The sizes make the middle a whole number of chunks, so no grid tail joins
    the window."""
    Q, K, V = _small_case(29, T=512)
    T = 512
    n_sink, n_win, bq = 16, 48, 16
    p = ref.Params(bq, (16,), (0,), n_sink, n_win)
    scale = ref.default_scale(16)
    t = np.arange(T)
    e_of = (t // bq + 1) * bq                       # block end of each query
    ok = (t[None, :] <= t[:, None]) & ((t[None, :] < n_sink) |
                                        (t[None, :] >= e_of[:, None] - n_win))
    expect = _sdpa(Q, K, V, scale, mask=ok)
    for m in range(T // bq):
        s, e = ref.block_bounds(m, T, p, decode=False)
        row = ref.prune_block(Q[:, s:e], K, s, e, p)
        assert np.array_equal(row, np.flatnonzero(ok[e - 1]))
        out = ref.attend_block(Q[:, s:e], K, V, row, s, scale)
        np.testing.assert_allclose(out, expect[:, s:e], rtol=2e-6, atol=2e-6)


def test_query_without_visible_key_outputs_zero():
    """A row whose keys all lie after some of the block's queries: those
    queries see nothing and output 0 (the empty sum); the others equal a
    library attention restricted to the row's keys."""
    Q, K, V = _small_case(37, T=128)
    scale = ref.default_scale(16)
    s, e = 64, 96
    row = np.array([70, 75, 80, 90], dtype=np.int64)       # queries 64..69 see none
    out = ref.attend_block(Q[:, s:e], K, V, row, s, scale)
    t = np.arange(s, e)
    ok = (row[None, :] <= t[:, None])
    assert np.all(out[:, ~ok.any(axis=1)] == 0)
    mask = np.zeros((e - s, K.shape[1]), dtype=bool)
    mask[:, row] = ok
    seen = ok.any(axis=1)
    expect = _sdpa(Q[:, s:e][:, seen], K, V, scale, mask=mask[seen])
    np.testing.assert_allclose(out[:, seen], expect, rtol=2e-6, atol=2e-6)
    assert np.all(ref.attend_block(Q[:, s:e], K, V, np.array([], dtype=np.int64), s, scale) == 0)


def test_no_causal_leak():
    Q, K, V = _small_case(31)
    T = Q.shape[1]
    p = ref.Params(32, (32, 8), (256, 64), 16, 64)
    scale = ref.default_scale(16)
    rng = np.random.default_rng(99)
    for m in (3, 12, 30):
        s, e = ref.block_bounds(m, T, p, decode=False)
        row = ref.prune_block(Q[:, s:e], K, s, e, p)
        out = ref.attend_block(Q[:, s:e], K, V, row, s, scale)
        K2, V2 = K.copy(), V.copy()
        K2[:, e:] = grid(rng, K2[:, e:].shape)
        V2[:, e:] = rng.standard_normal(V2[:, e:].shape)
        row2 = ref.prune_block(Q[:, s:e], K2, s, e, p)
        assert np.array_equal(row, row2)
        assert np.array_equal(out, ref.attend_block(Q[:, s:e], K2, V2, row2, s, scale))
        # and within the block: future keys of each query are ignored
        for tq in range(s, e, 7):
            K3, V3 = K.copy(), V.copy()
            K3[:, tq + 1:] = grid(rng, K3[:, tq + 1:].shape)
            V3[:, tq + 1:] = rng.standard_normal(V3[:, tq + 1:].shape)
            o3 = ref.attend_block(Q[:, tq:tq + 1], K3, V3, row, tq, scale)
            assert np.array_equal(o3[:, 0], out[:, tq - s])


def test_decode_is_last_query_of_prefill():
    Q, K, V = _small_case(37, T=700)
    T = 700
    p = ref.Params(1, (32, 8), (128, 64), 16, 64)
    scale = ref.default_scale(16)
    s, e = ref.block_bounds(0, T, p, decode=True)
    assert (s, e) == (T - 1, T)
    row = ref.prune_block(Q[:, s:e], K, s, e, p)
    out = ref.attend_block(Q[:, s:e], K, V, row, s, scale)
    mask = np.zeros((1, T), dtype=bool)
    mask[0, row] = True
    expect = _sdpa(Q[:, s:e], K, V, scale, mask=mask)
    np.testing.assert_allclose(out, expect, rtol=2e-6, atol=2e-6)


# --------------------------------------------------------------------------- #
# workloads: planted structure is found                                       #
# --------------------------------------------------------------------------- #
def test_needles_survive_pruning_prefill_32k():
    case = gen.make_case("c2")
    cfg = case.cfg
    p = ref.Params(cfg.block_q, cfg.chunk, cfg.keep, cfg.n_sink, cfg.n_window)
    for nd in case.needles:
        m = nd.query // cfg.block_q
        s, e = ref.block_bounds(m, cfg.t, p, decode=False)
        Q = case.q.sub(nd.b)[:, s:e]
        row = ref.prune_block(Q, case.k[nd.b], s, e, p)
        geo = ref.geometry(s, e, p)
        assert geo.n1 * cfg.chunk[0] > cfg.keep[-1]                  # pruning really happens
        assert set(range(nd.slot_start, nd.slot_start + nd.length)) <= set(row.tolist())


def test_visited_rows_bounds():
    rng = np.random.default_rng(41)
    Hq, Hkv, d, T = 8, 2, 16, 4096
    Q = grid(rng, (Hq, 1, d))
    K = grid(rng, (Hkv, T, d))
    p = ref.Params(1, (64, 8), (1024, 256), 16, 64)
    s, e = ref.block_bounds(0, T, p, decode=True)
    vis = ref.visited_rows(Q, K, s, e, p)
    geo = ref.geometry(s, e, p)
    nc = [geo.n1, 1024 // 8]
    G = Hq // Hkv
    for i, (n, l) in enumerate(zip(nc, p.chunk)):
        lo = n * Hkv * (1 + int(math.log2(l)))
        hi = n * Hkv * min(G * int(math.log2(l)) + 1, l)
        assert lo <= vis[i] <= hi
    # identical queries in a GQA group share every representative
    Q2 = np.repeat(Q[::G], G, axis=0)
    vis2 = ref.visited_rows(Q2, K, s, e, p)
    assert vis2[0] == nc[0] * Hkv * (1 + int(math.log2(p.chunk[0])))


# --------------------------------------------------------------------------- #
# mask caching across decode steps (InfiniteHiP "Sparse Attention Mask        #
# Caching"): the refresh schedule of Figure 7, and reductions to the uncached #
# pruning                                                                     #
# --------------------------------------------------------------------------- #
def test_refresh_schedule_matches_figure_7():
    g = _load("p1_fig7_refresh.json")
    refresh = tuple(g["presets"]["default"])
    n = g["fig7_steps"]
    for i in range(3):
        got = [st for st in range(n) if ref.stages_due(st, refresh)[i]]
        assert got == g["fig7_refresh_steps"][str(i + 1)]
    assert ref.stages_due(g["fig7_only_stage3_step"], refresh) == [False, False, True]
    # the same schedule seen through the cached pruning itself
    rng = np.random.default_rng(5)
    Hq, Hkv, d, T = 4, 2, 16, 1600
    K = grid(rng, (Hkv, T + n, d))
    p = ref.Params(1, (32, 8, 4), (256, 128, 64), 16, 64)
    cache = [None, None, None]
    for st in range(n):
        trace = []
        ref.prune_decode_cached(grid(rng, (Hq, d)), K, T + st, p, refresh, st, cache, trace)
        assert trace == [i for i in range(3) if st in g["fig7_refresh_steps"][str(i + 1)]]
    for name, iv in g["presets"].items():
        assert all(ref.stages_due(0, iv)) and not any(ref.stages_due(1, iv)), name


def test_cached_with_refresh_every_step_is_uncached():
    rng = np.random.default_rng(6)
    Hq, Hkv, d, T = 4, 2, 16, 1500
    K = grid(rng, (Hkv, T + 40, d))
    p = ref.Params(1, (32, 8), (256, 64), 16, 64)
    cache = [None, None]
    for st in range(40):
        q = grid(rng, (Hq, d))
        e = T + st
        got = ref.prune_decode_cached(q, K, e, p, (1, 1), st, cache)
        want = ref.prune_block(q[:, None, :], K, e - 1, e, p)
        assert np.array_equal(got, want), st


def test_cached_constant_query_equals_uncached():
    # With the same query and a middle that does not move (the context grows
    # inside one stage-1 chunk), every remembered stage equals a fresh one, so
    # the cached row must equal the uncached row at every step.
    rng = np.random.default_rng(7)
    Hq, Hkv, d = 8, 2, 16
    p = ref.Params(1, (64, 16, 4), (512, 256, 64), 16, 64)
    e0 = 16 + 64 + 40 * 64                       # middle ends exactly at a chunk boundary
    K = grid(rng, (Hkv, e0 + 64, d))
    q = grid(rng, (Hq, d))
    cache = [None, None, None]
    for st in range(63):
        e = e0 + st
        got = ref.prune_decode_cached(q, K, e, p, (16, 8, 4), st, cache)
        want = ref.prune_block(q[:, None, :], K, e - 1, e, p)
        assert np.array_equal(got, want), st


def test_cached_stage3_refresh_is_token_topk_of_remembered_stage2():
    # Keys constant over every stage-3 chunk make SelectRep irrelevant there:
    # a stage-3 refresh must keep the remembered stage-2 chunks whose token
    # score max_h q_h . k is among the top keep3/l3 (ties to lower positions),
    # computed here with a library sort, plus sinks and everything from the
    # stage-1 middle end up to the newest token.
    rng = np.random.default_rng(8)
    Hq, Hkv, d = 4, 2, 16
    p = ref.Params(1, (64, 32, 8), (1024, 512, 128), 16, 64)
    T = 16 + 64 + 60 * 64 + 37
    codes = rng.integers(-2, 3, size=(Hkv, (T + 16) // 8 + 1, d))
    K = np.repeat(codes, 8, axis=1)[:, :T + 16].astype(np.float32) / 8
    cache = [None, None, None]
    ref.prune_decode_cached(grid(rng, (Hq, d)), K, T, p, (16, 8, 4), 0, cache)
    stage2 = cache[1].kept.copy()
    mid_end = cache[0].mid_end
    # stage 2's record equals a fresh two-stage pruning of the step-0 context
    assert mid_end == ref.geometry(T - 1, T, p).mid_hi
    for st in (1, 2, 3, 4):
        q = grid(rng, (Hq, d))
        e = T + st
        got = ref.prune_decode_cached(q, K, e, p, (16, 8, 4), st, cache)
        assert np.array_equal(cache[1].kept, stage2)
        tail = np.arange(mid_end, e)
        if st < 4:                               # nothing due: the row only grows
            continue
        ch = stage2.reshape(-1, 8)[:, 0]
        Kf = K.astype(np.float64)
        G = Hq // Hkv
        sc = np.max([Kf[h // G, ch] @ q[h].astype(np.float64) for h in range(Hq)], axis=0)
        order = np.lexsort((np.arange(len(ch)), -sc))[:128 // 8]
        kept = np.sort(ch[order])
        want = np.concatenate([np.arange(16), (kept[:, None] + np.arange(8)).reshape(-1), tail])
        assert np.array_equal(got, want)


def test_cached_row_keeps_keys_that_left_the_window():
    rng = np.random.default_rng(9)
    Hq, Hkv, d = 4, 2, 16
    p = ref.Params(1, (32, 8), (256, 64), 16, 64)
    T = 2000
    K = grid(rng, (Hkv, T + 100, d))
    cache = [None, None]
    refresh = (48, 8)
    for st in range(100):
        e = T + st
        row = ref.prune_decode_cached(grid(rng, (Hq, d)), K, e, p, refresh, st, cache)
        mid_end = cache[0].mid_end
        assert np.all(np.diff(row) > 0) and row[-1] == e - 1
        assert set(range(16)) <= set(row.tolist())
        assert set(range(mid_end, e)) <= set(row.tolist())       # nothing was dropped
        assert set(range(e - 64, e)) <= set(row.tolist())        # the window is always there
        assert len(row) == 16 + 64 + (e - mid_end)
        growth = e - (T + (st // 48) * 48)
        assert len(row) <= ref.cached_row_bound(p, growth)


def test_cached_decode_rejects_missing_records():
    rng = np.random.default_rng(10)
    K = grid(rng, (2, 1200, 16))
    p = ref.Params(1, (32, 8), (256, 64), 16, 64)
    with pytest.raises(ValueError):
        ref.prune_decode_cached(grid(rng, (4, 16)), K, 1100, p, (16, 4), 3, [None, None])


# --------------------------------------------------------------------------- #
# f2: block-sparse estimation (MInference page, "Online Dynamic Index         #
# Estimation: Block-Sparse Heads (Algorithm 3)")                              #
# --------------------------------------------------------------------------- #
def _int_grid(rng, shape):
    return rng.integers(-8, 9, size=shape)


def test_block_sparse_pool_is_integer_block_mean():
    rng = np.random.default_rng(40)
    X = _int_grid(rng, (3, 64 * 7, 16))
    P = ref.bs_pool(X.astype(np.float32) / 8, 64)
    assert P.shape == (3, 7, 16)
    csum = np.concatenate([np.zeros((3, 1, 16), np.int64), np.cumsum(X, axis=1)], axis=1)
    sums = csum[:, 64::64] - csum[:, 0:-1:64]                  # integer block sums
    assert np.array_equal(P * 512, sums.astype(np.float64))   # mean of k/8 over 64 = sum/512
    const = np.broadcast_to(np.arange(5, dtype=np.float32)[None, :, None, None], (2, 5, 64, 4))
    assert np.array_equal(ref.bs_pool(const.reshape(2, 320, 4), 64)[0, :, 0], np.arange(5.0))


def test_block_sparse_scores_are_exact_block_causal_logits():
    rng = np.random.default_rng(41)
    Hq, Hkv, nb, d = 4, 2, 9, 32
    Qi, Ki = _int_grid(rng, (Hq, 64 * nb, d)), _int_grid(rng, (Hkv, 64 * nb, d))
    Qp = ref.bs_pool(Qi.astype(np.float32) / 8, 64)
    Kp = ref.bs_pool(Ki.astype(np.float32) / 8, 64)
    for h in range(Hq):
        for m in range(nb):
            sc = ref.bs_block_scores(Qp, Kp, h, m)
            assert sc.dtype == np.float32 and len(sc) == m + 1      # no key block after m
            qs = [int(v) for v in Qi[h, 64 * m:64 * m + 64].sum(axis=0)]
            for j in range(m + 1):
                ks = [int(v) for v in Ki[h // 2, 64 * j:64 * j + 64].sum(axis=0)]
                exact = sum(a * b for a, b in zip(qs, ks))           # integer numerator over 2^18
                assert sc[j] == np.float32(exact / 2.0 ** 18)


def test_block_sparse_select_is_argtopk_of_block_softmax():
    """Ranking pooled logits equals ranking the masked block softmax of step 2
    (scale 1/sqrt(d), future blocks at -inf), checked against a full sort."""
    rng = np.random.default_rng(42)
    nb, d, kb = 40, 16, 7
    Qp = rng.normal(size=(1, nb, d))
    Kp = rng.normal(size=(1, nb, d))
    for m in range(nb):
        sc = ref.bs_block_scores(Qp, Kp, 0, m)
        sel = ref.bs_select(sc, kb)
        logits = np.full(nb, -np.inf)
        logits[:m + 1] = (Kp[0, :m + 1] @ Qp[0, m]) / math.sqrt(d)
        A = np.exp(logits - logits.max())
        A /= A.sum()
        want = sorted(range(nb), key=lambda j: (-A[j], j))[:min(kb, m + 1)]
        assert list(sel) == sorted(want)
        assert A[sel].min() >= np.sort(A)[::-1][min(kb, m + 1) - 1]


def test_block_sparse_select_ties_go_to_lower_blocks():
    sc = np.array([1, 3, 3, 2, 3, 3], dtype=np.float32)
    assert list(ref.bs_select(sc, 3)) == [1, 2, 4]
    assert list(ref.bs_select(sc, 10)) == list(range(6))
    brute = sorted(range(6), key=lambda j: (-sc[j], j))[:4]
    assert list(ref.bs_select(sc, 4)) == sorted(brute)


def test_block_sparse_rows_structure():
    rng = np.random.default_rng(43)
    Q = grid(rng, (2, 64 * 12, 8))
    K = grid(rng, (1, 64 * 12, 8))
    kb = 5
    rows = ref.bs_rows(Q, K, 64, kb)
    assert len(rows) == 2 and all(len(r) == 12 for r in rows)
    for h in range(2):
        for m, row in enumerate(rows[h]):
            assert len(row) == 64 * min(m + 1, kb)
            assert np.all(np.diff(row) > 0) and row.max() < 64 * (m + 1)
            blocks = row.reshape(-1, 64)
            assert np.array_equal(blocks, blocks[:, :1] + np.arange(64))   # whole 64-runs
            assert np.all(blocks[:, 0] % 64 == 0)
    assert ref.bs_index_width(64, 100) == 6400 and ref.bs_index_width(16, 5) == 128


def test_block_sparse_full_budget_is_dense_causal_attention():
    """k_b >= number of blocks keeps every causal block, so block-sparse
    attention of every head is dense causal attention (library softmax)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(44)
    Hq, Hkv, nb, d = 4, 2, 4, 16
    T = 64 * nb
    Q, K = grid(rng, (Hq, T, d)), grid(rng, (Hkv, T, d))
    V = rng.normal(size=(Hkv, T, d)).astype(np.float32)
    rows = ref.bs_rows(Q, K, 64, nb)
    scale = ref.default_scale(d)
    out = np.zeros((Hq, T, d), np.float32)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        for m in range(nb):
            out[h:h + 1, 64 * m:64 * m + 64] = ref.attend_block(
                Q[h:h + 1, 64 * m:64 * m + 64], K[g:g + 1], V[g:g + 1], rows[h][m], 64 * m, scale)
    Kx = torch.from_numpy(np.repeat(K, 2, axis=0)).double()
    Vx = torch.from_numpy(np.repeat(V, 2, axis=0)).double()
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q).double(), Kx, Vx, is_causal=True, scale=scale).numpy()
    assert np.abs(out - want).max() < 1e-5


def test_block_sparse_planted_block_is_found():
    """A key block built to align with one query block's mean direction wins
    that row (and every later row whose query block shares the direction)."""
    rng = np.random.default_rng(45)
    nb, d = 24, 32
    Q = grid(rng, (1, 64 * nb, d)) * np.float32(0.25)
    K = grid(rng, (1, 64 * nb, d)) * np.float32(0.25)
    u = np.sign(rng.normal(size=d)).astype(np.float32)
    Q[0, 64 * 17:64 * 18] += u
    K[0, 64 * 3:64 * 4] += u
    rows = ref.bs_rows(Q, K, 64, 2)
    assert 64 * 3 in rows[0][17][::64]
    assert ref.bs_block_scores(ref.bs_pool(Q, 64), ref.bs_pool(K, 64), 0, 17).argmax() == 3


def test_block_sparse_equation_3_speedup():
    """The page's Equation 3: the pairs the rows admit under the causal mask,
    against dense causal attention, approach S / (2 B k_b) for S >> B k_b;
    the page's 1M-token figures follow from the same geometry."""
    g = _load("p3_block_sparse.json")
    B, kb = g["block"], g["k_blocks"]
    S = g["S_1m"]
    assert abs(S / B - g["blocks_per_row_1m_approx"]) < 1
    assert abs((S / B) ** 2 * g["d_h"] / g["pooled_matmul_flops_per_head_1m_approx"] - 1) < 0.02
    assert abs(S / (2 * B * kb) / g["speedup_eq3_1m_approx"] - 1) < 0.01
    rng = np.random.default_rng(46)
    nb, kb_s = 320, 8
    S_s = 64 * nb
    Q, K = grid(rng, (1, S_s, 4)), grid(rng, (1, S_s, 4))
    rows = ref.bs_rows(Q, K, 64, kb_s)
    pairs = 0
    for m, row in enumerate(rows[0]):
        t = 64 * m + np.arange(64)
        pairs += int((row[None, :] <= t[:, None]).sum())
    dense = S_s * (S_s + 1) // 2
    assert abs((dense / pairs) / (S_s / (2 * 64 * kb_s)) - 1) < 0.03


# --------------------------------------------------------------------------- #
# f3: vertical-slash estimation and index building (MInference page,         #
# "Online Dynamic Index Estimation: Vertical-Slash Heads (Algorithm 2)",      #
# "Vertical-Slash Hybrid Kernel (Appendix C.4.2)")                            #
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("T", [40, 64, 300])
def test_vs_sums_are_attention_mass(T):
    """Every estimation query's causal softmax sums to one and each (query,
    key) pair lies on exactly one column and one offset: both sums total the
    number of estimation queries."""
    rng = np.random.default_rng(T)
    Q, K = grid(rng, (2, T, 16)), grid(rng, (1, T, 16))
    for h in range(2):
        sv, ss = ref.vs_sums(Q, K, h)
        nq = min(64, T)
        assert abs(sv.sum() - nq) < 1e-10 and abs(ss.sum() - nq) < 1e-10
        assert sv.min() >= 0 and ss.min() >= 0 and len(sv) == len(ss) == T


def test_vs_constant_keys_closed_form():
    """Identical keys make every causal row uniform: query t gives 1/(t+1) to
    each key <= t, so column j and offset d both collect sum over the
    estimation queries t >= j (t >= d) of 1/(t+1)."""
    T = 200
    rng = np.random.default_rng(3)
    Q = grid(rng, (1, T, 8))
    K = np.broadcast_to(grid(rng, (1, 1, 8)), (1, T, 8)).copy()
    sv, ss = ref.vs_sums(Q, K, 0)
    t = np.arange(T - 64, T)
    want = np.array([sum(1.0 / (x + 1) for x in t if x >= j) for j in range(T)])
    assert np.abs(sv - want).max() < 1e-12 and np.abs(ss - want).max() < 1e-12


def test_vs_planted_column_and_offset_are_found():
    """A key aligned with every estimation query is the top column; keys that
    each align with one estimation query at the same distance behind it make
    that distance the top offset."""
    rng = np.random.default_rng(5)
    T, d = 512, 32
    Q = grid(rng, (1, T, d)) * np.float32(0.25)
    K = grid(rng, (1, T, d)) * np.float32(0.25)
    u = np.sign(rng.normal(size=d)).astype(np.float32)
    Kv = K.copy()
    Qv = Q.copy()
    Qv[0, T - 64:] += u                          # every estimation query points along u
    Kv[0, 137] = u                               # a vertical line at key 137
    sv, _ = ref.vs_sums(Qv, Kv, 0)
    assert list(ref.vs_select(sv, 1)) == [137]
    d_star = 300
    for t in range(T - 64, T):                  # a slash line at offset 300
        K[0, t - d_star] = np.sign(Q[0, t]) * np.float32(4)
    _, ss = ref.vs_sums(Q, K, 0)
    assert list(ref.vs_select(ss, 1)) == [d_star]


def test_vs_select_ranks_in_fp32_with_lower_index_ties():
    base = 0.1
    sums = np.array([base, base * (1 + 1e-12), 0.05, base, 0.2])   # 0, 1, 3 tie in fp32
    assert list(ref.vs_select(sums, 2)) == [0, 4]
    assert list(ref.vs_select(sums, 3)) == [0, 1, 4]
    assert list(ref.vs_select(sums, 0)) == []


def test_vs_row_worked_example():
    g = _load("p3_vs_rows_example.json")
    iv, is_ = np.array(g["i_v"]), np.array(g["i_s"])
    for r in g["rows"]:
        want = sorted([64 * b + x for b in r["blocks"] for x in range(64)] + r["columns"])
        assert list(ref.vs_row(iv, is_, r["m"])) == want, r["why"]


def test_vs_row_structure_and_width():
    rng = np.random.default_rng(9)
    T = 64 * 20
    for k_v, k_s in [(7, 3), (30, 11), (0, 5), (12, 0)]:
        iv = np.sort(rng.choice(T, size=k_v, replace=False))
        is_ = np.sort(rng.choice(T, size=k_s, replace=False))
        L = ref.vs_index_width(T, k_v, k_s)
        assert L % 64 == 0 and L <= T
        for m in range(T // 64):
            row = ref.vs_row(iv, is_, m)
            assert len(row) <= L and np.all(np.diff(row) > 0) and (len(row) == 0 or row.max() < 64 * (m + 1))
            cols = [p for p in row if not np.all(np.isin(p - p % 64 + np.arange(64), row))]
            assert set(cols) <= set(iv.tolist())               # everything else is whole blocks
            for v in iv:                                       # every visible vertical is present
                if v < 64 * (m + 1):
                    assert v in set(row.tolist())


def test_vs_lists_worked_example():
    """The hybrid kernel's two lists on the hand-worked example: the blocks
    and the columns of each query block as worked out by hand."""
    g = _load("p3_vs_rows_example.json")
    iv, is_ = np.array(g["i_v"]), np.array(g["i_s"])
    for r in g["rows"]:
        blocks, cols = ref.vs_lists(iv, is_, r["m"])
        assert list(blocks) == r["blocks"], r["why"]
        assert list(cols) == r["columns"], r["why"]


def test_vs_lists_are_the_row():
    """Blocks and columns are disjoint, ascending, causal, and together give
    exactly the positions of vs_row (two independent restatements of the
    index-building step)."""
    rng = np.random.default_rng(21)
    T = 64 * 24
    for k_v, k_s in [(7, 3), (40, 11), (0, 5), (12, 0), (200, 60)]:
        iv = np.sort(rng.choice(T, size=k_v, replace=False))
        is_ = np.sort(rng.choice(T, size=k_s, replace=False))
        for m in range(T // 64):
            blocks, cols = ref.vs_lists(iv, is_, m)
            assert np.all(np.diff(blocks) > 0) and (len(blocks) == 0 or (blocks.min() >= 0 and blocks.max() <= m))
            assert np.all(np.diff(cols) > 0) and (len(cols) == 0 or cols.max() < 64 * (m + 1))
            assert not np.isin(cols // 64, blocks).any()
            assert len(blocks) <= min(m + 1, 2 * k_s) and len(cols) <= k_v
            assert np.array_equal(ref.list_positions(blocks, cols), ref.vs_row(iv, is_, m))
    # offsets on block boundaries: offset 64 covers exactly key block m - 1,
    # offset 192 exactly block m - 3 (one key more would reach the next block)
    for m in range(T // 64):
        blocks, cols = ref.vs_lists(np.array([5, 700]), np.array([64, 192]), m)
        assert list(blocks) == [x for x in (m - 3, m - 1) if x >= 0]
        assert list(cols) == [c for c in (5, 700) if c < 64 * (m + 1) and c // 64 not in blocks]


def test_bs_lists_are_the_rows():
    """The block-sparse block lists expand to the block-sparse index rows."""
    rng = np.random.default_rng(22)
    Hq, Hkv, T, d = 4, 2, 64 * 9, 16
    Q, K = grid(rng, (Hq, T, d)), grid(rng, (Hkv, T, d))
    for kb in (1, 3, 20):
        rows, lists = ref.bs_rows(Q, K, 64, kb), ref.bs_lists(Q, K, 64, kb)
        for h in range(Hq):
            for m in range(T // 64):
                assert len(lists[h][m]) == min(m + 1, kb)
                assert np.array_equal(ref.list_positions(lists[h][m], np.array([], np.int64)), rows[h][m])


def test_vs_every_offset_is_dense_causal_attention():
    """k_s covering every offset keeps every causal block: vertical-slash
    attention is then dense causal attention (library SDPA)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(12)
    Hq, T, d = 2, 192, 16
    Q, K = grid(rng, (Hq, T, d)), grid(rng, (1, T, d))
    V = rng.normal(size=(1, T, d)).astype(np.float32)
    rows = ref.vs_rows(Q, K, 3, T)
    scale = ref.default_scale(d)
    out = np.zeros((Hq, T, d), np.float32)
    for h in range(Hq):
        for m in range(T // 64):
            out[h:h + 1, 64 * m:64 * m + 64] = ref.attend_block(Q[h:h + 1, 64 * m:64 * m + 64], K, V,
                                                                rows[h][m], 64 * m, scale)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q).double(), torch.from_numpy(np.repeat(K, Hq, 0)).double(),
        torch.from_numpy(np.repeat(V, Hq, 0)).double(), is_causal=True, scale=scale).numpy()
    assert np.abs(out - want).max() < 1e-5


def test_vs_diagonal_plus_columns_matches_masked_sdpa():
    """Offset 0 alone keeps each query block's own block; with vertical columns
    the attended set of query t is {j <= t: j in t's block or j a column},
    checked against library SDPA with that boolean mask."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(13)
    T, d = 256, 16
    Q, K = grid(rng, (1, T, d)), grid(rng, (1, T, d))
    V = rng.normal(size=(1, T, d)).astype(np.float32)
    iv = np.array([3, 70, 71, 200])
    scale = ref.default_scale(d)
    out = np.zeros((1, T, d), np.float32)
    for m in range(T // 64):
        row = ref.vs_row(iv, np.array([0]), m)
        out[:, 64 * m:64 * m + 64] = ref.attend_block(Q[:, 64 * m:64 * m + 64], K, V, row, 64 * m, scale)
    t, j = np.arange(T)[:, None], np.arange(T)[None, :]
    mask = (j <= t) & ((j // 64 == t // 64) | np.isin(j, iv))
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q).double(), torch.from_numpy(K).double(), torch.from_numpy(V).double(),
        attn_mask=torch.from_numpy(mask), scale=scale).numpy()
    assert np.abs(out - want).max() < 1e-5


def test_vs_page_numbers():
    g = _load("p3_vertical_slash.json")
    assert ref.VS_LAST_Q == g["last_q"] and ref.VS_BLOCK == 64
    assert abs(g["last_q"] * g["S_1m"] * g["d_h"] / g["estimation_multiply_adds_1m_approx"] - 1) < 0.01
    k_v, k_s = g["search_space_vs"][0]
    assert k_v + k_s == g["example_lines"]
    assert g["S_1m"] // 64 == g["blocks_per_row_1m"]
    assert abs((k_v + k_s) / g["blocks_per_row_1m"] - g["example_fraction_approx"]) < 0.001


# --------------------------------------------------------------------------- #
# f4: relative RoPE in SelectRep (InfiniteHiP page, "Four RoPE Styles for     #
# Context Pruning", Relative; "Layer-Specific Strategy Assignment")           #
# --------------------------------------------------------------------------- #
def _rope_complex(x, pos, base):
    """Independent form: pairs (x_i, x_{i+d/2}) as complex numbers times
    exp(i pos theta_i)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    z = x[..., :half] + 1j * x[..., half:]
    theta = np.array([base ** (-2.0 * i / d) for i in range(half)])
    w = z * np.exp(1j * pos * theta)
    return np.concatenate([w.real, w.imag], axis=-1)


def test_rope_rotation_matches_complex_form_and_is_relative():
    rng = np.random.default_rng(30)
    base = 10000.0
    q, k = rng.normal(size=(5, 32)), rng.normal(size=(7, 32))
    for pos in (0, 1, 17, 1025):
        assert np.abs(ref.rope_rotate(q, pos, base) - _rope_complex(q, pos, base)).max() < 1e-12
    assert np.array_equal(ref.rope_rotate(q, 0, base), q)
    assert np.abs(np.linalg.norm(ref.rope_rotate(q, 77, base), axis=1) - np.linalg.norm(q, axis=1)).max() < 1e-12
    lhs = ref.rope_rotate(q, 1025, base) @ ref.rope_rotate(k, 3, base).T     # absolute positions
    rhs = ref.rope_rotate(q, 1022, base) @ k.T                               # their difference only
    assert np.abs(lhs - rhs).max() < 1e-9


def test_rt_queries_use_the_page_offsets_and_stay_exact():
    g = _load("p1_rope_rt.json")
    rng = np.random.default_rng(31)
    q = grid(rng, (64, 128))
    n_stream, base = 1024, 500000.0
    ql, qr = ref.rt_queries(q, n_stream, base)
    off_l = n_stream + g["query_position_minus_n_stream"] - g["left_branch_key_position"]
    off_r = n_stream + g["query_position_minus_n_stream"] - g["right_branch_key_position"]
    assert np.array_equal(ql, np.rint(_rope_complex(q, off_l, base) * 128) / 128)
    assert np.array_equal(qr, np.rint(_rope_complex(q, off_r, base) * 128) / 128)
    for x in (ql, qr):
        n = x.astype(np.float64) * 128
        assert np.array_equal(n, np.rint(n)) and np.abs(n).max() < 256      # bf16-exact
    K = rng.integers(-8, 9, size=(300, 128))
    exact = (np.rint(ql.astype(np.float64) * 128).astype(np.int64) @ K.T).max(axis=0) / 1024.0
    assert np.array_equal(ref.rep_score(ql, K.astype(np.float32) / 8).astype(np.float64), exact)


def test_rt_tournament_with_one_query_set_is_selectrep():
    rng = np.random.default_rng(32)
    q = grid(rng, (4, 16))
    K = grid(rng, (1, 256, 16))
    P2 = np.arange(256).reshape(8, 32)
    reps, win = ref.select_rep_rt_all(q, q, K, 0, P2)
    assert np.array_equal(reps, ref.select_rep_all(q, K, 0, P2))
    assert np.array_equal(win, ref.rep_score(q, K[0, reps]))


def test_rt_tournament_hand_example():
    """Two-dimensional keys with the left queries reading coordinate 0 and the
    right queries coordinate 1: the right half wins twice and the chunk scores
    its last right win; when the final split goes left the chunk keeps the
    representative's left score."""
    ql, qr = np.array([[1.0, 0.0]], np.float32), np.array([[0.0, 1.0]], np.float32)
    K = np.array([[[1, 0], [5, 5], [0, 2], [0, 3], [1, 0], [5, 5], [0, 2], [0, -1]]], np.float32)
    reps, win = ref.select_rep_rt_all(ql, qr, K, 0, np.arange(8).reshape(2, 4))
    assert list(reps) == [3, 6] and list(win) == [3.0, 0.0]
    plain = ref.select_rep_all(ql, K, 0, np.arange(8).reshape(2, 4))      # without RoPE: key 1
    assert list(plain) == [1, 5]


# --------------------------------------------------------------------------- #
# f4: chunk-indexed RoPE in SelectRep (InfiniteHiP page, "Four RoPE Styles for #
# Context Pruning", Chunk-indexed; "Layer-Specific Strategy Assignment")       #
# --------------------------------------------------------------------------- #
def test_rope_rows_match_complex_form():
    rng = np.random.default_rng(40)
    x = rng.normal(size=(6, 16))
    pos = np.array([0, 1, 5, 99, 1000, 123457])
    got = ref.rope_rotate_rows(x, pos, 10000.0)
    for i in range(6):
        assert np.abs(got[i] - _rope_complex(x[i], pos[i], 10000.0)).max() < 1e-9
    assert np.array_equal(ref.rope_round(np.array([0.3, -1.0 / 256 - 1e-9, 1.999])) * 128, [38.0, -1.0, 256.0])


def test_ci_positions_follow_the_page():
    g = _load("p1_rope_ci.json")
    p = ref.Params(1, (64, 8), (1024, 256), 16, 1024)
    e = 100_000
    geo = ref.geometry(e - 1, e, p)
    for l in p.chunk:
        pos = np.arange(geo.mid_lo, geo.mid_hi)
        c = ref.ci_chunk_index(pos, p.n_sink, l)
        assert g["keys_in_one_chunk_share_id"] and np.all(c.reshape(-1, l) == c[::l][:, None])
        assert np.all(np.diff(c[::l]) == g["consecutive_chunks_id_step"]) and c[0] == 0
        qpos = ref.ci_query_positions(np.array([e - 1]), geo.mid_hi, p.n_sink, p.n_window, l)
        assert g["query_id_minus_last_chunk_id"] == "n_stream" and qpos[0] - c[-1] == p.n_window
    # the cap: single-key chunks and no sinks put the last chunk's ID past
    # the first queries of a block
    p1 = ref.Params(64, (1,), (8,), 0, 64)
    geo = ref.geometry(128, 192, p1)
    qpos = ref.ci_query_positions(np.arange(128, 192), geo.mid_hi, 0, 64, 1)
    assert g["query_id_cap"] == "i_orig"
    assert np.array_equal(qpos, np.minimum(np.arange(128, 192), geo.mid_hi - 1 + 64)) and qpos[0] == 128


def test_ci_rotated_scores_are_exact():
    rng = np.random.default_rng(41)
    Q = grid(rng, (64, 128))
    K = grid(rng, (1, 512, 128))
    qr = ref.rope_round(ref.rope_rotate_rows(Q, np.full(64, 4321), 500000.0))
    kr = ref.CiKeys(K, 0, 8, 500000.0)[0, np.arange(512)]
    for x in (qr, kr):
        n = x.astype(np.float64) * 128
        assert np.array_equal(n, np.rint(n)) and np.abs(n).max() < 256            # bf16-exact
    exact = (np.rint(qr.astype(np.float64) * 128).astype(np.int64)
             @ np.rint(kr.astype(np.float64) * 128).astype(np.int64).T).max(axis=0) / 16384.0
    assert np.array_equal(ref.rep_score(qr, kr).astype(np.float64), exact)


def test_ci_with_trivial_rotation_is_plain_pruning():
    """Pair 0 (the only frequency that turns at any base) zero in Q and K and
    a base so large that every other angle rounds away: chunk-indexed pruning
    equals the plain pruning, in both modes and over three stages."""
    rng = np.random.default_rng(42)
    d = 32
    K = grid(rng, (2, 4096, d))
    K[:, :, 0] = K[:, :, d // 2] = 0
    p = ref.Params(64, (64, 8, 1), (1024, 256, 64), 16, 128)
    for s, e in ((4032, 4096), (4095, 4096), (1984, 2048)):
        Q = grid(rng, (4, e - s, d))
        Q[:, :, 0] = Q[:, :, d // 2] = 0
        assert np.array_equal(ref.prune_block_ci(Q, K, s, e, p, 1e300), ref.prune_block(Q, K, s, e, p))


def test_ci_hand_example_two_stages():
    """d = 2 (one pair, angle = position): identical keys (1, 0) and query
    (1, 0), so each chunk's score is the rounded cos(query ID - chunk ID); the
    plain pruning ties everywhere and keeps the first chunks."""
    n_sink, n_stream = 4, 8
    p = ref.Params(1, (8, 4), (32, 8), n_sink, n_stream)
    e = 4 + 10 * 8 + 8
    K = np.tile(np.array([1.0, 0.0], np.float32), (1, e, 1))
    Q = np.array([[[1.0, 0.0]]], np.float32)

    def rnd(v):
        return round(v * 128) / 128

    def score(qid, cid):
        return rnd(math.cos(qid)) * rnd(math.cos(cid)) + rnd(math.sin(qid)) * rnd(math.sin(cid))

    # stage 1: ten chunks of 8 (IDs 0..9), query ID 9 + n_stream; keep 4
    s1 = [score(9 + n_stream, c) for c in range(10)]
    keep1 = sorted(sorted(range(10), key=lambda c: (-s1[c], c))[:4])
    # stage 2: chunks of 4 of the kept ones (IDs (pos - n_sink) / 4), query ID 19 + n_stream; keep 2
    c2 = [2 * c + h for c in keep1 for h in (0, 1)]
    s2 = {c: score(19 + n_stream, c) for c in c2}
    keep2 = sorted(sorted(c2, key=lambda c: (-s2[c], c))[:2])
    want = list(range(n_sink)) + [n_sink + 4 * c + i for c in keep2 for i in range(4)] + list(range(84, e))
    got = ref.prune_block_ci(Q, K, e - 1, e, p, 10000.0)
    assert keep1 == [3, 4, 5, 6] and keep2 == [8, 9]
    assert list(got) == want
    plain = ref.prune_block(Q, K, e - 1, e, p)
    assert list(plain[n_sink:n_sink + 8]) == list(range(n_sink, n_sink + 8))


def test_streamed_active_count_follows_closed_form():
    """The InfLLM page's test idea (stream 10,000 tokens, watch the number of
    active keys), for this method: a decode row holds the sinks, min(M, k_N)
    middle keys (M = the whole stage-1 chunks of the middle; the stages keep
    k_1 >= ... >= k_N), the window, and the chunk-grid tail (the part of the
    middle that does not fill a stage-1 chunk), which cycles through [0, l_1)
    as tokens arrive; once M exceeds k_N the count is that constant plus the
    tail."""
    rng = np.random.default_rng(50)
    d, T0, n = 8, 64, 10_000
    p = ref.Params(1, (8, 2), (64, 16), 4, 32)
    K = grid(rng, (1, T0 + n, d))
    seen = set()
    for e in range(T0 + 1, T0 + n + 1):
        q = grid(rng, (1, 1, d))
        row = ref.prune_block(q, K, e - 1, e, p)
        rem = (e - p.n_window - p.n_sink) % p.chunk[0]
        M = (e - p.n_window - p.n_sink) // p.chunk[0] * p.chunk[0]
        assert len(row) == p.n_sink + min(M, p.keep[-1]) + p.n_window + rem, e
        if M > p.keep[-1]:
            seen.add(rem)
    assert seen == set(range(p.chunk[0]))
