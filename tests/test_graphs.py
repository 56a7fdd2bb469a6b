"""HIP graph capture of the decode step (pruning + attention), as bench.py
times it: each replay, run after new inputs are written into the captured
buffers and after eager calls of its own, must equal the eager result bit for
bit (the library allocates and clears nothing inside the calls)."""
import pytest
import torch

import helpers as H
from dynamic_sparse_attention_query_amd import api, gen
from dynamic_sparse_attention_query_amd.inputs import params_of, to_device

pytestmark = pytest.mark.gpu

BASE = 500000.0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from dynamic_sparse_attention_query_amd import _lib
    _lib.load()


@pytest.mark.parametrize("style", ["plain", "relative", "chunk_indexed"])
def test_decode_step_graph_replays_match_eager(style):
    case = gen.make_case("c3", t=65536, n_queries=4)
    H.say(f"graph replays of the decode step ({style})")
    dev = to_device(case)
    p = params_of(case.cfg)
    kw = dict(seq_lens=dev.seq_lens, block_table=dev.block_table, t=dev.t)
    q_buf = dev.q[0].contiguous().clone()

    def prune(out=None):
        if style == "plain":
            return api.prune_select(q_buf, dev.k, p, out=out, **kw)
        return api.prune_select_rope(q_buf, dev.k, p, BASE, out=out, style=style, **kw)

    idx = prune()
    out = api.sparse_attn(q_buf, dev.k, dev.v, idx, p, **kw)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        prune(out=idx.view(-1))
        api.sparse_attn(q_buf, dev.k, dev.v, idx, p, out=out, **kw)
    for qi in (1, 2, 3, 1):
        q_buf.copy_(dev.q[qi])
        idx_e = prune()
        out_e = api.sparse_attn(q_buf, dev.k, dev.v, idx_e, p, **kw)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, idx_e), f"query {qi}: index rows differ"
        assert torch.equal(out, out_e), f"query {qi}: outputs differ"


def test_cached_decode_graph_replays_match_eager():
    """Decoding with remembered stages (refresh 16, 8, 4) as bench.py times it:
    one captured graph per step of a refresh cycle, each with its own context
    length, replayed in order on a second cache with plain eager calls in
    between; every step's rows and outputs equal the eager stream's."""
    n, T = 16, 65536
    case = gen.make_case("c3", t=T, n_queries=n)
    H.say("graph replays of the remembered-stage decode cycle")
    dev = to_device(case)
    p = params_of(case.cfg)
    q_buf = dev.q[0].contiguous().clone()
    sls = [torch.full((1,), T - n + 1 + i, dtype=torch.int32, device="cuda") for i in range(n)]

    def make_cache():
        return api.MaskCache(q_buf, dev.k, p, (16, 8, 4), seq_lens=sls[-1], t=T)

    def step(cache, i, idx, out):
        api.prune_select_cached(q_buf, dev.k, cache, i, seq_lens=sls[i], t=T, out=idx.view(-1))
        api.sparse_attn(q_buf, dev.k, dev.v, idx, p, seq_lens=sls[i], t=T, out=out)

    eager = make_cache()
    want = []
    for i in range(n):
        q_buf.copy_(dev.q[i])
        idx = torch.empty(1, eager.width, dtype=torch.int32, device="cuda")
        out = torch.empty(q_buf.shape, dtype=torch.float32, device="cuda")
        step(eager, i, idx, out)
        want.append((idx, out))
    torch.cuda.synchronize()

    cached = make_cache()
    idx_g = torch.empty(1, cached.width, dtype=torch.int32, device="cuda")
    out_g = torch.empty(q_buf.shape, dtype=torch.float32, device="cuda")
    graphs = []
    for i in range(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(cached, i, idx_g, out_g)
        graphs.append(g)
    torch.cuda.synchronize()
    for i in range(n):
        q_buf.copy_(dev.q[i])
        graphs[i].replay()
        torch.cuda.synchronize()
        assert torch.equal(idx_g, want[i][0]), f"step {i}: index rows differ"
        assert torch.equal(out_g, want[i][1]), f"step {i}: outputs differ"
        api.prune_select(dev.q[(i + 1) % n].contiguous(), dev.k, p, seq_lens=sls[i], t=T)   # eager work between
    assert int(cached.status.item()) == 0
