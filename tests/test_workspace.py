"""Workspaces of the tensor-level entry points (GPU).

Each (device, stream) has its own workspace; a workspace that grows is
replaced, but the old buffer stays alive, so a HIP graph captured with it
keeps working; callers may also pass their own buffer (ws=).
"""
import pytest
import torch

from dynamic_sparse_attention_query_amd import api, gen
from dynamic_sparse_attention_query_amd.inputs import params_of, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(t, seed):
    cfg = gen.Config(f"ws-{t}", "decode", 1, 32, 8, 128, t, "bf16", 1, (64, 16, 4), (4096, 1024, 256), 32, 256,
                     seed=seed, n_queries=1)
    case = gen.make_case(cfg)
    return params_of(cfg), to_device(case)


def test_graph_replay_survives_workspace_growth():
    p, dev = _case(20000, 31)
    pb, devb = _case(300000, 32)
    s = torch.cuda.Stream()
    q = dev.q[0].contiguous()
    idx = torch.empty(api._lib.index_width(p), dtype=torch.int32, device="cuda")
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    with torch.cuda.stream(s):
        want_idx, want_out = api.prune_attend(q, dev.k, dev.v, p, seq_lens=dev.seq_lens)
    s.synchronize()
    key = (torch.cuda.current_device(), s.cuda_stream)
    small = api._WS[key].data_ptr()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        api.prune_attend(q, dev.k, dev.v, p, seq_lens=dev.seq_lens, idx=idx, out=out)
    s.synchronize()
    # a larger call on the same stream grows its workspace
    with torch.cuda.stream(s):
        api.prune_attend(devb.q[0].contiguous(), devb.k, devb.v, pb, seq_lens=devb.seq_lens)
    s.synchronize()
    assert api._WS[key].data_ptr() != small, "the workspace did not grow"
    assert any(b.data_ptr() == small for b in api._RETIRED), "the captured workspace was released"
    # fresh allocations that would reuse a released buffer, filled with junk
    junk = [torch.full((1 << 20,), 0x7F7F7F7F, dtype=torch.int32, device="cuda") for _ in range(16)]
    for rep in range(3):
        idx.fill_(-7)
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, want_idx.view(-1)), f"replay {rep}: index row changed"
        assert torch.equal(out, want_out), f"replay {rep}: output changed"
    del junk


def test_streams_have_their_own_workspace():
    p, dev = _case(20000, 33)
    q = dev.q[0].contiguous()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(s1):
        api.prune_attend(q, dev.k, dev.v, p, seq_lens=dev.seq_lens)
    with torch.cuda.stream(s2):
        api.prune_attend(q, dev.k, dev.v, p, seq_lens=dev.seq_lens)
    torch.cuda.synchronize()
    d = torch.cuda.current_device()
    assert api._WS[(d, s1.cuda_stream)].data_ptr() != api._WS[(d, s2.cuda_stream)].data_ptr()


def test_caller_workspace():
    p, dev = _case(20000, 34)
    q = dev.q[0].contiguous()
    shape = api.make_shape(q, dev.k, seq_lens=dev.seq_lens)
    need = api.workspace_bytes(shape, p)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    a_idx, a_out = api.prune_attend(q, dev.k, dev.v, p, seq_lens=dev.seq_lens, ws=ws)
    b_idx, b_out = api.prune_attend(q, dev.k, dev.v, p, seq_lens=dev.seq_lens)
    torch.cuda.synchronize()
    assert torch.equal(a_idx, b_idx) and torch.equal(a_out, b_out)
    with pytest.raises(ValueError):
        api.prune_attend(q, dev.k, dev.v, p, seq_lens=dev.seq_lens, ws=ws[: need // 2])
