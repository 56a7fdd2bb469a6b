"""dsa_prune_attend_static (the entry point for callers that cannot allocate)
against dsa_prune_attend with a caller workspace, through the C ABI, on
consecutive calls of decreasing size (the static scratch keeps the previous
call's contents), and under HIP graph capture."""
import ctypes

import pytest
import torch

from dynamic_sparse_attention_query_amd import _lib, api, gen
from dynamic_sparse_attention_query_amd.inputs import params_of, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _decode(t, seed):
    cfg = gen.Config(f"static-{t}", "decode", 1, 32, 8, 128, t, "bf16", 1, (256, 32, 8), (32768, 8192, 4096),
                     64, 1024, seed=seed, n_queries=1)
    return params_of(cfg), to_device(gen.make_case(cfg))


def _call(lib, entry, shape, q, k, v, p, ws=None):
    L = _lib.index_width(p)
    rows = shape.batch * (1 if shape.mode == _lib.DSA_DECODE else shape.t // p.block_q)
    idx = torch.full((rows * L,), -7, dtype=torch.int32, device="cuda")
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    cs, cp = shape.c(), p.c()
    sp = torch.cuda.current_stream().cuda_stream
    if entry == "static":
        st = lib.dsa_prune_attend_static(ctypes.byref(cs), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                         ctypes.byref(cp), 0.0, idx.data_ptr(), out.data_ptr(), None, sp)
    else:
        st = lib.dsa_prune_attend(ctypes.byref(cs), q.data_ptr(), k.data_ptr(), v.data_ptr(), ctypes.byref(cp),
                                  0.0, idx.data_ptr(), out.data_ptr(), ws.data_ptr(), ws.numel(), None, sp)
    assert st == 0, lib.dsa_last_error().decode()
    return idx, out


def test_static_entry_matches_workspace_entry():
    lib = _lib.load()
    cases = [("decode 200K", *_decode(200000, 41)), ("decode 20K", *_decode(20000, 42))]
    pre = gen.make_case("c2", t=4096, keep=(1024, 512, 256), n_window=128, n_needles=1)
    cases.append(("prefill 4K", params_of(pre.cfg), to_device(pre)))
    for name, p, dev in cases:                                  # sizes decrease call after call
        q = dev.q[0].contiguous() if name.startswith("decode") else dev.q
        kw = dict(seq_lens=dev.seq_lens) if name.startswith("decode") else {}
        shape = api.make_shape(q, dev.k, **kw)
        ws = torch.empty(_lib.workspace_bytes(shape, p), dtype=torch.uint8, device="cuda")
        a_idx, a_out = _call(lib, "static", shape, q, dev.k, dev.v, p)
        b_idx, b_out = _call(lib, "ws", shape, q, dev.k, dev.v, p, ws)
        torch.cuda.synchronize()
        assert torch.equal(a_idx, b_idx), f"{name}: index rows differ"
        assert torch.equal(a_out, b_out), f"{name}: outputs differ"


def test_static_entry_under_graph_capture():
    lib = _lib.load()
    p, dev = _decode(60000, 43)
    q = dev.q[0].contiguous()
    shape = api.make_shape(q, dev.k, seq_lens=dev.seq_lens)
    L = _lib.index_width(p)
    idx = torch.empty(L, dtype=torch.int32, device="cuda")
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    cs, cp = shape.c(), p.c()
    want_idx, want_out = _call(lib, "static", shape, q, dev.k, dev.v, p)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = lib.dsa_prune_attend_static(ctypes.byref(cs), q.data_ptr(), dev.k.data_ptr(), dev.v.data_ptr(),
                                         ctypes.byref(cp), 0.0, idx.data_ptr(), out.data_ptr(), None,
                                         torch.cuda.current_stream().cuda_stream)
        assert st == 0
    for rep in range(3):
        idx.fill_(-7)
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, want_idx), f"replay {rep}"
        assert torch.equal(out, want_out), f"replay {rep}"
