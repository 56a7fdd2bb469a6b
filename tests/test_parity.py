"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

Index rows must match bit-exactly (dot products are exact on the input grid,
so both sides make the same selections). Attention outputs (fp32) must be
within max-abs 1e-2 and relative-L2 5e-3 of the oracle's fp64 softmax.
"""
import numpy as np
import pytest
import torch

import helpers as H
from dynamic_sparse_attention_query_amd import api, gen
from dynamic_sparse_attention_query_amd.inputs import params_of, to_device
from oracle import ref

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from dynamic_sparse_attention_query_amd import _lib
    _lib.load()


def gpu_prefill(dev, p):
    idx = api.prune_select(dev.q, dev.k, p)
    out = api.sparse_attn(dev.q, dev.k, dev.v, idx, p)
    torch.cuda.synchronize()
    return idx, out


def gpu_decode(dev, p, qi=0, visited=None):
    q = dev.q[qi].contiguous()
    kw = dict(seq_lens=dev.seq_lens, block_table=dev.block_table, t=dev.t)
    idx = api.prune_select(q, dev.k, p, visited=visited, **kw)
    out = api.sparse_attn(q, dev.k, dev.v, idx, p, **kw)
    torch.cuda.synchronize()
    return idx, out


def check_prefill_blocks(case, idx, out, blocks, attn_blocks=None, b=0):
    """Index rows of `blocks` bit for bit, attention of `attn_blocks` (default:
    the same) within tolerance; each oracle row is computed once, and only
    the checked blocks' outputs are copied to the host."""
    idx_np = idx.cpu().numpy()
    cfg = case.cfg
    rows = set(blocks)
    attn = set(attn_blocks if attn_blocks is not None else blocks)
    for m in sorted(rows | attn):
        want = H.oracle_row(case, b, m)
        if m in rows:
            got = idx_np[b, m]
            assert np.array_equal(got, want), f"block {m}: first diff at {np.flatnonzero(got != want)[:5]}"
        if m in attn:
            s, e = m * cfg.block_q, (m + 1) * cfg.block_q
            got_out = out[b, :, s:e].cpu().numpy()
            H.assert_close(got_out, H.oracle_attend(case, b, m, want), f"block {m} attention")


# --------------------------------------------------------------------------- #
# prefill                                                                     #
# --------------------------------------------------------------------------- #
def test_c1_tiny_prefill_full():
    case = gen.make_case("c1")
    H.say("c1: full index array + every block's attention")
    dev = to_device(case)
    p = params_of(case.cfg)
    idx, out = gpu_prefill(dev, p)
    nblk = case.cfg.t // case.cfg.block_q
    check_prefill_blocks(case, idx, out, range(nblk))
    dense = api.dense_attn(dev.q, dev.k, dev.v).cpu().numpy()
    for m in range(0, nblk, 9):
        s, e = m * 32, m * 32 + 32
        H.assert_close(dense[0, :, s:e], H.oracle_dense(case, 0, m), f"dense block {m}")
    # planted chunks are found
    idx_np = idx.cpu().numpy()
    found = sum(all(x in set(idx_np[0, m].tolist()) for x in range(st, st + 16))
                for (b, m), starts in case.planted.items() for st in starts)
    total = sum(len(v) for v in case.planted.values())
    H.say(f"c1 planted-chunk recall {found}/{total}")


def small_three_stage():
    return gen.make_case("c2", t=4096, keep=(1024, 512, 256), n_window=256, n_needles=2)


def test_prefill_three_stages_full_array():
    case = small_three_stage()
    H.say("c2-shape at T=4096, keeps 1024/512/256: full index array + attention")
    dev = to_device(case)
    p = params_of(case.cfg)
    idx, out = gpu_prefill(dev, p)
    nblk = case.cfg.t // case.cfg.block_q
    check_prefill_blocks(case, idx, out, range(nblk), attn_blocks=range(0, nblk, 5))
    # determinism
    idx2, out2 = gpu_prefill(dev, p)
    assert torch.equal(idx, idx2)
    assert torch.equal(out, out2)


@pytest.mark.parametrize("hq,hkv,d,batch", [(8, 4, 64, 2), (4, 4, 128, 1), (16, 2, 128, 1)])
def test_prefill_bf16_group_shapes(hq, hkv, d, batch):
    """bf16 prefill on the matrix-core kernels for the other GQA group sizes
    (2, 1, 8), head size 64 and a batch of two sequences."""
    case = gen.make_case("c2", t=2048, hq=hq, hkv=hkv, d=d, batch=batch, keep=(512, 256, 128),
                         n_window=128, n_needles=2)
    H.say(f"bf16 prefill Hq={hq} Hkv={hkv} d={d} B={batch}")
    dev = to_device(case)
    p = params_of(case.cfg)
    idx, out = gpu_prefill(dev, p)
    nblk = case.cfg.t // case.cfg.block_q
    for b in range(batch):
        check_prefill_blocks(case, idx, out, range(nblk), attn_blocks=range(b, nblk, 7), b=b)


def test_prefill_dense_matches_oracle():
    case = gen.make_case("c2", t=2048, n_needles=0)
    dev = to_device(case)
    dense = api.dense_attn(dev.q, dev.k, dev.v).cpu().numpy()
    for m in (0, 7, 19, 31):
        s, e = m * 64, m * 64 + 64
        H.assert_close(dense[0, :, s:e], H.oracle_dense(case, 0, m), f"dense block {m}")


def test_full_budget_prefill_is_dense():
    case = gen.make_case("c2", t=2048, keep=(2048, 2048, 2048), n_needles=0)
    dev = to_device(case)
    p = params_of(case.cfg)
    idx, out = gpu_prefill(dev, p)
    idx_np = idx.cpu().numpy()
    for m in range(32):
        e = 64 * (m + 1)
        assert np.array_equal(idx_np[0, m, :e], np.arange(e))
        assert np.all(idx_np[0, m, e:] == -1)
    dense = api.dense_attn(dev.q, dev.k, dev.v)
    torch.cuda.synchronize()
    H.assert_close(out.cpu().numpy(), dense.cpu().numpy(), "sparse(full budget) vs dense")


def test_c2_prefill_32k_sampled():
    case = gen.make_case("c2")
    cfg = case.cfg
    H.say("c2: 32K prefill, sampled blocks")
    dev = to_device(case)
    p = params_of(cfg)
    idx, out = gpu_prefill(dev, p)
    nblk = cfg.t // cfg.block_q
    blocks = gen.sample_blocks(nblk, 64, cfg.seed)
    last8 = list(range(nblk - 8, nblk))                   # the widest rows
    blocks = sorted(set(blocks) | set(last8))
    # index rows and attention on every sampled block and the last eight
    check_prefill_blocks(case, idx, out, blocks, attn_blocks=blocks)
    idx_np = idx.cpu().numpy()
    for nd in case.needles:
        row = set(idx_np[nd.b, nd.query // cfg.block_q].tolist())
        assert set(range(nd.slot_start, nd.slot_start + nd.length)) <= row


def test_c2_prefill_128k_sampled():
    """The 128K prefill the bench times (same shape, inputs and launches):
    index rows and attention on about 35 sampled query blocks, among them the
    first rows whose stage 1 prunes and the widest (last) rows."""
    case = gen.make_case("c2_128k")
    cfg = case.cfg
    H.say("c2: 128K prefill, sampled blocks")
    dev = to_device(case)
    p = params_of(cfg)
    idx, out = gpu_prefill(dev, p)
    nblk = cfg.t // cfg.block_q
    blocks = sorted(set(gen.sample_blocks(nblk, 32, cfg.seed + 1)) | {300, nblk - 2, nblk - 1})
    check_prefill_blocks(case, idx, out, blocks, attn_blocks=blocks)


# --------------------------------------------------------------------------- #
# decode                                                                      #
# --------------------------------------------------------------------------- #
def check_decode(case, dev, b_list, qi=0, visited=False):
    p = params_of(case.cfg)
    vis = torch.zeros(len(p.chunk), dtype=torch.int64, device="cuda") if visited else None
    idx, out = gpu_decode(dev, p, qi, vis)
    idx_np, out_np = idx.cpu().numpy(), out.cpu().numpy()
    for b in b_list:
        want = H.oracle_row(case, b, 0, qi)
        assert np.array_equal(idx_np[b], want), \
            f"seq {b}: first diff at {np.flatnonzero(idx_np[b] != want)[:5]}"
        H.assert_close(out_np[b], H.oracle_attend(case, b, 0, want, qi)[:, 0], f"seq {b} attention")
    return idx, out, vis


def test_decode_small_edge_lengths():
    # ragged contiguous batch: lengths below the sink, inside sink+window, a
    # chunk-grid tail, and long enough for all three stages to prune
    cfg = gen.Config("decode-edge", "decode", 6, 8, 2, 128, 9000, "bf16", 1,
                     (64, 16, 4), (2048, 512, 128), 16, 64, seed=11, n_queries=2)
    case = gen.make_case(cfg)
    case.seq_lens[:] = [1, 7, 80, 300, 5000, 9000]
    for b, L in enumerate(case.seq_lens):
        case.k[b] = case.k[b].sub((slice(None), slice(0, int(L))))
        case.v[b] = case.v[b].sub((slice(None), slice(0, int(L))))
    dev = to_device(case)
    for qi in range(2):
        check_decode(case, dev, range(6), qi)


def test_decode_streamed_lengths_active_count():
    """The InfLLM page's streaming test idea on the GPU: one decode step for
    each of 250 context lengths 40 + 41 i (i = 0..249, up to 10,249 tokens) in
    one ragged batch; every row holds the sinks, min(M, k_N) middle keys, the
    window and the chunk-grid tail (the closed form pinned on the oracle), and
    sampled rows equal the oracle's."""
    n = 250
    cfg = gen.Config("decode-stream", "decode", n, 4, 1, 64, 40 + 41 * (n - 1), "bf16", 1,
                     (8, 2), (64, 16), 4, 32, seed=13, n_queries=1)
    case = gen.make_case(cfg)
    case.seq_lens[:] = 40 + 41 * np.arange(n)
    for b, L in enumerate(case.seq_lens):
        case.k[b] = case.k[b].sub((slice(None), slice(0, int(L))))
        case.v[b] = case.v[b].sub((slice(None), slice(0, int(L))))
    dev = to_device(case)
    idx, _, _ = check_decode(case, dev, [0, 1, 2, 17, 128, n - 1])
    counts = (idx.cpu().numpy() >= 0).sum(axis=1)
    e = case.seq_lens.astype(np.int64)
    rem = (e - 32 - 4) % 8
    M = (e - 32 - 4) // 8 * 8
    assert np.array_equal(counts, 4 + np.minimum(M, 16) + 32 + rem)
    assert len(set(rem[M > 16].tolist())) == 8                    # the tail takes every value


def test_decode_zero_budget_and_full_budget():
    base = gen.Config("decode-budget", "decode", 2, 8, 2, 64, 3000, "bf16", 1,
                      (32, 8), (0, 0), 8, 64, seed=12, n_queries=1)
    for keep in ((0, 0), (4096, 4096)):
        case = gen.make_case(base.replace(keep=keep))
        dev = to_device(case)
        idx, out, _ = check_decode(case, dev, range(2))
        if keep[0] == 0:
            row = idx.cpu().numpy()[0]
            T = 3000
            mid_hi = 8 + ((T - 64 - 8) // 32) * 32
            assert np.array_equal(row[row >= 0], np.r_[np.arange(8), np.arange(mid_hi, T)])
        else:
            dense = api.dense_attn(dev.q[0].contiguous(), dev.k, dev.v, seq_lens=dev.seq_lens)
            H.assert_close(out.cpu().numpy(), dense.cpu().numpy(), "full budget vs dense")


@pytest.mark.parametrize("hq,hkv,d,page", [(16, 8, 128, 0), (32, 8, 128, 64), (64, 8, 128, 0),
                                           (8, 8, 128, 0), (32, 8, 64, 0)])
def test_dense_decode_ragged_shapes(hq, hkv, d, page):
    """Dense decode over a ragged batch whose longest sequence spans several
    chunks per split (100,000 keys: splits of 256 entries), at 1, 2, 4 and 8
    query heads per kv head, d = 64 and 128, paged and contiguous: sequences
    of one key and of fewer keys than a split leave most splits empty."""
    cfg = gen.Config("decode-dense", "decode", 4, hq, hkv, d, 100000, "bf16", 1,
                     (64,), (0,), 0, 64, seed=21, n_queries=1, page_size=page)
    case = gen.make_case(cfg)
    case.seq_lens[:] = [1, 70, 5000, 100000]
    for b, L in enumerate(case.seq_lens):
        case.k[b] = case.k[b].sub((slice(None), slice(0, int(L))))
        case.v[b] = case.v[b].sub((slice(None), slice(0, int(L))))
    dev = to_device(case)
    q = dev.q[0].contiguous()
    out = api.dense_attn(q, dev.k, dev.v, seq_lens=dev.seq_lens, block_table=dev.block_table,
                         t=dev.t).cpu().numpy()
    for b in range(4):
        H.assert_close(out[b], H.oracle_dense(case, b, 0)[:, 0], f"dense decode seq {b}")


@pytest.mark.parametrize("page", [0, 64])
def test_decode_wide_rows(page):
    """Two-call decode over index rows wider than 65,536 entries (a one-stage
    budget of 80,000 keys in 100,000): the attention takes spans of several
    128-entry chunks per split; contiguous and paged, one sequence shorter
    than the budget (everything kept)."""
    cfg = gen.Config("decode-wide", "decode", 2, 32, 8, 128, 100000, "bf16", 1,
                     (64,), (80000,), 64, 1024, seed=22, n_queries=1, page_size=page)
    case = gen.make_case(cfg)
    case.seq_lens[:] = [100000, 60000]
    for b, L in enumerate(case.seq_lens):
        case.k[b] = case.k[b].sub((slice(None), slice(0, int(L))))
        case.v[b] = case.v[b].sub((slice(None), slice(0, int(L))))
    dev = to_device(case)
    assert _lib_width(case) > 65536
    check_decode(case, dev, range(2))


@pytest.mark.parametrize("hq,hkv,d,page,batch", [(32, 32, 128, 0, 1), (32, 32, 128, 64, 2), (24, 12, 64, 0, 2),
                                                 (64, 64, 128, 0, 1)])
def test_decode_head_slices(hq, hkv, d, page, batch):
    """Decode pruning with more kv heads than the 16 lane groups of a scoring
    workgroup hold (32 and 64: a score list per slice of 16 heads, maxed by
    the readers) or a head count that does not divide 16 (12 heads, one chunk
    per workgroup); one sequence takes the fused top-K kernels, two the
    per-row selection; the one-call step gives the same rows and outputs."""
    cfg = gen.Config("decode-slices", "decode", batch, hq, hkv, d, 24000, "bf16", 1,
                     (64, 16, 4), (2048, 512, 128), 16, 64, seed=31, n_queries=1, page_size=page)
    case = gen.make_case(cfg)
    if batch == 2:
        case.seq_lens[:] = [24000, 15000]
        for b, L in enumerate(case.seq_lens):
            case.k[b] = case.k[b].sub((slice(None), slice(0, int(L))))
            case.v[b] = case.v[b].sub((slice(None), slice(0, int(L))))
    H.say(f"decode head slices {hq}/{hkv} d={d} page={page} batch={batch}")
    dev = to_device(case)
    idx, out, _ = check_decode(case, dev, range(batch))
    q = dev.q[0].contiguous()
    idx1, out1 = api.prune_attend(q, dev.k, dev.v, params_of(cfg), seq_lens=dev.seq_lens,
                                  block_table=dev.block_table, t=dev.t)
    torch.cuda.synchronize()
    assert np.array_equal(idx1.cpu().numpy().reshape(idx.shape), idx.cpu().numpy())
    H.assert_close(out1.cpu().numpy(), out.cpu().numpy(), "one-call step vs two calls")


@pytest.mark.parametrize("page", [4, 8, 16, 256])
def test_decode_page_sizes(page):
    """Paged decode across page sizes: 64-key stage-1 chunks over sixteen,
    eight or four pages (row reads through the page table, or page ids held
    in registers), later chunks resolved from the pages the top-K recorded
    (pages of 8 keys and more), 256-key pages that chunks cross; 96 ragged
    sequences; rows and outputs match the oracle, and the one-call step
    (index rows resolved to pool rows for the attention) equals the two calls
    bit for bit."""
    # 96 sequences: the one-call step's tail is too wide for the fused kernel,
    # so it takes the per-row top-K and the split attention over index rows
    B = 96
    cfg = gen.Config("decode-pages", "decode", B, 32, 8, 128, 6000, "bf16", 1,
                     (64, 16, 4), (2048, 512, 128), 16, 64, seed=33, n_queries=1, page_size=page)
    case = gen.make_case(cfg)
    case.seq_lens[:] = [6000, 3500] + [6000 - 37 * b for b in range(2, B)]
    for b, L in enumerate(case.seq_lens):
        case.k[b] = case.k[b].sub((slice(None), slice(0, int(L))))
        case.v[b] = case.v[b].sub((slice(None), slice(0, int(L))))
    H.say(f"decode page size {page}")
    dev = to_device(case)
    idx, out, _ = check_decode(case, dev, [0, 1, 50, B - 1])
    q = dev.q[0].contiguous()
    idx1, out1 = api.prune_attend(q, dev.k, dev.v, params_of(cfg), seq_lens=dev.seq_lens,
                                  block_table=dev.block_table, t=dev.t)
    torch.cuda.synchronize()
    assert torch.equal(idx1.view(idx.shape), idx)
    assert torch.equal(out1, out)


def _lib_width(case):
    from dynamic_sparse_attention_query_amd import _lib
    return _lib.index_width(params_of(case.cfg))


@pytest.fixture(scope="module")
def c3():
    H.say("generating c3 (1M-token decode)")
    case = gen.make_case("c3", n_queries=3)
    dev = to_device(case)
    return case, dev


def test_c3_decode_1m(c3):
    case, dev = c3
    for qi in range(2):
        idx, out, vis = check_decode(case, dev, [0], qi, visited=True)
        Q, s, e = H.decode_query(case, 0, qi)
        want = ref.visited_rows(Q, case.k[0], s, e, H.oracle_params(case.cfg))
        assert vis.cpu().tolist() == want, (vis.cpu().tolist(), want)


def test_c3_dense_decode_1m(c3):
    case, dev = c3
    q = dev.q[2].contiguous()
    out = api.dense_attn(q, dev.k, dev.v, seq_lens=dev.seq_lens).cpu().numpy()
    H.assert_close(out[0], H.oracle_dense(case, 0, 0, qi=2)[:, 0], "dense 1M decode")


def test_c4_paged_ragged_batch():
    H.say("generating c4 (32 ragged sequences, paged)")
    case = gen.make_case("c4")
    dev = to_device(case)
    bs = sorted({0, 31, *np.random.default_rng(7).choice(32, 5, replace=False).tolist()})
    idx, out, _ = check_decode(case, dev, bs)
    # the one-call step resolves the pages of its index rows while selecting;
    # the attention over them is the two-call path's, bit for bit
    q = dev.q[0].contiguous()
    idx1, out1 = api.prune_attend(q, dev.k, dev.v, params_of(case.cfg), seq_lens=dev.seq_lens,
                                  block_table=dev.block_table, t=dev.t)
    torch.cuda.synchronize()
    assert torch.equal(idx1.view(idx.shape), idx)
    assert torch.equal(out1, out)


def test_c5_decode_3m_needles():
    H.say("generating c5 (3M-token decode)")
    case = gen.make_case("c5")
    dev = to_device(case)
    idx, out, _ = check_decode(case, dev, [0])
    row = set(idx.cpu().numpy()[0].tolist())
    for nd in case.needles:
        assert set(range(nd.slot_start, nd.slot_start + nd.length)) <= row
