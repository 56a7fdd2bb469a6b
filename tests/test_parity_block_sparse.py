"""GPU parity of the block-sparse heads (MInference page, "Online Dynamic Index
Estimation: Block-Sparse Heads (Algorithm 3)" and "Block-Sparse FlashAttention
Kernel (Appendix C.4.1)"): dsa_block_sparse_select and dsa_sparse_attn_heads
through the C ABI against the CPU oracle, and the block-list forms
(dsa_block_sparse_select_lists, dsa_sparse_attn_lists).

Index rows are compared bit-exactly (the pooled logits are exact fp64 numbers
on the input grid, rounded once to fp32 on both sides); attention outputs
within max-abs 1e-2 and relative-L2 5e-3.
"""
import numpy as np
import pytest
import torch

import helpers as H
from dynamic_sparse_attention_query_amd import api, gen
from dynamic_sparse_attention_query_amd.inputs import to_device
from oracle import ref

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from dynamic_sparse_attention_query_amd import _lib
    _lib.load()


class Host:
    """fp32 host copies of one sequence's inputs and its pooled rows."""

    def __init__(self, Q, K, V):
        self.Q, self.K, self.V = Q, K, V                     # [Hq,T,d], [Hkv,T,d], [Hkv,T,d]
        self.Qp = ref.bs_pool(Q, 64)
        self.Kp = ref.bs_pool(K, 64)
        self.G = Q.shape[0] // K.shape[0]

    def row(self, h, m, kb, L):
        sel = ref.bs_select(ref.bs_block_scores(self.Qp, self.Kp, h, m), kb)
        pos = (sel[:, None] * 64 + np.arange(64)[None, :]).reshape(-1)
        return ref.pad_row(pos, L)

    def attend(self, h, m, row):
        g = h // self.G
        s = 64 * m
        return ref.attend_block(self.Q[h:h + 1, s:s + 64], self.K[g:g + 1], self.V[g:g + 1], row, s,
                                ref.default_scale(self.Q.shape[2]))[0]


def host_of_case(case, b=0):
    return Host(case.q.sub(b).f32(), case.k[b].f32(), case.v[b].f32())


def run_gpu(q, k, v, kb):
    idx = api.block_sparse_select(q, k, kb)
    out = api.sparse_attn_heads(q, k, v, idx)
    torch.cuda.synchronize()
    return idx, out


def check(host, idx, out, kb, rows, attn_rows, b=0, what=""):
    L = idx.shape[-1]
    idx_np = idx[b].cpu().numpy()
    for h, m in rows:
        want = host.row(h, m, kb, L)
        got = idx_np[h, m]
        assert np.array_equal(got, want), f"{what} row (h={h}, m={m}): first diff at {np.flatnonzero(got != want)[:5]}"
    out_np = out[b].cpu().numpy()
    for h, m in attn_rows:
        H.assert_close(out_np[h, 64 * m:64 * m + 64], host.attend(h, m, host.row(h, m, kb, L)),
                       f"{what} attention (h={h}, m={m})")


def all_rows(Hq, nblk):
    return [(h, m) for h in range(Hq) for m in range(nblk)]


# --------------------------------------------------------------------------- #
def test_bs_fp32_one_head_full():
    """The tiny fp32 workload (one head, d = 64, T = 4096): every row and every
    block's attention, k_b = 8 of 64 blocks."""
    case = gen.make_case("c1")
    H.say("bs fp32 T=4096 k_b=8: all rows and outputs")
    dev = to_device(case)
    idx, out = run_gpu(dev.q, dev.k, dev.v, 8)
    assert tuple(idx.shape) == (1, 1, 64, 512)
    host = host_of_case(case)
    rows = all_rows(1, 64)
    check(host, idx, out, 8, rows, rows, what="fp32")


def test_bs_bf16_gqa_4k_full():
    """Llama-shaped heads (32 q / 8 kv, d = 128) at T = 4096: every row, k_b = 16;
    attention of every head in six blocks."""
    case = gen.make_case("c2", t=4096, n_needles=3)
    H.say("bs bf16 32/8 heads T=4096 k_b=16: all rows, 192 attention blocks")
    dev = to_device(case)
    idx, out = run_gpu(dev.q, dev.k, dev.v, 16)
    host = host_of_case(case)
    check(host, idx, out, 16, all_rows(32, 64),
          [(h, m) for h in range(32) for m in (0, 1, 15, 16, 40, 63)], what="4k")
    idx2, out2 = run_gpu(dev.q, dev.k, dev.v, 16)
    assert torch.equal(idx, idx2) and torch.equal(out, out2), "not deterministic"


def test_bs_c2_32k_sampled():
    """The 32K Llama-shaped workload with the page's k_b = 100: 96 sampled rows
    (first and last blocks included) bit-exact, 24 of them through attention;
    the planted needle blocks are reported."""
    case = gen.make_case("c2")
    H.say("bs c2 32K k_b=100: sampled rows")
    dev = to_device(case)
    idx, out = run_gpu(dev.q, dev.k, dev.v, 100)
    host = host_of_case(case)
    rng = np.random.default_rng(7)
    nblk = 512
    rows = [(0, 0), (31, nblk - 1), (5, 99), (6, 100)] + [
        (int(h), int(m)) for h, m in zip(rng.integers(0, 32, 92), rng.integers(0, nblk, 92))]
    check(host, idx, out, 100, rows, rows[:24], what="32k")
    idx_np = idx[0].cpu().numpy()
    hit = sum(int(n.slot_start in set(idx_np[n.q_head, n.query // 64].tolist())) for n in case.needles)
    H.say(f"bs c2 32K needle blocks kept {hit}/{len(case.needles)}")


@pytest.mark.parametrize("dtype,hq,hkv,d,nblk,batch,kb", [
    ("bf16", 4, 2, 64, 37, 2, 5),        # ragged block tiles (37 = 2 x 16 + 5), two sequences
    ("f32", 8, 1, 128, 21, 1, 3),        # group of 8, fp32 at d = 128
    ("bf16", 2, 2, 128, 20, 1, 1),       # k_b = 1
    ("bf16", 4, 4, 64, 9, 1, 12),        # k_b above the block count: every causal block
])
def test_bs_shapes(dtype, hq, hkv, d, nblk, batch, kb):
    t = 64 * nblk
    case = gen.make_case("c2", hq=hq, hkv=hkv, d=d, t=t, batch=batch, dtype=dtype, structure="plain",
                         n_needles=0, n_sink=64, n_window=64, chunk=(64,), keep=(128,))
    H.say(f"bs {dtype} {hq}/{hkv} heads d={d} blocks={nblk} batch={batch} k_b={kb}")
    dev = to_device(case)
    idx, out = run_gpu(dev.q, dev.k, dev.v, kb)
    for b in range(batch):
        host = host_of_case(case, b)
        rows = all_rows(hq, nblk)
        check(host, idx, out, kb, rows, rows, b=b, what=f"seq {b}")
    if kb >= nblk:                                       # every causal block: dense attention
        dense = api.dense_attn(dev.q, dev.k, dev.v)
        torch.cuda.synchronize()
        H.assert_close(out.cpu().numpy(), dense.cpu().numpy(), "k_b >= blocks vs dense path")


def test_bs_ties_go_to_lower_blocks():
    """Every key block identical: all pooled logits of a row tie exactly, so the
    first k_b blocks are kept."""
    rng = np.random.default_rng(11)
    nblk, d, kb = 24, 64, 6
    Q = rng.integers(-8, 9, size=(2, 64 * nblk, d)).astype(np.float32) / 8
    K = np.tile(rng.integers(-8, 9, size=(1, 64, d)).astype(np.float32) / 8, (1, nblk, 1))
    V = rng.normal(size=(1, 64 * nblk, d)).astype(np.float32)
    q, k, v = (torch.from_numpy(x).unsqueeze(0).to("cuda", torch.bfloat16) for x in (Q, K, V))
    H.say("bs ties: identical key blocks")
    idx, out = run_gpu(q, k, v, kb)
    host = Host(Q, K, v[0].float().cpu().numpy())
    rows = all_rows(2, nblk)
    check(host, idx, out, kb, rows, rows[:8], what="ties")
    for m in range(nblk):
        want = np.arange(64 * min(m + 1, kb))
        assert np.array_equal(idx[0, 0, m].cpu().numpy()[:len(want)], want)


@pytest.mark.parametrize("width,d", [(100, 128), (50, 128), (72, 64)])
def test_heads_attention_arbitrary_rows(width, d):
    """Per-head rows that are not whole 64-key blocks: ascending causal
    positions of each head's own choosing, -1 padded, widths that end inside a
    tile (100), are not a multiple of 4 (50, the register-staged kernel) or use
    d = 64."""
    rng = np.random.default_rng(width)
    hq, hkv, nblk = 4, 2, 6
    t = 64 * nblk
    Q = rng.integers(-8, 9, size=(1, hq, t, d)).astype(np.float32) / 8
    K = rng.integers(-8, 9, size=(1, hkv, t, d)).astype(np.float32) / 8
    V = rng.normal(size=(1, hkv, t, d)).astype(np.float32)
    idx = np.full((1, hq, nblk, width), -1, dtype=np.int32)
    for h in range(hq):
        for m in range(nblk):
            e = 64 * (m + 1)
            n = int(rng.integers(1, min(width, e) + 1))
            # key 0 in every row: each query sees at least one key
            pos = np.union1d([0], rng.choice(np.arange(1, e), size=n - 1, replace=False))
            idx[0, h, m, :n] = pos
    q, k, v = (torch.from_numpy(x).to("cuda", torch.bfloat16) for x in (Q, K, V))
    H.say(f"per-head rows width={width} d={d}")
    out = api.sparse_attn_heads(q, k, v, torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    host = Host(Q[0], K[0], v[0].float().cpu().numpy())
    out_np = out[0].cpu().numpy()
    for h in range(hq):
        for m in range(nblk):
            H.assert_close(out_np[h, 64 * m:64 * m + 64], host.attend(h, m, idx[0, h, m]), f"(h={h}, m={m})")


# --------------------------------------------------------------------------- #
# block lists (the page's kernel takes block ids) and attention over them     #
# --------------------------------------------------------------------------- #
def run_lists(q, k, v, kb, attend=True):
    blocks, counts = api.block_sparse_select_lists(q, k, kb)
    out = api.sparse_attn_lists(q, k, v, blocks, counts) if attend else None
    torch.cuda.synchronize()
    return blocks, counts, out


def check_lists(host, blocks, counts, out, kb, rows, attn_rows, b=0, what=""):
    bl, cn = blocks[b].cpu().numpy(), counts[b].cpu().numpy()
    wb = bl.shape[-1]
    assert wb == (kb + 3) // 4 * 4
    for h, m in rows:
        sel = ref.bs_select(ref.bs_block_scores(host.Qp, host.Kp, h, m), kb)
        assert tuple(cn[h, m]) == (len(sel), 0), f"{what} counts (h={h}, m={m})"
        assert np.array_equal(bl[h, m], ref.pad_row(sel, wb)), f"{what} block list (h={h}, m={m})"
    if out is None:
        return
    o = out[b].cpu().numpy()
    for h, m in attn_rows:
        sel = ref.bs_select(ref.bs_block_scores(host.Qp, host.Kp, h, m), kb)
        row = ref.list_positions(sel, np.array([], np.int64))
        H.assert_close(o[h, 64 * m:64 * m + 64], host.attend(h, m, row), f"{what} list attention (h={h}, m={m})")


def test_bs_lists_fp32_selection_full():
    """fp32 inputs (one head, d = 64): every block list bit-exact; attention
    over lists takes bf16 with d = 128 and rejects this shape before launch."""
    from dynamic_sparse_attention_query_amd import _lib
    case = gen.make_case("c1")
    dev = to_device(case)
    blocks, counts, _ = run_lists(dev.q, dev.k, dev.v, 8, attend=False)
    check_lists(host_of_case(case), blocks, counts, None, 8, all_rows(1, 64), [], what="fp32 lists")
    with pytest.raises(_lib.DsaError) as ei:
        api.sparse_attn_lists(dev.q, dev.k, dev.v, blocks, counts)
    assert ei.value.status == _lib.DSA_ERR_UNSUPPORTED


def test_bs_lists_bf16_gqa_4k_full():
    """Llama-shaped heads at T = 4096, k_b = 16: every block list; list
    attention of every head in six blocks against the oracle, and the whole
    output against the row path (same keys, another order)."""
    case = gen.make_case("c2", t=4096, n_needles=3)
    H.say("bs lists bf16 32/8 heads T=4096 k_b=16")
    dev = to_device(case)
    blocks, counts, out = run_lists(dev.q, dev.k, dev.v, 16)
    check_lists(host_of_case(case), blocks, counts, out, 16, all_rows(32, 64),
                [(h, m) for h in range(32) for m in (0, 1, 15, 16, 40, 63)], what="4k lists")
    _, out_rows = run_gpu(dev.q, dev.k, dev.v, 16)
    H.assert_close(out.cpu().numpy(), out_rows.cpu().numpy(), "list vs row attention")
    b2, c2, out2 = run_lists(dev.q, dev.k, dev.v, 16)
    assert torch.equal(blocks, b2) and torch.equal(counts, c2) and torch.equal(out, out2), "not deterministic"


def test_bs_lists_c2_32k_sampled():
    """The 32K workload with k_b = 100: 96 sampled block lists bit-exact, 24
    through list attention."""
    case = gen.make_case("c2")
    H.say("bs lists c2 32K k_b=100: sampled")
    dev = to_device(case)
    blocks, counts, out = run_lists(dev.q, dev.k, dev.v, 100)
    rng = np.random.default_rng(8)
    nblk = 512
    rows = [(0, 0), (31, nblk - 1), (5, 99), (6, 100)] + [
        (int(h), int(m)) for h, m in zip(rng.integers(0, 32, 92), rng.integers(0, nblk, 92))]
    check_lists(host_of_case(case), blocks, counts, out, 100, rows, rows[:24], what="32k lists")
