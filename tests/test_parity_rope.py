"""GPU parity of pruning with RoPE inside SelectRep (InfiniteHiP page, "Four
RoPE Styles for Context Pruning": Relative and Chunk-indexed):
dsa_prune_select_rope through the C ABI against the CPU oracle. Rotated
vectors are rounded to multiples of 1/128, so every SelectRep score is exact
on both sides and the index rows are compared bit-exactly."""
import numpy as np
import pytest
import torch

import helpers as H
from dynamic_sparse_attention_query_amd import api, gen
from dynamic_sparse_attention_query_amd.inputs import params_of, to_device
from oracle import ref

pytestmark = pytest.mark.gpu

BASE = 500000.0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from dynamic_sparse_attention_query_amd import _lib
    _lib.load()


STYLES = ["relative", "chunk_indexed"]


def oracle_row_rt(case, b, m, qi=0, style="relative"):
    cfg = case.cfg
    p = H.oracle_params(cfg)
    if cfg.mode == "prefill":
        Q, s, e = H.prefill_block(case, b, m)
    else:
        Q, s, e = H.decode_query(case, b, qi)
    prune = ref.prune_block_rt if style == "relative" else ref.prune_block_ci
    return ref.pad_row(prune(Q, case.k[b], s, e, p, BASE), ref.index_width(p))


@pytest.mark.parametrize("style", STYLES)
def test_rope_prefill_fp32_full(style):
    """The tiny fp32 workload: every block's row; RoPE changes some rows."""
    case = gen.make_case("c1")
    H.say(f"rope {style} c1: all 128 rows")
    dev = to_device(case)
    p = params_of(case.cfg)
    idx = api.prune_select_rope(dev.q, dev.k, p, BASE, style=style).cpu().numpy()
    plain = api.prune_select(dev.q, dev.k, p).cpu().numpy()
    for m in range(case.cfg.t // case.cfg.block_q):
        want = oracle_row_rt(case, 0, m, style=style)
        assert np.array_equal(idx[0, m], want), f"block {m}: first diff {np.flatnonzero(idx[0, m] != want)[:5]}"
    changed = int((idx != plain).any(axis=-1).sum())
    H.say(f"rope {style} c1: {changed} of {idx.shape[1]} rows differ from plain SelectRep")
    assert changed > 0


@pytest.mark.parametrize("style", STYLES)
def test_rope_prefill_llama_heads_4k(style):
    """32 q / 8 kv heads, d = 128, bf16, three stages at T = 4096: 20 blocks."""
    case = gen.make_case("c2", t=4096, keep=(1024, 512, 256), n_window=256, n_needles=2)
    H.say(f"rope {style} c2 4K: sampled rows")
    dev = to_device(case)
    idx = api.prune_select_rope(dev.q, dev.k, params_of(case.cfg), BASE, style=style).cpu().numpy()
    for m in gen.sample_blocks(64, 18, 5):
        want = oracle_row_rt(case, 0, m, style=style)
        assert np.array_equal(idx[0, m], want), f"block {m}: first diff {np.flatnonzero(idx[0, m] != want)[:5]}"


@pytest.mark.parametrize("style", STYLES)
@pytest.mark.parametrize("paged", [False, True])
def test_rope_decode(paged, style):
    """Decode with relative-RoPE SelectRep: a 64K-token sequence (contiguous)
    and a ragged batch of 3 over a paged pool."""
    if paged:
        case = gen.make_case("c4", batch=3, ragged=(20000, 70000), t=70000)
    else:
        case = gen.make_case("c3", t=65536, n_queries=1)
    H.say(f"rope {style} decode paged={paged}")
    dev = to_device(case)
    q = dev.q[0].contiguous()
    idx = api.prune_select_rope(q, dev.k, params_of(case.cfg), BASE, seq_lens=dev.seq_lens,
                                block_table=dev.block_table, t=dev.t, style=style).cpu().numpy()
    for b in range(case.cfg.batch):
        want = oracle_row_rt(case, b, 0, style=style)
        assert np.array_equal(idx[b], want), f"sequence {b}: first diff {np.flatnonzero(idx[b] != want)[:5]}"


@pytest.mark.parametrize("dtype,hq,hkv,d,chunk,keep,paged", [
    ("f32", 8, 8, 64, (64, 4, 1), (2048, 512, 128), False),      # one head per group; 8-key, 4-key, 1-key chunks
    ("bf16", 16, 2, 128, (128, 16, 2), (2048, 512, 64), True),   # groups of 8; 2-key chunks take no first round
    ("bf16", 8, 4, 64, (32, 8, 4), (1024, 256, 64), False),      # groups of 2 at d = 64
    ("bf16", 32, 32, 128, (64, 16, 4), (2048, 512, 128), False),  # 32 kv heads: two score slices
    ("bf16", 24, 12, 64, (32, 8, 4), (1024, 256, 64), True),     # 12 kv heads per scoring workgroup
])
@pytest.mark.parametrize("style", STYLES)
def test_rope_decode_shapes(dtype, hq, hkv, d, chunk, keep, paged, style):
    """Decode tournaments across group sizes, head dims, key types and chunk
    lengths (every first-round form: 4 and 8 keys, none, single keys)."""
    kw = dict(batch=2, ragged=(9000, 16384), page_size=64) if paged else dict(batch=1)
    case = gen.make_case("c4" if paged else "c3", hq=hq, hkv=hkv, d=d, t=16384, dtype=dtype, chunk=chunk,
                         keep=keep, n_queries=1, **kw)
    H.say(f"rope {style} decode {dtype} {hq}/{hkv} d={d} chunk={chunk} paged={paged}")
    dev = to_device(case)
    q = dev.q[0].contiguous()
    idx = api.prune_select_rope(q, dev.k, params_of(case.cfg), BASE, seq_lens=dev.seq_lens,
                                block_table=dev.block_table, t=dev.t, style=style).cpu().numpy()
    for b in range(case.cfg.batch):
        want = oracle_row_rt(case, b, 0, style=style)
        assert np.array_equal(idx[b], want), f"sequence {b}: first diff {np.flatnonzero(idx[b] != want)[:5]}"


@pytest.mark.parametrize("hq,hkv,d,chunk,keep", [
    (8, 1, 64, (32, 8, 1), (512, 256, 64)),      # matrix-core tournaments at d = 64, group of 8, single keys
    (4, 2, 128, (16, 2), (512, 128)),            # 2-key chunks
])
@pytest.mark.parametrize("style", STYLES)
def test_rope_prefill_shapes(hq, hkv, d, chunk, keep, style):
    """bf16 prefill (the matrix-core tournaments) across head layouts and
    chunk lengths: every block's row."""
    case = gen.make_case("c2", hq=hq, hkv=hkv, d=d, t=2048, chunk=chunk, keep=keep, n_window=64,
                         n_sink=64, n_needles=0, structure="plain")
    H.say(f"rope {style} prefill {hq}/{hkv} d={d} chunk={chunk}")
    dev = to_device(case)
    idx = api.prune_select_rope(dev.q, dev.k, params_of(case.cfg), BASE, style=style).cpu().numpy()
    for m in range(case.cfg.t // case.cfg.block_q):
        want = oracle_row_rt(case, 0, m, style=style)
        assert np.array_equal(idx[0, m], want), f"block {m}: first diff {np.flatnonzero(idx[0, m] != want)[:5]}"


def test_ci_query_ids_capped_at_own_position():
    """Chunk-indexed RoPE with 4 sinks and single-key chunks in the last stage:
    the stage's query ID passes most queries' own positions, so each of them
    is rotated to its own position (the cap); every block's row."""
    case = gen.make_case("c2", hq=4, hkv=2, d=64, t=1024, chunk=(16, 1), keep=(256, 32), n_window=64,
                         n_sink=4, n_needles=0, structure="plain")
    cfg = case.cfg
    H.say("rope chunk_indexed prefill with capped query IDs")
    p = H.oracle_params(cfg)
    geo = ref.geometry(1024 - 64, 1024, p)
    ids = ref.ci_query_positions(np.arange(1024 - 64, 1024), geo.mid_hi, p.n_sink, p.n_window, 1)
    assert (ids < np.arange(1024 - 64, 1024)).sum() < 64 and (ids == np.arange(1024 - 64, 1024)).sum() > 32
    dev = to_device(case)
    idx = api.prune_select_rope(dev.q, dev.k, params_of(cfg), BASE, style="chunk_indexed").cpu().numpy()
    for m in range(cfg.t // cfg.block_q):
        want = oracle_row_rt(case, 0, m, style="chunk_indexed")
        assert np.array_equal(idx[0, m], want), f"block {m}: first diff {np.flatnonzero(idx[0, m] != want)[:5]}"


@pytest.mark.parametrize("style", STYLES)
def test_rope_decode_edge_lengths_and_budgets(style):
    """Ragged contiguous decode batch with lengths below the sinks, inside
    sinks + window, on a chunk-grid tail and long enough for all three stages;
    then a zero budget (sinks and window only) and a budget above every length
    (nothing pruned)."""
    cfg = gen.Config("decode-edge", "decode", 6, 8, 2, 128, 9000, "bf16", 1,
                     (64, 16, 4), (2048, 512, 128), 16, 64, seed=11, n_queries=1)
    case = gen.make_case(cfg)
    case.seq_lens[:] = [1, 7, 80, 300, 5000, 9000]
    for b, L in enumerate(case.seq_lens):
        case.k[b] = case.k[b].sub((slice(None), slice(0, int(L))))
        case.v[b] = case.v[b].sub((slice(None), slice(0, int(L))))
    for keep in ((2048, 512, 128), (0, 0, 0), (16384, 16384, 16384)):
        case.cfg = cfg.replace(keep=keep)
        H.say(f"rope {style} decode edge lengths, keep={keep}")
        dev = to_device(case)
        q = dev.q[0].contiguous()
        idx = api.prune_select_rope(q, dev.k, params_of(case.cfg), BASE, seq_lens=dev.seq_lens,
                                    block_table=dev.block_table, t=dev.t, style=style).cpu().numpy()
        for b in range(cfg.batch):
            want = oracle_row_rt(case, b, 0, style=style)
            assert np.array_equal(idx[b], want), f"keep {keep} sequence {b}: first diff {np.flatnonzero(idx[b] != want)[:5]}"
        if keep[0] == 0:
            T = 9000
            mid_hi = 16 + ((T - 64 - 16) // 64) * 64
            row = idx[5]
            assert np.array_equal(row[row >= 0], np.r_[np.arange(16), np.arange(mid_hi, T)])


@pytest.fixture(scope="module")
def c4_full():
    case = gen.make_case("c4", n_queries=1)
    return case, to_device(case)


@pytest.mark.parametrize("style", STYLES)
def test_rope_decode_batch32_paged_full(c4_full, style):
    """The batch-32 ragged paged workload at full size (lengths 65,536 to
    262,144): the launches exceed one sequence's worth of workgroups, so each
    stage's top-K runs as its own kernel; three sampled sequences against the
    oracle, every row's shape checked."""
    case, dev = c4_full
    H.say(f"rope {style} decode batch-32 paged full size")
    q = dev.q[0].contiguous()
    idx = api.prune_select_rope(q, dev.k, params_of(case.cfg), BASE, seq_lens=dev.seq_lens,
                                block_table=dev.block_table, t=dev.t, style=style).cpu().numpy()
    p = H.oracle_params(case.cfg)
    for b in (0, 17, 31):
        want = oracle_row_rt(case, b, 0, style=style)
        assert np.array_equal(idx[b], want), f"sequence {b}: first diff {np.flatnonzero(idx[b] != want)[:5]}"
    for b in range(case.cfg.batch):
        row = idx[b][idx[b] >= 0]
        e = int(case.seq_lens[b])
        rem = (e - p.n_window - p.n_sink) % p.chunk[0]
        assert len(row) == p.n_sink + p.keep[-1] + p.n_window + rem and np.all(np.diff(row) > 0), b
        assert np.array_equal(row[:p.n_sink], np.arange(p.n_sink)) and row[-1] == e - 1, b


@pytest.mark.parametrize("style", STYLES)
def test_rope_prefill_two_sequences(style):
    """Two prefill sequences in one call (the key rotation and the rotated
    query copies index sequence and kv head): every block of both."""
    case = gen.make_case("c2", hq=8, hkv=2, d=128, t=1024, batch=2, chunk=(16, 4), keep=(256, 64), n_window=64,
                         n_sink=16, n_needles=0, structure="plain")
    H.say(f"rope {style} prefill, two sequences")
    dev = to_device(case)
    idx = api.prune_select_rope(dev.q, dev.k, params_of(case.cfg), BASE, style=style).cpu().numpy()
    for b in range(2):
        for m in range(case.cfg.t // case.cfg.block_q):
            want = oracle_row_rt(case, b, m, style=style)
            assert np.array_equal(idx[b, m], want), f"seq {b} block {m}: first diff {np.flatnonzero(idx[b, m] != want)[:5]}"


def _rotated_keys_step(case, dev, p, q, pieces=1):
    """Chunk-indexed decode over keys rotated once (dsa_rope_rotate_keys, in
    `pieces` consecutive position ranges), then dsa_prune_select_rope_keys."""
    k_rot = api.rope_key_copies(dev.k, p)
    T = dev.k.shape[2]
    cuts = np.linspace(0, T, pieces + 1).astype(int)
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        api.rope_rotate_keys(dev.k, p, BASE, k_rot, pos_begin=int(lo), pos_end=int(hi), seq_lens=dev.seq_lens)
    idx = api.prune_select_rope_keys(q, k_rot, p, BASE, seq_lens=dev.seq_lens)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), k_rot


@pytest.mark.parametrize("dtype,hq,hkv,d,chunk,keep", [
    ("bf16", 32, 8, 128, (256, 32, 8), (8192, 2048, 1024)),     # the 1M configuration's stage shapes
    ("bf16", 8, 2, 64, (64, 16, 4), (2048, 512, 128)),
    ("f32", 8, 8, 64, (64, 4, 1), (2048, 512, 128)),           # fp32 inputs, one-key chunks
])
def test_ci_decode_over_rotated_keys(dtype, hq, hkv, d, chunk, keep):
    """Keys rotated once per stage give the rows of the chunk-indexed decode
    that rotates them every step, bit for bit, and those of the oracle; the
    rotation written in three position ranges equals one pass over all."""
    case = gen.make_case("c3", hq=hq, hkv=hkv, d=d, t=40000, dtype=dtype, chunk=chunk, keep=keep, batch=2,
                         n_queries=1)
    case.seq_lens[:] = [40000, 23456]
    H.say(f"rope chunk_indexed decode over rotated keys {dtype} {hq}/{hkv} d={d} chunk={chunk}")
    dev = to_device(case)
    p = params_of(case.cfg)
    q = dev.q[0].contiguous()
    want = api.prune_select_rope(q, dev.k, p, BASE, seq_lens=dev.seq_lens, style="chunk_indexed").cpu().numpy()
    got, k1 = _rotated_keys_step(case, dev, p, q)
    assert np.array_equal(got, want), f"first diff {np.flatnonzero(got != want)[:5]}"
    for b in range(case.cfg.batch):
        assert np.array_equal(got[b], oracle_row_rt(case, b, 0, style="chunk_indexed")), f"sequence {b}"
    got3, k3 = _rotated_keys_step(case, dev, p, q, pieces=3)
    assert np.array_equal(got3, want)
    ns = case.cfg.n_sink
    for s in range(len(k1)):
        assert torch.equal(k1[s][:, :, ns:], k3[s][:, :, ns:]), f"stage {s}: rotated rows differ by range split"
