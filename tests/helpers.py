"""Glue between the seeded workloads, the CPU oracle and the GPU library (tests only)."""
from __future__ import annotations

import os
import sys

import numpy as np

from dynamic_sparse_attention_query_amd import gen
from oracle import ref

MAX_ABS = 1e-2      # fp32 attention outputs vs the oracle
REL_L2 = 5e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def oracle_params(cfg: gen.Config) -> ref.Params:
    return ref.Params(cfg.block_q, tuple(cfg.chunk), tuple(cfg.keep), cfg.n_sink, cfg.n_window)


def prefill_block(case: gen.Case, b: int, m: int):
    """(Q block [Hq, b_q, d] float32, s, e) of prefill block m of sequence b."""
    cfg = case.cfg
    s, e = m * cfg.block_q, (m + 1) * cfg.block_q
    return case.q.sub(b)[:, s:e], s, e


def decode_query(case: gen.Case, b: int, qi: int = 0):
    T = int(case.seq_lens[b])
    return case.q.sub((qi, b))[:, None, :], T - 1, T


def oracle_row(case, b, m, qi=0):
    cfg = case.cfg
    p = oracle_params(cfg)
    if cfg.mode == "prefill":
        Q, s, e = prefill_block(case, b, m)
    else:
        Q, s, e = decode_query(case, b, qi)
    return ref.pad_row(ref.prune_block(Q, case.k[b], s, e, p), ref.index_width(p))


def oracle_attend(case, b, m, row, qi=0):
    cfg = case.cfg
    if cfg.mode == "prefill":
        Q, s, e = prefill_block(case, b, m)
    else:
        Q, s, e = decode_query(case, b, qi)
    return ref.attend_block(Q, case.k[b], case.v[b], row, s, ref.default_scale(cfg.d))


def oracle_dense(case, b, m, qi=0):
    cfg = case.cfg
    if cfg.mode == "prefill":
        Q, s, e = prefill_block(case, b, m)
    else:
        Q, s, e = decode_query(case, b, qi)
    return ref.dense_block(Q, case.k[b], case.v[b], s, e, ref.default_scale(cfg.d))


def assert_close(got: np.ndarray, want: np.ndarray, what: str):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - want).max()
    rel = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30)
    assert err <= MAX_ABS and rel <= REL_L2, f"{what}: max-abs {err:.3e}, rel-L2 {rel:.3e}"
    return err, rel
