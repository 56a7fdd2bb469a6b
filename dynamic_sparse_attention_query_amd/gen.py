"""Seeded synthetic inputs for the sparse-attention workloads.

This module holds input *data* only: shapes, value distributions and planted
structure. It contains none of the attention or pruning arithmetic, so the CPU
oracle (under ``oracle/``) and the GPU tests can both draw their inputs from it
without sharing any of the method's code.

Value grids
-----------
* Q and K are integer codes in ``[-8, 8]`` scaled by 1/8. Every product of two
  such values is a multiple of 1/64 with magnitude <= 1, so every partial sum
  of a length-d dot product (d <= 128) is a multiple of 1/64 of magnitude <= 128.
  That fits in 13 significant bits, so a dot product is exact in fp32 in any
  summation order, and the values are exact in bf16 too.
* V is standard normal. For the bf16 workloads it is rounded once to bf16
  (round to nearest even) and stored as bf16 bit patterns; the float32 values
  handed to any consumer are those rounded values.

Workload shapes follow the pages: Llama-3-8B-shaped attention (32 query heads,
8 KV heads, d=128), 32K/128K prefill, and 1M/3M-token decode contexts
(InfiniteHiP page, sections "Formal Background" and "Latency Details").
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np

GRID_DEN = 8          # Q/K value = code / GRID_DEN
GRID_MAX = 8          # codes lie in [-GRID_MAX, GRID_MAX]


# --------------------------------------------------------------------------- #
# value containers                                                            #
# --------------------------------------------------------------------------- #
def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns, round to nearest even."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + r) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


class Values:
    """A read-only float32 view over a compact storage array.

    ``kind`` is ``"grid"`` (int8 codes, value = code/8), ``"bf16"`` (uint16 bit
    patterns) or ``"f32"``. Indexing returns float32 numpy arrays with the
    exact stored values.
    """

    def __init__(self, data: np.ndarray, kind: str):
        assert kind in ("grid", "bf16", "f32")
        self.data = data
        self.kind = kind

    @property
    def shape(self):
        return self.data.shape

    def __len__(self):
        return self.data.shape[0]

    def _conv(self, a):
        if self.kind == "grid":
            return np.asarray(a, dtype=np.float32) * np.float32(1.0 / GRID_DEN)
        if self.kind == "bf16":
            return bf16_bits_to_f32(a)
        return np.asarray(a, dtype=np.float32)

    def __getitem__(self, key):
        return self._conv(self.data[key])

    def sub(self, key) -> "Values":
        return Values(self.data[key], self.kind)

    def f32(self) -> np.ndarray:
        return self._conv(self.data)


# --------------------------------------------------------------------------- #
# configurations                                                              #
# --------------------------------------------------------------------------- #
@dataclass(frozen=True)
class Config:
    name: str
    mode: str                       # "prefill" | "decode"
    batch: int
    hq: int
    hkv: int
    d: int
    t: int                          # prefill length / decode context (or max for ragged)
    dtype: str                      # "f32" | "bf16"
    block_q: int
    chunk: Tuple[int, ...]
    keep: Tuple[int, ...]
    n_sink: int
    n_window: int
    seed: int
    structure: str = "plain"        # "planted" | "needles" | "local" | "plain"
    n_needles: int = 0
    ragged: Optional[Tuple[int, int]] = None   # decode: lengths ~ U[lo, hi]
    page_size: int = 0              # decode: > 0 -> paged KV pool
    n_queries: int = 1              # decode: distinct queries drawn (step i uses query i)

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


# The five workloads plus the 128K prefill measurement shape.
CONFIGS = {
    # Tiny single-layer causal prefill, fp32, one head.
    "c1": Config("c1-tiny-prefill-4k", "prefill", 1, 1, 1, 64, 4096, "f32", 32,
                 (16, 4), (2048, 512), 16, 64, seed=1, structure="planted"),
    # Llama-3-8B-shaped prefill at 32K, needles in 1% of stage-1 chunks.
    "c2": Config("c2-llama3-8b-prefill-32k", "prefill", 1, 32, 8, 128, 32768, "bf16", 64,
                 (64, 32, 8), (16384, 8192, 4096), 64, 1024, seed=2,
                 structure="needles", n_needles=5),
    # Same shape at 128K: the sparse-prefill throughput measurement.
    "c2_128k": Config("c2-llama3-8b-prefill-128k", "prefill", 1, 32, 8, 128, 131072, "bf16", 64,
                      (64, 32, 8), (16384, 8192, 4096), 64, 1024, seed=6,
                      structure="needles", n_needles=20),
    # 1M-token single-sequence decode.
    "c3": Config("c3-decode-1m", "decode", 1, 32, 8, 128, 1048576, "bf16", 1,
                 (256, 32, 8), (32768, 8192, 4096), 64, 1024, seed=3, n_queries=64),
    # Batch-32 ragged decode over a paged KV pool.
    "c4": Config("c4-decode-b32-ragged-paged", "decode", 32, 32, 8, 128, 262144, "bf16", 1,
                 (256, 32, 8), (32768, 8192, 4096), 64, 1024, seed=4,
                 ragged=(65536, 262144), page_size=64),
    # 3M-token single-sequence decode with 10 needles.
    "c5": Config("c5-decode-3m", "decode", 1, 32, 8, 128, 3000000, "bf16", 1,
                 (256, 32, 8), (32768, 8192, 4096), 64, 1024, seed=5,
                 structure="needles", n_needles=10),
}


@dataclass
class Needle:
    """A planted chunk of identical keys equal to sign(q) of one query/head."""
    b: int
    slot_start: int     # first key position of the planted run
    length: int
    kv_head: int
    q_head: int
    query: int          # absolute query position (prefill) / query index (decode)


@dataclass
class Case:
    cfg: Config
    q: Values                       # prefill [B,Hq,T,d]; decode [NQ,B,Hq,d]
    k: List[Values]                 # per sequence [Hkv, T_b, d]
    v: List[Values]                 # per sequence [Hkv, T_b, d]
    seq_lens: np.ndarray            # [B] int32 (prefill: all == t)
    needles: List[Needle] = field(default_factory=list)
    planted: dict = field(default_factory=dict)   # c1: block -> list of slot starts
    # paged decode
    block_table: Optional[np.ndarray] = None      # [B, max_pages] int32
    n_pages: int = 0

    @property
    def batch(self):
        return self.cfg.batch


BLOCK = 1 << 22          # values per independently seeded block
_NORMAL_LEVELS = None


def _pool_map(fn, n):
    workers = max(1, min(16, os.cpu_count() or 1))
    if n <= 1 or workers == 1:
        return [fn(i) for i in range(n)]
    with ThreadPoolExecutor(workers) as ex:
        return list(ex.map(fn, range(n)))


def _grid_fill(shape, seed: int, tag: int) -> np.ndarray:
    """Uniform integer codes in [-8, 8]. Block i of BLOCK values is drawn from
    SeedSequence([seed, tag, i]): 15 base-17 digits of one uniform draw below
    17**15 give 15 exactly uniform codes."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.int8)

    def block(i):
        lo, hi = i * BLOCK, min(n, (i + 1) * BLOCK)
        m = hi - lo
        rng = np.random.default_rng([seed, tag, i])
        x = rng.integers(0, 17 ** 15, size=(m + 14) // 15, dtype=np.uint64)
        dig = np.empty((15, x.size), dtype=np.int8)
        for r in range(15):
            dig[r] = (x % np.uint64(17)).astype(np.int8) - GRID_MAX
            x //= np.uint64(17)
        out[lo:hi] = dig.reshape(-1)[:m]

    _pool_map(block, (n + BLOCK - 1) // BLOCK)
    return out.reshape(shape)


def _normal_levels() -> np.ndarray:
    """bf16 bit patterns of the standard-normal quantiles at (i + 0.5) / 65536."""
    global _NORMAL_LEVELS
    if _NORMAL_LEVELS is None:
        from scipy.special import ndtri
        u = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
        _NORMAL_LEVELS = bf16_round_bits(ndtri(u).astype(np.float32))
    return _NORMAL_LEVELS


def _normal_fill(shape, seed: int, tag: int, dtype: str) -> "Values":
    """Standard-normal values. fp32: numpy normals per seeded block. bf16:
    inverse-CDF sampling on a 65536-level quantile grid (finer than bf16's
    resolution), stored as bf16 bit patterns."""
    n = int(np.prod(shape))
    if dtype == "f32":
        out32 = np.empty(n, dtype=np.float32)

        def block32(i):
            lo, hi = i * BLOCK, min(n, (i + 1) * BLOCK)
            out32[lo:hi] = np.random.default_rng([seed, tag, i]).standard_normal(size=hi - lo, dtype=np.float32)

        _pool_map(block32, (n + BLOCK - 1) // BLOCK)
        return Values(out32.reshape(shape), "f32")
    lv = _normal_levels()
    out = np.empty(n, dtype=np.uint16)

    def block(i):
        lo, hi = i * BLOCK, min(n, (i + 1) * BLOCK)
        u = np.random.default_rng([seed, tag, i]).integers(0, 65536, size=hi - lo, dtype=np.uint16)
        out[lo:hi] = lv[u]

    _pool_map(block, (n + BLOCK - 1) // BLOCK)
    return Values(out.reshape(shape), "bf16")


def _sign_codes(codes: np.ndarray) -> np.ndarray:
    return (np.sign(codes.astype(np.int16)) * GRID_DEN).astype(np.int8)


def eligible_slots(origin: int, align: int, limit: int) -> int:
    """Number of aligned slots [origin + align*j, origin + align*(j+1)) that end at or before limit."""
    return max(0, (limit - origin) // align)


def make_case(cfg: Config | str, **overrides) -> Case:
    """Draw the seeded inputs of a workload.

    Every array is drawn from its own seed stream: tag 1 lengths, 2 Q, 3 the
    Q block directions and perturbations (planted structure), 100 + b the keys
    of sequence b, 200 + b its values, 4 the planted structure, 5 the page
    permutation.
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    if overrides:
        cfg = cfg.replace(**overrides)
    B, Hq, Hkv, d = cfg.batch, cfg.hq, cfg.hkv, cfg.d
    seed = cfg.seed

    if cfg.ragged is not None:
        lo, hi = cfg.ragged
        seq_lens = np.random.default_rng([seed, 1]).integers(lo, hi + 1, size=B).astype(np.int32)
    else:
        seq_lens = np.full(B, cfg.t, dtype=np.int32)

    # ---- Q ------------------------------------------------------------------
    planted = {}
    if cfg.mode == "prefill":
        if cfg.structure == "planted":
            nblk = cfg.t // cfg.block_q
            u = _grid_fill((B, Hq, nblk, d), seed, 3).astype(np.int16)
            eps = np.random.default_rng([seed, 3, 1]).integers(-2, 3, size=(B, Hq, cfg.t, d)).astype(np.int16)
            qc = np.clip(np.repeat(u, cfg.block_q, axis=2) + eps, -GRID_MAX, GRID_MAX).astype(np.int8)
        else:
            qc = _grid_fill((B, Hq, cfg.t, d), seed, 2)
    else:
        qc = _grid_fill((cfg.n_queries, B, Hq, d), seed, 2)
    q = Values(qc, "grid")

    # ---- K, V ---------------------------------------------------------------
    k_list, v_list = [], []
    for b in range(B):
        k_list.append(Values(_grid_fill((Hkv, int(seq_lens[b]), d), seed, 100 + b), "grid"))
    for b in range(B):
        v_list.append(_normal_fill((Hkv, int(seq_lens[b]), d), seed, 200 + b, cfg.dtype))
    rng = np.random.default_rng([seed, 4])

    case = Case(cfg=cfg, q=q, k=k_list, v=v_list, seq_lens=seq_lens)

    # ---- planted structure --------------------------------------------------
    # Slots are aligned runs of keys laid out from `origin` in steps of `align`;
    # a slot is planted for a query only if it ends at least `lag` keys before
    # the query's block ends, so that it sits among the prunable middle keys.
    if cfg.structure == "planted":
        # Each query block owns up to 4 slots of `chunk[0]` keys, drawn without
        # replacement from the not-yet-owned eligible slots, in block order; the
        # slot keys are the sign pattern of the block's mean query direction u_m.
        origin, align, lag = cfg.n_sink, cfg.chunk[0], cfg.n_window
        nblk = cfg.t // cfg.block_q
        for b in range(B):
            owned = np.zeros(eligible_slots(origin, align, cfg.t), dtype=bool)
            for m in range(nblk):
                ns = eligible_slots(origin, align, (m + 1) * cfg.block_q - lag)
                free = np.flatnonzero(~owned[:ns])
                if free.size == 0:
                    continue
                take = rng.choice(free, size=min(4, free.size), replace=False)
                owned[take] = True
                starts = sorted(int(origin + align * j) for j in take)
                planted[(b, m)] = starts
                for h in range(Hq):
                    g = h * Hkv // Hq
                    sgn = _sign_codes(u[b, h, m].astype(np.int8))
                    for st in starts:
                        k_list[b].data[g, st:st + align, :] = sgn
        case.planted = planted
    elif cfg.structure == "local":
        # Every key points along the summed queries of its own position in its
        # kv group: each query's largest logit is its own position, the local
        # structure of attention heads (a strong diagonal).
        for b in range(B):
            for g in range(Hkv):
                qs = q.data[b, g * (Hq // Hkv):(g + 1) * (Hq // Hkv)].astype(np.int32).sum(axis=0)
                k_list[b].data[g] = _sign_codes(np.sign(qs).astype(np.int8))
    elif cfg.structure == "needles":
        origin, align = cfg.n_sink, cfg.chunk[0]
        lag = cfg.n_window + cfg.block_q
        needles = []
        for _ in range(cfg.n_needles):
            b = int(rng.integers(0, B))
            T = int(seq_lens[b])
            h = int(rng.integers(0, Hq))
            g = h * Hkv // Hq
            if cfg.mode == "prefill":
                # random target query t* in the second half of the sequence,
                # where the middle is long enough to be pruned
                tq = int(rng.integers(max(T // 2, origin + align + lag + cfg.block_q), T))
                ns = eligible_slots(origin, align, (tq // cfg.block_q) * cfg.block_q - lag)
                j = int(rng.integers(0, ns))
                qsrc = qc[b, h, tq]
                qid = tq
            else:
                ns = eligible_slots(origin, align, T - lag)
                j = int(rng.integers(0, ns))
                qsrc = qc[0, b, h]
                qid = 0
            st = origin + align * j
            k_list[b].data[g, st:st + align, :] = _sign_codes(qsrc)
            needles.append(Needle(b, st, align, g, h, qid))
        case.needles = needles

    # ---- paging -------------------------------------------------------------
    if cfg.page_size:
        ps = cfg.page_size
        pages = [-(-int(L) // ps) for L in seq_lens]
        total = int(sum(pages))
        perm = np.random.default_rng([seed, 5]).permutation(total).astype(np.int32)
        maxp = max(pages)
        bt = np.zeros((B, maxp), dtype=np.int32)
        off = 0
        for b in range(B):
            bt[b, :pages[b]] = perm[off:off + pages[b]]
            off += pages[b]
        case.block_table = bt
        case.n_pages = total
    return case


def page_pool(case: Case, which: str) -> np.ndarray:
    """Scatter the per-sequence K codes or V storage into the physical page pool
    [n_pages, Hkv, page_size, d] given by the case's block table (pure data
    movement; unused tail slots of the last page of each sequence are zero)."""
    cfg = case.cfg
    ps = cfg.page_size
    src = case.k if which == "k" else case.v
    dt = src[0].data.dtype
    pool = np.zeros((case.n_pages, cfg.hkv, ps, cfg.d), dtype=dt)
    for b in range(cfg.batch):
        L = int(case.seq_lens[b])
        npg = -(-L // ps)
        data = src[b].data
        for i in range(npg):
            lo, hi = i * ps, min(L, (i + 1) * ps)
            pool[case.block_table[b, i], :, :hi - lo, :] = data[:, lo:hi, :]
    return pool


def sample_blocks(n_blocks: int, count: int, seed: int) -> List[int]:
    """A seeded sample of block indices that always includes the first and last."""
    rng = np.random.default_rng(seed + 1000)
    if n_blocks <= count + 2:
        return list(range(n_blocks))
    pick = set(rng.choice(n_blocks, size=count, replace=False).tolist())
    pick.update({0, n_blocks - 1})
    return sorted(pick)
