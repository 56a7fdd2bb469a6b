"""Move a generated workload (gen.Case) into GPU tensors in the library's layouts.

Pure data movement: integer grid codes become bf16/fp32 values (exact), bf16
bit patterns are reinterpreted, and paged decode scatters each sequence's
pages into the pool at the ids of its block table.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from ._lib import Params
from .gen import Case, Config, Values


def params_of(cfg: Config) -> Params:
    return Params(cfg.block_q, tuple(cfg.chunk), tuple(cfg.keep), cfg.n_sink, cfg.n_window)


def torch_dtype(cfg: Config) -> torch.dtype:
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def values_to_device(v: Values, dtype: torch.dtype, device) -> torch.Tensor:
    if v.kind == "grid":
        t = torch.from_numpy(np.ascontiguousarray(v.data)).to(device)
        return (t.to(torch.float32) * 0.125).to(dtype)
    if v.kind == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(v.data).view(np.int16)).to(device)
        t = t.view(torch.bfloat16)
        return t if dtype == torch.bfloat16 else t.to(dtype)
    return torch.from_numpy(np.ascontiguousarray(v.data)).to(device).to(dtype)


@dataclass
class DeviceCase:
    q: torch.Tensor                     # prefill [B,Hq,T,d]; decode [NQ,B,Hq,d]
    k: torch.Tensor                     # [B,Hkv,t,d] or pool [n_pages,Hkv,ps,d]
    v: torch.Tensor
    seq_lens: Optional[torch.Tensor]    # decode [B] int32
    block_table: Optional[torch.Tensor] # paged decode [B,max_pages] int32
    t: int                              # shape.t: prefill length / decode capacity


def to_device(case: Case, device="cuda") -> DeviceCase:
    cfg = case.cfg
    dt = torch_dtype(cfg)
    q = values_to_device(case.q, dt, device)
    if cfg.mode == "prefill" or cfg.page_size == 0:
        T = int(max(case.seq_lens))
        def padded(x):
            t = values_to_device(x, dt, device)
            return t if t.shape[1] == T else torch.nn.functional.pad(t, (0, 0, 0, T - t.shape[1]))
        k = torch.stack([padded(x) for x in case.k])
        v = torch.stack([padded(x) for x in case.v])
        sl = bt = None
        if cfg.mode == "decode":
            sl = torch.from_numpy(case.seq_lens.astype(np.int32)).to(device)
        return DeviceCase(q, k, v, sl, bt, int(k.shape[2]))
    ps = cfg.page_size
    bt_np = case.block_table
    kpool = torch.zeros((case.n_pages, cfg.hkv, ps, cfg.d), dtype=dt, device=device)
    vpool = torch.zeros_like(kpool)
    for b in range(cfg.batch):
        L = int(case.seq_lens[b])
        npg = -(-L // ps)
        ids = torch.from_numpy(bt_np[b, :npg].astype(np.int64)).to(device)
        for src, pool in ((case.k[b], kpool), (case.v[b], vpool)):
            x = values_to_device(src, dt, device)                     # [Hkv, L, d]
            if npg * ps != L:
                x = torch.nn.functional.pad(x, (0, 0, 0, npg * ps - L))
            pool[ids] = x.view(cfg.hkv, npg, ps, cfg.d).permute(1, 0, 2, 3)
            del x
    sl = torch.from_numpy(case.seq_lens.astype(np.int32)).to(device)
    bt = torch.from_numpy(bt_np.astype(np.int32)).to(device)
    return DeviceCase(q, kpool, vpool, sl, bt, int(bt_np.shape[1]) * ps)
