"""Tensor-level entry points over the C ABI (PyTorch supplies memory and streams).

    idx = prune_select(q, k, params)                    # prefill, or decode with seq_lens=
    out = sparse_attn(q, k, v, idx, params)
    out = dense_attn(q, k, v)

Layouts are those of include/dsa.h. Prefill: q [B,Hq,T,d], k/v [B,Hkv,T,d].
Decode: q [B,Hq,d] with seq_lens [B] (int32, on the GPU) and either contiguous
k/v [B,Hkv,t,d] or page pools [n_pages,Hkv,page_size,d] with block_table
[B,max_pages]. Outputs are float32.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Tuple

import torch

from . import _lib
from ._lib import DSA_BF16, DSA_DECODE, DSA_F32, DSA_PREFILL, Params, Shape

# Workspaces: one per (device, stream), so calls on different streams never
# share scratch memory. A workspace that is too small is replaced by a larger
# one, but the old buffer is kept alive (never returned to the allocator): a
# HIP graph captured earlier may still hold its address. Callers that want
# full control pass their own buffer (ws=, at least workspace_bytes()).
_WS: Dict[Tuple[int, int], torch.Tensor] = {}
_RETIRED: List[torch.Tensor] = []


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DSA_BF16
    if t.dtype == torch.float32:
        return DSA_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _need(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def make_shape(q: torch.Tensor, k: torch.Tensor, *, seq_lens: Optional[torch.Tensor] = None,
               block_table: Optional[torch.Tensor] = None, t: Optional[int] = None) -> Shape:
    """Describe the problem from the tensors (see the module docstring)."""
    _need(q, "q")
    _need(k, "k")
    dt = _dtype_code(q)
    if k.dtype != q.dtype:
        raise TypeError("q and k must share a dtype")
    if seq_lens is None:
        if q.dim() != 4 or k.dim() != 4:
            raise ValueError("prefill expects q [B,Hq,T,d] and k [B,Hkv,T,d]")
        B, Hq, T, d = q.shape
        if k.shape[0] != B or k.shape[2] != T or k.shape[3] != d:
            raise ValueError("k shape does not match q")
        return Shape(DSA_PREFILL, dt, B, Hq, k.shape[1], d, T)
    _need(seq_lens, "seq_lens")
    if seq_lens.dtype != torch.int32:
        raise TypeError("seq_lens must be int32")
    if q.dim() != 3:
        raise ValueError("decode expects q [B,Hq,d]")
    B, Hq, d = q.shape
    if seq_lens.numel() != B:
        raise ValueError("seq_lens must have B entries")
    if block_table is None:
        if k.dim() != 4 or k.shape[0] != B or k.shape[3] != d:
            raise ValueError("contiguous decode expects k [B,Hkv,t,d]")
        return Shape(DSA_DECODE, dt, B, Hq, k.shape[1], d, k.shape[2], seq_lens.data_ptr())
    _need(block_table, "block_table")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [B, max_pages]")
    if k.dim() != 4 or k.shape[3] != d:
        raise ValueError("paged decode expects k [n_pages,Hkv,page_size,d]")
    ps = k.shape[2]
    maxp = block_table.shape[1]
    return Shape(DSA_DECODE, dt, B, Hq, k.shape[1], d, t if t is not None else maxp * ps,
                 seq_lens.data_ptr(), block_table.data_ptr(), ps, maxp)


def workspace_bytes(shape: Shape, params: Optional[Params]) -> int:
    """Bytes of the scratch buffer the calls on this shape need."""
    return _lib.workspace_bytes(shape, params)


def workspace(shape: Shape, params: Optional[Params], device: torch.device,
              ws: Optional[torch.Tensor] = None) -> Tuple[int, int]:
    """Scratch buffer for one call: the caller's `ws`, else the workspace of
    (device, current stream), grown on demand."""
    return _scratch(_lib.workspace_bytes(shape, params), device, ws)


def _scratch(nbytes: int, device: torch.device, ws: Optional[torch.Tensor] = None) -> Tuple[int, int]:
    if ws is not None:
        if not ws.is_cuda or not ws.is_contiguous():
            raise ValueError("ws must be a contiguous GPU tensor")
        size = ws.numel() * ws.element_size()
        if size < nbytes:
            raise ValueError(f"ws holds {size} bytes; this call needs {nbytes}")
        return ws.data_ptr(), size
    dev = device.index if device.index is not None else torch.cuda.current_device()
    key = (dev, torch.cuda.current_stream(dev).cuda_stream)
    buf = _WS.get(key)
    if buf is None or buf.numel() < nbytes:
        if buf is not None:
            _RETIRED.append(buf)
        grow = 0 if buf is None else 2 * buf.numel()
        buf = torch.empty(max(nbytes, grow, 256), dtype=torch.uint8, device=device)
        _WS[key] = buf
    return buf.data_ptr(), buf.numel()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def prune_select(q: torch.Tensor, k: torch.Tensor, params: Params, *,
                 seq_lens: Optional[torch.Tensor] = None, block_table: Optional[torch.Tensor] = None,
                 t: Optional[int] = None, out: Optional[torch.Tensor] = None,
                 visited: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    shape = make_shape(q, k, seq_lens=seq_lens, block_table=block_table, t=t)
    L = _lib.index_width(params)
    if L < 0:
        raise _lib.DsaError(_lib.DSA_ERR_INVALID_ARG, "invalid params")
    rows = shape.batch * (1 if shape.mode == DSA_DECODE else shape.t // params.block_q)
    if out is None:
        out = torch.empty(rows * L, dtype=torch.int32, device=q.device)
    if out.numel() != rows * L or out.dtype != torch.int32:
        raise ValueError("idx buffer has the wrong size or dtype")
    wsp, wsb = workspace(shape, params, q.device, ws)
    vis = 0
    if visited is not None:
        if visited.dtype != torch.int64 or visited.numel() < len(params.chunk):
            raise ValueError("visited must be int64 with one entry per stage")
        vis = visited.data_ptr()
    _lib.prune_select_raw(shape, q.data_ptr(), k.data_ptr(), params, out.data_ptr(), wsp, wsb, vis, _stream())
    if shape.mode == DSA_DECODE:
        return out.view(shape.batch, L)
    return out.view(shape.batch, shape.t // params.block_q, L)


def prune_attend(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, params: Params, *, scale: float = 0.0,
                 seq_lens: Optional[torch.Tensor] = None, block_table: Optional[torch.Tensor] = None,
                 t: Optional[int] = None, idx: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                 visited: Optional[torch.Tensor] = None,
                 ws: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """prune_select followed by sparse_attn in one call: (idx, out)."""
    shape = make_shape(q, k, seq_lens=seq_lens, block_table=block_table, t=t)
    _need(v, "v")
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("v must match k")
    L = _lib.index_width(params)
    if L < 0:
        raise _lib.DsaError(_lib.DSA_ERR_INVALID_ARG, "invalid params")
    rows = shape.batch * (1 if shape.mode == DSA_DECODE else shape.t // params.block_q)
    if idx is None:
        idx = torch.empty(rows * L, dtype=torch.int32, device=q.device)
    if idx.numel() != rows * L or idx.dtype != torch.int32:
        raise ValueError("idx buffer has the wrong size or dtype")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    wsp, wsb = workspace(shape, params, q.device, ws)
    vis = 0
    if visited is not None:
        if visited.dtype != torch.int64 or visited.numel() < len(params.chunk):
            raise ValueError("visited must be int64 with one entry per stage")
        vis = visited.data_ptr()
    _lib.prune_attend_raw(shape, q.data_ptr(), k.data_ptr(), v.data_ptr(), params, scale, idx.data_ptr(),
                          out.data_ptr(), wsp, wsb, vis, _stream())
    if shape.mode == DSA_DECODE:
        return idx.view(shape.batch, L), out
    return idx.view(shape.batch, shape.t // params.block_q, L), out


def check_decode_inputs(q: torch.Tensor, k: torch.Tensor, *, seq_lens: torch.Tensor,
                        block_table: Optional[torch.Tensor] = None, t: Optional[int] = None) -> None:
    """Checked mode: copies seq_lens and the block table to the host (this
    synchronises with their producers) and validates every length and every
    page id a length reaches against the K pool; raises DsaError naming the
    first bad entry."""
    shape = make_shape(q, k, seq_lens=seq_lens, block_table=block_table, t=t)
    n_pages = k.shape[0] if block_table is not None else 0
    _lib.check_decode_inputs(shape, seq_lens.cpu().numpy(),
                             block_table.cpu().numpy() if block_table is not None else None, n_pages)


class MaskCache:
    """Remembered stage outputs of one stream of decode steps (mask caching).

    Holds the device buffer the library reads and writes, the refresh
    intervals and the row width; `status` views the per-sequence overflow flags.
    Allocate it for the largest context the stream will reach (`t`).
    """

    def __init__(self, q: torch.Tensor, k: torch.Tensor, params: Params, refresh, *,
                 seq_lens: torch.Tensor, block_table: Optional[torch.Tensor] = None,
                 t: Optional[int] = None, max_growth: Optional[int] = None):
        if len(refresh) != len(params.chunk):
            raise ValueError("one refresh interval per stage")
        shape = make_shape(q, k, seq_lens=seq_lens, block_table=block_table, t=t)
        self.params = params
        self.refresh = tuple(int(x) for x in refresh)
        self.batch = shape.batch
        growth = self.refresh[0] - 1 if max_growth is None else max_growth
        self.width = _lib.cached_index_width(params, growth)
        if self.width < 0:
            raise _lib.DsaError(_lib.DSA_ERR_INVALID_ARG, "invalid params or growth")
        self.buf = torch.zeros(_lib.mask_cache_bytes(shape, params), dtype=torch.uint8, device=q.device)

    @property
    def status(self) -> torch.Tensor:
        return self.buf[: 4 * self.batch].view(torch.int32)


def prune_select_cached(q: torch.Tensor, k: torch.Tensor, cache: MaskCache, step: int, *,
                        seq_lens: torch.Tensor, block_table: Optional[torch.Tensor] = None,
                        t: Optional[int] = None, out: Optional[torch.Tensor] = None,
                        visited: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One decode step of pruning with remembered stages: [B, cache.width] rows."""
    shape = make_shape(q, k, seq_lens=seq_lens, block_table=block_table, t=t)
    params = cache.params
    L = cache.width
    if out is None:
        out = torch.empty(shape.batch * L, dtype=torch.int32, device=q.device)
    if out.numel() != shape.batch * L or out.dtype != torch.int32:
        raise ValueError("idx buffer has the wrong size or dtype")
    wsp, wsb = workspace(shape, params, q.device, ws)
    vis = 0
    if visited is not None:
        if visited.dtype != torch.int64 or visited.numel() < len(params.chunk):
            raise ValueError("visited must be int64 with one entry per stage")
        vis = visited.data_ptr()
    _lib.prune_select_cached_raw(shape, q.data_ptr(), k.data_ptr(), params, cache.refresh, step,
                                 cache.buf.data_ptr(), cache.buf.numel(), out.data_ptr(), L, wsp, wsb, vis,
                                 _stream())
    return out.view(shape.batch, L)


def sparse_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor, params: Params, *,
                scale: float = 0.0, seq_lens: Optional[torch.Tensor] = None,
                block_table: Optional[torch.Tensor] = None, t: Optional[int] = None,
                out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Attention over the index rows written by prune_select with the same params."""
    shape = make_shape(q, k, seq_lens=seq_lens, block_table=block_table, t=t)
    _need(v, "v")
    _need(idx, "idx")
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("v must match k")
    if idx.dtype != torch.int32:
        raise TypeError("idx must be int32")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    wsp, wsb = workspace(shape, params, q.device, ws)
    _lib.sparse_attn_raw(shape, q.data_ptr(), k.data_ptr(), v.data_ptr(), idx.data_ptr(), idx.shape[-1],
                         params.block_q, scale, out.data_ptr(), wsp, wsb, _stream())
    return out


def dense_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, scale: float = 0.0,
               seq_lens: Optional[torch.Tensor] = None, block_table: Optional[torch.Tensor] = None,
               t: Optional[int] = None, out: Optional[torch.Tensor] = None,
               ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    shape = make_shape(q, k, seq_lens=seq_lens, block_table=block_table, t=t)
    _need(v, "v")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    wsp, wsb = workspace(shape, None, q.device, ws)
    _lib.dense_attn_raw(shape, q.data_ptr(), k.data_ptr(), v.data_ptr(), scale, out.data_ptr(), wsp, wsb,
                        _stream())
    return out


# --------------------------------------------------------------------------- #
# block-sparse heads                                                          #
# --------------------------------------------------------------------------- #
def block_sparse_select(q: torch.Tensor, k: torch.Tensor, k_blocks: int, *,
                        out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-head block index estimation (prefill): [B, Hq, T/64, 64*k_blocks] rows."""
    shape = make_shape(q, k)
    if shape.mode != DSA_PREFILL:
        raise ValueError("block-sparse estimation is a prefill call")
    L = _lib.block_sparse_index_width(k_blocks)
    nblk = shape.t // 64
    n = shape.batch * shape.hq * nblk * L
    if out is None:
        out = torch.empty(n, dtype=torch.int32, device=q.device)
    if out.numel() != n or out.dtype != torch.int32 or not out.is_contiguous():
        raise ValueError("idx buffer has the wrong size, dtype or layout")
    wsp, wsb = _scratch(_lib.block_sparse_workspace_bytes(shape, k_blocks), q.device, ws)
    _lib.block_sparse_select_raw(shape, q.data_ptr(), k.data_ptr(), k_blocks, out.data_ptr(), wsp, wsb, _stream())
    return out.view(shape.batch, shape.hq, nblk, L)


def sparse_attn_heads(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor, *,
                      scale: float = 0.0, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Prefill attention over per-head index rows idx [B, Hq, T/64, L]."""
    shape = make_shape(q, k)
    _need(v, "v")
    _need(idx, "idx")
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("v must match k")
    if idx.dtype != torch.int32:
        raise TypeError("idx must be int32")
    if tuple(idx.shape[:3]) != (shape.batch, shape.hq, shape.t // 64):
        raise ValueError("idx must be [B, Hq, T/64, L]")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    _lib.sparse_attn_heads_raw(shape, q.data_ptr(), k.data_ptr(), v.data_ptr(), idx.data_ptr(), idx.shape[-1],
                               scale, out.data_ptr(), _stream())
    return out


def _out_i32(t: Optional[torch.Tensor], shape, device, name: str) -> torch.Tensor:
    """A caller's int32 output buffer of this shape, or a new one."""
    if t is None:
        return torch.empty(shape, dtype=torch.int32, device=device)
    if tuple(t.shape) != tuple(shape) or t.dtype != torch.int32 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 tensor of shape {tuple(shape)}")
    return t


def block_sparse_select_lists(q: torch.Tensor, k: torch.Tensor, k_blocks: int, *,
                              blocks: Optional[torch.Tensor] = None, counts: Optional[torch.Tensor] = None,
                              ws: Optional[torch.Tensor] = None):
    """Per-head block index estimation (prefill) as block lists: (blocks
    [B, Hq, T/64, wb] ascending ids then -1, counts [B, Hq, T/64, 2])."""
    shape = make_shape(q, k)
    if shape.mode != DSA_PREFILL:
        raise ValueError("block-sparse estimation is a prefill call")
    wb = _lib.block_sparse_list_width(k_blocks)
    nblk = shape.t // 64
    blocks = _out_i32(blocks, (shape.batch, shape.hq, nblk, wb), q.device, "blocks")
    counts = _out_i32(counts, (shape.batch, shape.hq, nblk, 2), q.device, "counts")
    wsp, wsb = _scratch(_lib.block_sparse_workspace_bytes(shape, k_blocks), q.device, ws)
    _lib.block_sparse_select_lists_raw(shape, q.data_ptr(), k.data_ptr(), k_blocks, blocks.data_ptr(),
                                       counts.data_ptr(), wsp, wsb, _stream())
    return blocks, counts


def sparse_attn_lists(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, blocks: torch.Tensor,
                      counts: torch.Tensor, cols: Optional[torch.Tensor] = None, *, scale: float = 0.0,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Prefill attention over per-head block lists [B, Hq, T/64, wb] and
    (optionally) column lists [B, Hq, T/64, wc], counts [B, Hq, T/64, 2]."""
    shape = make_shape(q, k)
    _need(v, "v")
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("v must match k")
    lead = (shape.batch, shape.hq, shape.t // 64)
    for name, x in (("blocks", blocks), ("counts", counts)) + ((("cols", cols),) if cols is not None else ()):
        _need(x, name)
        if x.dtype != torch.int32 or tuple(x.shape[:3]) != lead:
            raise ValueError(f"{name} must be int32 [B, Hq, T/64, ...]")
    if counts.shape[-1] != 2:
        raise ValueError("counts must be [B, Hq, T/64, 2]")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    _lib.sparse_attn_lists_raw(shape, q.data_ptr(), k.data_ptr(), v.data_ptr(), blocks.data_ptr(), blocks.shape[-1],
                               cols.data_ptr() if cols is not None else 0, cols.shape[-1] if cols is not None else 0,
                               counts.data_ptr(), scale, out.data_ptr(), _stream())
    return out


# --------------------------------------------------------------------------- #
# vertical-slash heads                                                        #
# --------------------------------------------------------------------------- #
def vertical_slash_select(q: torch.Tensor, k: torch.Tensor, k_v: int, k_s: int, *,
                          out: Optional[torch.Tensor] = None, return_lines: bool = False,
                          ws: Optional[torch.Tensor] = None):
    """Per-head vertical-slash index estimation (prefill, bf16): rows
    [B, Hq, T/64, L]; with return_lines also the kept columns [B, Hq, k_v] and
    offsets [B, Hq, k_s]."""
    shape = make_shape(q, k)
    if shape.mode != DSA_PREFILL:
        raise ValueError("vertical-slash estimation is a prefill call")
    L = _lib.vertical_slash_index_width(shape.t, k_v, k_s)
    nblk = shape.t // 64
    n = shape.batch * shape.hq * nblk * L
    if out is None:
        out = torch.empty(n, dtype=torch.int32, device=q.device)
    if out.numel() != n or out.dtype != torch.int32 or not out.is_contiguous():
        raise ValueError("idx buffer has the wrong size, dtype or layout")
    cols = torch.empty((shape.batch, shape.hq, max(k_v, 1)), dtype=torch.int32, device=q.device) if return_lines else None
    offs = torch.empty((shape.batch, shape.hq, k_s), dtype=torch.int32, device=q.device) if return_lines else None
    wsp, wsb = _scratch(_lib.vertical_slash_workspace_bytes(shape, k_v, k_s), q.device, ws)
    _lib.vertical_slash_select_raw(shape, q.data_ptr(), k.data_ptr(), k_v, k_s, out.data_ptr(),
                                   cols.data_ptr() if cols is not None else 0,
                                   offs.data_ptr() if offs is not None else 0, wsp, wsb, _stream())
    idx = out.view(shape.batch, shape.hq, nblk, L)
    if return_lines:
        return idx, cols[..., :k_v], offs
    return idx


def vertical_slash_select_lists(q: torch.Tensor, k: torch.Tensor, k_v: int, k_s: int, *,
                                blocks: Optional[torch.Tensor] = None, cols: Optional[torch.Tensor] = None,
                                counts: Optional[torch.Tensor] = None, return_lines: bool = False,
                                ws: Optional[torch.Tensor] = None):
    """Per-head vertical-slash index estimation (prefill, bf16) as the hybrid
    kernel's lists: (blocks [B, Hq, T/64, wb], cols [B, Hq, T/64, wc], counts
    [B, Hq, T/64, 2]); with return_lines also the kept columns and offsets."""
    shape = make_shape(q, k)
    if shape.mode != DSA_PREFILL:
        raise ValueError("vertical-slash estimation is a prefill call")
    wb, wc = _lib.vertical_slash_list_widths(shape.t, k_v, k_s)
    lead = (shape.batch, shape.hq, shape.t // 64)
    blocks = _out_i32(blocks, lead + (wb,), q.device, "blocks")
    cols = _out_i32(cols, lead + (wc,), q.device, "cols")
    counts = _out_i32(counts, lead + (2,), q.device, "counts")
    kc = torch.empty((shape.batch, shape.hq, max(k_v, 1)), dtype=torch.int32, device=q.device) if return_lines else None
    ko = torch.empty((shape.batch, shape.hq, k_s), dtype=torch.int32, device=q.device) if return_lines else None
    wsp, wsb = _scratch(_lib.vertical_slash_workspace_bytes(shape, k_v, k_s), q.device, ws)
    _lib.vertical_slash_select_lists_raw(shape, q.data_ptr(), k.data_ptr(), k_v, k_s, blocks.data_ptr(),
                                         cols.data_ptr(), counts.data_ptr(), kc.data_ptr() if kc is not None else 0,
                                         ko.data_ptr() if ko is not None else 0, wsp, wsb, _stream())
    if return_lines:
        return blocks, cols, counts, kc[..., :k_v], ko
    return blocks, cols, counts


# --------------------------------------------------------------------------- #
# pruning with RoPE inside SelectRep (relative or chunk-indexed)              #
# --------------------------------------------------------------------------- #
def rope_style_for_layer(layer: int, n_chunk_indexed: int = 3) -> str:
    """RoPE style of a model layer (1-based) under the InfiniteHiP page's
    layer-specific assignment ("Layer-Specific Strategy Assignment"): the
    chunk-indexed style for the first three layers, the relative style for
    the rest."""
    if layer < 1:
        raise ValueError(f"layer {layer}: layers are numbered from 1")
    return "chunk_indexed" if layer <= n_chunk_indexed else "relative"


def rope_key_copies(k: torch.Tensor, params: Params) -> list:
    """Buffers for the chunk-indexed rotated keys: one bf16 tensor shaped like
    k per stage (filled by rope_rotate_keys)."""
    return [torch.empty(k.shape, dtype=torch.bfloat16, device=k.device) for _ in range(len(params.chunk))]


def rope_rotate_keys(k: torch.Tensor, params: Params, base: float, k_rot: list, *, pos_begin: int = 0,
                     pos_end: Optional[int] = None, seq_lens: Optional[torch.Tensor] = None,
                     t: Optional[int] = None) -> list:
    """Chunk-indexed RoPE: write every stage's rotated rows of the keys at
    positions [pos_begin, pos_end) into k_rot (decode layout, contiguous k)."""
    if seq_lens is None:
        raise ValueError("rope_rotate_keys is a decode call: pass seq_lens")
    if len(k_rot) != len(params.chunk):
        raise ValueError("one rotated key buffer per stage")
    for x in k_rot:
        if x.shape != k.shape or x.dtype != torch.bfloat16 or not x.is_contiguous():
            raise ValueError("rotated key buffers are contiguous bf16 tensors shaped like k")
    q_dummy = torch.empty((k.shape[0], k.shape[1], k.shape[3]), dtype=k.dtype, device=k.device)
    shape = make_shape(q_dummy, k, seq_lens=seq_lens, t=t)
    end = shape.t if pos_end is None else pos_end
    _lib.rope_rotate_keys_raw(shape, k.data_ptr(), params, base, pos_begin, end, [x.data_ptr() for x in k_rot],
                              _stream())
    return k_rot


def prune_select_rope_keys(q: torch.Tensor, k_rot: list, params: Params, base: float, *,
                           seq_lens: torch.Tensor, t: Optional[int] = None, out: Optional[torch.Tensor] = None,
                           ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Chunk-indexed decode pruning over the rotated key copies of
    rope_rotate_keys; idx as prune_select_rope(style="chunk_indexed")."""
    if len(k_rot) != len(params.chunk):
        raise ValueError("one rotated key buffer per stage")
    _need(q, "q")
    _need(seq_lens, "seq_lens")
    if q.dim() != 3 or seq_lens.dtype != torch.int32 or seq_lens.numel() != q.shape[0]:
        raise ValueError("decode expects q [B,Hq,d] and int32 seq_lens [B]")
    kr = k_rot[0]
    if kr.dim() != 4 or kr.shape[0] != q.shape[0] or kr.shape[3] != q.shape[2]:
        raise ValueError("rotated key buffers must be [B,Hkv,t,d]")
    # q's dtype describes the call; the rotated keys are bf16 either way
    shape = Shape(DSA_DECODE, _dtype_code(q), q.shape[0], q.shape[1], kr.shape[1], q.shape[2],
                  kr.shape[2] if t is None else t, seq_lens.data_ptr())
    L = _lib.index_width(params)
    if L < 0:
        raise _lib.DsaError(_lib.DSA_ERR_INVALID_ARG, "invalid params")
    if out is None:
        out = torch.empty(shape.batch * L, dtype=torch.int32, device=q.device)
    if out.numel() != shape.batch * L or out.dtype != torch.int32:
        raise ValueError("idx buffer has the wrong size or dtype")
    wsp, wsb = _scratch(_lib.prune_rope_workspace_bytes(shape, params, _lib.DSA_ROPE_CHUNK_INDEXED, base), q.device, ws)
    _lib.prune_select_rope_keys_raw(shape, q.data_ptr(), [x.data_ptr() for x in k_rot], params, base, out.data_ptr(),
                                    wsp, wsb, _stream())
    return out.view(shape.batch, L)


def prune_select_rope(q: torch.Tensor, k: torch.Tensor, params: Params, base: float, *,
                      seq_lens: Optional[torch.Tensor] = None, block_table: Optional[torch.Tensor] = None,
                      t: Optional[int] = None, out: Optional[torch.Tensor] = None,
                      style: str = "relative", ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """prune_select with RoPE inside SelectRep (q, k taken before any rotary
    embedding); style "relative" or "chunk_indexed"."""
    styles = {"relative": _lib.DSA_ROPE_RELATIVE, "chunk_indexed": _lib.DSA_ROPE_CHUNK_INDEXED}
    if style not in styles:
        raise ValueError(f"rope style {style!r}; expected one of {sorted(styles)}")
    shape = make_shape(q, k, seq_lens=seq_lens, block_table=block_table, t=t)
    L = _lib.index_width(params)
    if L < 0:
        raise _lib.DsaError(_lib.DSA_ERR_INVALID_ARG, "invalid params")
    rows = shape.batch * (1 if shape.mode == DSA_DECODE else shape.t // params.block_q)
    if out is None:
        out = torch.empty(rows * L, dtype=torch.int32, device=q.device)
    if out.numel() != rows * L or out.dtype != torch.int32:
        raise ValueError("idx buffer has the wrong size or dtype")
    wsp, wsb = _scratch(_lib.prune_rope_workspace_bytes(shape, params, styles[style], base), q.device, ws)
    _lib.prune_select_rope_raw(shape, q.data_ptr(), k.data_ptr(), params, base, out.data_ptr(), wsp, wsb, _stream(),
                               style=styles[style])
    if shape.mode == DSA_DECODE:
        return out.view(shape.batch, L)
    return out.view(shape.batch, shape.t // params.block_q, L)

