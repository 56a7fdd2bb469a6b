"""ctypes binding of libdsa (include/dsa.h): argument marshalling only.

Every computation runs in the HIP library. PyTorch supplies device memory and
streams; tensors are passed as raw device pointers. If libdsa.so has not been
built, importing the binding raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdsa.so")

DSA_OK, DSA_ERR_INVALID_ARG, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE, DSA_ERR_HIP = range(5)
DSA_F32, DSA_BF16 = 0, 1
DSA_PREFILL, DSA_DECODE = 0, 1
MAX_STAGES = 4

EXPORTS = ("dsa_index_width", "dsa_workspace_bytes", "dsa_prune_select", "dsa_sparse_attn", "dsa_prune_attend",
           "dsa_prune_attend_static",
           "dsa_dense_attn", "dsa_mask_cache_bytes", "dsa_cached_index_width", "dsa_prune_select_cached",
           "dsa_block_sparse_index_width", "dsa_block_sparse_workspace_bytes", "dsa_block_sparse_select",
           "dsa_sparse_attn_heads", "dsa_vertical_slash_index_width", "dsa_vertical_slash_workspace_bytes",
           "dsa_vertical_slash_select", "dsa_prune_rope_workspace_bytes", "dsa_prune_select_rope",
           "dsa_rope_rotate_keys", "dsa_prune_select_rope_keys",
           "dsa_block_sparse_list_width", "dsa_block_sparse_select_lists", "dsa_sparse_attn_lists",
           "dsa_vertical_slash_list_widths", "dsa_vertical_slash_select_lists",
           "dsa_check_decode_inputs", "dsa_profile_begin", "dsa_profile_end", "dsa_status_str", "dsa_last_error")


class CParams(ctypes.Structure):
    _fields_ = [("n_stages", ctypes.c_int32), ("block_q", ctypes.c_int32),
                ("chunk", ctypes.c_int32 * MAX_STAGES), ("keep", ctypes.c_int32 * MAX_STAGES),
                ("n_sink", ctypes.c_int32), ("n_window", ctypes.c_int32)]


class CShape(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("batch", ctypes.c_int32), ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("t", ctypes.c_int32),
                ("seq_lens", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("page_size", ctypes.c_int32), ("max_pages", ctypes.c_int32)]


class CRope(ctypes.Structure):
    _fields_ = [("style", ctypes.c_int32), ("base", ctypes.c_double)]


DSA_ROPE_RELATIVE = 1
DSA_ROPE_CHUNK_INDEXED = 2


class CKernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double)]


class DsaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{status_str(status)}: {msg}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdsa.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m dynamic_sparse_attention_query_amd.build`")
    lib = ctypes.CDLL(path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.dsa_index_width.argtypes = [ctypes.POINTER(CParams)]
    lib.dsa_index_width.restype = ctypes.c_int32
    lib.dsa_workspace_bytes.argtypes = [ctypes.POINTER(CShape), ctypes.POINTER(CParams), ctypes.POINTER(sz)]
    lib.dsa_workspace_bytes.restype = ctypes.c_int
    lib.dsa_prune_select.argtypes = [ctypes.POINTER(CShape), vp, vp, ctypes.POINTER(CParams), vp, vp, sz, vp, vp]
    lib.dsa_prune_attend.argtypes = [ctypes.POINTER(CShape), vp, vp, vp, ctypes.POINTER(CParams), ctypes.c_float,
                                     vp, vp, vp, sz, vp, vp]
    lib.dsa_prune_attend.restype = ctypes.c_int
    lib.dsa_prune_attend_static.argtypes = [ctypes.POINTER(CShape), vp, vp, vp, ctypes.POINTER(CParams),
                                            ctypes.c_float, vp, vp, vp, vp]
    lib.dsa_prune_attend_static.restype = ctypes.c_int
    lib.dsa_check_decode_inputs.argtypes = [ctypes.POINTER(CShape), vp, vp, ctypes.c_int64]
    lib.dsa_check_decode_inputs.restype = ctypes.c_int
    lib.dsa_prune_select.restype = ctypes.c_int
    lib.dsa_mask_cache_bytes.argtypes = [ctypes.POINTER(CShape), ctypes.POINTER(CParams), ctypes.POINTER(sz)]
    lib.dsa_mask_cache_bytes.restype = ctypes.c_int
    lib.dsa_cached_index_width.argtypes = [ctypes.POINTER(CParams), ctypes.c_int32]
    lib.dsa_cached_index_width.restype = ctypes.c_int32
    lib.dsa_prune_select_cached.argtypes = [ctypes.POINTER(CShape), vp, vp, ctypes.POINTER(CParams),
                                            ctypes.POINTER(ctypes.c_int32), ctypes.c_int64, vp, sz, vp,
                                            ctypes.c_int32, vp, sz, vp, vp]
    lib.dsa_prune_select_cached.restype = ctypes.c_int
    lib.dsa_sparse_attn.argtypes = [ctypes.POINTER(CShape), vp, vp, vp, vp, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_float, vp, vp, sz, vp]
    lib.dsa_sparse_attn.restype = ctypes.c_int
    lib.dsa_dense_attn.argtypes = [ctypes.POINTER(CShape), vp, vp, vp, ctypes.c_float, vp, vp, sz, vp]
    lib.dsa_dense_attn.restype = ctypes.c_int
    lib.dsa_block_sparse_index_width.argtypes = [ctypes.c_int32]
    lib.dsa_block_sparse_index_width.restype = ctypes.c_int32
    lib.dsa_block_sparse_workspace_bytes.argtypes = [ctypes.POINTER(CShape), ctypes.c_int32, ctypes.POINTER(sz)]
    lib.dsa_block_sparse_workspace_bytes.restype = ctypes.c_int
    lib.dsa_block_sparse_select.argtypes = [ctypes.POINTER(CShape), vp, vp, ctypes.c_int32, vp, vp, sz, vp]
    lib.dsa_block_sparse_select.restype = ctypes.c_int
    lib.dsa_sparse_attn_heads.argtypes = [ctypes.POINTER(CShape), vp, vp, vp, vp, ctypes.c_int32, ctypes.c_float,
                                          vp, vp]
    lib.dsa_sparse_attn_heads.restype = ctypes.c_int
    lib.dsa_vertical_slash_index_width.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    lib.dsa_vertical_slash_index_width.restype = ctypes.c_int32
    lib.dsa_vertical_slash_workspace_bytes.argtypes = [ctypes.POINTER(CShape), ctypes.c_int32, ctypes.c_int32,
                                                       ctypes.POINTER(sz)]
    lib.dsa_vertical_slash_workspace_bytes.restype = ctypes.c_int
    lib.dsa_vertical_slash_select.argtypes = [ctypes.POINTER(CShape), vp, vp, ctypes.c_int32, ctypes.c_int32, vp, vp,
                                              vp, vp, sz, vp]
    lib.dsa_vertical_slash_select.restype = ctypes.c_int
    lib.dsa_block_sparse_list_width.argtypes = [ctypes.c_int32]
    lib.dsa_block_sparse_list_width.restype = ctypes.c_int32
    lib.dsa_block_sparse_select_lists.argtypes = [ctypes.POINTER(CShape), vp, vp, ctypes.c_int32, vp, vp, vp, sz, vp]
    lib.dsa_block_sparse_select_lists.restype = ctypes.c_int
    lib.dsa_sparse_attn_lists.argtypes = [ctypes.POINTER(CShape), vp, vp, vp, vp, ctypes.c_int32, vp, ctypes.c_int32,
                                          vp, ctypes.c_float, vp, vp]
    lib.dsa_sparse_attn_lists.restype = ctypes.c_int
    lib.dsa_vertical_slash_list_widths.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                   ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
    lib.dsa_vertical_slash_list_widths.restype = ctypes.c_int
    lib.dsa_vertical_slash_select_lists.argtypes = [ctypes.POINTER(CShape), vp, vp, ctypes.c_int32, ctypes.c_int32,
                                                    vp, vp, vp, vp, vp, vp, sz, vp]
    lib.dsa_vertical_slash_select_lists.restype = ctypes.c_int
    lib.dsa_prune_rope_workspace_bytes.argtypes = [ctypes.POINTER(CShape), ctypes.POINTER(CParams),
                                                   ctypes.POINTER(CRope), ctypes.POINTER(sz)]
    lib.dsa_prune_rope_workspace_bytes.restype = ctypes.c_int
    lib.dsa_prune_select_rope.argtypes = [ctypes.POINTER(CShape), vp, vp, ctypes.POINTER(CParams),
                                          ctypes.POINTER(CRope), vp, vp, sz, vp]
    lib.dsa_prune_select_rope.restype = ctypes.c_int
    lib.dsa_rope_rotate_keys.argtypes = [ctypes.POINTER(CShape), vp, ctypes.POINTER(CParams), ctypes.POINTER(CRope),
                                         ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(vp), vp]
    lib.dsa_rope_rotate_keys.restype = ctypes.c_int
    lib.dsa_prune_select_rope_keys.argtypes = [ctypes.POINTER(CShape), vp, ctypes.POINTER(vp), ctypes.POINTER(CParams),
                                               ctypes.POINTER(CRope), vp, vp, sz, vp]
    lib.dsa_prune_select_rope_keys.restype = ctypes.c_int
    lib.dsa_profile_begin.argtypes = []
    lib.dsa_profile_begin.restype = ctypes.c_int
    lib.dsa_profile_end.argtypes = [ctypes.POINTER(CKernelTime), ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]
    lib.dsa_profile_end.restype = ctypes.c_int
    lib.dsa_status_str.argtypes = [ctypes.c_int]
    lib.dsa_status_str.restype = ctypes.c_char_p
    lib.dsa_last_error.argtypes = []
    lib.dsa_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_str(st: int) -> str:
    return load().dsa_status_str(st).decode()


def _check(st: int):
    if st != DSA_OK:
        raise DsaError(st, load().dsa_last_error().decode())


# --------------------------------------------------------------------------- #
# parameter / shape records                                                   #
# --------------------------------------------------------------------------- #
@dataclass(frozen=True)
class Params:
    block_q: int
    chunk: Sequence[int]
    keep: Sequence[int]
    n_sink: int
    n_window: int

    def c(self) -> CParams:
        p = CParams()
        p.n_stages = len(self.chunk)
        p.block_q = self.block_q
        for i in range(MAX_STAGES):
            p.chunk[i] = self.chunk[i] if i < len(self.chunk) else 0
            p.keep[i] = self.keep[i] if i < len(self.keep) else 0
        p.n_sink = self.n_sink
        p.n_window = self.n_window
        return p


@dataclass
class Shape:
    mode: int
    dtype: int
    batch: int
    hq: int
    hkv: int
    d: int
    t: int
    seq_lens: int = 0          # device pointer
    block_table: int = 0       # device pointer
    page_size: int = 0
    max_pages: int = 0

    def c(self) -> CShape:
        s = CShape()
        s.mode, s.dtype = self.mode, self.dtype
        s.batch, s.hq, s.hkv, s.d, s.t = self.batch, self.hq, self.hkv, self.d, self.t
        s.seq_lens = self.seq_lens or None
        s.block_table = self.block_table or None
        s.page_size, s.max_pages = self.page_size, self.max_pages
        return s


# --------------------------------------------------------------------------- #
# raw entry points (pointers in, status checked)                              #
# --------------------------------------------------------------------------- #
def index_width(p: Params) -> int:
    cp = p.c()
    return load().dsa_index_width(ctypes.byref(cp))


def workspace_bytes(shape: Shape, p: Optional[Params]) -> int:
    cs = shape.c()
    cp = p.c() if p is not None else None
    out = ctypes.c_size_t(0)
    _check(load().dsa_workspace_bytes(ctypes.byref(cs), ctypes.byref(cp) if cp is not None else None,
                                      ctypes.byref(out)))
    return out.value


def prune_select_raw(shape: Shape, q: int, k: int, p: Params, idx: int, ws: int, ws_bytes: int,
                     visited: int = 0, stream: int = 0):
    cs, cp = shape.c(), p.c()
    _check(load().dsa_prune_select(ctypes.byref(cs), q, k, ctypes.byref(cp), idx, ws, ws_bytes,
                                   visited or None, stream or None))


def prune_attend_raw(shape: Shape, q: int, k: int, v: int, p: Params, scale: float, idx: int, out: int,
                     ws: int, ws_bytes: int, visited: int = 0, stream: int = 0):
    cs, cp = shape.c(), p.c()
    _check(load().dsa_prune_attend(ctypes.byref(cs), q, k, v, ctypes.byref(cp), scale, idx, out, ws, ws_bytes,
                                   visited or None, stream or None))


def check_decode_inputs(shape: Shape, seq_lens, block_table=None, n_pages: int = 0):
    """Checked mode: validate host copies of seq_lens (int32 [B]) and the
    block table (int32 [B, max_pages]); raises DsaError on the first bad entry."""
    import numpy as np
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    bt = None if block_table is None else np.ascontiguousarray(block_table, dtype=np.int32)
    cs = shape.c()
    _check(load().dsa_check_decode_inputs(ctypes.byref(cs), sl.ctypes.data,
                                          bt.ctypes.data if bt is not None else None, int(n_pages)))


def mask_cache_bytes(shape: Shape, p: Params) -> int:
    cs, cp = shape.c(), p.c()
    out = ctypes.c_size_t(0)
    _check(load().dsa_mask_cache_bytes(ctypes.byref(cs), ctypes.byref(cp), ctypes.byref(out)))
    return out.value


def cached_index_width(p: Params, max_growth: int) -> int:
    cp = p.c()
    return load().dsa_cached_index_width(ctypes.byref(cp), max_growth)


def prune_select_cached_raw(shape: Shape, q: int, k: int, p: Params, refresh: Sequence[int], step: int,
                            cache: int, cache_bytes: int, idx: int, idx_width: int, ws: int, ws_bytes: int,
                            visited: int = 0, stream: int = 0):
    cs, cp = shape.c(), p.c()
    rf = (ctypes.c_int32 * MAX_STAGES)(*([int(x) for x in refresh] + [1] * (MAX_STAGES - len(refresh))))
    _check(load().dsa_prune_select_cached(ctypes.byref(cs), q, k, ctypes.byref(cp), rf, step, cache or None,
                                          cache_bytes, idx, idx_width, ws, ws_bytes, visited or None,
                                          stream or None))


def sparse_attn_raw(shape: Shape, q: int, k: int, v: int, idx: int, idx_width: int, block_q: int,
                    scale: float, out: int, ws: int, ws_bytes: int, stream: int = 0):
    cs = shape.c()
    _check(load().dsa_sparse_attn(ctypes.byref(cs), q, k, v, idx, idx_width, block_q, scale, out,
                                  ws or None, ws_bytes, stream or None))


def dense_attn_raw(shape: Shape, q: int, k: int, v: int, scale: float, out: int, ws: int, ws_bytes: int,
                   stream: int = 0):
    cs = shape.c()
    _check(load().dsa_dense_attn(ctypes.byref(cs), q, k, v, scale, out, ws or None, ws_bytes,
                                 stream or None))


def block_sparse_index_width(k_blocks: int) -> int:
    w = load().dsa_block_sparse_index_width(k_blocks)
    if w < 0:
        raise DsaError(1, f"invalid k_blocks {k_blocks}")
    return w


def block_sparse_workspace_bytes(shape: Shape, k_blocks: int) -> int:
    cs, n = shape.c(), ctypes.c_size_t(0)
    _check(load().dsa_block_sparse_workspace_bytes(ctypes.byref(cs), k_blocks, ctypes.byref(n)))
    return n.value


def block_sparse_select_raw(shape: Shape, q: int, k: int, k_blocks: int, idx: int, ws: int, ws_bytes: int,
                            stream: int = 0):
    cs = shape.c()
    _check(load().dsa_block_sparse_select(ctypes.byref(cs), q, k, k_blocks, idx, ws or None, ws_bytes,
                                          stream or None))


def sparse_attn_heads_raw(shape: Shape, q: int, k: int, v: int, idx: int, idx_width: int, scale: float,
                          out: int, stream: int = 0):
    cs = shape.c()
    _check(load().dsa_sparse_attn_heads(ctypes.byref(cs), q, k, v, idx, idx_width, scale, out,
                                        stream or None))


def block_sparse_list_width(k_blocks: int) -> int:
    w = load().dsa_block_sparse_list_width(k_blocks)
    if w < 0:
        raise DsaError(1, f"invalid k_blocks {k_blocks}")
    return w


def block_sparse_select_lists_raw(shape: Shape, q: int, k: int, k_blocks: int, blocks: int, counts: int, ws: int,
                                  ws_bytes: int, stream: int = 0):
    cs = shape.c()
    _check(load().dsa_block_sparse_select_lists(ctypes.byref(cs), q, k, k_blocks, blocks, counts, ws or None,
                                                ws_bytes, stream or None))


def sparse_attn_lists_raw(shape: Shape, q: int, k: int, v: int, blocks: int, wb: int, cols: int, wc: int,
                          counts: int, scale: float, out: int, stream: int = 0):
    cs = shape.c()
    _check(load().dsa_sparse_attn_lists(ctypes.byref(cs), q, k, v, blocks, wb, cols or None, wc, counts, scale, out,
                                        stream or None))


def vertical_slash_list_widths(t: int, k_v: int, k_s: int):
    wb, wc = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(load().dsa_vertical_slash_list_widths(t, k_v, k_s, ctypes.byref(wb), ctypes.byref(wc)))
    return wb.value, wc.value


def vertical_slash_select_lists_raw(shape: Shape, q: int, k: int, k_v: int, k_s: int, blocks: int, cols: int,
                                    counts: int, kept_cols: int, kept_offsets: int, ws: int, ws_bytes: int,
                                    stream: int = 0):
    cs = shape.c()
    _check(load().dsa_vertical_slash_select_lists(ctypes.byref(cs), q, k, k_v, k_s, blocks, cols, counts,
                                                  kept_cols or None, kept_offsets or None, ws or None, ws_bytes,
                                                  stream or None))


def vertical_slash_index_width(t: int, k_v: int, k_s: int) -> int:
    w = load().dsa_vertical_slash_index_width(t, k_v, k_s)
    if w < 0:
        raise DsaError(1, f"invalid vertical-slash sizes t={t} k_v={k_v} k_s={k_s}")
    return w


def vertical_slash_workspace_bytes(shape: Shape, k_v: int, k_s: int) -> int:
    cs, n = shape.c(), ctypes.c_size_t(0)
    _check(load().dsa_vertical_slash_workspace_bytes(ctypes.byref(cs), k_v, k_s, ctypes.byref(n)))
    return n.value


def vertical_slash_select_raw(shape: Shape, q: int, k: int, k_v: int, k_s: int, idx: int, cols: int, offsets: int,
                              ws: int, ws_bytes: int, stream: int = 0):
    cs = shape.c()
    _check(load().dsa_vertical_slash_select(ctypes.byref(cs), q, k, k_v, k_s, idx, cols or None, offsets or None,
                                            ws or None, ws_bytes, stream or None))


def prune_rope_workspace_bytes(shape: Shape, p: Params, style: int = DSA_ROPE_RELATIVE, base: float = 10000.0) -> int:
    cs, cp, n = shape.c(), p.c(), ctypes.c_size_t(0)
    rope = CRope(style, base)
    _check(load().dsa_prune_rope_workspace_bytes(ctypes.byref(cs), ctypes.byref(cp), ctypes.byref(rope),
                                                 ctypes.byref(n)))
    return n.value


def prune_select_rope_raw(shape: Shape, q: int, k: int, p: Params, base: float, idx: int, ws: int, ws_bytes: int,
                          stream: int = 0, style: int = DSA_ROPE_RELATIVE):
    cs, cp = shape.c(), p.c()
    rope = CRope(style, base)
    _check(load().dsa_prune_select_rope(ctypes.byref(cs), q, k, ctypes.byref(cp), ctypes.byref(rope), idx,
                                        ws or None, ws_bytes, stream or None))


def rope_rotate_keys_raw(shape: Shape, k: int, p: Params, base: float, pos_begin: int, pos_end: int,
                         k_rot: list, stream: int = 0):
    cs, cp = shape.c(), p.c()
    rope = CRope(DSA_ROPE_CHUNK_INDEXED, base)
    ptrs = (ctypes.c_void_p * MAX_STAGES)(*[ctypes.c_void_p(x) for x in k_rot])
    _check(load().dsa_rope_rotate_keys(ctypes.byref(cs), k, ctypes.byref(cp), ctypes.byref(rope), pos_begin, pos_end,
                                       ptrs, stream or None))


def prune_select_rope_keys_raw(shape: Shape, q: int, k_rot: list, p: Params, base: float, idx: int, ws: int,
                               ws_bytes: int, stream: int = 0):
    cs, cp = shape.c(), p.c()
    rope = CRope(DSA_ROPE_CHUNK_INDEXED, base)
    ptrs = (ctypes.c_void_p * MAX_STAGES)(*[ctypes.c_void_p(x) for x in k_rot])
    _check(load().dsa_prune_select_rope_keys(ctypes.byref(cs), q, ptrs, ctypes.byref(cp), ctypes.byref(rope), idx,
                                             ws or None, ws_bytes, stream or None))


def profile_begin():
    _check(load().dsa_profile_begin())


def profile_end() -> dict:
    """{kernel name: (launches, total ms)} recorded since profile_begin()."""
    buf = (CKernelTime * 64)()
    n = ctypes.c_int32(0)
    _check(load().dsa_profile_end(buf, 64, ctypes.byref(n)))
    return {buf[i].name.decode(): (int(buf[i].launches), float(buf[i].total_ms)) for i in range(min(n.value, 64))}
