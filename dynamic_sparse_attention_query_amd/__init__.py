"""Dynamic, per-input block-sparse attention for AMD MI355X (gfx950).

Hierarchical chunk pruning with SelectRep representatives (prune_select) and a
gathered sparse attention pass over the surviving keys plus sink and window
keys (sparse_attn), with an exact dense path (dense_attn) for comparison. All
computation runs in the HIP library libdsa.so behind the C ABI of
include/dsa.h; this package only marshals tensors.
"""
from ._lib import Params, Shape, DsaError, index_width, workspace_bytes  # noqa: F401

__all__ = ["Params", "Shape", "DsaError", "index_width", "workspace_bytes",
           "prune_select", "sparse_attn", "dense_attn"]


def __getattr__(name):
    if name in ("prune_select", "sparse_attn", "dense_attn", "make_shape"):
        from . import api
        return getattr(api, name)
    raise AttributeError(name)
