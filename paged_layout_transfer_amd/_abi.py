"""Constants, structures and descriptor builders of the C ABI in include/kvxfer.h.

Pure ctypes: importing this module loads nothing, so code that only builds
descriptors (or drives another build of the library) can use it without the HIP
runtime.  paged_layout_transfer_amd.kvxfer re-exports everything here.
"""
from __future__ import annotations

import ctypes
from typing import Iterable, Sequence

# ---- constants (mirror include/kvxfer.h) ---------------------------------------------
KV_OK = 0
KV_ERR_ARG = -1
KV_ERR_ALIGN = -2
KV_ERR_RANGE = -3
KV_ERR_OOM = -4
KV_ERR_RING = -5
KV_ERR_HIP = -6
KV_ERR_DEVICE = -7
KV_ERR_DUP = -8
KV_ERR_SCRATCH = -9
KV_ERR_CAPTURE = -10
KV_LAYER_FIRST = 0
KV_PAGE_FIRST = 1
KV_PAGE_TOKEN_MAJOR = 0
KV_PAGE_HEAD_MAJOR = 1
KV_GATHER = 0
KV_SCATTER = 1
KV_FLAG_VALIDATE = 0x1
KV_FLAG_DMA_STRIDED = 0x2
KV_FLAG_CACHED = 0x4
KV_FLAG_PAGE_RUNS = 0x8
KV_DEVERR_BLOCK_RANGE = 0x1
KV_RING_COHERENT = 0x0
KV_RING_NONCOHERENT = 0x1
KV_MAX_SPANS = 4096
KV_VERSION = 200


class kv_pool_desc(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("num_kv", ctypes.c_int32),
                ("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("elem_bytes", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("page_layout", ctypes.c_int32),
                ("num_blocks", ctypes.c_int64), ("block_stride", ctypes.c_int64),
                ("bases", ctypes.POINTER(ctypes.c_void_p))]


class kv_span(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("table_len", ctypes.c_int64),
                ("t_begin", ctypes.c_int64), ("t_end", ctypes.c_int64),
                ("first_chunk", ctypes.c_int64)]


class kv_chunk_spec(ctypes.Structure):
    _fields_ = [("layout", ctypes.c_int32), ("chunk_layers", ctypes.c_int32),
                ("chunk_tokens", ctypes.c_int64), ("layer_begin", ctypes.c_int32),
                ("layer_end", ctypes.c_int32), ("base", ctypes.c_void_p),
                ("slot_bytes", ctypes.c_int64), ("n_slots", ctypes.c_int64),
                ("max_workgroups", ctypes.c_int32), ("flags", ctypes.c_int32)]


class kv_transfer_info(ctypes.Structure):
    _fields_ = [("tiles", ctypes.c_int64), ("chunks", ctypes.c_int64),
                ("payload_bytes", ctypes.c_int64), ("max_chunk_bytes", ctypes.c_int64)]


def _addr(x) -> int:
    if x is None:
        return 0
    if hasattr(x, "data_ptr"):
        return int(x.data_ptr())
    return int(x)


# ---- descriptor builders ---------------------------------------------------------------

def make_pool_desc(num_layers: int, num_kv: int, num_heads: int, head_dim: int, elem_bytes: int,
                   block_size: int, num_blocks: int, block_stride: int,
                   bases: Sequence, page_layout: int = KV_PAGE_TOKEN_MAJOR) -> kv_pool_desc:
    """A kv_pool_desc; bases holds num_layers*num_kv device addresses (index l*num_kv+kv)."""
    arr = (ctypes.c_void_p * len(bases))(*[_addr(b) for b in bases])
    d = kv_pool_desc(num_layers, num_kv, num_heads, head_dim, elem_bytes, block_size, page_layout,
                     num_blocks, block_stride, ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)))
    d._bases_keepalive = arr
    return d


def make_spans(spans: Iterable) -> ctypes.Array:
    """spans: (block_table, table_len, t_begin, t_end, first_chunk) tuples; block_table
    is a device address or tensor (a host address for kv_validate_targets)."""
    spans = list(spans)
    arr = (kv_span * max(1, len(spans)))()
    for i, (tbl, n, t0, t1, fc) in enumerate(spans):
        arr[i] = kv_span(_addr(tbl), int(n), int(t0), int(t1), int(fc))
    arr._n = len(spans)
    return arr


def make_chunk_spec(layout: int, chunk_layers: int, chunk_tokens: int, layer_begin: int,
                    layer_end: int, base, slot_bytes: int, n_slots: int,
                    max_workgroups: int = 0, flags: int = 0) -> kv_chunk_spec:
    return kv_chunk_spec(layout, chunk_layers, chunk_tokens, layer_begin, layer_end, _addr(base),
                         slot_bytes, n_slots, max_workgroups, flags)


def _nspans(spans) -> int:
    return getattr(spans, "_n", len(spans))
