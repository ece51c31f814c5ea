"""CPU oracle for paged-KV gather/scatter -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package.  The HIP library never imports, links or calls it,
and it imports nothing from the HIP library.

The arithmetic lives in ``oracle.c`` (plain nested loops, see its header for the
definition and the passages of the Strata guide and the Tutti summary it
follows).  This module only builds and loads it and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

GATHER = 0
SCATTER = 1
LAYER_FIRST = 0
PAGE_FIRST = 1


CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp"]


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (plain -O2, OpenMP over the (span, layer) pairs)
    into liboracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


class _Pool(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "num_layers", "num_kv", "num_heads", "head_dim", "elem_bytes",
        "block_size", "num_blocks", "block_stride", "page_layout")]


class _Span(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("t_begin", ctypes.c_int64),
                ("t_end", ctypes.c_int64), ("first_chunk", ctypes.c_int64)]


class _Chunks(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "layout", "chunk_layers", "chunk_tokens", "layer_begin", "layer_end",
        "slot_bytes", "n_slots")]


_lib = None


def _load(path: str | None = None):
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(path or _LIB)
        lib.orc_transfer.restype = ctypes.c_int64
        lib.orc_transfer.argtypes = [
            ctypes.c_int, ctypes.POINTER(_Pool), ctypes.POINTER(ctypes.c_void_p),
            ctypes.POINTER(_Span), ctypes.c_int64, ctypes.POINTER(_Chunks), ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64]
        lib.orc_set_threads.argtypes = [ctypes.c_int]
        lib.orc_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def load_library(path: str):
    """Load an oracle build from an explicit path (used to run planted-mistake builds)."""
    lib = ctypes.CDLL(path)
    lib.orc_transfer.restype = ctypes.c_int64
    lib.orc_transfer.argtypes = _load().orc_transfer.argtypes
    lib.orc_set_threads.argtypes = [ctypes.c_int]
    lib.orc_max_threads.restype = ctypes.c_int
    return lib


def set_threads(n: int, lib=None) -> None:
    """Threads the following oracle calls share their (span, layer) pairs between."""
    (lib or _load()).orc_set_threads(int(n))


def max_threads(lib=None) -> int:
    """Threads the oracle uses now (OpenMP's current maximum; 1 without OpenMP)."""
    return int((lib or _load()).orc_max_threads())


def transfer(direction: int, pool: dict, regions, spans, chunks: dict, chunk_buf: np.ndarray,
             only_layers: tuple[int, int] | None = None, lib=None) -> int:
    """Run the oracle in place.

    pool     : dict with num_layers, num_kv, num_heads, head_dim, elem_bytes,
               block_size, num_blocks, block_stride and optionally page_layout
               (0 token-major pages, the default; 1 head-major)
    regions  : sequence of L*KV writable uint8 numpy arrays (one per (layer, kv),
               index l*KV+kv), each covering every block it addresses, or a
               2-D uint8 array whose rows are the regions; with only_layers, the
               entries of layers outside that range may be None
    spans    : sequence of (int32 block table, t_begin, t_end, first_chunk)
    chunks   : dict with layout, chunk_layers, chunk_tokens, layer_begin,
               layer_end, slot_bytes, n_slots
    chunk_buf: writable uint8 array of n_slots*slot_bytes bytes
    Returns the number of bytes copied; raises ValueError on a broken precondition.
    """
    lib = lib or _load()
    p = _Pool(**{k: int(pool.get(k, 0)) for k, _ in _Pool._fields_})
    c = _Chunks(**{k: int(chunks[k]) for k, _ in _Chunks._fields_})
    nreg = p.num_layers * p.num_kv
    if len(regions) != nreg:
        raise ValueError("need one region per (layer, kv)")
    need = (p.num_blocks - 1) * p.block_stride + p.block_size * p.num_heads * p.head_dim * p.elem_bytes
    l0, l1 = only_layers if only_layers is not None else (0, p.num_layers)
    ptrs = (ctypes.c_void_p * nreg)()
    for i in range(nreg):
        r = regions[i]
        if r is None and not (l0 <= i // p.num_kv < l1):
            continue  # a layer outside the evaluated range is never touched
        if r is None or r.dtype != np.uint8 or not r.flags.c_contiguous or r.size < need:
            raise ValueError("region %d must be a contiguous uint8 array of >= %d bytes" % (i, need))
        ptrs[i] = r.ctypes.data
    if chunk_buf.dtype != np.uint8 or not chunk_buf.flags.c_contiguous:
        raise ValueError("chunk_buf must be contiguous uint8")
    if chunk_buf.size < c.n_slots * c.slot_bytes:
        raise ValueError("chunk_buf smaller than n_slots*slot_bytes")
    tables = []
    sp = (_Span * max(1, len(spans)))()
    for i, (tbl, t0, t1, fc) in enumerate(spans):
        tbl = np.ascontiguousarray(tbl, dtype=np.int32)
        if tbl.size * p.block_size < t1:
            raise ValueError("span %d: block table shorter than ceil(t_end/block_size)" % i)
        tables.append(tbl)
        sp[i] = _Span(tbl.ctypes.data, int(t0), int(t1), int(fc))
    n = lib.orc_transfer(int(direction), ctypes.byref(p), ptrs, sp, len(spans), ctypes.byref(c),
                         chunk_buf.ctypes.data, int(l0), int(l1))
    if n < 0:
        raise ValueError("oracle rejected the call (precondition broken)")
    return int(n)


def gather(pool, regions, spans, chunks, chunk_buf, **kw) -> int:
    return transfer(GATHER, pool, regions, spans, chunks, chunk_buf, **kw)


def scatter(pool, regions, spans, chunks, chunk_buf, **kw) -> int:
    return transfer(SCATTER, pool, regions, spans, chunks, chunk_buf, **kw)
