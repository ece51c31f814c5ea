"""Python binding of the C ABI in include/kvxfer.h (ctypes; argument marshalling only).

Every function here has the name of the C entry point it calls and does nothing
but convert arguments and raise on error codes; all transfer work runs in the
HIP library.  Device buffers are passed as integer addresses or as objects with
``data_ptr()`` (torch tensors), streams as integer ``hipStream_t`` handles
(``torch.cuda.current_stream().cuda_stream``) or objects with ``cuda_stream``.

Importing this module loads ``libkvxfer.so`` from this package directory and
raises ImportError if it has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvxfer.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(
        "libkvxfer.so is not built (%s); build it with __graft_entry__.build() or "
        "python -m paged_layout_transfer_amd._build" % _LIB_PATH)
# A process must hold one HIP runtime.  PyTorch ships its own copy and its libraries
# ask for it under a name that does not match an already loaded /opt/rocm copy, so
# loading this library first would leave two runtimes, and the second sees no
# device.  Loading torch first makes this library bind to torch's runtime.
try:
    import torch  # noqa: F401
except ImportError:
    pass
_lib = ctypes.CDLL(_LIB_PATH)

from ._abi import *  # noqa: E402,F401,F403  (constants, structures, descriptor builders)
from ._abi import _addr, _nspans  # noqa: E402

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64


def _sig(name, res, *args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_sig("kv_pool_create", ctypes.c_int, ctypes.POINTER(kv_pool_desc), ctypes.POINTER(_P))
_sig("kv_pool_destroy", ctypes.c_int, _P)
_sig("kv_pool_alloc_blocks", ctypes.c_int, _P, _I32, _P)
_sig("kv_pool_free_blocks", ctypes.c_int, _P, _I32, _P)
_sig("kv_pool_free_count", ctypes.c_int, _P, ctypes.POINTER(_I64))
_sig("kv_check_transfer", ctypes.c_int, ctypes.POINTER(kv_pool_desc), ctypes.POINTER(kv_span), _I32,
     ctypes.POINTER(kv_chunk_spec), ctypes.POINTER(kv_transfer_info))
_sig("kv_chunk_bytes", ctypes.c_int, ctypes.POINTER(kv_pool_desc), ctypes.POINTER(kv_chunk_spec), _I64,
     ctypes.POINTER(_I64))
_sig("kv_validate_targets", ctypes.c_int, ctypes.POINTER(kv_pool_desc), ctypes.POINTER(kv_span), _I32,
     ctypes.POINTER(_P), _I32)
_sig("kv_gather_chunks", ctypes.c_int, _P, ctypes.POINTER(kv_span), _I32, ctypes.POINTER(kv_chunk_spec), _P)
_sig("kv_scatter_chunks", ctypes.c_int, _P, ctypes.POINTER(kv_span), _I32, ctypes.POINTER(kv_chunk_spec), _P)
_sig("kv_transfer_chunks_noalloc", ctypes.c_int, _P, _I32, ctypes.POINTER(kv_span), _I32,
     ctypes.POINTER(kv_chunk_spec), _P, _P)
_sig("kv_gather_chunks_dma", ctypes.c_int, _P, ctypes.POINTER(kv_span), _I32, ctypes.POINTER(kv_chunk_spec), _P)
_sig("kv_scatter_chunks_dma", ctypes.c_int, _P, ctypes.POINTER(kv_span), _I32, ctypes.POINTER(kv_chunk_spec), _P)
_sig("kv_pool_get_error", ctypes.c_int, _P, _P, ctypes.POINTER(_I32))
_sig("kv_pool_timing_start", ctypes.c_int, _P)
_sig("kv_pool_timing_read", ctypes.c_int, _P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_I64))
_sig("kv_pool_timing_read_each", ctypes.c_int, _P, _P, _I64, ctypes.POINTER(_I64))
_sig("kv_ring_create", ctypes.c_int, _I64, _I64, _I32, ctypes.POINTER(_P))
_sig("kv_ring_slot", ctypes.c_int, _P, _I64, ctypes.POINTER(_P), ctypes.POINTER(_P))
_sig("kv_ring_destroy", ctypes.c_int, _P)
_sig("kv_ring_record", ctypes.c_int, _P, _I64, _I64, _P)
_sig("kv_ring_wait", ctypes.c_int, _P, _I64, _I64)
_sig("kv_ring_stream_wait", ctypes.c_int, _P, _I64, _I64, _P)
_sig("kv_strerror", ctypes.c_char_p, ctypes.c_int)
_sig("kv_version", ctypes.c_int)
_sig("kv_last_hip_error", ctypes.c_int, ctypes.POINTER(ctypes.c_char_p))

LIBRARY_PATH = _LIB_PATH
EXPORTED = ("kv_pool_create", "kv_pool_destroy", "kv_pool_alloc_blocks", "kv_pool_free_blocks",
            "kv_pool_free_count", "kv_check_transfer", "kv_chunk_bytes", "kv_validate_targets",
            "kv_gather_chunks", "kv_scatter_chunks", "kv_transfer_chunks_noalloc",
            "kv_gather_chunks_dma", "kv_scatter_chunks_dma",
            "kv_pool_get_error", "kv_pool_timing_start",
            "kv_pool_timing_read", "kv_pool_timing_read_each", "kv_ring_create", "kv_ring_slot", "kv_ring_destroy",
            "kv_ring_record", "kv_ring_wait", "kv_ring_stream_wait",
            "kv_strerror", "kv_version", "kv_last_hip_error")


class KvError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = int(code)
        msg = "%s: %s (%d)" % (where, kv_strerror(code), code)
        if self.code == KV_ERR_HIP:
            err, call = kv_last_hip_error()
            msg += "; last failing HIP call: %s -> hipError %d" % (call, err)
        super().__init__(msg)


def _check(rc: int, where: str) -> None:
    if rc != KV_OK:
        raise KvError(rc, where)


def _stream(s) -> int:
    if s is None:
        return 0
    if hasattr(s, "cuda_stream"):
        return int(s.cuda_stream)
    return int(s)


# ---- entry points ------------------------------------------------------------------------

def kv_pool_create(desc: kv_pool_desc) -> int:
    h = ctypes.c_void_p()
    _check(_lib.kv_pool_create(ctypes.byref(desc), ctypes.byref(h)), "kv_pool_create")
    return h.value


def kv_pool_destroy(pool: int) -> None:
    _check(_lib.kv_pool_destroy(pool), "kv_pool_destroy")


def kv_pool_alloc_blocks(pool: int, n: int) -> np.ndarray:
    out = np.empty(max(1, n), dtype=np.int32)
    _check(_lib.kv_pool_alloc_blocks(pool, n, out.ctypes.data), "kv_pool_alloc_blocks")
    return out[:n]


def kv_pool_free_blocks(pool: int, ids) -> None:
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    _check(_lib.kv_pool_free_blocks(pool, ids.size, ids.ctypes.data), "kv_pool_free_blocks")


def kv_pool_free_count(pool: int) -> int:
    n = ctypes.c_int64()
    _check(_lib.kv_pool_free_count(pool, ctypes.byref(n)), "kv_pool_free_count")
    return n.value


def kv_check_transfer(desc: kv_pool_desc, spans, spec: kv_chunk_spec) -> kv_transfer_info:
    info = kv_transfer_info()
    _check(_lib.kv_check_transfer(ctypes.byref(desc), spans, _nspans(spans), ctypes.byref(spec),
                                  ctypes.byref(info)), "kv_check_transfer")
    return info


def kv_chunk_bytes(desc: kv_pool_desc, spec: kv_chunk_spec, tokens: int) -> int:
    n = ctypes.c_int64()
    _check(_lib.kv_chunk_bytes(ctypes.byref(desc), ctypes.byref(spec), tokens, ctypes.byref(n)),
           "kv_chunk_bytes")
    return n.value


def kv_validate_targets(desc: kv_pool_desc, spans, host_tables: Sequence[np.ndarray],
                        direction: int) -> None:
    tabs = [np.ascontiguousarray(t, dtype=np.int32) for t in host_tables]
    ptrs = (ctypes.c_void_p * max(1, len(tabs)))(*[t.ctypes.data for t in tabs])
    _check(_lib.kv_validate_targets(ctypes.byref(desc), spans, _nspans(spans), ptrs, direction),
           "kv_validate_targets")


def kv_gather_chunks(pool: int, spans, spec: kv_chunk_spec, stream=None) -> None:
    _check(_lib.kv_gather_chunks(pool, spans, _nspans(spans), ctypes.byref(spec), _stream(stream)),
           "kv_gather_chunks")


def kv_scatter_chunks(pool: int, spans, spec: kv_chunk_spec, stream=None) -> None:
    _check(_lib.kv_scatter_chunks(pool, spans, _nspans(spans), ctypes.byref(spec), _stream(stream)),
           "kv_scatter_chunks")


def kv_transfer_chunks_noalloc(pool: int, direction: int, spans, spec: kv_chunk_spec, err_word=None,
                               stream=None) -> None:
    """Gather or scatter with no allocation (static device scratch); err_word is a
    caller-owned device int32 (address or tensor) that receives KV_DEVERR_* bits, or None."""
    _check(_lib.kv_transfer_chunks_noalloc(pool, direction, spans, _nspans(spans), ctypes.byref(spec),
                                           _addr(err_word) if err_word is not None else None,
                                           _stream(stream)),
           "kv_transfer_chunks_noalloc")


def kv_gather_chunks_dma(pool: int, spans, spec: kv_chunk_spec, stream=None) -> None:
    """Copy-engine gather (one hipMemcpyAsync per tile, or one strided copy per chunk page
    with KV_FLAG_DMA_STRIDED); the spans' block tables are host arrays."""
    _check(_lib.kv_gather_chunks_dma(pool, spans, _nspans(spans), ctypes.byref(spec), _stream(stream)),
           "kv_gather_chunks_dma")


def kv_scatter_chunks_dma(pool: int, spans, spec: kv_chunk_spec, stream=None) -> None:
    """Copy-engine scatter (one hipMemcpyAsync per tile, or one strided copy per chunk page
    with KV_FLAG_DMA_STRIDED); the spans' block tables are host arrays."""
    _check(_lib.kv_scatter_chunks_dma(pool, spans, _nspans(spans), ctypes.byref(spec), _stream(stream)),
           "kv_scatter_chunks_dma")


def kv_pool_get_error(pool: int, stream=None) -> int:
    """Synchronizes the stream; returns (and clears) the device error bits (0 if none)."""
    bits = ctypes.c_int32()
    rc = _lib.kv_pool_get_error(pool, _stream(stream), ctypes.byref(bits))
    if rc not in (KV_OK, KV_ERR_DEVICE):
        raise KvError(rc, "kv_pool_get_error")
    return bits.value


def kv_pool_timing_start(pool: int) -> None:
    _check(_lib.kv_pool_timing_start(pool), "kv_pool_timing_start")


def kv_pool_timing_read(pool: int) -> tuple[float, int]:
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(_lib.kv_pool_timing_read(pool, ctypes.byref(ms), ctypes.byref(n)), "kv_pool_timing_read")
    return ms.value, n.value


def kv_pool_timing_read_each(pool: int, cap: int = 4096) -> np.ndarray:
    """Each timed launch's kernel time in milliseconds, in launch order; stops timing."""
    out = np.empty(max(1, cap), dtype=np.float64)
    n = ctypes.c_int64()
    _check(_lib.kv_pool_timing_read_each(pool, out.ctypes.data, cap, ctypes.byref(n)),
           "kv_pool_timing_read_each")
    return out[:min(n.value, cap)].copy()


def kv_ring_create(slot_bytes: int, n_slots: int, flags: int = KV_RING_COHERENT) -> int:
    h = ctypes.c_void_p()
    _check(_lib.kv_ring_create(slot_bytes, n_slots, flags, ctypes.byref(h)), "kv_ring_create")
    return h.value


def kv_ring_slot(ring: int, i: int) -> tuple[int, int]:
    hp, dp = ctypes.c_void_p(), ctypes.c_void_p()
    _check(_lib.kv_ring_slot(ring, i, ctypes.byref(hp), ctypes.byref(dp)), "kv_ring_slot")
    return hp.value, dp.value


def kv_ring_destroy(ring: int) -> None:
    _check(_lib.kv_ring_destroy(ring), "kv_ring_destroy")


def kv_ring_record(ring: int, first: int, count: int, stream=None) -> None:
    _check(_lib.kv_ring_record(ring, first, count, _stream(stream)), "kv_ring_record")


def kv_ring_wait(ring: int, first: int, count: int) -> None:
    _check(_lib.kv_ring_wait(ring, first, count), "kv_ring_wait")


def kv_ring_stream_wait(ring: int, first: int, count: int, stream=None) -> None:
    _check(_lib.kv_ring_stream_wait(ring, first, count, _stream(stream)), "kv_ring_stream_wait")


def kv_strerror(code: int) -> str:
    return _lib.kv_strerror(code).decode()


def kv_version() -> int:
    return int(_lib.kv_version())


def kv_last_hip_error() -> tuple[int, str]:
    where = ctypes.c_char_p()
    code = _lib.kv_last_hip_error(ctypes.byref(where))
    return int(code), (where.value or b"").decode()


def hip_runtime() -> ctypes.CDLL:
    """The HIP runtime library this process already has mapped -- the one this
    library and torch are bound to -- for direct runtime calls (memory queries,
    copies, CU-masked streams).  A second copy loaded by soname would be a separate
    runtime that sees no device, so there is no fallback: if none is mapped,
    RuntimeError."""
    with open("/proc/self/maps") as f:
        for line in f:
            path = line.split()[-1]
            if "libamdhip64.so" in path:
                return ctypes.CDLL(path)
    raise RuntimeError("no HIP runtime is mapped in this process")


def ring_host_array(ring: int, nbytes: int) -> np.ndarray:
    """A numpy uint8 view of a ring's host mapping (first nbytes), for filling and reading."""
    host, _ = kv_ring_slot(ring, 0)
    return np.ctypeslib.as_array((ctypes.c_uint8 * nbytes).from_address(host))
