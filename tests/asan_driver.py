"""Runs the library's host code under AddressSanitizer and UBSan (no GPU, no torch).

Started by tests/test_host_sanitizers.py in a child process whose LD_PRELOAD holds
the sanitizer runtime; argv[1] is a build of the library's sources plus
tests/kernel_emu.cpp with host-side instrumentation.  It drives, on small random
cases, the host preparation and the kernel's tile walk (emu_transfer, copying the
bytes), the copy-engine plan (emu_dma, per tile and strided), the span-record arena
bookkeeping (emu_arena), the block allocator against a set model, and the host
validation's error paths (kv_check_transfer), and compares every copied result with
the oracle.  Prints "ok" at the end; any
sanitizer report aborts the process.
"""
from __future__ import annotations

import ctypes
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import cases  # noqa: E402
import oracle  # noqa: E402
from paged_layout_transfer_amd import _abi as A  # noqa: E402

lib = ctypes.CDLL(sys.argv[1])
I64P = ctypes.POINTER(ctypes.c_int64)
lib.emu_transfer.argtypes = [ctypes.c_int, ctypes.POINTER(A.kv_pool_desc), ctypes.POINTER(A.kv_span), ctypes.c_int32,
                             ctypes.POINTER(A.kv_chunk_spec), ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                             I64P, I64P, I64P]
lib.emu_dma.argtypes = [ctypes.c_int, ctypes.POINTER(A.kv_pool_desc), ctypes.POINTER(A.kv_span), ctypes.c_int32,
                        ctypes.POINTER(A.kv_chunk_spec), ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                        I64P, I64P, I64P]
lib.emu_arena.restype = ctypes.c_int64
lib.emu_arena.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32]
lib.kv_check_transfer.argtypes = [ctypes.POINTER(A.kv_pool_desc), ctypes.POINTER(A.kv_span), ctypes.c_int32,
                                  ctypes.POINTER(A.kv_chunk_spec), ctypes.POINTER(A.kv_transfer_info)]


def run_case(seed: int) -> None:
    rng = np.random.default_rng(41_000 + seed)
    pool, spans, chunks = cases.make_case(rng, tok_multiple=16, medium=bool(seed % 3 == 0),
                                          max_bytes=4 << 20, head_major=None)
    regions = cases.regions_for(pool, rng)
    staging = cases.staging_for(chunks, rng=rng)
    n = regions.shape[0]
    tabs = [np.ascontiguousarray(t, dtype=np.int32) for t, _, _, _ in spans]
    sp = A.make_spans([(t.ctypes.data, t.size, t0, t1, fc) for t, (_, t0, t1, fc) in zip(tabs, spans)])
    rb = np.full(n, regions.shape[1], dtype=np.int64)
    for d in (A.KV_GATHER, A.KV_SCATTER):
        r_or, s_or = regions.copy(), staging.copy()
        oracle.transfer(d, pool, r_or, spans, chunks, s_or)
        for mode in ("kernel", "dma", "dma_strided"):
            r, s = regions.copy(), staging.copy()
            desc = A.make_pool_desc(pool["num_layers"], pool["num_kv"], pool["num_heads"], pool["head_dim"],
                                    pool["elem_bytes"], pool["block_size"], pool["num_blocks"],
                                    pool["block_stride"], [r[i].ctypes.data for i in range(n)],
                                    pool.get("page_layout", 0))
            strided = mode == "dma_strided"
            spec = A.make_chunk_spec(chunks["layout"], chunks["chunk_layers"], chunks["chunk_tokens"],
                                     chunks["layer_begin"], chunks["layer_end"], s.ctypes.data,
                                     chunks["slot_bytes"], chunks["n_slots"], int(seed % 4),
                                     A.KV_FLAG_DMA_STRIDED if strided else 0)
            a, b, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
            fn = lib.emu_transfer if mode == "kernel" else lib.emu_dma
            last = 1 if mode == "kernel" else int(strided)
            rc = fn(d, ctypes.byref(desc), sp, len(spans), ctypes.byref(spec), rb.ctypes.data, s.size, last,
                    ctypes.byref(a), ctypes.byref(b), ctypes.byref(c))
            assert rc == 0 and a.value == 0, (seed, mode, rc, a.value)
            assert np.array_equal(r, r_or) and np.array_equal(s, s_or), (seed, d, mode)


def error_paths() -> None:
    base = np.zeros(1 << 16, dtype=np.uint8)
    stg = np.zeros(1 << 16, dtype=np.uint8)
    tab = np.arange(8, dtype=np.int32)
    info = A.kv_transfer_info()

    def check(expect, *, bases=None, stride=2048, t0=0, t1=64, table_len=8, ct=16, cl=1, L=2, slot=4096,
              n_slots=8, stg_addr=None, flags=0):
        bases = bases if bases is not None else [base.ctypes.data, base.ctypes.data + 16384]
        desc = A.make_pool_desc(L, 1, 1, 64, 2, 16, 8, stride, bases)
        sp = A.make_spans([(tab.ctypes.data, table_len, t0, t1, 0)])
        spec = A.make_chunk_spec(0, cl, ct, 0, L, stg.ctypes.data if stg_addr is None else stg_addr, slot,
                                 n_slots, 0, flags)
        rc = lib.kv_check_transfer(ctypes.byref(desc), sp, 1, ctypes.byref(spec), ctypes.byref(info))
        assert rc == expect, (expect, rc)

    check(A.KV_OK)
    check(A.KV_ERR_ALIGN, bases=[base.ctypes.data + 8, base.ctypes.data + 16384])
    check(A.KV_ERR_ARG, bases=[0, base.ctypes.data])
    check(A.KV_ERR_ARG, t0=8)                      # not on a page boundary
    check(A.KV_ERR_ARG, ct=24)                     # chunk tokens not a multiple of the page
    check(A.KV_ERR_ARG, cl=3, L=2)                 # chunk layers do not divide the layers
    check(A.KV_ERR_ARG, t0=64, t1=32)              # inverted range
    check(A.KV_ERR_RANGE, table_len=3)             # span past its table
    check(A.KV_ERR_RING, n_slots=1)                # more chunks than slots
    check(A.KV_ERR_RANGE, slot=1024)               # slot smaller than a chunk
    check(A.KV_ERR_ALIGN, stg_addr=stg.ctypes.data + 4)
    check(A.KV_ERR_ARG, flags=0x40)                # unknown flag
    check(A.KV_ERR_ARG, stride=1024)               # blocks overlap


def allocator() -> None:
    lib.kv_pool_create.argtypes = [ctypes.POINTER(A.kv_pool_desc), ctypes.POINTER(ctypes.c_void_p)]
    lib.kv_pool_alloc_blocks.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    lib.kv_pool_free_blocks.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    lib.kv_pool_destroy.argtypes = [ctypes.c_void_p]
    region = np.zeros(16, dtype=np.uint8)
    for n_blocks in (1, 63, 64, 65, 1000):
        desc = A.make_pool_desc(1, 1, 1, 8, 2, 1, n_blocks, 16, [region.ctypes.data])
        h = ctypes.c_void_p()
        assert lib.kv_pool_create(ctypes.byref(desc), ctypes.byref(h)) == 0
        rng = np.random.default_rng(43_000 + n_blocks)
        held = set()
        for _ in range(300):
            if held and rng.random() < 0.5:
                ids = rng.permutation(sorted(held))[:int(rng.integers(1, len(held) + 1))].astype(np.int32)
                assert lib.kv_pool_free_blocks(h, ids.size, ids.ctypes.data) == 0
                held -= set(ids.tolist())
            else:
                free = sorted(set(range(n_blocks)) - held)
                k = int(rng.integers(0, len(free) + 2))
                out = np.full(max(1, k), -1, dtype=np.int32)
                rc = lib.kv_pool_alloc_blocks(h, k, out.ctypes.data)
                if k > len(free):
                    assert rc == A.KV_ERR_OOM
                else:
                    assert rc == 0 and out[:k].tolist() == free[:k]
                    held |= set(out[:k].tolist())
            # out of range, or one id twice (free or held): rejected, nothing freed
            bad = np.array([n_blocks, -1] if rng.random() < 0.5 else [0, 0], dtype=np.int32)
            assert lib.kv_pool_free_blocks(h, 2, bad.ctypes.data) == A.KV_ERR_RANGE
        assert lib.kv_pool_destroy(h) == 0


def arena() -> None:
    rng = np.random.default_rng(42_000)
    for lag in (0, 5, 300):
        spans = [int(x) for x in rng.choice([1, 7, 64, 1000, 4096], size=3000)]
        sizes = np.array([(64 * k + 255) // 256 * 256 for k in spans], dtype=np.int64)
        assert lib.emu_arena(4 << 20, sizes.ctypes.data, sizes.size, lag) == 0


if __name__ == "__main__":
    for seed in range(int(os.environ.get("ASAN_CASES", "24"))):
        run_case(seed)
    error_paths()
    allocator()
    arena()
    print("ok", flush=True)
