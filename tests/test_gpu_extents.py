"""Declared buffer extents against the allocations that hold them.

A transfer trusts the sizes its arguments declare (num_blocks per region,
n_slots * slot_bytes of staging, table_len entries per block table).  Where the
HIP runtime knows the allocation behind a pointer, a declared extent that runs
past its end must be refused with KV_ERR_RANGE before anything is enqueued.

Every refused call here touches only bytes inside the real buffers (slot 0, low
block ids, the first table entries), so it would be harmless even if it were
launched; the tests then check that nothing was written and that valid calls on
the same buffers still work.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import gpu_harness as G
from paged_layout_transfer_amd import kvxfer as K
from paged_layout_transfer_amd import workloads as W

pytestmark = pytest.mark.gpu

L, KV, H, D, E, BS, N = 2, 2, 1, 64, 2, 16, 64
TOK = H * D * E
TILE = BS * TOK


def _alloc_end(ptr: int) -> int:
    """How far the runtime's allocations reach from ptr without a gap (a torch block
    lies inside one allocation; virtual-memory mappings count one by one), as the
    library itself walks them."""
    hip = G.hip_runtime()
    cur = ptr
    for i in range(1 << 16):
        base, size = ctypes.c_void_p(), ctypes.c_size_t()
        rc = hip.hipMemGetAddressRange(ctypes.byref(base), ctypes.byref(size), ctypes.c_void_p(cur))
        if rc != 0:
            hip.hipGetLastError()
            assert i > 0, "hipMemGetAddressRange does not know the buffer (%d)" % rc
            return cur
        cur = base.value + size.value
    raise AssertionError("allocations reach too far to follow")


def _setup():
    dev = torch.device("cuda", 0)
    pool_t = torch.full((L * KV, N * TILE), 7, dtype=torch.uint8, device=dev)
    stg = torch.full((4 * L * KV * TILE,), W.SENTINEL, dtype=torch.uint8, device=dev)
    tab = torch.arange(4, dtype=torch.int32, device=dev)
    return dev, pool_t, stg, tab


def _pool(pool_t, num_blocks=N):
    bases = [pool_t.data_ptr() + i * pool_t.stride(0) for i in range(L * KV)]
    return K.kv_pool_create(K.make_pool_desc(L, KV, H, D, E, BS, num_blocks, TILE, bases))


def _spec(stg, n_slots):
    slot = L * KV * BS * TOK          # one page per chunk
    return K.make_chunk_spec(K.KV_LAYER_FIRST, L, BS, 0, L, stg, slot, n_slots)


def test_valid_call_passes_and_moves_bytes():
    _, pool_t, stg, tab = _setup()
    p = _pool(pool_t)
    stream = torch.cuda.current_stream()
    try:
        K.kv_gather_chunks(p, K.make_spans([(tab, 4, 0, BS, 0)]), _spec(stg, 4), stream)
        assert K.kv_pool_get_error(p, stream) == 0
        torch.cuda.synchronize()
        assert int((stg[:L * KV * TILE] == 7).sum()) == L * KV * TILE
    finally:
        K.kv_pool_destroy(p)


def test_staging_declared_past_its_allocation_is_refused():
    _, pool_t, stg, tab = _setup()
    slot = L * KV * BS * TOK
    avail = _alloc_end(stg.data_ptr()) - stg.data_ptr()
    too_many = avail // slot + 1                       # n_slots * slot_bytes > what the allocation holds
    p = _pool(pool_t)
    stream = torch.cuda.current_stream()
    spans = K.make_spans([(tab, 4, 0, BS, 0)])         # one chunk, slot 0: inside the buffer
    try:
        for fn in (K.kv_gather_chunks, K.kv_scatter_chunks):
            with pytest.raises(K.KvError) as e:
                fn(p, spans, _spec(stg, too_many), stream)
            assert e.value.code == K.KV_ERR_RANGE
        torch.cuda.synchronize()
        assert bool((stg == W.SENTINEL).all()), "a refused gather wrote the staging"
        assert bool((pool_t == 7).all()), "a refused scatter wrote the pool"
        # the largest slot count that fits is accepted
        K.kv_gather_chunks(p, spans, _spec(stg, avail // slot), stream)
        assert K.kv_pool_get_error(p, stream) == 0
        torch.cuda.synchronize()
        assert int((stg[:slot] == 7).sum()) == slot
    finally:
        K.kv_pool_destroy(p)


def test_regions_declared_past_their_allocation_are_refused():
    _, pool_t, stg, tab = _setup()
    last = pool_t.data_ptr() + (L * KV - 1) * pool_t.stride(0)
    fits = (_alloc_end(last) - last - TILE) // TILE + 1  # blocks the last region can hold
    if fits + 1 > 2**31 - 1:
        pytest.skip("the allocations after the pool reach past a 31-bit block count")
    stream = torch.cuda.current_stream()
    spans = K.make_spans([(tab, 4, 0, BS, 0)])          # block 0 only
    bad = _pool(pool_t, num_blocks=fits + 1)
    try:
        for fn in (K.kv_scatter_chunks, K.kv_gather_chunks):
            with pytest.raises(K.KvError) as e:
                fn(bad, spans, _spec(stg, 4), stream)
            assert e.value.code == K.KV_ERR_RANGE
        torch.cuda.synchronize()
        assert bool((pool_t == 7).all()) and bool((stg == W.SENTINEL).all())
    finally:
        K.kv_pool_destroy(bad)
    good = _pool(pool_t, num_blocks=fits)
    try:
        K.kv_gather_chunks(good, spans, _spec(stg, 4), stream)
        assert K.kv_pool_get_error(good, stream) == 0
    finally:
        K.kv_pool_destroy(good)


def test_block_table_declared_past_its_allocation_is_refused():
    _, pool_t, stg, tab = _setup()
    entries = (_alloc_end(tab.data_ptr()) - tab.data_ptr()) // 4
    if entries + 1 > 2**31 - 1:
        pytest.skip("the allocations after the table reach past a 31-bit table length")
    p = _pool(pool_t)
    stream = torch.cuda.current_stream()
    try:
        # one page read (entry 0), table declared one entry longer than its allocation
        spans = K.make_spans([(tab, entries + 1, 0, BS, 0)])
        for fn in (K.kv_gather_chunks, K.kv_scatter_chunks):
            with pytest.raises(K.KvError) as e:
                fn(p, spans, _spec(stg, 4), stream)
            assert e.value.code == K.KV_ERR_RANGE
        torch.cuda.synchronize()
        assert bool((pool_t == 7).all()) and bool((stg == W.SENTINEL).all())
        K.kv_gather_chunks(p, K.make_spans([(tab, entries, 0, BS, 0)]), _spec(stg, 4), stream)
        assert K.kv_pool_get_error(p, stream) == 0
    finally:
        K.kv_pool_destroy(p)
