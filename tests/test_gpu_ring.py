"""A small pinned ring used as a double-buffered queue, fenced with kv_ring_record /
kv_ring_wait, for an offload and a reload that are larger than the ring.

Offload: window i (two layers) is gathered into half i % 2 of the ring and
recorded; the gather of window i + 1 is queued before the host drains window i
(after waiting on its slots), so GPU writes and host reads of the two halves
overlap.  Reload: the host refills a half only after waiting for the scatter that
last read it.  The drained host copy must equal the oracle's gather of the whole
call, and the reloaded pool the oracle's scatter of it.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import cases
import oracle
from paged_layout_transfer_amd import kvxfer as K
from paged_layout_transfer_amd import workloads as W

pytestmark = pytest.mark.gpu


def test_double_buffered_ring_offload_and_reload():
    dev = torch.device("cuda", 0)
    L, KV, H, D, E, bs, N = 6, 2, 2, 64, 2, 16, 64
    tok = H * D * E
    T = 600                         # 38 pages, last one partial
    CT, CL, win = 256, 1, 2         # 3 token chunks per layer, 2 layers per window
    n_tc = cases.cdiv(T, CT)
    per_win = win * n_tc            # 6 slots per half
    slot = CL * KV * CT * tok
    pool = dict(num_layers=L, num_kv=KV, num_heads=H, head_dim=D, elem_bytes=E, block_size=bs,
                num_blocks=N, block_stride=bs * tok)
    rng = np.random.default_rng(80_000)
    table = rng.permutation(N)[:cases.cdiv(T, bs)].astype(np.int32)
    regions = rng.integers(0, 256, size=(L * KV, N * bs * tok), dtype=np.uint8)

    pool_d = torch.from_numpy(regions).to(dev)
    fresh_d = torch.full_like(pool_d, W.SENTINEL)
    tab_d = torch.from_numpy(table).to(dev)

    def make(t):
        return K.kv_pool_create(K.make_pool_desc(L, KV, H, D, E, bs, N, bs * tok,
                                                 [t.data_ptr() + i * t.stride(0) for i in range(L * KV)]))

    src, dst = make(pool_d), make(fresh_d)
    ring = K.kv_ring_create(slot, 2 * per_win)
    host = K.ring_host_array(ring, slot * 2 * per_win)
    stream = torch.cuda.current_stream()
    cache = np.empty(slot * per_win * (L // win), dtype=np.uint8)   # the host's copy of the context
    try:
        ring_dev = K.kv_ring_slot(ring, 0)[1]

        def spec(i):
            return K.make_chunk_spec(K.KV_LAYER_FIRST, CL, CT, i * win, (i + 1) * win, ring_dev, slot,
                                     2 * per_win)

        def span(i):
            return K.make_spans([(tab_d, table.size, 0, T, (i % 2) * per_win)])

        def drain(i):
            h = i % 2
            K.kv_ring_wait(ring, h * per_win, per_win)
            cache[i * per_win * slot:(i + 1) * per_win * slot] = host[h * per_win * slot:(h + 1) * per_win * slot]

        print("[ring] offload through a 2 x %d-slot ring" % per_win, flush=True)
        for i in range(L // win):
            K.kv_gather_chunks(src, span(i), spec(i), stream)
            K.kv_ring_record(ring, (i % 2) * per_win, per_win, stream)
            if i > 0:
                drain(i - 1)             # overlaps with the gather just queued
        drain(L // win - 1)
        assert K.kv_pool_get_error(src, stream) == 0

        print("[ring] reload through the ring", flush=True)
        host[:] = 0
        for i in range(L // win):
            h = i % 2
            K.kv_ring_wait(ring, h * per_win, per_win)   # the scatter that last read this half is done
            host[h * per_win * slot:(h + 1) * per_win * slot] = cache[i * per_win * slot:(i + 1) * per_win * slot]
            K.kv_scatter_chunks(dst, span(i), spec(i), stream)
            K.kv_ring_record(ring, h * per_win, per_win, stream)
        assert K.kv_pool_get_error(dst, stream) == 0
        torch.cuda.synchronize()
        got_pool = fresh_d.cpu().numpy()
    finally:
        torch.cuda.synchronize()
        K.kv_pool_destroy(src)
        K.kv_pool_destroy(dst)
        K.kv_ring_destroy(ring)

    chunks = dict(layout=0, chunk_layers=CL, chunk_tokens=CT, layer_begin=0, layer_end=L,
                  slot_bytes=slot, n_slots=L * n_tc)
    # the oracle's gather over two different fills: where both agree, it wrote
    expect = np.full(slot * L * n_tc, 0xEE, dtype=np.uint8)
    expect2 = np.full(slot * L * n_tc, 0x11, dtype=np.uint8)
    oracle.gather(pool, regions, [(table, 0, T, 0)], chunks, expect)
    oracle.gather(pool, regions, [(table, 0, T, 0)], chunks, expect2)
    written = expect == expect2
    assert np.array_equal(cache[written], expect[written])
    # the reload read only written bytes, so it must equal the oracle's scatter of its own gather
    exp_pool = np.full_like(regions, W.SENTINEL)
    oracle.scatter(pool, exp_pool, [(table, 0, T, 0)], chunks, expect)
    assert np.array_equal(got_pool, exp_pool)


def test_ring_fencing_rejects_bad_ranges():
    ring = K.kv_ring_create(4096, 8)
    try:
        for first, count in ((-1, 1), (8, 1), (0, 0), (0, 9)):
            with pytest.raises(K.KvError) as e:
                K.kv_ring_record(ring, first, count, 0)
            assert e.value.code == K.KV_ERR_ARG
            with pytest.raises(K.KvError):
                K.kv_ring_wait(ring, first, count)
        K.kv_ring_wait(ring, 0, 8)            # nothing recorded yet: returns at once
        K.kv_ring_record(ring, 6, 4, 0)       # wraps to slots 6, 7, 0, 1
        K.kv_ring_wait(ring, 7, 2)
        K.kv_ring_stream_wait(ring, 0, 8, 0)
        torch.cuda.synchronize()
    finally:
        K.kv_ring_destroy(ring)


@pytest.mark.parametrize("grids", [(0, 0), (6, 2)])
def test_offload_and_reload_at_once_on_two_streams(grids):
    """A reload (scatter of layers [0, 4) from one pinned ring) and an offload (gather of
    layers [4, 8) into another) queued on two streams with nothing ordering them, so
    both directions of the host link are in use at once; several windows each.  The
    default grids and the 6 / 2 split that measured fastest for such a pair.  The
    pool must equal the oracle's scatter of the reload rings (the offloaded layers and
    every block outside the table unchanged), and each offload ring the oracle's
    gather."""
    dev = torch.device("cuda", 0)
    L, KV, H, D, E, bs, N = 8, 2, 4, 64, 2, 16, 96
    tok = H * D * E
    T = 1000                        # 63 pages, last one partial
    CT, CL, win = 256, 1, 2
    n_tc = cases.cdiv(T, CT)
    n_slots = win * n_tc
    slot = CL * KV * CT * tok
    pool = dict(num_layers=L, num_kv=KV, num_heads=H, head_dim=D, elem_bytes=E, block_size=bs,
                num_blocks=N, block_stride=bs * tok)
    rng = np.random.default_rng(80_500 + grids[0])
    table = rng.permutation(N)[:cases.cdiv(T, bs)].astype(np.int32)
    regions = rng.integers(0, 256, size=(L * KV, N * bs * tok), dtype=np.uint8)
    src = rng.integers(0, 256, size=(L // 2 // win, slot * n_slots), dtype=np.uint8)   # per reload window
    pool_d = torch.from_numpy(regions).to(dev)
    tab_d = torch.from_numpy(table).to(dev)
    h = K.kv_pool_create(K.make_pool_desc(L, KV, H, D, E, bs, N, bs * tok,
                                          [pool_d.data_ptr() + i * pool_d.stride(0) for i in range(L * KV)]))
    n_win = L // 2 // win
    rings_in = [K.kv_ring_create(slot, n_slots) for _ in range(n_win)]
    rings_out = [K.kv_ring_create(slot, n_slots) for _ in range(n_win)]
    s_in, s_out = torch.cuda.Stream(), torch.cuda.Stream()
    try:
        for i, r in enumerate(rings_in):
            K.ring_host_array(r, slot * n_slots)[:] = src[i]
        for r in rings_out:
            K.ring_host_array(r, slot * n_slots)[:] = W.SENTINEL
        spans = K.make_spans([(tab_d, tab_d.numel(), 0, T, 0)])

        def spec(l0, ring, wg):
            return K.make_chunk_spec(K.KV_LAYER_FIRST, CL, CT, l0, l0 + win, K.kv_ring_slot(ring, 0)[1], slot,
                                     n_slots, wg)

        torch.cuda.synchronize()
        print("[gpu] reload layers 0-3 and offload layers 4-7 at once, grids %s" % (grids,), flush=True)
        for i in range(n_win):
            K.kv_scatter_chunks(h, spans, spec(i * win, rings_in[i], grids[0]), s_in)
            K.kv_gather_chunks(h, spans, spec(L // 2 + i * win, rings_out[i], grids[1]), s_out)
        torch.cuda.synchronize()
        assert K.kv_pool_get_error(h, torch.cuda.current_stream()) == 0
        got = pool_d.cpu().numpy()
        exp = regions.copy()
        for i in range(n_win):
            ch = dict(layout=K.KV_LAYER_FIRST, chunk_layers=CL, chunk_tokens=CT, layer_begin=i * win,
                      layer_end=(i + 1) * win, slot_bytes=slot, n_slots=n_slots)
            oracle.scatter(pool, [exp[r] for r in range(L * KV)], [(table, 0, T, 0)], ch, src[i].copy(),
                           only_layers=(i * win, (i + 1) * win))
        assert np.array_equal(got, exp), "pool after the reload differs from the oracle"
        for i in range(n_win):
            ch = dict(layout=K.KV_LAYER_FIRST, chunk_layers=CL, chunk_tokens=CT, layer_begin=L // 2 + i * win,
                      layer_end=L // 2 + (i + 1) * win, slot_bytes=slot, n_slots=n_slots)
            want = np.full(slot * n_slots, W.SENTINEL, dtype=np.uint8)
            oracle.gather(pool, [regions[r] for r in range(L * KV)], [(table, 0, T, 0)], ch, want,
                          only_layers=(L // 2 + i * win, L // 2 + (i + 1) * win))
            assert np.array_equal(K.ring_host_array(rings_out[i], slot * n_slots), want), \
                "offload window %d differs from the oracle" % i
    finally:
        torch.cuda.synchronize()
        for r in rings_in + rings_out:
            K.kv_ring_destroy(r)
        K.kv_pool_destroy(h)
