"""Many transfer calls queued back to back with no synchronisation in between.

320 calls exceed the 256 calls the library keeps in flight.  Most move one
three-page request; every eighth call carries 4096 one-page requests, i.e. 4096
span records, which go through the pool's 4 MiB device span-record arena
(256 KiB per such call), so the arena wraps several times while earlier calls are
still queued and its stretches are reused only after their calls have finished.
Every request owns distinct pages and staging slots, and some end in a partial
page.  The result must equal the oracle's single call over all requests, in both
directions.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from paged_layout_transfer_amd import kvxfer as K
from paged_layout_transfer_amd import workloads as W

pytestmark = pytest.mark.gpu


def test_deep_queue_of_calls_through_the_record_arena():
    dev = torch.device("cuda", 0)
    L, KV, H, D, E, bs, calls = 2, 1, 1, 32, 2, 2, 320
    tok = H * D * E
    big = K.KV_MAX_SPANS
    n_req = (calls // 8) * big + (calls - calls // 8) * 1
    n_pages = (calls // 8) * big + (calls - calls // 8) * 3
    N = n_pages + 1000
    slot = L * KV * bs * tok                 # one page of every layer per chunk
    pool = dict(num_layers=L, num_kv=KV, num_heads=H, head_dim=D, elem_bytes=E, block_size=bs,
                num_blocks=N, block_stride=bs * tok)
    rng = np.random.default_rng(90_000)
    table = rng.permutation(N).astype(np.int32)
    regions = rng.integers(0, 256, size=(L * KV, N * bs * tok), dtype=np.uint8)
    pool_d = torch.from_numpy(regions).to(dev)
    fresh_d = torch.full_like(pool_d, W.SENTINEL)
    tab_d = torch.from_numpy(table).to(dev)

    # requests: (t_begin, t_end, first_chunk) over the one shared table, pages in order
    page = chunk = 0
    call_spans, host_spans = [], []
    for i in range(calls):
        reqs = []
        for _ in range(big if i % 8 == 0 else 1):
            n = 1 if i % 8 == 0 else 3
            t0 = page * bs
            t1 = t0 + n * bs - int(rng.integers(0, 2))      # some end in a partial page
            reqs.append((t0, t1, chunk))
            page += n
            chunk += n
        call_spans.append(K.make_spans([(tab_d, N, t0, t1, fc) for t0, t1, fc in reqs]))
        host_spans += [(table, t0, t1, fc) for t0, t1, fc in reqs]
    assert page == n_pages and len(host_spans) == n_req
    stg_d = torch.full((chunk * slot,), W.SENTINEL, dtype=torch.uint8, device=dev)
    spec = K.make_chunk_spec(K.KV_LAYER_FIRST, L, bs, 0, L, stg_d, slot, chunk)

    def make(t):
        return K.kv_pool_create(K.make_pool_desc(L, KV, H, D, E, bs, N, bs * tok,
                                                 [t.data_ptr() + i * t.stride(0) for i in range(L * KV)]))

    src, dst = make(pool_d), make(fresh_d)
    stream = torch.cuda.current_stream()
    try:
        print("[queue] %d gathers, then %d scatters, %d requests, no sync between calls" % (
            calls, calls, n_req), flush=True)
        for sp in call_spans:
            K.kv_gather_chunks(src, sp, spec, stream)
        for sp in call_spans:
            K.kv_scatter_chunks(dst, sp, spec, stream)
        assert K.kv_pool_get_error(src, stream) == 0 and K.kv_pool_get_error(dst, stream) == 0
        torch.cuda.synchronize()
        got_stg = stg_d.cpu().numpy()
        got_pool = fresh_d.cpu().numpy()
    finally:
        K.kv_pool_destroy(src)
        K.kv_pool_destroy(dst)

    chunks = dict(layout=0, chunk_layers=L, chunk_tokens=bs, layer_begin=0, layer_end=L,
                  slot_bytes=slot, n_slots=chunk)
    exp_stg = np.full(chunk * slot, W.SENTINEL, dtype=np.uint8)
    oracle.gather(pool, regions, host_spans, chunks, exp_stg)
    assert np.array_equal(got_stg, exp_stg)
    exp_pool = np.full_like(regions, W.SENTINEL)
    oracle.scatter(pool, exp_pool, host_spans, chunks, exp_stg)
    assert np.array_equal(got_pool, exp_pool)


def test_timing_reports_each_launch():
    dev = torch.device("cuda", 0)
    L, KV, H, D, E, bs, N = 2, 2, 2, 64, 2, 16, 64
    tok = H * D * E
    pool_d = torch.zeros((L * KV, N * bs * tok), dtype=torch.uint8, device=dev)
    stg = torch.zeros(L * KV * 256 * tok, dtype=torch.uint8, device=dev)
    tab = torch.arange(16, dtype=torch.int32, device=dev)
    h = K.kv_pool_create(K.make_pool_desc(L, KV, H, D, E, bs, N, bs * tok,
                                          [pool_d.data_ptr() + i * pool_d.stride(0) for i in range(L * KV)]))
    spans = K.make_spans([(tab, 16, 0, 256, 0)])
    spec = K.make_chunk_spec(K.KV_LAYER_FIRST, L, 256, 0, L, stg, stg.numel(), 1)
    stream = torch.cuda.current_stream()
    try:
        print("[timing] 3 gathers, per-launch read; 2 scatters, summed read", flush=True)
        K.kv_pool_timing_start(h)
        for _ in range(3):
            K.kv_gather_chunks(h, spans, spec, stream)
        each = K.kv_pool_timing_read_each(h)
        assert each.size == 3 and np.all(each > 0)
        K.kv_pool_timing_start(h)
        for _ in range(2):
            K.kv_scatter_chunks(h, spans, spec, stream)
        total, n = K.kv_pool_timing_read(h)
        assert n == 2 and total > 0
        assert K.kv_pool_get_error(h, stream) == 0
    finally:
        torch.cuda.synchronize()
        K.kv_pool_destroy(h)


def test_one_pool_on_two_streams():
    """One pool handle used from two streams at once: gathers of two halves of a request
    on stream A and stream B, 60 calls each without synchronisation (they share the
    pool's span-record arena and error word), then scatters of both halves into a
    second pool, again split over the two streams.  Every result equals the oracle."""
    dev = torch.device("cuda", 0)
    L, KV, H, D, E, bs, N = 2, 2, 2, 64, 2, 16, 256
    tok = H * D * E
    pool = dict(num_layers=L, num_kv=KV, num_heads=H, head_dim=D, elem_bytes=E, block_size=bs,
                num_blocks=N, block_stride=bs * tok)
    rng = np.random.default_rng(91_000)
    table = rng.permutation(N)[:64].astype(np.int32)           # a 1024-token request
    regions = rng.integers(0, 256, size=(L * KV, N * bs * tok), dtype=np.uint8)
    src_d = torch.from_numpy(regions).to(dev)
    dst_d = torch.full_like(src_d, W.SENTINEL)
    tab_d = torch.from_numpy(table).to(dev)
    CT = 256
    slot = L * KV * CT * tok
    halves = [(0, 512), (512, 1024)]
    stg = [torch.full((2 * slot,), W.SENTINEL, dtype=torch.uint8, device=dev) for _ in halves]

    def make(t):
        return K.kv_pool_create(K.make_pool_desc(L, KV, H, D, E, bs, N, bs * tok,
                                                 [t.data_ptr() + i * t.stride(0) for i in range(L * KV)]))

    src, dst = make(src_d), make(dst_d)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    spans = [K.make_spans([(tab_d, 64, t0, t1, 0)]) for t0, t1 in halves]
    specs = [K.make_chunk_spec(K.KV_LAYER_FIRST, L, CT, 0, L, s, slot, 2) for s in stg]
    try:
        print("[streams] 2 x 60 gathers on two streams, then scatters on both", flush=True)
        torch.cuda.synchronize()
        for _ in range(60):
            for h in range(2):
                K.kv_gather_chunks(src, spans[h], specs[h], streams[h])
        for h in range(2):
            K.kv_scatter_chunks(dst, spans[h], specs[h], streams[h])
        torch.cuda.synchronize()
        assert K.kv_pool_get_error(src, streams[0]) == 0 and K.kv_pool_get_error(dst, streams[1]) == 0
        got_stg = [s.cpu().numpy() for s in stg]
        got_pool = dst_d.cpu().numpy()
    finally:
        torch.cuda.synchronize()
        K.kv_pool_destroy(src)
        K.kv_pool_destroy(dst)

    chunks = dict(layout=0, chunk_layers=L, chunk_tokens=CT, layer_begin=0, layer_end=L, slot_bytes=slot,
                  n_slots=2)
    exp_pool = np.full_like(regions, W.SENTINEL)
    for h, (t0, t1) in enumerate(halves):
        exp = np.full(2 * slot, W.SENTINEL, dtype=np.uint8)
        oracle.gather(pool, regions, [(table, t0, t1, 0)], chunks, exp)
        assert np.array_equal(got_stg[h], exp), "gather half %d" % h
        oracle.scatter(pool, exp_pool, [(table, t0, t1, 0)], chunks, exp)
    assert np.array_equal(got_pool, exp_pool)
