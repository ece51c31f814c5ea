"""Host-side tests of the C ABI (no GPU): exports, validation, decomposition sizes,
allocator, ring-slot ownership, table checks.  Every check here runs before the
library makes any HIP call, so it works in a CPU-only container."""
from __future__ import annotations

import ctypes
import json
import os
import re

import numpy as np
import pytest

from paged_layout_transfer_amd import kvxfer as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvxfer.h")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

FAKE = 0x7F0000000000  # 16-byte aligned stand-in device addresses, never dereferenced


def _desc(L=2, KV=2, H=2, D=64, E=2, bs=16, N=64, stride=None, bases=None, page_layout=0):
    tok = H * D * E
    if stride is None:
        stride = bs * tok
    if bases is None:
        bases = [FAKE + i * (1 << 30) for i in range(L * KV)]
    return K.make_pool_desc(L, KV, H, D, E, bs, N, stride, bases, page_layout)


def _spec(**kw):
    a = dict(layout=K.KV_LAYER_FIRST, chunk_layers=2, chunk_tokens=256, layer_begin=0, layer_end=2,
             base=FAKE + (1 << 40), slot_bytes=256 * 1024, n_slots=1, max_workgroups=0, flags=0)
    a.update(kw)
    return K.make_chunk_spec(**a)


def _span(t0=0, t1=256, fc=0, tbl=FAKE + (1 << 39), n=None, bs=16):
    return (tbl, -(-t1 // bs) if n is None else n, t0, t1, fc)


def test_header_symbols_are_exported():
    decl = set(re.findall(r"KV_API\s+[\w\s\*]*?\b(kv_\w+)\s*\(", open(HEADER).read()))
    assert decl == set(K.EXPORTED)
    for name in decl:
        assert hasattr(K._lib, name)


def test_header_constants_match_binding():
    text = open(HEADER).read()
    for name, val in re.findall(r"#define\s+(KV_[A-Z_0-9]+)\s+\(?(-?(?:0x)?[0-9a-fA-F]+)\)?", text):
        if name == "KV_API":
            continue
        assert getattr(K, name) == int(val, 0), name


def test_version_and_strerror():
    assert K.kv_version() == K.KV_VERSION
    codes = [K.KV_OK, K.KV_ERR_ARG, K.KV_ERR_ALIGN, K.KV_ERR_RANGE, K.KV_ERR_OOM, K.KV_ERR_RING,
             K.KV_ERR_HIP, K.KV_ERR_DEVICE, K.KV_ERR_DUP, K.KV_ERR_SCRATCH,
             K.KV_ERR_CAPTURE]
    msgs = [K.kv_strerror(c) for c in codes]
    assert len(set(msgs)) == len(codes)
    assert K.kv_strerror(12345) == "unknown error"


def test_valid_call_sizes_tiny():
    info = K.kv_check_transfer(_desc(), K.make_spans([_span()]), _spec())
    assert (info.tiles, info.chunks) == (2 * 2 * 16, 1)
    assert info.payload_bytes == info.max_chunk_bytes == 256 * 1024


def test_tile_counts_from_the_pages():
    fx = json.load(open(os.path.join(GOLDEN, "page_sizes.json")))["fragmentation_example"]
    bs, T, L = fx["page_tokens"], fx["context_tokens"], fx["layers"]
    d = _desc(L=L, KV=1, H=8, D=128, E=2, bs=bs, N=T // bs)
    spec = _spec(chunk_layers=1, chunk_tokens=T, layer_end=L, slot_bytes=T * 2048, n_slots=L)
    info = K.kv_check_transfer(d, K.make_spans([_span(0, T, bs=bs)]), spec)
    assert info.tiles == fx["transfers_per_request"]
    assert info.tiles // L == fx["transfers_per_layer"]
    assert info.payload_bytes // info.tiles == fx["approx_bytes_per_layer_page"]
    one_layer = _spec(chunk_layers=1, chunk_tokens=T, layer_begin=3, layer_end=4, slot_bytes=T * 2048)
    assert K.kv_check_transfer(d, K.make_spans([_span(0, T, bs=bs)]), one_layer).tiles == fx["transfers_per_layer"]


@pytest.mark.parametrize("layout,tokens,expect", [
    (K.KV_LAYER_FIRST, 256, 32 * 2 * 256 * 2048),   # llama8b chunk: 32 MiB
    (K.KV_LAYER_FIRST, 100, 32 * 2 * 100 * 2048),   # short last chunk stays dense
    (K.KV_PAGE_FIRST, 256, 32 * 2 * 256 * 2048),
    (K.KV_PAGE_FIRST, 100, 7 * 32 * 2 * 16 * 2048),  # page-first pads to whole pages
])
def test_chunk_bytes(layout, tokens, expect):
    d = _desc(L=32, KV=2, H=8, D=128, E=2, bs=16, N=16)
    assert K.kv_chunk_bytes(d, _spec(layout=layout, chunk_layers=32, layer_end=32), tokens) == expect


def test_chunk_bytes_of_the_workloads():
    llama70b = _desc(L=80, KV=2, H=8, D=128, E=2, bs=16, N=16)
    assert K.kv_chunk_bytes(llama70b, _spec(chunk_layers=1, chunk_tokens=512, layer_end=80), 512) == 2 << 20
    mla = _desc(L=61, KV=1, H=1, D=576, E=1, bs=64, N=16)
    assert K.kv_chunk_bytes(mla, _spec(layout=1, chunk_layers=61, chunk_tokens=64, layer_end=61), 64) == 61 * 64 * 576
    i8 = _desc(L=61, KV=2, H=8, D=128, E=1, bs=64, N=16)
    assert K.kv_chunk_bytes(i8, _spec(layout=1, chunk_layers=61, chunk_tokens=64, layer_end=61), 64) == 61 * 2 * 64 * 1024


# ---- validation matrix ---------------------------------------------------------------

POOL_CASES = [
    (dict(KV=3), K.KV_ERR_ARG),
    (dict(L=0), K.KV_ERR_ARG),
    (dict(E=3), K.KV_ERR_ARG),
    (dict(N=0), K.KV_ERR_ARG),
    (dict(H=1, D=4, E=2), K.KV_ERR_ALIGN),            # 8-byte tokens
    (dict(stride=4096 - 16), K.KV_ERR_ARG),          # stride below the page
    (dict(stride=4096 + 8), K.KV_ERR_ALIGN),
    (dict(bases=[FAKE, FAKE + 8, FAKE, FAKE]), K.KV_ERR_ALIGN),
    (dict(bases=[FAKE, 0, FAKE, FAKE]), K.KV_ERR_ARG),
    (dict(page_layout=2), K.KV_ERR_ARG),
    (dict(H=8, D=1, E=2, page_layout=1), K.KV_ERR_ALIGN),   # 2-byte head rows
    (dict(H=8, D=3, E=2, page_layout=1), K.KV_ERR_ALIGN),   # 6-byte head rows (tokens of 48 B)
    (dict(H=1026, D=8, E=1, page_layout=1), K.KV_ERR_ARG),  # 8-byte rows, token over 8 KiB
]


@pytest.mark.parametrize("kw,code", POOL_CASES)
def test_pool_create_rejects(kw, code):
    with pytest.raises(K.KvError) as e:
        K.kv_pool_create(_desc(**kw))
    assert e.value.code == code


CALL_CASES = [
    (dict(), [_span(t0=3)], K.KV_ERR_ARG),                    # t_begin not on a page boundary
    (dict(), [_span(t0=32, t1=16)], K.KV_ERR_ARG),            # inverted range
    (dict(), [_span(fc=-1)], K.KV_ERR_ARG),
    (dict(), [_span(n=15)], K.KV_ERR_RANGE),                  # span past its table
    (dict(), [_span(tbl=0)], K.KV_ERR_ARG),                   # null table
    (dict(chunk_tokens=250), [_span()], K.KV_ERR_ARG),        # chunk_tokens not whole pages
    (dict(chunk_tokens=8), [_span()], K.KV_ERR_ARG),          # below one page
    (dict(chunk_layers=3, layer_end=2), [_span()], K.KV_ERR_ARG),
    (dict(layer_begin=1, layer_end=1), [_span()], K.KV_ERR_ARG),
    (dict(layer_end=3), [_span()], K.KV_ERR_ARG),
    (dict(layout=2), [_span()], K.KV_ERR_ARG),
    (dict(base=0), [_span()], K.KV_ERR_ARG),
    (dict(base=FAKE + 4), [_span()], K.KV_ERR_ALIGN),
    (dict(slot_bytes=256 * 1024 - 16), [_span()], K.KV_ERR_RANGE),  # chunk does not fit
    (dict(), [_span(n=1 << 31)], K.KV_ERR_RANGE),   # declared table length past the 31-bit limit
    (dict(slot_bytes=256 * 1024 + 8), [_span()], K.KV_ERR_ALIGN),
    (dict(n_slots=0), [_span()], K.KV_ERR_ARG),
    (dict(max_workgroups=-1), [_span()], K.KV_ERR_ARG),
    (dict(flags=0x100), [_span()], K.KV_ERR_ARG),
    (dict(flags=0x10), [_span()], K.KV_ERR_ARG),     # the first bit past KV_FLAG_PAGE_RUNS
    # ring ownership: two spans, one chunk each, same slot
    (dict(n_slots=4), [_span(fc=1), _span(fc=5)], K.KV_ERR_RING),
    (dict(n_slots=1), [_span(fc=0), _span(fc=1)], K.KV_ERR_RING),   # more chunks than slots
    (dict(n_slots=4, chunk_tokens=64), [_span(fc=3), _span(t1=64, fc=0)], K.KV_ERR_RING),  # wraps onto slot 0
]


@pytest.mark.parametrize("spec_kw,spans,code", CALL_CASES)
def test_call_validation(spec_kw, spans, code):
    d = _desc()
    sp = K.make_spans(spans)
    with pytest.raises(K.KvError) as e:
        K.kv_check_transfer(d, sp, _spec(**spec_kw))
    assert e.value.code == code
    # the transfer entry points reject the same call before touching the GPU
    pool = K.kv_pool_create(d)
    try:
        for fn in (K.kv_gather_chunks, K.kv_scatter_chunks):
            with pytest.raises(K.KvError) as e2:
                fn(pool, sp, _spec(**spec_kw))
            assert e2.value.code == code
    finally:
        K.kv_pool_destroy(pool)


def test_ring_arcs():
    d = _desc()
    ok = K.make_spans([_span(fc=6, t1=64), _span(fc=0, t1=32), _span(fc=1, t1=96)])  # slots {6,7},{0},{1,2,3}
    info = K.kv_check_transfer(d, ok, _spec(n_slots=8, chunk_tokens=32))
    assert info.chunks == 6
    wrap = K.make_spans([_span(fc=7, t1=64), _span(fc=1, t1=32)])  # slots {7,0},{1}
    assert K.kv_check_transfer(d, wrap, _spec(n_slots=8, chunk_tokens=32)).chunks == 3
    clash = K.make_spans([_span(fc=7, t1=64), _span(fc=8, t1=32)])  # slot 0 twice (8 mod 8)
    with pytest.raises(K.KvError) as e:
        K.kv_check_transfer(d, clash, _spec(n_slots=8, chunk_tokens=32))
    assert e.value.code == K.KV_ERR_RING


def test_empty_calls_need_no_gpu():
    d = _desc()
    pool = K.kv_pool_create(d)
    try:
        K.kv_gather_chunks(pool, K.make_spans([]), _spec())             # no spans
        K.kv_scatter_chunks(pool, K.make_spans([_span(32, 32)]), _spec())  # one empty span
        assert K.kv_pool_get_error(pool) == 0                            # never touched a device
    finally:
        K.kv_pool_destroy(pool)
    info = K.kv_check_transfer(d, K.make_spans([_span(32, 32)]), _spec())
    assert (info.tiles, info.chunks, info.payload_bytes) == (0, 0, 0)


def test_partial_pages_and_layer_ranges():
    d = _desc(L=4, KV=2, N=64)
    sp = K.make_spans([_span(16, 16 + 33)])     # 33 tokens: 3 pages, last has 1 token
    info = K.kv_check_transfer(d, sp, _spec(chunk_layers=1, layer_begin=1, layer_end=3, chunk_tokens=32,
                                            slot_bytes=32 * 2 * 256, n_slots=4))
    assert info.tiles == 2 * 2 * 3
    assert info.chunks == 2 * 2
    assert info.payload_bytes == 2 * 2 * 33 * 256


def test_spans_limit():
    d = _desc()
    too_many = K.make_spans([_span(0, 0)] * (K.KV_MAX_SPANS + 1))
    with pytest.raises(K.KvError) as e:
        K.kv_check_transfer(d, too_many, _spec())
    assert e.value.code == K.KV_ERR_ARG


def test_timing_read_each_rejects_bad_arguments():
    """Argument errors are caught before any HIP call (so this runs without a GPU)."""
    pool = K.kv_pool_create(_desc(N=10))
    try:
        n = ctypes.c_int64()
        assert K._lib.kv_pool_timing_read_each(pool, None, -1, ctypes.byref(n)) == K.KV_ERR_ARG
        assert K._lib.kv_pool_timing_read_each(pool, None, 4, ctypes.byref(n)) == K.KV_ERR_ARG
        assert K._lib.kv_pool_timing_read_each(pool, None, 0, None) == K.KV_ERR_ARG
        assert K._lib.kv_pool_timing_read_each(None, None, 0, ctypes.byref(n)) == K.KV_ERR_ARG
        # nothing timed yet: no launches, no HIP call
        assert K._lib.kv_pool_timing_read_each(pool, None, 0, ctypes.byref(n)) == K.KV_OK and n.value == 0
    finally:
        K.kv_pool_destroy(pool)


# ---- allocator --------------------------------------------------------------------------

def test_allocator_hands_out_lowest_free_ids_in_order():
    """Lowest free ids first, ascending, whatever order they were freed in; across
    64-bit bitmap words; against a plain set model over a random alloc/free history."""
    N = 300
    pool = K.kv_pool_create(_desc(N=N))
    try:
        assert K.kv_pool_alloc_blocks(pool, 5).tolist() == [0, 1, 2, 3, 4]
        rng = np.random.default_rng(5)
        held = set(range(5))
        for _ in range(400):
            if held and rng.random() < 0.5:
                k = int(rng.integers(1, len(held) + 1))
                ids = rng.permutation(sorted(held))[:k]
                K.kv_pool_free_blocks(pool, ids)
                held -= set(ids.tolist())
            else:
                free = sorted(set(range(N)) - held)
                k = int(rng.integers(0, min(len(free), 70) + 1))
                got = K.kv_pool_alloc_blocks(pool, k).tolist()
                assert got == free[:k]
                held |= set(got)
            assert K.kv_pool_free_count(pool) == N - len(held)
    finally:
        K.kv_pool_destroy(pool)


def test_allocator():
    pool = K.kv_pool_create(_desc(N=10))
    try:
        a = K.kv_pool_alloc_blocks(pool, 4)
        assert len(set(a.tolist())) == 4 and all(0 <= x < 10 for x in a)
        assert K.kv_pool_free_count(pool) == 6
        with pytest.raises(K.KvError) as e:
            K.kv_pool_alloc_blocks(pool, 7)
        assert e.value.code == K.KV_ERR_OOM
        assert K.kv_pool_free_count(pool) == 6                     # failed alloc took nothing
        b = K.kv_pool_alloc_blocks(pool, 6)
        assert set(a.tolist()) | set(b.tolist()) == set(range(10))
        K.kv_pool_free_blocks(pool, a[:2])
        with pytest.raises(K.KvError) as e:
            K.kv_pool_free_blocks(pool, a[1:3])                    # a[1] already free
        assert e.value.code == K.KV_ERR_RANGE
        assert K.kv_pool_free_count(pool) == 2                     # nothing freed by the bad call
        with pytest.raises(K.KvError):
            K.kv_pool_free_blocks(pool, [a[2], a[2]])              # duplicate within a call
        with pytest.raises(K.KvError):
            K.kv_pool_free_blocks(pool, [10])                      # out of range
        assert K.kv_pool_free_count(pool) == 2
        K.kv_pool_free_blocks(pool, np.concatenate([a[2:], b]))
        assert K.kv_pool_free_count(pool) == 10
        assert sorted(K.kv_pool_alloc_blocks(pool, 10).tolist()) == list(range(10))
    finally:
        K.kv_pool_destroy(pool)


# ---- host table checks --------------------------------------------------------------------

def test_validate_targets():
    d = _desc(N=8, bs=4, D=8, H=1, E=2)  # 16-byte tokens
    t_ok = np.array([0, 1, 2, 3], dtype=np.int32)
    t_bad = np.array([0, 1, 8, 3], dtype=np.int32)
    spans = K.make_spans([(0, 4, 0, 16, 0)])
    K.kv_validate_targets(d, spans, [t_ok], K.KV_SCATTER)
    with pytest.raises(K.KvError) as e:
        K.kv_validate_targets(d, spans, [t_bad], K.KV_GATHER)
    assert e.value.code == K.KV_ERR_RANGE
    # a page shared by two spans: fine to read twice, not to write twice
    two = K.make_spans([(0, 4, 0, 16, 0), (0, 2, 4, 8, 4)])
    t2 = np.array([5, 1], dtype=np.int32)
    K.kv_validate_targets(d, two, [t_ok, t2], K.KV_GATHER)
    with pytest.raises(K.KvError) as e:
        K.kv_validate_targets(d, two, [t_ok, t2], K.KV_SCATTER)
    assert e.value.code == K.KV_ERR_DUP
    # only the pages a span touches are checked: the prefix page before t_begin may be anything
    tail = K.make_spans([(0, 4, 8, 16, 0)])
    K.kv_validate_targets(d, tail, [np.array([-5, 99, 6, 7], dtype=np.int32)], K.KV_SCATTER)


def test_per_tile_dma_validates_host_tables_before_any_hip_call():
    d = _desc(N=8, bs=4, D=8, H=1, E=2)  # 16-byte tokens
    pool = K.kv_pool_create(d)
    try:
        bad = np.array([0, 1, 8, 3], dtype=np.int32)
        dup = np.array([0, 1, 1, 3], dtype=np.int32)
        spec = _spec(chunk_layers=2, chunk_tokens=16, slot_bytes=2 * 2 * 16 * 16, n_slots=1)
        for tbl, fn, code in ((bad, K.kv_gather_chunks_dma, K.KV_ERR_RANGE),
                              (dup, K.kv_scatter_chunks_dma, K.KV_ERR_DUP)):
            with pytest.raises(K.KvError) as e:
                fn(pool, K.make_spans([(tbl.ctypes.data, 4, 0, 16, 0)]), spec)
            assert e.value.code == code
        good = np.array([0, 1, 2, 3], dtype=np.int32)
        with pytest.raises(K.KvError) as e:   # valid: gets as far as the first copy, no device here
            K.kv_gather_chunks_dma(pool, K.make_spans([(good.ctypes.data, 4, 0, 16, 0)]), spec)
        assert e.value.code == K.KV_ERR_HIP
    finally:
        K.kv_pool_destroy(pool)


def test_ring_functions_reject_null_handles():
    for fn, args in ((K._lib.kv_ring_record, (None, 0, 1, None)), (K._lib.kv_ring_wait, (None, 0, 1)),
                     (K._lib.kv_ring_stream_wait, (None, 0, 1, None)), (K._lib.kv_ring_slot, (None, 0, None, None))):
        assert fn(*args) == K.KV_ERR_ARG
    assert K._lib.kv_ring_destroy(None) == K.KV_OK
    assert K._lib.kv_pool_destroy(None) == K.KV_OK


def test_noalloc_entry_refuses_before_any_hip_call():
    """The no-allocation entry point's own limits are checked on the host first: a bad
    direction, KV_FLAG_VALIDATE (its table check copies to the host), more regions than
    its static scratch holds, a misaligned error word; an empty call is a no-op."""
    h = K.kv_pool_create(_desc())
    try:
        sp = K.make_spans([_span()])
        for direction, spec, err, code in ((7, _spec(), None, K.KV_ERR_ARG),
                                           (K.KV_GATHER, _spec(flags=K.KV_FLAG_VALIDATE), None, K.KV_ERR_ARG),
                                           (K.KV_SCATTER, _spec(), FAKE + 2, K.KV_ERR_ALIGN)):
            with pytest.raises(K.KvError) as e:
                K.kv_transfer_chunks_noalloc(h, direction, sp, spec, err)
            assert e.value.code == code
        K.kv_transfer_chunks_noalloc(h, K.KV_GATHER, K.make_spans([_span(t1=0)]), _spec())
    finally:
        K.kv_pool_destroy(h)
    L = 513  # 1026 regions
    big = K.kv_pool_create(_desc(L=L, bases=[FAKE + i * (1 << 24) for i in range(2 * L)]))
    try:
        with pytest.raises(K.KvError) as e:
            K.kv_transfer_chunks_noalloc(big, K.KV_SCATTER, K.make_spans([_span()]),
                                         _spec(chunk_layers=L, layer_end=L, slot_bytes=L * 2 * 256 * 256))
        assert e.value.code == K.KV_ERR_SCRATCH
    finally:
        K.kv_pool_destroy(big)
