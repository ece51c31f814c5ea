"""CPU check of the kernel's tile indexing (no GPU).

tests/kernel_emu.cpp is compiled here together with the library's sources and
walks the exact grid-stride loop the kernel runs -- the library's own launch
preparation, span search and tile resolution -- on host buffers: every address
must stay inside its buffer and every tile must be visited once.  Small cases
also copy the bytes and must match the oracle; the workload-sized calls are
walked without copying (addresses and coverage only).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import pytest

import cases
import oracle
from paged_layout_transfer_amd import _build
from paged_layout_transfer_amd import kvxfer as K
from paged_layout_transfer_amd import workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))


def _build_emu(tmp_path_factory, defines=()):
    out = str(tmp_path_factory.mktemp("emu") / "libemu.so")
    cmd = [_build.HIPCC, *[f for f in _build.FLAGS if f != "-fvisibility=hidden"], *defines,
           "-I", os.path.join(_build.ROOT, "include"), "-I", _build.CSRC,
           *_build.SOURCES, os.path.join(HERE, "kernel_emu.cpp"), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    lib = ctypes.CDLL(out)
    lib.emu_transfer.restype = ctypes.c_int
    lib.emu_transfer.argtypes = [ctypes.c_int, ctypes.POINTER(K.kv_pool_desc), ctypes.POINTER(K.kv_span),
                                 ctypes.c_int32, ctypes.POINTER(K.kv_chunk_spec), ctypes.c_void_p,
                                 ctypes.c_int64, ctypes.c_int32, ctypes.POINTER(ctypes.c_int64),
                                 ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]
    lib.emu_arena.restype = ctypes.c_int64
    lib.emu_arena.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32]
    lib.emu_launch_block.restype = ctypes.c_uint32
    lib.emu_launch_block.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32]
    lib.emu_launch_rule.restype = ctypes.c_int
    lib.emu_launch_rule.argtypes = [ctypes.c_int, ctypes.POINTER(K.kv_pool_desc), ctypes.POINTER(K.kv_span),
                                    ctypes.c_int32, ctypes.POINTER(K.kv_chunk_spec), ctypes.POINTER(ctypes.c_int64)]
    lib.emu_gather_seg_unroll.restype = ctypes.c_int
    lib.emu_gather_seg_unroll.argtypes = [ctypes.c_int64, ctypes.c_int64]
    lib.emu_hm_page_ok.restype = ctypes.c_int32
    lib.emu_hm_page_ok.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
    lib.emu_hm_lds_tokens.restype = ctypes.c_uint32
    lib.emu_hm_lds_tokens.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_uint32]
    lib.emu_hm_lds_head_slab.restype = None
    lib.emu_hm_lds_head_slab.argtypes = [ctypes.c_int, ctypes.c_uint32, ctypes.c_int64, ctypes.c_int64, ctypes.c_uint32,
                                         ctypes.POINTER(ctypes.c_uint32), ctypes.POINTER(ctypes.c_uint32)]
    lib.emu_dma.restype = ctypes.c_int
    lib.emu_dma.argtypes = [ctypes.c_int, ctypes.POINTER(K.kv_pool_desc), ctypes.POINTER(K.kv_span),
                            ctypes.c_int32, ctypes.POINTER(K.kv_chunk_spec), ctypes.c_void_p, ctypes.c_int64,
                            ctypes.c_int32, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64),
                            ctypes.POINTER(ctypes.c_int64)]
    lib.emu_set_allocs.restype = None
    lib.emu_set_allocs.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32]
    lib.emu_covered_end.restype = ctypes.c_uint64
    lib.emu_covered_end.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int32]
    lib.emu_cache_reset.restype = None
    lib.emu_cache_covers.restype = ctypes.c_int32
    lib.emu_cache_covers.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)]
    return lib


@pytest.fixture(scope="module")
def emu(tmp_path_factory):
    return _build_emu(tmp_path_factory)


@pytest.fixture(scope="module")
def emu_split(tmp_path_factory):
    """The same walk with small parts, so tiles are split between 2-4 waves in both directions."""
    return _build_emu(tmp_path_factory, ("-DKVX_GATHER_PART_BYTES=256", "-DKVX_SCATTER_PART_BYTES=128",
                                         "-DKVX_GATHER_SPLIT_MIN=512", "-DKVX_SCATTER_SPLIT_MIN=256"))


def _emulate(lib, direction, pool, spans, chunks, bases, region_bytes, staging_ptr, staging_bytes,
             copy, max_workgroups=0):
    desc = K.make_pool_desc(pool["num_layers"], pool["num_kv"], pool["num_heads"], pool["head_dim"],
                            pool["elem_bytes"], pool["block_size"], pool["num_blocks"],
                            pool["block_stride"], bases, pool.get("page_layout", 0))
    tabs = [np.ascontiguousarray(t, dtype=np.int32) for t, _, _, _ in spans]
    sp = K.make_spans([(t.ctypes.data, t.size, t0, t1, fc) for t, (_, t0, t1, fc) in zip(tabs, spans)])
    spec = K.make_chunk_spec(chunks["layout"], chunks["chunk_layers"], chunks["chunk_tokens"],
                             chunks["layer_begin"], chunks["layer_end"], staging_ptr,
                             chunks["slot_bytes"], chunks["n_slots"], max_workgroups, 0)
    rb = np.ascontiguousarray(region_bytes, dtype=np.int64)
    viol, tiles, grid = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    rc = lib.emu_transfer(direction, ctypes.byref(desc), sp, len(spans), ctypes.byref(spec),
                          rb.ctypes.data, staging_bytes, int(copy), ctypes.byref(viol),
                          ctypes.byref(tiles), ctypes.byref(grid))
    assert rc == 0, K.kv_strerror(rc)
    return viol.value, tiles.value, grid.value


def _copy_case(lib, pool, spans, chunks, seed, max_workgroups=0):
    rng = np.random.default_rng(seed)
    regions = cases.regions_for(pool, rng)
    staging = cases.staging_for(chunks, rng=rng)
    n = regions.shape[0]
    for d in (K.KV_GATHER, K.KV_SCATTER):
        r_emu, s_emu = regions.copy(), staging.copy()
        bases = [r_emu[i].ctypes.data for i in range(n)]
        viol, _, _ = _emulate(lib, d, pool, spans, chunks, bases, [r_emu.shape[1]] * n,
                              s_emu.ctypes.data, s_emu.size, True, max_workgroups)
        assert viol == 0
        r_or, s_or = regions.copy(), staging.copy()
        oracle.transfer(d, pool, r_or, spans, chunks, s_or)
        assert np.array_equal(s_emu, s_or) and np.array_equal(r_emu, r_or)


@pytest.mark.parametrize("seed", range(60))
def test_emulated_kernel_matches_oracle_small(emu, seed):
    pool, spans, chunks = cases.make_case(np.random.default_rng(10_000 + seed), tok_multiple=16)
    _copy_case(emu, pool, spans, chunks, seed)


@pytest.mark.parametrize("seed", range(30))
def test_emulated_kernel_matches_oracle_medium(emu, seed):
    pool, spans, chunks = cases.make_case(np.random.default_rng(20_000 + seed), tok_multiple=16,
                                          medium=True, max_bytes=48 << 20)
    _copy_case(emu, pool, spans, chunks, seed, max_workgroups=int(seed % 4))


@pytest.mark.parametrize("seed", range(30))
def test_emulated_head_major_matches_oracle(emu, seed):
    pool, spans, chunks = cases.make_case(np.random.default_rng(27_000 + seed), tok_multiple=16,
                                          medium=bool(seed % 2), max_bytes=24 << 20, head_major=True)
    assert pool["page_layout"] == 1
    _copy_case(emu, pool, spans, chunks, seed, max_workgroups=int(seed % 3))


@pytest.mark.parametrize("seed", range(20))
def test_emulated_split_tiles_match_oracle(emu_split, seed):
    pool, spans, chunks = cases.make_case(np.random.default_rng(25_000 + seed), tok_multiple=16,
                                          medium=True, max_bytes=48 << 20, head_major=None)
    _copy_case(emu_split, pool, spans, chunks, seed, max_workgroups=int(seed % 3))


@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("name", sorted(cases.RULE_SHAPES))
def test_emulated_launch_rule_shapes_match_oracle(emu, name, layout):
    """The calls the GPU parity test runs at each launch rule's boundary: every access
    inside its buffer and the bytes equal to the oracle's."""
    pool, spans, chunks = cases.rule_case(name, layout)
    _copy_case(emu, pool, spans, chunks, 98_500 + layout)


@pytest.mark.parametrize("wg", [1, 7, 9])
@pytest.mark.parametrize("name", ["tm_24k", "tm_32k", "tm_36k", "tm_48k", "tm_64k", "tm_80k", "hm_16k_t4"])
def test_emulated_launch_rule_shapes_on_capped_grids(emu, name, wg):
    """The same calls on grids of 1, 7 and 9 workgroups: every item taken once, every
    access inside its buffer, the bytes equal to the oracle's."""
    pool, spans, chunks = cases.rule_case(name, 1)
    _copy_case(emu, pool, spans, chunks, 98_700 + wg, max_workgroups=wg)


FULL = ["tiny", "llama8b", "llama70b", "mixed", "mla_fp8", "int8_kv", "llama8b_hnd", "fp8_hnd_d64", "llama8b_tp8",
        "hnd_rows24", "hnd_h100_r12", "llama8b_tp2", "llama8b_tp4", "llama8b_hnd_tp4"]


@pytest.mark.parametrize("name", FULL)
def test_workload_addresses_stay_in_bounds(emu, name):
    """Full-size calls of every workload, walked without copying: addresses stay inside
    a pool of exactly num_blocks blocks and a staging buffer of exactly n_slots slots."""
    w = W.resolve(W.WORKLOADS[name])
    tok = W.token_bytes(w)
    pool = {k: w[k] for k in ("num_layers", "num_kv", "num_heads", "head_dim", "elem_bytes",
                              "block_size", "num_blocks")}
    pool["block_stride"] = w["block_size"] * tok
    pool["page_layout"] = w.get("page_layout", 0)
    plan = W.staging_plan(w)
    chunks = dict(layout=w["layout"], chunk_layers=w["chunk_layers"], chunk_tokens=w["chunk_tokens"],
                  layer_begin=0, layer_end=w["num_layers"], slot_bytes=plan["slot_bytes"],
                  n_slots=plan["n_chunks"])
    spans = [(t, t0, t1, fc) for t, (t0, t1), fc in zip(w["block_tables"], w["requests"], plan["first_chunk"])]
    n = pool["num_layers"] * pool["num_kv"]
    fake = 1 << 44
    bases = [fake + i * (1 << 38) for i in range(n)]
    grids = (0,) if pool["page_layout"] else (0, 2)   # a head-major walk visits every vector
    for d in (K.KV_GATHER, K.KV_SCATTER):
        for wg in grids:
            viol, tiles, grid = _emulate(emu, d, pool, spans, chunks, bases,
                                         [pool["num_blocks"] * pool["block_stride"]] * n, 1 << 45,
                                         plan["slot_bytes"] * plan["n_chunks"], False, wg)
            assert viol == 0
            assert tiles == sum(n * -(-(t1 - t0) // w["block_size"]) for t0, t1 in w["requests"])


def _extreme_case(name, layout, page_layout):
    from test_gpu_parity import EXTREMES
    c = EXTREMES[name]
    tok = c["H"] * c["D"] * c["E"]
    pool = dict(num_layers=c["L"], num_kv=c["KV"], num_heads=c["H"], head_dim=c["D"], elem_bytes=c["E"],
                block_size=c["bs"], num_blocks=c["N"], block_stride=c["bs"] * tok, page_layout=page_layout)
    rng = np.random.default_rng(95_000 + 7 * layout + page_layout)
    perm = rng.permutation(c["N"]).astype(np.int32)
    spans, used, fc = [], 0, 0
    for t0, t1 in c["spans"]:
        n_pages = cases.cdiv(t1, c["bs"])
        tbl = np.concatenate([np.full(t0 // c["bs"], -1, np.int32), perm[used:used + n_pages - t0 // c["bs"]]])
        used += n_pages - t0 // c["bs"]
        spans.append((tbl, t0, t1, fc))
        fc += (c["L"] // c["CL"]) * cases.cdiv(t1 - t0, c["CT"])
    chunks = dict(layout=layout, chunk_layers=c["CL"], chunk_tokens=c["CT"], layer_begin=0, layer_end=c["L"],
                  slot_bytes=c["CL"] * c["KV"] * c["CT"] * tok, n_slots=fc)
    return pool, spans, chunks


@pytest.mark.parametrize("name", ["one_token_pages", "huge_pages", "deep_start", "word_rows"])
@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("page_layout", [0, 1])
def test_emulated_extreme_shapes(emu, name, layout, page_layout):
    """The GPU extreme-shape cases, walked on the CPU first (prefix table entries are -1
    and must never be read)."""
    pool, spans, chunks = _extreme_case(name, layout, page_layout)
    _copy_case(emu, pool, spans, chunks, 3)


def _dma_case(lib, pool, spans, chunks, seed, strided, even_regions=True):
    """The copy-engine plan carried out on host buffers must equal the oracle; returns
    (copies, rows) of the gather."""
    rng = np.random.default_rng(seed)
    regions = cases.regions_for(pool, rng)
    staging = cases.staging_for(chunks, rng=rng)
    n = regions.shape[0]
    tabs = [np.ascontiguousarray(t, dtype=np.int32) for t, _, _, _ in spans]
    sp = K.make_spans([(t.ctypes.data, t.size, t0, t1, fc) for t, (_, t0, t1, fc) in zip(tabs, spans)])
    counts = None
    for d in (K.KV_GATHER, K.KV_SCATTER):
        # region i lives in row order[i]; reversed rows are not evenly spaced in ascending order
        order = list(range(n)) if even_regions else list(range(n))[::-1]
        r_emu, s_emu = regions[order].copy(), staging.copy()
        bases = [r_emu[order[i]].ctypes.data for i in range(n)]
        desc = K.make_pool_desc(pool["num_layers"], pool["num_kv"], pool["num_heads"], pool["head_dim"],
                                pool["elem_bytes"], pool["block_size"], pool["num_blocks"],
                                pool["block_stride"], bases, pool.get("page_layout", 0))
        spec = K.make_chunk_spec(chunks["layout"], chunks["chunk_layers"], chunks["chunk_tokens"],
                                 chunks["layer_begin"], chunks["layer_end"], s_emu.ctypes.data,
                                 chunks["slot_bytes"], chunks["n_slots"], 0, K.KV_FLAG_DMA_STRIDED if strided else 0)
        rb = np.full(n, r_emu.shape[1], dtype=np.int64)
        viol, copies, rows = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        rc = lib.emu_dma(d, ctypes.byref(desc), sp, len(spans), ctypes.byref(spec), rb.ctypes.data,
                         s_emu.size, int(strided), ctypes.byref(viol), ctypes.byref(copies), ctypes.byref(rows))
        assert rc == 0, K.kv_strerror(rc)
        assert viol.value == 0
        r_emu = r_emu[order]          # back to region order (order is its own inverse)
        r_or, s_or = regions.copy(), staging.copy()
        oracle.transfer(d, pool, r_or, spans, chunks, s_or)
        assert np.array_equal(s_emu, s_or) and np.array_equal(r_emu, r_or)
        if counts is None:
            counts = (copies.value, rows.value)
    return counts


@pytest.mark.parametrize("seed", range(40))
@pytest.mark.parametrize("strided", [False, True])
def test_dma_plan_matches_oracle(emu, seed, strided):
    """Per-tile and strided copy-engine plans, both chunk layouts, both page layouts."""
    pool, spans, chunks = cases.make_case(np.random.default_rng(29_000 + seed), tok_multiple=16,
                                          medium=bool(seed % 2), max_bytes=24 << 20, head_major=None)
    copies, rows = _dma_case(emu, pool, spans, chunks, seed, strided)
    tiles = sum((chunks["layer_end"] - chunks["layer_begin"]) * pool["num_kv"] * cases.cdiv(t1 - t0, pool["block_size"])
                for _, t0, t1, _ in spans)
    per_tile = tiles * (pool["num_heads"] if pool.get("page_layout", 0) else 1)
    group = chunks["chunk_layers"] * pool["num_kv"]
    if strided and not pool.get("page_layout", 0) and group > 1:
        assert copies * group == tiles
    else:
        assert copies == per_tile


@pytest.mark.parametrize("seed", range(6))
def test_dma_strided_plan_falls_back_on_uneven_regions(emu, seed):
    pool, spans, chunks = cases.make_case(np.random.default_rng(29_500 + seed), tok_multiple=16,
                                          max_bytes=8 << 20, head_major=False)
    copies, _ = _dma_case(emu, pool, spans, chunks, seed, True, even_regions=False)
    tiles = sum((chunks["layer_end"] - chunks["layer_begin"]) * pool["num_kv"] * cases.cdiv(t1 - t0, pool["block_size"])
                for _, t0, t1, _ in spans)
    assert copies == tiles


@pytest.mark.parametrize("lag", [0, 3, 40, 200])
@pytest.mark.parametrize("pattern", ["queue_test", "random", "large_only"])
def test_span_record_arena_never_overwrites_calls_in_flight(emu, pattern, lag):
    """The arena bookkeeping the transfer calls use (kvx::ArenaRing, 4 MiB, 256 calls in
    flight): no reservation may overlap a call that has not finished.  Record sizes are
    64 bytes per span rounded up to 256, as the library reserves them."""
    rng = np.random.default_rng(31_000 + lag)
    if pattern == "queue_test":        # every eighth call carries 4096 spans
        spans = [4096 if i % 8 == 0 else 1 for i in range(5000)]
    elif pattern == "large_only":
        spans = [int(x) for x in rng.integers(3000, 4097, size=3000)]
    else:
        spans = [int(x) for x in rng.choice([1, 2, 17, 300, 1000, 4096], size=5000)]
    sizes = np.array([(64 * n + 255) // 256 * 256 for n in spans], dtype=np.int64)
    assert emu.emu_arena(4 << 20, sizes.ctypes.data, sizes.size, lag) == 0


T4_SHAPES = [(4, 128, 2, 4), (8, 256, 1, 16), (12, 128, 2, 8), (4, 128, 2, 32)]   # H, D, E, bs: 256-B head rows


@pytest.mark.parametrize("seed", range(16))
def test_emulated_head_major_blocks_match_oracle(emu, seed):
    """Head-major pages with 256-byte head rows take the 4x4-block walk with the register
    transpose (emulated with the measured lane swaps): bytes equal the oracle's."""
    rng = np.random.default_rng(33_000 + seed)
    pool, spans, chunks = cases.head_major_case(rng, *T4_SHAPES[seed % len(T4_SHAPES)])
    _copy_case(emu, pool, spans, chunks, seed, max_workgroups=int(seed % 3))


LDS_SHAPES = cases.HM_LDS_SHAPES


@pytest.mark.parametrize("seed", range(32))
def test_emulated_head_major_lds_matches_oracle(emu, seed):
    """Head-major pages whose rows are not whole 16-byte vectors take the LDS slab walk
    (the kernel's lanes, magic-multiply divisions and slice indices replayed on the CPU):
    every word lands once, no slice word is read stale, bytes equal the oracle's."""
    rng = np.random.default_rng(35_000 + seed)
    pool, spans, chunks = cases.head_major_case(rng, *LDS_SHAPES[seed % len(LDS_SHAPES)])
    _copy_case(emu, pool, spans, chunks, seed, max_workgroups=int(seed % 3))


@pytest.mark.parametrize("seed", range(16))
def test_emulated_head_major_lds_split_match_oracle(emu_split, seed):
    """The same with tiles split between waves (parts are ranges of slabs)."""
    rng = np.random.default_rng(36_000 + seed)
    pool, spans, chunks = cases.head_major_case(rng, *LDS_SHAPES[seed % len(LDS_SHAPES)])
    _copy_case(emu_split, pool, spans, chunks, seed)


@pytest.mark.parametrize("tile_kib,unroll", [(36, 4), (28, 4), (24, 8), (40, 8), (72, 8), (18, 2), (20, 4)])
def test_segment_group_size(emu, tile_kib, unroll):
    """The segment walk's group size is the largest of 8, 4, 2 KiB dividing the pieces a
    32 KiB segment cuts from the tiles, i.e. gcd(tile, 32 KiB)."""
    assert emu.emu_gather_seg_unroll(tile_kib * 1024, 32768) == unroll


@pytest.mark.parametrize("row,heads,bs,tj", [
    (24, 16, 64, 16),    # 21 tokens fit; 16 make 384-byte (whole-line) head runs
    (12, 20, 64, 32),    # 34 fit; 32 make 384 bytes
    (100, 4, 128, 20),   # 20 fit; whole lines need 32, so all 20
    (8, 32, 16, 16),     # a whole page fits
    (100, 64, 4, 1),     # one token
])
def test_lds_slab_tokens(emu, row, heads, bs, tj):
    got = emu.emu_hm_lds_tokens(row, row * heads, bs)
    assert got == tj
    assert got * row * heads <= 8192 and 1 <= got <= bs


@pytest.mark.parametrize("row,heads,bs,whole", [
    (12, 100, 16, True),    # 19200-byte pages: more than a token slab's 8 KiB, within 20 KiB
    (12, 20, 64, True),     # 15360
    (8, 32, 48, True),      # 12288
    (8, 8, 16, False),      # 1 KiB pages fit a token slab whole already
    (24, 16, 64, False),    # 24 KiB pages: token slabs
    (12, 100, 32, False),   # 37.5 KiB pages: token and head-group slabs
    (16, 100, 16, False),   # rows of whole 16-byte vectors take no LDS at all
])
def test_whole_page_rule(emu, row, heads, bs, whole):
    assert bool(emu.emu_hm_page_ok(row, row * heads, row * heads * bs)) == whole


@pytest.mark.parametrize("row,heads,bs,gather,scatter", [
    (24, 16, 64, (0, 16), (0, 16)),      # token slabs of whole lines in both directions
    (12, 100, 16, (0, 6), (25, 16)),     # scatter: 25 heads x whole pages; gather keeps tokens
    (8, 128, 32, (32, 32), (32, 32)),    # both: 32 heads x 8 bytes = 256-byte chunk runs
    (100, 4, 128, (0, 20), (1, 64)),     # scatter: one head, 64 of its 128 rows (50 lines)
    (100, 64, 4, (0, 1), (16, 4)),       # scatter: 20 pages fit, 16 divides 64
])
def test_lds_head_group_slabs(emu, row, heads, bs, gather, scatter):
    """Where token slabs would split pool lines, scatter takes whole pages of a head
    group (the largest divisor of H that fits, or one head and part of its page) and
    gather does so only when the group's chunk runs are whole 128-byte lines."""
    hg, tj = ctypes.c_uint32(), ctypes.c_uint32()
    for d, want in ((K.KV_GATHER, gather), (K.KV_SCATTER, scatter)):
        emu.emu_hm_lds_head_slab(d, heads, row, row * heads, bs, ctypes.byref(hg), ctypes.byref(tj))
        assert (hg.value, tj.value) == want, (d, hg.value, tj.value)
        if hg.value:
            assert heads % hg.value == 0 and hg.value * tj.value * row <= 8192


def test_magic_division_is_exact():
    """The multiply that replaces division by d in the LDS walk (ceil(2^32/d), high
    word of the product) equals floor division for every numerator below 2^16, checked
    for every divisor the walk can use (row words and slab words up to 2048) against
    numpy's integer division."""
    n = np.arange(1 << 16, dtype=np.uint64)
    for d in range(1, 2049):
        m = np.uint64(((1 << 32) + d - 1) // d)
        assert np.array_equal((n * m) >> np.uint64(32), n // np.uint64(d)), d


@pytest.mark.parametrize("seed", range(8))
def test_emulated_head_major_blocks_split_match_oracle(emu_split, seed):
    """The same with tiles split between waves (parts are ranges of 4x4 blocks)."""
    rng = np.random.default_rng(34_000 + seed)
    pool, spans, chunks = cases.head_major_case(rng, *T4_SHAPES[seed % len(T4_SHAPES)])
    _copy_case(emu_split, pool, spans, chunks, seed)


# ---- declared extents against a fake allocation table ------------------------------

def _allocs(lib, pieces):
    bases = np.array([b for b, _ in pieces], dtype=np.uint64)
    sizes = np.array([n for _, n in pieces], dtype=np.uint64)
    lib.emu_set_allocs(bases.ctypes.data, sizes.ctypes.data, len(pieces))
    return bases, sizes   # keep alive


def test_extent_walk_follows_adjoining_allocations_and_stops_at_gaps(emu):
    MB = 1 << 20
    A = 0x7F0000000000
    # one 4 MiB allocation; three adjoining 2 MiB mappings; then a gap; then 1 MiB
    keep = _allocs(emu, [(A, 4 * MB), (A + 16 * MB, 2 * MB), (A + 18 * MB, 2 * MB), (A + 20 * MB, 2 * MB),
                         (A + 23 * MB, MB)])
    UMAX = 2**64 - 1
    assert emu.emu_covered_end(A, A + MB, 1 << 16) == A + 4 * MB                 # inside one allocation
    assert emu.emu_covered_end(A + MB, A + 4 * MB, 1 << 16) == A + 4 * MB         # ends exactly at its end
    assert emu.emu_covered_end(A, A + 4 * MB + 1, 1 << 16) == A + 4 * MB          # one byte past: short
    assert emu.emu_covered_end(A + 17 * MB, A + 22 * MB, 1 << 16) == A + 22 * MB  # across three mappings
    assert emu.emu_covered_end(A + 17 * MB, A + 23 * MB, 1 << 16) == A + 22 * MB  # the gap stops the walk
    assert emu.emu_covered_end(A + 8 * MB, A + 9 * MB, 1 << 16) == 0              # unknown memory
    assert emu.emu_covered_end(A + 16 * MB, A + 22 * MB, 2) == UMAX               # too many pieces: trusted
    assert emu.emu_covered_end(A + 16 * MB, A + 22 * MB, 3) == A + 22 * MB
    del keep


def test_extent_check_sees_each_allocation_as_it_is_now(emu):
    MB = 1 << 20
    A = 0x7F0000000000
    n = ctypes.c_int64()
    emu.emu_cache_reset()
    keep = _allocs(emu, [(A, 4 * MB)])
    assert emu.emu_cache_covers(A, 4 * MB, ctypes.byref(n)) == 1 and n.value == 1
    assert emu.emu_cache_covers(A, 2 * MB, ctypes.byref(n)) == 1 and n.value == 1
    assert emu.emu_cache_covers(A, 4 * MB + 16, ctypes.byref(n)) == 0
    # freed and made again smaller at the same address: the old 4 MiB extent is refused
    keep = _allocs(emu, [(A, 2 * MB)])
    assert emu.emu_cache_covers(A, 4 * MB, ctypes.byref(n)) == 0
    assert emu.emu_cache_covers(A, 2 * MB, ctypes.byref(n)) == 1
    # made again larger: accepted
    keep = _allocs(emu, [(A, 8 * MB)])
    assert emu.emu_cache_covers(A, 6 * MB, ctypes.byref(n)) == 1 and n.value == 1
    # memory the runtime does not know is taken on trust
    B = A + 64 * MB
    assert emu.emu_cache_covers(B, 1 << 40, ctypes.byref(n)) == 1 and n.value == 1
    del keep


def test_extent_check_reuses_a_walk_over_pieces_while_its_ends_stand(emu):
    MB = 1 << 20
    A = 0x7F0000000000
    n = ctypes.c_int64()
    emu.emu_cache_reset()
    keep = _allocs(emu, [(A, 2 * MB), (A + 2 * MB, 2 * MB), (A + 4 * MB, 2 * MB)])
    assert emu.emu_cache_covers(A, 6 * MB, ctypes.byref(n)) == 1 and n.value == 3   # walked
    assert emu.emu_cache_covers(A, 6 * MB, ctypes.byref(n)) == 1 and n.value == 2   # first + last checked
    # the last piece unmapped and mapped again smaller: the walk runs again and refuses
    keep = _allocs(emu, [(A, 2 * MB), (A + 2 * MB, 2 * MB), (A + 4 * MB, MB)])
    assert emu.emu_cache_covers(A, 6 * MB, ctypes.byref(n)) == 0
    # the first piece replaced by a smaller allocation (a gap after it): refused
    keep = _allocs(emu, [(A, MB), (A + 2 * MB, 2 * MB), (A + 4 * MB, 2 * MB)])
    assert emu.emu_cache_covers(A, 6 * MB, ctypes.byref(n)) == 0
    # whole again
    keep = _allocs(emu, [(A, 2 * MB), (A + 2 * MB, 2 * MB), (A + 4 * MB, 2 * MB)])
    assert emu.emu_cache_covers(A, 6 * MB, ctypes.byref(n)) == 1
    del keep


FAKE_BASE = 1 << 40   # addresses are only formed, never dereferenced, by the launch rules


def _rule(lib, direction, H, D, E, bs=16, page_layout=0, flags=0, layout=K.KV_LAYER_FIRST):
    """The launch decisions for a one-page call of a pool with H x D x E-byte rows."""
    tok = H * D * E
    desc = K.make_pool_desc(2, 2, H, D, E, bs, 4, bs * tok, [FAKE_BASE + i * (1 << 24) for i in range(4)],
                            page_layout)
    tab = np.arange(4, dtype=np.int32)
    sp = K.make_spans([(tab.ctypes.data, 4, 0, bs, 0)])
    spec = K.make_chunk_spec(layout, 2, bs, 0, 2, FAKE_BASE + (1 << 30), 2 * 2 * bs * tok, 1, 0, flags)
    out = (ctypes.c_int64 * 8)()
    assert lib.emu_launch_rule(direction, ctypes.byref(desc), sp, 1, ctypes.byref(spec), out) == 0
    return dict(shift=out[0], seg=out[1], lds=out[2], page=out[3], t4=out[4], xcd=out[5], sbuf=out[6],
                part=out[7])


@pytest.mark.parametrize("H,D,E,gather,scatter", [
    # token-major tiles: 4 KiB one wave; 8-12 KiB gathers and 8-18 KiB scatters in 4 parts
    # of 2 KiB or more; 16 KiB gathers, and those of 64 KiB or more that are not powers of
    # two, in 32 KiB segments; 20-64 KiB gathers that are not powers of two, and 20-64 KiB
    # scatters, in 4 KiB parts; 64 KiB gathers in 2 parts, 64 and 128 KiB scatters in 4,
    # and 80 and 96 KiB scatters (multiples of 16 KiB that are not powers of two) in 16 KiB
    # parts.  (split shift, segment bytes, XCD remap, fixed part bytes): gathers of 8 KiB
    # tiles or more outside the segment walk remap their workgroups, and so do scatters in
    # 4 KiB parts other than 32 KiB tiles with layer-first chunks (these calls are
    # layer-first); scatters split in 2^k parts or in 4 KiB parts go through buffer
    # instructions
    (1, 128, 2, (0, 0, 0, 0), (0, 0, 0, 0)),
    (2, 128, 2, (2, 0, 1, 0), (2, 0, 0, 0)),
    (3, 128, 2, (2, 0, 1, 0), (2, 0, 0, 0)),
    (4, 128, 2, (None, 32768, 0, 0), (2, 0, 0, 0)),
    (5, 128, 2, (0, 0, 1, 4096), (0, 0, 1, 4096)),
    (8, 128, 2, (0, 0, 1, 0), (0, 0, 0, 4096)),
    (16, 128, 2, (1, 0, 1, 0), (2, 0, 0, 0)),
    (9, 128, 2, (0, 0, 1, 4096), (0, 0, 1, 4096)),
    (12, 128, 2, (0, 0, 1, 4096), (0, 0, 1, 4096)),
    (20, 128, 2, (None, 32768, 0, 0), (0, 0, 0, 16384)),
    (24, 128, 2, (None, 32768, 0, 0), (0, 0, 0, 16384)),
    (32, 128, 2, (2, 0, 1, 0), (2, 0, 0, 0)),
])
def test_token_major_launch_rules(emu, H, D, E, gather, scatter):
    """The measured split, segment, part and workgroup-order rules, pinned to worked
    tile sizes."""
    for d, (shift, seg, xcd, part) in ((K.KV_GATHER, gather), (K.KV_SCATTER, scatter)):
        r = _rule(emu, d, H, D, E)
        assert r["seg"] == seg, (d, r)
        if shift is not None:
            assert r["shift"] == shift, (d, r)
        assert r["xcd"] == xcd, (d, r)
        assert r["part"] == part, (d, r)
        buffer_form = d == K.KV_SCATTER and (r["shift"] > 0 or r["part"] == 4096)
        assert r["sbuf"] == int(buffer_form), (d, r)
        assert not (r["lds"] or r["page"] or r["t4"])


@pytest.mark.parametrize("H,D,E,lf,pf", [(5, 128, 2, 1, 1), (8, 128, 2, 0, 1), (9, 128, 2, 1, 1), (16, 128, 2, 0, 0),
                                         (2, 128, 2, 0, 0), (20, 128, 2, 0, 0)])
def test_scatter_workgroup_order_by_chunk_layout(emu, H, D, E, lf, pf):
    """Scatters in 4 KiB parts remap their workgroups per XCD, except 32 KiB tiles with
    layer-first chunks; other scatters keep the plain order in either layout."""
    assert _rule(emu, K.KV_SCATTER, H, D, E)["xcd"] == lf
    assert _rule(emu, K.KV_SCATTER, H, D, E, layout=K.KV_PAGE_FIRST)["xcd"] == pf


@pytest.mark.parametrize("H,D,E,part", [(5, 128, 2, 4096), (8, 128, 2, 4096), (9, 128, 2, 4096), (12, 128, 2, 4096),
                                         (20, 128, 2, 16384), (16, 128, 2, 0), (4, 128, 2, 0)])
def test_page_runs_hint_keeps_20_to_64_kib_scatter_tiles_whole(emu, H, D, E, part):
    """KV_FLAG_PAGE_RUNS takes the 4 KiB parts away from 20-64 KiB scatter tiles (copied
    whole, in the global form) and changes nothing else."""
    plain = _rule(emu, K.KV_SCATTER, H, D, E)
    runs = _rule(emu, K.KV_SCATTER, H, D, E, flags=K.KV_FLAG_PAGE_RUNS)
    assert plain["part"] == part
    if part == 4096:
        assert runs["part"] == 0 and runs["shift"] == 0 and runs["sbuf"] == 0
    else:
        assert runs == plain
    # gathers ignore the hint
    assert _rule(emu, K.KV_GATHER, H, D, E, flags=K.KV_FLAG_PAGE_RUNS) == _rule(emu, K.KV_GATHER, H, D, E)


@pytest.mark.parametrize("H,D,E,bs,path", [
    (8, 128, 2, 16, "t4"),        # 256-byte rows, heads and tokens multiples of 4
    (8, 64, 1, 16, "lds"),        # 64-byte rows, 8 KiB page: token slab
    (8, 64, 2, 16, "page"),       # 128-byte rows, 16 KiB page: whole page
    (16, 64, 2, 16, "lds"),       # 128-byte rows, 32 KiB page: slabs
    (2, 128, 2, 16, "lds"),       # 256-byte rows, 2 heads, 8 KiB page
    (1, 256, 2, 16, "lds"),       # 512-byte rows, 8 KiB page
    (3, 128, 2, 16, "cursor"),    # 256-byte rows, 12 KiB page, heads not a multiple of 4
    (1, 128, 2, 32, "lds"),       # 256-byte rows, 1 head, 8 KiB page
    (2, 256, 2, 16, "cursor"),    # 512-byte rows, 16 KiB page
    (130, 32, 2, 16, "cursor"),   # 64-byte rows, but a token (8320 bytes) exceeds the slice
    (64, 128, 2, 16, "t4"),       # 16 KiB tokens, 256-byte rows: the 4 x 4 transpose needs no slice
    (6, 12, 2, 64, "page"),       # 24-byte rows (4-byte words), 9 KiB page: whole page
])
def test_head_major_path_rules(emu, H, D, E, bs, path):
    """Which head-major path a pool takes, pinned to worked shapes (both directions)."""
    for d in (K.KV_GATHER, K.KV_SCATTER):
        r = _rule(emu, d, H, D, E, bs, page_layout=1)
        got = "t4" if r["t4"] else "page" if r["page"] else "lds" if r["lds"] else "cursor"
        assert got == path, (H, D, E, bs, r)
        # LDS-staged pages (not whole) of 16 KiB or more go in 4 parts
        if path == "lds":
            assert r["shift"] == (2 if H * D * E * bs >= 16384 else 0), (d, r)
        # 4 x 4-transposed pages of 32 to under 64 KiB are scattered in 8 parts (one 4 KiB
        # block of 4 tokens x 4 heads each for 32 KiB pages), gathered whole
        if path == "t4" and H * D * E * bs < 65536:
            assert r["shift"] == (3 if d == K.KV_SCATTER and H * D * E * bs >= 32768 else 0), (d, r)
        # only the 4 x 4 gather remaps its workgroups per XCD; head-major scatters keep
        # their own copy loops
        assert r["xcd"] == int(d == K.KV_GATHER and path == "t4"), (d, r)
        assert r["sbuf"] == 0 and r["part"] == 0, (d, r)


@pytest.mark.parametrize("grid", [1, 7, 8, 9, 15, 16, 17, 64, 100, 1000, 4096 + 5, 32768, 65535])
def test_xcd_launch_order_is_a_permutation(emu, grid):
    """Remapped workgroup ids cover [0, grid) exactly once; workgroups b and b + 8 (one
    XCD's consecutive workgroups) take consecutive ids below the last grid % 8; without
    the remap the order is the identity."""
    got = [emu.emu_launch_block(b, grid, 1) for b in range(grid)]
    assert sorted(got) == list(range(grid))
    g8 = grid - grid % 8
    for b in range(g8 - 8):
        assert got[b + 8] == got[b] + 1
    assert got[g8:] == list(range(g8, grid))
    assert [emu.emu_launch_block(b, grid, 0) for b in range(grid)] == list(range(grid))
