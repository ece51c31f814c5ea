"""GPU parity: the HIP path through the C ABI against the CPU oracle, byte for byte.

Every case starts from random pool bytes and random staging bytes (so NaN, Inf,
-0.0 and subnormal fp16/bf16/fp8 patterns all occur), runs one call on the GPU
and the same call in the oracle, and compares the *whole* pool and the *whole*
staging buffer: moved bytes must match and every other byte must keep its prior
value.  Sizes are small enough for the oracle to finish in seconds while still
spanning many tiles, ragged last pages and short last chunks.
"""
from __future__ import annotations

import numpy as np
import pytest

import cases
import gpu_harness as G
import oracle
from paged_layout_transfer_amd import kvxfer as K
from paged_layout_transfer_amd import workloads as W

pytestmark = pytest.mark.gpu

DIRS = (K.KV_GATHER, K.KV_SCATTER)


def _oracle(direction, pool, spans, chunks, regions, staging, views=None):
    regs = regions.copy()
    stg = staging.copy()
    if views is None:
        rows = [regs[i] for i in range(regs.shape[0])]
    else:
        need = (pool["num_blocks"] - 1) * pool["block_stride"] + \
            pool["block_size"] * pool["num_heads"] * pool["head_dim"] * pool["elem_bytes"]
        rows = [regs[o:o + need] for o in views]
    oracle.transfer(direction, pool, rows, spans, chunks, stg)
    return regs, stg


def _compare(direction, pool, spans, chunks, regions, staging, label, views=None, **kw):
    exp_r, exp_s = _oracle(direction, pool, spans, chunks, regions, staging, views)
    got_r, got_s, bits = G.run_transfer(direction, pool, spans, chunks, regions, staging,
                                        label=label, region_views=views, **kw)
    assert bits == 0, "device reported error bits %#x" % bits
    assert np.array_equal(got_s, exp_s), "staging differs from the oracle"
    assert np.array_equal(got_r, exp_r), "pool differs from the oracle"


def _random(pool, chunks, seed):
    rng = np.random.default_rng(seed)
    return cases.regions_for(pool, rng), cases.staging_for(chunks, rng=rng)


@pytest.mark.parametrize("seed", range(40))
def test_small_random_cases(seed):
    pool, spans, chunks = cases.make_case(np.random.default_rng(10_000 + seed), tok_multiple=16)
    regions, staging = _random(pool, chunks, seed)
    for d in DIRS:
        _compare(d, pool, spans, chunks, regions, staging, "small-%d" % seed)


def test_many_random_cases_with_random_options():
    """200 more small random cases in one test, each with a random choice of page layout,
    staging (HBM or pinned ring), cache policy and grid cap."""
    for seed in range(200):
        rng = np.random.default_rng(60_000 + seed)
        pool, spans, chunks = cases.make_case(rng, tok_multiple=16, head_major=None)
        regions, staging = _random(pool, chunks, seed)
        flags = K.KV_FLAG_CACHED if rng.random() < 0.3 else 0
        ring = bool(rng.random() < 0.25)
        wg = int(rng.choice([0, 0, 1, 3, 7]))
        for d in DIRS:
            _compare(d, pool, spans, chunks, regions, staging, "many-%d" % seed, ring=ring, flags=flags,
                     max_workgroups=wg)


@pytest.mark.parametrize("n_records", [15, 16, 17, 18, 40])
def test_span_record_count_around_the_inline_limit(n_records):
    """A call with at most 16 span records passes them in the kernel arguments; one with
    more uploads them to the pool's device arena.  Whole-buffer parity on both sides of
    that limit, both directions, both chunk layouts, with empty spans mixed in (an
    empty span makes no record, so they must not count towards the limit)."""
    for layout in (K.KV_LAYER_FIRST, K.KV_PAGE_FIRST):
        rng = np.random.default_rng(70_000 + 10 * n_records + layout)
        pool, spans, chunks = cases.make_case(rng, tok_multiple=16, n_spans=n_records, layout=layout,
                                              max_bytes=16 << 20)
        empty = (np.zeros(0, dtype=np.int32), 0, 0, 0)
        for _ in range(int(rng.integers(1, 6))):
            spans.insert(int(rng.integers(0, len(spans) + 1)), empty)
        assert sum(1 for _, t0, t1, _ in spans if t1 > t0) == n_records
        regions, staging = _random(pool, chunks, n_records)
        for d in DIRS:
            _compare(d, pool, spans, chunks, regions, staging, "records-%d-layout%d" % (n_records, layout))


@pytest.mark.parametrize("seed", range(24))
def test_medium_random_cases(seed):
    pool, spans, chunks = cases.make_case(np.random.default_rng(20_000 + seed), tok_multiple=16,
                                          medium=True, max_bytes=48 << 20)
    regions, staging = _random(pool, chunks, seed)
    for d in DIRS:
        _compare(d, pool, spans, chunks, regions, staging, "medium-%d" % seed)


@pytest.mark.parametrize("seed", range(8))
def test_pinned_host_ring_cases(seed):
    """Chunks in pinned host memory, read (scatter) and written (gather) by the kernel."""
    pool, spans, chunks = cases.make_case(np.random.default_rng(30_000 + seed), tok_multiple=16,
                                          medium=True, max_bytes=32 << 20)
    regions, staging = _random(pool, chunks, seed)
    flags = K.KV_RING_NONCOHERENT if seed % 2 else K.KV_RING_COHERENT
    for d in DIRS:
        _compare(d, pool, spans, chunks, regions, staging, "ring-%d" % seed, ring=True, ring_flags=flags)


@pytest.mark.parametrize("wg", [1, 2, 3, 5])
def test_capped_grid(wg):
    """A grid of a few workgroups walks every tile through the grid-stride loop."""
    pool = dict(num_layers=3, num_kv=2, num_heads=8, head_dim=128, elem_bytes=2, block_size=16,
                num_blocks=64, block_stride=16 * 2048)
    rng = np.random.default_rng(40_000 + wg)
    tables = [rng.permutation(64)[:20].astype(np.int32), rng.permutation(64)[20:40].astype(np.int32)]
    tables[1] = np.setdiff1d(np.arange(64, dtype=np.int32), tables[0])[:20]
    spans = [(tables[0], 0, 311, 0), (tables[1], 48, 301, 6)]
    chunks = dict(layout=0, chunk_layers=3, chunk_tokens=128, layer_begin=0, layer_end=3,
                  slot_bytes=3 * 2 * 128 * 2048, n_slots=9)
    regions, staging = _random(pool, chunks, wg)
    for d in DIRS:
        _compare(d, pool, spans, chunks, regions, staging, "grid-%d" % wg, max_workgroups=wg)


def test_tiny_workload_gather_then_scatter():
    w = W.resolve(W.WORKLOADS["tiny"])
    tok = W.token_bytes(w)
    pool = {k: w[k] for k in ("num_layers", "num_kv", "num_heads", "head_dim", "elem_bytes",
                              "block_size", "num_blocks")}
    pool["block_stride"] = w["block_size"] * tok
    plan = W.staging_plan(w)
    chunks = dict(layout=w["layout"], chunk_layers=w["chunk_layers"], chunk_tokens=w["chunk_tokens"],
                  layer_begin=0, layer_end=w["num_layers"], slot_bytes=plan["slot_bytes"],
                  n_slots=plan["n_chunks"])
    spans = [(w["block_tables"][0], 0, w["tokens"], 0)]
    n = w["num_layers"] * w["num_kv"]
    regions = W.host_fill(n * w["num_blocks"] * pool["block_stride"], w["fill"], w["k"]).reshape(n, -1)
    staging = np.full(plan["slot_bytes"] * plan["n_chunks"], W.SENTINEL, dtype=np.uint8)
    exp_r, exp_s = _oracle(K.KV_GATHER, pool, spans, chunks, regions, staging)
    _, got_s, bits = G.run_transfer(K.KV_GATHER, pool, spans, chunks, regions, staging, label="tiny")
    assert bits == 0 and np.array_equal(got_s, exp_s)
    fresh = np.full_like(regions, W.SENTINEL)
    exp_r2, _ = _oracle(K.KV_SCATTER, pool, spans, chunks, fresh, got_s)
    got_r2, _, bits = G.run_transfer(K.KV_SCATTER, pool, spans, chunks, fresh, got_s, label="tiny")
    assert bits == 0 and np.array_equal(got_r2, exp_r2)
    # the round trip restores every referenced token and leaves the rest at the sentinel
    moved = got_r2 != W.SENTINEL
    assert np.array_equal(got_r2[moved], regions[moved])


REDUCED = {
    "llama8b": dict(num_layers=4, chunk_layers=4, tokens=2085, num_blocks=200),
    "llama70b": dict(num_layers=3, chunk_layers=1, tokens=4096 + 21, num_blocks=300),
    "mixed": dict(num_layers=3, chunk_layers=3, n_requests=6, median=600, min_len=100,
                  max_len=3000),
    "mla_fp8": dict(num_layers=5, chunk_layers=5, tokens=64 * 9 + 13, num_blocks=40),
    "int8_kv": dict(num_layers=3, chunk_layers=3, tokens=64 * 7 + 1, num_blocks=30),
    "llama8b_tp8": dict(num_layers=4, chunk_layers=2, tokens=16 * 37 + 9, num_blocks=80),
    "llama8b_tp2": dict(num_layers=4, chunk_layers=4, tokens=16 * 41 + 3, num_blocks=90),
    "llama8b_tp4": dict(num_layers=4, chunk_layers=2, tokens=16 * 45 + 7, num_blocks=100),
}


def reduced_call(name):
    w = dict(W.WORKLOADS[name])
    w.update(REDUCED[name])
    w = W.resolve(w)
    tok = W.token_bytes(w)
    pool = {k: w[k] for k in ("num_layers", "num_kv", "num_heads", "head_dim", "elem_bytes",
                              "block_size", "num_blocks")}
    pool["block_stride"] = w["block_size"] * tok
    plan = W.staging_plan(w)
    chunks = dict(layout=w["layout"], chunk_layers=w["chunk_layers"], chunk_tokens=w["chunk_tokens"],
                  layer_begin=0, layer_end=w["num_layers"], slot_bytes=plan["slot_bytes"],
                  n_slots=plan["n_chunks"])
    spans = [(tbl, t0, t1, fc) for tbl, (t0, t1), fc in
             zip(w["block_tables"], w["requests"], plan["first_chunk"])]
    return w, pool, spans, chunks


@pytest.mark.parametrize("name", sorted(REDUCED))
def test_reduced_workloads(name):
    w, pool, spans, chunks = reduced_call(name)
    n = pool["num_layers"] * pool["num_kv"]
    regions = W.host_fill(n * pool["num_blocks"] * pool["block_stride"], w["fill"], w["k"]).reshape(n, -1)
    staging = W.host_fill(chunks["slot_bytes"] * chunks["n_slots"], "bytes", 100 + w["k"])
    ring = w["staging"] == "host"
    for d in DIRS:
        _compare(d, pool, spans, chunks, regions, staging, "reduced-" + name, ring=ring)


def test_interleaved_kv_pool():
    """A per-layer [blocks][K/V][page] pool: block_stride = 2 pages, V regions offset by a page."""
    L, KV, H, D, E, bs, N = 3, 2, 2, 128, 2, 32, 24
    tile = bs * H * D * E
    pool = dict(num_layers=L, num_kv=KV, num_heads=H, head_dim=D, elem_bytes=E, block_size=bs,
                num_blocks=N, block_stride=KV * tile)
    views = [l * N * KV * tile + kv * tile for l in range(L) for kv in range(KV)]
    rng = np.random.default_rng(50_000)
    flat = rng.integers(0, 256, size=L * N * KV * tile, dtype=np.uint8)
    tbl = rng.permutation(N)[:7].astype(np.int32)
    spans = [(tbl, 32, 32 * 6 + 17, 0)]
    for layout in (0, 1):
        chunks = dict(layout=layout, chunk_layers=1, chunk_tokens=64, layer_begin=0, layer_end=L,
                      slot_bytes=KV * 64 * H * D * E, n_slots=L * 3)
        staging = cases.staging_for(chunks, rng=rng)
        for d in DIRS:
            _compare(d, pool, spans, chunks, flat, staging, "interleaved-%d" % layout, views=views)


@pytest.mark.parametrize("H,D,bs,page_layout", [(1, 64, 16, 0), (2, 288, 16, 0), (8, 4, 16, 1)])
def test_bad_block_id_is_skipped_and_reported(H, D, bs, page_layout):
    """A table entry past the pool: that page's tiles are skipped, the sticky error bit is
    set, and every other tile still moves (page-first, one chunk per page).  The second
    shape has 18 KiB tiles, so the gather takes the segment walk; the third is head-major
    with 8-byte rows (the LDS slab walk)."""
    L, KV, E, N = 2, 2, 2, 32
    tok = H * D * E
    pool = dict(num_layers=L, num_kv=KV, num_heads=H, head_dim=D, elem_bytes=E, block_size=bs,
                num_blocks=N, block_stride=bs * tok, page_layout=page_layout)
    rng = np.random.default_rng(60_000)
    good = rng.permutation(N)[:6].astype(np.int32)
    bad = good.copy()
    bad[4] = N + 3                                # page 4 is poisoned
    chunks = dict(layout=1, chunk_layers=L, chunk_tokens=bs, layer_begin=0, layer_end=L,
                  slot_bytes=L * KV * bs * tok, n_slots=6)
    regions, staging = _random(pool, chunks, 7)
    for d in DIRS:
        # expected: the oracle without page 4 (chunk 4 keeps its bytes, pool block untouched)
        part = [(good, 0, 64, 0), (good, 80, 96, 5)]
        exp_r, exp_s = _oracle(d, pool, part, chunks, regions, staging)
        got_r, got_s, bits = G.run_transfer(d, pool, [(bad, 0, 96, 0)], chunks, regions, staging,
                                            label="bad-block")
        assert bits == K.KV_DEVERR_BLOCK_RANGE
        assert np.array_equal(got_s, exp_s) and np.array_equal(got_r, exp_r)


def test_empty_span_moves_nothing():
    pool = dict(num_layers=2, num_kv=2, num_heads=1, head_dim=64, elem_bytes=2, block_size=16,
                num_blocks=8, block_stride=2048)
    chunks = dict(layout=0, chunk_layers=2, chunk_tokens=16, layer_begin=0, layer_end=2,
                  slot_bytes=2 * 2 * 16 * 128, n_slots=4)
    regions, staging = _random(pool, chunks, 3)
    tbl = np.arange(4, dtype=np.int32)
    spans = [(tbl, 32, 32, 0), (tbl, 0, 16, 0), (tbl, 64, 64, 3)]   # only the middle span moves
    for d in DIRS:
        _compare(d, pool, spans, chunks, regions, staging, "empty-spans")


def test_validate_flag_rejects_double_write():
    pool = dict(num_layers=1, num_kv=1, num_heads=1, head_dim=64, elem_bytes=2, block_size=16,
                num_blocks=8, block_stride=2048)
    chunks = dict(layout=0, chunk_layers=1, chunk_tokens=16, layer_begin=0, layer_end=1,
                  slot_bytes=2048, n_slots=4)
    regions, staging = _random(pool, chunks, 4)
    tbl = np.array([1, 2, 1, 3], dtype=np.int32)       # block 1 twice
    spans = [(tbl, 0, 64, 0)]
    with pytest.raises(K.KvError) as e:
        G.run_transfer(K.KV_SCATTER, pool, spans, chunks, regions, staging,
                       flags=K.KV_FLAG_VALIDATE, label="validate-dup")
    assert e.value.code == K.KV_ERR_DUP
    # a gather may read one page twice
    _compare(K.KV_GATHER, pool, spans, chunks, regions, staging, "validate-gather",
             flags=K.KV_FLAG_VALIDATE)


@pytest.mark.parametrize("seed", range(10))
def test_per_tile_dma_baseline_matches_oracle(seed):
    """The copy-engine comparison path (one hipMemcpyAsync per tile, host block tables)
    gives the same bytes as the oracle, in HBM and, for odd seeds, in pinned host memory."""
    pool, spans, chunks = cases.make_case(np.random.default_rng(70_000 + seed), tok_multiple=16,
                                          medium=bool(seed % 3), max_bytes=24 << 20)
    regions, staging = _random(pool, chunks, seed)
    for d in DIRS:
        _compare(d, pool, spans, chunks, regions, staging, "dma-%d" % seed, dma=True, ring=bool(seed % 2))


@pytest.mark.parametrize("seed", range(10))
def test_strided_dma_matches_oracle(seed):
    """KV_FLAG_DMA_STRIDED: one hipMemcpy2DAsync per (chunk, page) over the page's
    (layer, kv) tiles (the regions are rows of one tensor, so evenly spaced); head-major
    cases keep their per-head copies."""
    pool, spans, chunks = cases.make_case(np.random.default_rng(72_000 + seed), tok_multiple=16,
                                          medium=bool(seed % 3), max_bytes=24 << 20, head_major=None)
    regions, staging = _random(pool, chunks, seed)
    for d in DIRS:
        _compare(d, pool, spans, chunks, regions, staging, "dma-strided-%d" % seed, dma=True,
                 ring=bool(seed % 2), flags=K.KV_FLAG_DMA_STRIDED)


@pytest.mark.parametrize("seed", range(8))
def test_cached_policy_matches_oracle(seed):
    """KV_FLAG_CACHED (plain cached loads and stores) moves the same bytes: both page
    layouts, HBM and pinned-host staging."""
    pool, spans, chunks = cases.make_case(np.random.default_rng(74_000 + seed), tok_multiple=16,
                                          medium=bool(seed % 2), max_bytes=24 << 20, head_major=None)
    regions, staging = _random(pool, chunks, seed)
    for d in DIRS:
        _compare(d, pool, spans, chunks, regions, staging, "cached-%d" % seed, ring=seed % 4 == 3,
                 flags=K.KV_FLAG_CACHED)


def test_per_tile_dma_rejects_bad_ids_before_copying():
    pool = dict(num_layers=1, num_kv=1, num_heads=1, head_dim=64, elem_bytes=2, block_size=16,
                num_blocks=8, block_stride=2048)
    chunks = dict(layout=0, chunk_layers=1, chunk_tokens=16, layer_begin=0, layer_end=1,
                  slot_bytes=2048, n_slots=4)
    regions, staging = _random(pool, chunks, 5)
    for tbl, code in ((np.array([1, 2, 9, 3], dtype=np.int32), K.KV_ERR_RANGE),
                      (np.array([1, 2, 1, 3], dtype=np.int32), K.KV_ERR_DUP)):
        with pytest.raises(K.KvError) as e:
            G.run_transfer(K.KV_SCATTER, pool, [(tbl, 0, 64, 0)], chunks, regions, staging,
                           label="dma-bad", dma=True)
        assert e.value.code == code


@pytest.mark.parametrize("seed", range(16))
def test_head_major_pool_cases(seed):
    """Head-major pages ([H][bs][D]) against token-major chunks; odd seeds stage in
    pinned host memory, every fourth uses the per-tile copy-engine path."""
    pool, spans, chunks = cases.make_case(np.random.default_rng(85_000 + seed), tok_multiple=16,
                                          medium=bool(seed % 3), max_bytes=24 << 20, head_major=True)
    regions, staging = _random(pool, chunks, seed)
    for d in DIRS:
        _compare(d, pool, spans, chunks, regions, staging, "head-major-%d" % seed, ring=bool(seed % 2),
                 dma=seed % 4 == 0)


@pytest.mark.parametrize("seed", range(32))
def test_head_major_lds_cases(seed):
    """Head-major pages whose head rows are not whole 16-byte vectors (4 to 100 bytes),
    moved through LDS slabs: every slab shape of the list twice, odd seeds staged in pinned
    host memory, every third seed with cached accesses, every fourth through the per-tile
    copy-engine path."""
    rng = np.random.default_rng(86_000 + seed)
    pool, spans, chunks = cases.head_major_case(rng, *cases.HM_LDS_SHAPES[seed % len(cases.HM_LDS_SHAPES)])
    regions, staging = _random(pool, chunks, seed)
    flags = K.KV_FLAG_CACHED if seed % 3 == 0 else 0
    for d in DIRS:
        _compare(d, pool, spans, chunks, regions, staging, "head-major-lds-%d" % seed, ring=bool(seed % 2),
                 dma=seed % 4 == 0, flags=flags)


@pytest.mark.parametrize("flags", [0, K.KV_FLAG_CACHED, K.KV_FLAG_PAGE_RUNS])
@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("name", sorted(cases.RULE_SHAPES))
def test_launch_rule_boundaries(name, layout, flags):
    """Each launch path at the tile sizes around its rule, both chunk layouts, with 1-2
    spans that start 0-2 pages in and end in a partial page, with the default
    nontemporal accesses, with KV_FLAG_CACHED (each kernel form has both) and with the
    KV_FLAG_PAGE_RUNS hint (whole tiles where 4 KiB parts are the default); whole buffers
    compared."""
    pool, spans, chunks = cases.rule_case(name, layout)
    regions, staging = _random(pool, chunks, 98_500 + layout)
    for d in DIRS:
        _compare(d, pool, spans, chunks, regions, staging, "rule-%s-%d-%d" % (name, layout, flags), flags=flags)


@pytest.mark.parametrize("wg", [1, 7, 9])
@pytest.mark.parametrize("name", ["tm_24k", "tm_32k", "tm_36k", "tm_48k", "tm_64k", "tm_80k", "hm_16k_t4"])
def test_launch_rule_shapes_on_capped_grids(name, wg):
    """The fixed-part, buffer-form and per-XCD-ordered walks on grids of 1, 7 and 9
    workgroups (each wave loops over many items; 7 and 9 leave workgroups outside the
    per-XCD permutation's whole eighths), page-first chunks; whole buffers compared."""
    pool, spans, chunks = cases.rule_case(name, 1)
    regions, staging = _random(pool, chunks, 98_700 + wg)
    for d in DIRS:
        _compare(d, pool, spans, chunks, regions, staging, "rule-capped-%s-%d" % (name, wg), max_workgroups=wg)


EXTREMES = {
    # 1-token pages of 16-byte tokens: every tile is one vector
    "one_token_pages": dict(L=3, KV=2, H=1, D=16, E=1, bs=1, N=900, spans=[(0, 500), (0, 77)], CT=64, CL=3),
    # 512-token pages of 2 KiB tokens: 1 MiB tiles, split between waves in both directions
    "huge_pages": dict(L=2, KV=2, H=8, D=128, E=2, bs=512, N=8, spans=[(0, 1500), (512, 1100)], CT=1024, CL=1),
    # 64 heads x 100-byte rows: 400 KiB tiles, one token per LDS slab when head-major, split
    # between waves
    "word_rows": dict(L=2, KV=2, H=64, D=100, E=1, bs=64, N=24, spans=[(0, 700), (64, 300)], CT=128, CL=1),
    # a span that starts 300 pages into its table
    "deep_start": dict(L=2, KV=1, H=2, D=64, E=2, bs=16, N=400, spans=[(300 * 16, 300 * 16 + 70)], CT=32, CL=2),
}


def test_blocks_past_4_gib_in_one_region():
    """One 4.3 GiB region with 1 MiB between blocks: the spans' pages sit in blocks past
    the 4 GiB offset and near the start, so every pool address needs the 64-bit product
    of block id and stride (the chunk side is the same for either chunk layout, so
    layer-first chunks only).  Both directions, whole region and staging compared."""
    tok = 2 * 64 * 2
    pool = dict(num_layers=1, num_kv=1, num_heads=2, head_dim=64, elem_bytes=2, block_size=16,
                num_blocks=4400, block_stride=1 << 20, page_layout=0)
    rng = np.random.default_rng(97_000)
    far = rng.permutation(np.arange(4096, 4400))[:150]
    near = rng.permutation(np.arange(0, 64))[:20]
    ids = rng.permutation(np.concatenate([far, near])).astype(np.int32)
    spans = [(ids[:100], 0, 100 * 16 - 5, 0), (ids[100:], 0, 70 * 16, 7)]
    chunks = dict(layout=0, chunk_layers=1, chunk_tokens=256, layer_begin=0, layer_end=1,
                  slot_bytes=256 * tok, n_slots=12)
    regions = np.full((1, pool["num_blocks"] * pool["block_stride"]), 0xA5, dtype=np.uint8)
    for b in ids:
        o = int(b) * pool["block_stride"]
        regions[0, o:o + 16 * tok] = rng.integers(0, 256, 16 * tok, dtype=np.uint8)
    staging = cases.staging_for(chunks, rng=rng)
    for d in DIRS:
        _compare(d, pool, spans, chunks, regions, staging, "past-4gib")


@pytest.mark.parametrize("name", sorted(EXTREMES))
@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("page_layout", [0, 1])
def test_extreme_shapes(name, layout, page_layout):
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
    regions, staging = _random(pool, chunks, 3)
    for d in DIRS:
        _compare(d, pool, spans, chunks, regions, staging, "extreme-%s-%d-%d" % (name, layout, page_layout))
