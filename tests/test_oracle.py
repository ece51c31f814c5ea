"""Pins for the CPU oracle (no GPU).

Each test checks the oracle against something that is not the oracle:
  * brute force   -- tests/brute.py decodes every staging byte back to its pool
                     byte (the oracle encodes pool -> staging), on many random
                     tiny shapes, both layouts, both directions, ring wrap;
  * library call  -- torch CPU advanced indexing for one span of whole pages;
  * closed form   -- the index map of the transfer kernel printed in the Strata
                     guide ("Step 1: High-Performance GPU-Assisted I/O CUDA
                     Kernel"), evaluated with numpy on 16-byte items;
  * invariants    -- round trip into a fresh sentinel pool, untouched bytes keep
                     the sentinel, page-first = transpose of layer-first, byte
                     histogram conservation;
  * page sizes    -- the request sizes of the Strata guide's fragmentation figure
                     (tests/golden/page_sizes.json);
  * planted bugs  -- copies of oracle.c with one plausible mistake each must
                     fail at least one of the pins above.
"""
from __future__ import annotations

import json
import os
import subprocess
import sys
import tempfile

import numpy as np
import pytest
import torch

import brute
import cases
import oracle
from paged_layout_transfer_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _run_pair(direction, pool, spans, chunks, seed, lib=None):
    """Oracle and brute force on the same random inputs; returns (oracle_out, brute_out)."""
    rng = np.random.default_rng(seed)
    regions = cases.regions_for(pool, rng)
    if direction == oracle.GATHER:
        buf = cases.staging_for(chunks, rng=rng)
        exp = brute.gather(pool, regions, spans, chunks, buf)
        got = buf.copy()
        oracle.gather(pool, regions, spans, chunks, got, lib=lib)
        return got, exp
    buf = cases.staging_for(chunks, rng=rng)
    exp = brute.scatter(pool, regions, spans, chunks, buf)
    got = regions.copy()
    oracle.scatter(pool, got, spans, chunks, buf, lib=lib)
    return got, exp


@pytest.mark.parametrize("seed", range(120))
def test_oracle_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    pool, spans, chunks = cases.make_case(rng, head_major=None)
    for direction in (oracle.GATHER, oracle.SCATTER):
        got, exp = _run_pair(direction, pool, spans, chunks, seed * 7 + direction)
        assert np.array_equal(got, exp), (direction, pool, chunks)


def _tiny():
    w = W.resolve(W.WORKLOADS["tiny"])
    tok = W.token_bytes(w)
    pool = {k: w[k] for k in ("num_layers", "num_kv", "num_heads", "head_dim", "elem_bytes",
                              "block_size", "num_blocks")}
    pool["block_stride"] = w["block_size"] * tok
    chunks = dict(layout=w["layout"], chunk_layers=w["chunk_layers"], chunk_tokens=w["chunk_tokens"],
                  layer_begin=0, layer_end=w["num_layers"],
                  slot_bytes=w["chunk_layers"] * w["num_kv"] * w["chunk_tokens"] * tok, n_slots=1)
    spans = [(w["block_tables"][0], 0, w["tokens"], 0)]
    return w, pool, spans, chunks


def test_tiny_workload_brute_force_and_roundtrip():
    w, pool, spans, chunks = _tiny()
    n = pool["num_layers"] * pool["num_kv"]
    regions = W.host_fill(n * pool["num_blocks"] * pool["block_stride"], w["fill"], w["k"]).reshape(n, -1)
    buf = cases.staging_for(chunks)
    assert buf.size == 256 * 1024  # one [2,2,256,2,64] fp16 chunk
    exp = brute.gather(pool, regions, spans, chunks, buf)
    got = buf.copy()
    assert oracle.gather(pool, regions, spans, chunks, got) == 256 * 1024
    assert np.array_equal(got, exp)
    fresh = np.full_like(regions, W.SENTINEL)
    oracle.scatter(pool, fresh, spans, chunks, got)
    assert np.array_equal(fresh, brute.scatter(pool, np.full_like(regions, W.SENTINEL), spans, chunks, got))


def _referenced_mask(pool, spans, chunks):
    """Pool bytes the call touches, written from the page-table definition alone."""
    n = pool["num_layers"] * pool["num_kv"]
    mask = np.zeros((n, pool["num_blocks"] * pool["block_stride"]), dtype=bool)
    H, R = pool["num_heads"], pool["head_dim"] * pool["elem_bytes"]
    bs = pool["block_size"]
    for tbl, t0, t1, _ in spans:
        for t in range(t0, t1):
            b, j = int(tbl[t // bs]), t % bs
            for h in range(H):
                if pool.get("page_layout", 0) == 1:      # [H][bs][D]
                    o = b * pool["block_stride"] + (h * bs + j) * R
                else:                                    # [bs][H][D]
                    o = b * pool["block_stride"] + (j * H + h) * R
                for l in range(chunks["layer_begin"], chunks["layer_end"]):
                    for kv in range(pool["num_kv"]):
                        mask[l * pool["num_kv"] + kv, o:o + R] = True
    return mask


@pytest.mark.parametrize("seed", range(40))
def test_roundtrip_identity_and_sentinel(seed):
    rng = np.random.default_rng(1000 + seed)
    pool, spans, chunks = cases.make_case(rng, head_major=None)
    regions = cases.regions_for(pool, rng)
    buf = cases.staging_for(chunks)
    oracle.gather(pool, regions, spans, chunks, buf)
    fresh = np.full_like(regions, W.SENTINEL)
    oracle.scatter(pool, fresh, spans, chunks, buf)
    mask = _referenced_mask(pool, spans, chunks)
    assert np.array_equal(fresh[mask], regions[mask])
    assert np.all(fresh[~mask] == W.SENTINEL)


@pytest.mark.parametrize("seed", range(12))
def test_layer_first_equals_torch_indexing(seed):
    """One span of whole pages, layer-first, page-sized pool strides: each chunk is
    pool[l, kv][table[pages]] flattened to tokens, stacked over (layer, kv); for a
    head-major pool, with each page's [H][bs] axes permuted to [bs][H] first."""
    rng = np.random.default_rng(2000 + seed)
    head_major = seed % 2 == 1
    L, KV, H, D, E, bs = 3, 2, int(rng.integers(1, 4)), 16, 2, int(rng.choice([4, 16]))
    N, n_pages = 40, int(rng.integers(2, 9))
    CT = bs * int(rng.integers(1, 4))
    CL = int(rng.choice([1, 3]))
    pad = int(rng.choice([0, 32]))
    tok = H * D * E
    pool = dict(num_layers=L, num_kv=KV, num_heads=H, head_dim=D, elem_bytes=E, block_size=bs,
                num_blocks=N, block_stride=bs * tok + pad, page_layout=int(head_major))
    tbl = rng.permutation(N)[:n_pages].astype(np.int32)
    T = n_pages * bs
    n_tc = cases.cdiv(T, CT)
    chunks = dict(layout=0, chunk_layers=CL, chunk_tokens=CT, layer_begin=0, layer_end=L,
                  slot_bytes=CL * KV * CT * tok, n_slots=(L // CL) * n_tc)
    regions = cases.regions_for(pool, rng)
    buf = cases.staging_for(chunks)
    oracle.gather(pool, regions, [(tbl, 0, T, 0)], chunks, buf)

    t_regions = torch.from_numpy(regions).view(L, KV, N, -1)[:, :, :, :bs * tok]
    if head_major:
        t_regions = t_regions.reshape(L, KV, N, H, bs, D * E).permute(0, 1, 2, 4, 3, 5)
    t_regions = t_regions.reshape(L, KV, N, bs, tok)
    idx = torch.from_numpy(tbl.astype(np.int64))
    per_lkv = t_regions[:, :, idx].reshape(L, KV, T, tok)       # [L][KV][T][tok]
    for lc in range(L // CL):
        for tc in range(n_tc):
            c = lc * n_tc + tc
            lo, hi = tc * CT, min(T, (tc + 1) * CT)
            expect = per_lkv[lc * CL:(lc + 1) * CL, :, lo:hi].contiguous().view(-1).numpy()
            got = buf[c * chunks["slot_bytes"]: c * chunks["slot_bytes"] + expect.size]
            assert np.array_equal(got, expect)
            assert np.all(buf[c * chunks["slot_bytes"] + expect.size:(c + 1) * chunks["slot_bytes"]] == W.SENTINEL)


@pytest.mark.parametrize("seed", range(8))
def test_scatter_matches_printed_kernel_index_map(seed):
    """The Strata guide's load kernel: a page-first host buffer of 16-byte items
    [page][layer][item] lands in a layer-first HBM buffer [layer][gpu page][item]
    at item (layer*total_gpu_pages + page_indices[page])*items_per_page_layer +
    item_in_layer.  In this library's terms: one K/V object, per-layer pools laid
    end to end, one page-first chunk holding every page and every layer."""
    rng = np.random.default_rng(3000 + seed)
    num_pages, num_layers = int(rng.integers(1, 7)), int(rng.integers(1, 5))
    cppl = int(rng.choice([1, 4, 8]))            # 16-byte items per (page, layer)
    total_gpu_pages = num_pages + int(rng.integers(0, 6))
    page_indices = rng.permutation(total_gpu_pages)[:num_pages].astype(np.int32)
    src = rng.integers(0, 256, size=num_pages * num_layers * cppl * 16, dtype=np.uint8)

    # The printed map, written with numpy on 16-byte items.
    items = src.reshape(-1, 16)
    chunk_idx = np.arange(num_pages * num_layers * cppl, dtype=np.int64)
    p_offset = chunk_idx // (num_layers * cppl)
    rem = chunk_idx % (num_layers * cppl)
    layer_idx = rem // cppl
    chunk_in_layer = rem % cppl
    dst_idx = (layer_idx * total_gpu_pages * cppl + page_indices[p_offset].astype(np.int64) * cppl
               + chunk_in_layer)
    expect = np.full((num_layers * total_gpu_pages * cppl, 16), W.SENTINEL, dtype=np.uint8)
    expect[dst_idx] = items[chunk_idx]

    # The same move through the oracle: tokens of 16 bytes, a page = cppl tokens.
    pool = dict(num_layers=num_layers, num_kv=1, num_heads=1, head_dim=16, elem_bytes=1,
                block_size=cppl, num_blocks=total_gpu_pages, block_stride=cppl * 16)
    dst = np.full(num_layers * total_gpu_pages * cppl * 16, W.SENTINEL, dtype=np.uint8)
    regions = dst.reshape(num_layers, -1)
    chunks = dict(layout=1, chunk_layers=num_layers, chunk_tokens=num_pages * cppl, layer_begin=0,
                  layer_end=num_layers, slot_bytes=src.size, n_slots=1)
    oracle.scatter(pool, regions, [(page_indices, 0, num_pages * cppl, 0)], chunks, src.copy())
    assert np.array_equal(dst.reshape(-1, 16), expect)


@pytest.mark.parametrize("seed", range(10))
def test_page_first_is_transpose_of_layer_first(seed):
    rng = np.random.default_rng(4000 + seed)
    L, KV, H, D, E, bs = int(rng.integers(1, 4)), int(rng.integers(1, 3)), 2, 8, 2, 4
    n_pages, N = int(rng.integers(1, 6)), 24
    tok = H * D * E
    pool = dict(num_layers=L, num_kv=KV, num_heads=H, head_dim=D, elem_bytes=E, block_size=bs,
                num_blocks=N, block_stride=bs * tok)
    tbl = rng.permutation(N)[:n_pages].astype(np.int32)
    T = n_pages * bs
    regions = cases.regions_for(pool, rng)
    base = dict(chunk_layers=L, chunk_tokens=T, layer_begin=0, layer_end=L,
                slot_bytes=L * KV * T * tok, n_slots=1)
    lf = cases.staging_for(base)
    pf = cases.staging_for(base)
    oracle.gather(pool, regions, [(tbl, 0, T, 0)], dict(base, layout=0), lf)
    oracle.gather(pool, regions, [(tbl, 0, T, 0)], dict(base, layout=1), pf)
    lf6 = lf.reshape(L, KV, n_pages, bs, tok)
    assert np.array_equal(pf, np.ascontiguousarray(lf6.transpose(2, 0, 1, 3, 4)).reshape(-1))
    # and back: scattering either chunk restores the same pool
    a = np.full_like(regions, W.SENTINEL)
    b = np.full_like(regions, W.SENTINEL)
    oracle.scatter(pool, a, [(tbl, 0, T, 0)], dict(base, layout=0), lf)
    oracle.scatter(pool, b, [(tbl, 0, T, 0)], dict(base, layout=1), pf)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("seed", range(10))
def test_byte_histogram_is_conserved(seed):
    rng = np.random.default_rng(5000 + seed)
    pool, spans, chunks = cases.make_case(rng, head_major=None)
    regions = cases.regions_for(pool, rng)
    buf = cases.staging_for(chunks)
    written = oracle.gather(pool, regions, spans, chunks, buf)
    mask = _referenced_mask(pool, spans, chunks)
    assert written == int(mask.sum())
    after = np.bincount(buf, minlength=256).astype(np.int64)
    after[W.SENTINEL] -= buf.size - written
    assert np.array_equal(after, np.bincount(regions[mask], minlength=256))


def test_page_sizes_from_the_pages():
    g = json.load(open(os.path.join(GOLDEN, "page_sizes.json")))
    fx = g["fragmentation_example"]
    # One layer of the figure's request, Llama-3-8B-shaped K: 8 heads x 128 dims x 2 bytes.
    H, D, E, bs, T = 8, 128, 2, fx["page_tokens"], fx["context_tokens"]
    pages = T // bs
    pool = dict(num_layers=1, num_kv=1, num_heads=H, head_dim=D, elem_bytes=E, block_size=bs,
                num_blocks=pages, block_stride=bs * H * D * E)
    assert pool["block_stride"] == fx["approx_bytes_per_layer_page"]
    assert pages == fx["transfers_per_layer"]
    assert pages * fx["layers"] == fx["transfers_per_request"]
    rng = np.random.default_rng(7)
    tbl = rng.permutation(pages).astype(np.int32)
    regions = rng.integers(0, 256, size=(1, pages * pool["block_stride"]), dtype=np.uint8)
    chunks = dict(layout=1, chunk_layers=1, chunk_tokens=T, layer_begin=0, layer_end=1,
                  slot_bytes=T * H * D * E, n_slots=1)
    buf = cases.staging_for(chunks)
    n = oracle.gather(pool, regions, [(tbl, 0, T, 0)], chunks, buf)
    assert n == fx["transfers_per_layer"] * fx["approx_bytes_per_layer_page"]
    # each of the 256 page-sized pieces of the chunk is one whole pool block
    pieces = buf.reshape(pages, -1)
    blocks = regions.reshape(pages, -1)
    assert all(np.array_equal(pieces[i], blocks[tbl[i]]) for i in range(pages))
    g8 = g["llama8b_layer_page"]
    assert g8["page_tokens"] * g8["kv_heads"] * g8["head_dim"] * g8["elem_bytes"] == g8["bytes_per_layer_page"]


@pytest.mark.parametrize("bad", [
    dict(t_begin=3),                   # span must start on a page boundary
    dict(chunk_tokens=6),              # chunk_tokens must be whole pages
    dict(chunk_layers=2, layer_end=3),  # chunk_layers must divide the layer range
    dict(layer_end=0),                 # empty layer range
    dict(block_id=99),                 # block id past the pool
    dict(slot_bytes=64),               # chunk does not fit its slot
])
def test_oracle_rejects_broken_preconditions(bad):
    pool = dict(num_layers=3, num_kv=1, num_heads=1, head_dim=16, elem_bytes=1, block_size=4,
                num_blocks=8, block_stride=64)
    tbl = np.array([1, 2, 3, bad.get("block_id", 4)], dtype=np.int32)
    t0 = bad.get("t_begin", 0)
    chunks = dict(layout=0, chunk_layers=bad.get("chunk_layers", 1),
                  chunk_tokens=bad.get("chunk_tokens", 8), layer_begin=0,
                  layer_end=bad.get("layer_end", 3), slot_bytes=bad.get("slot_bytes", 256), n_slots=16)
    regions = np.zeros((3, 8 * 64), dtype=np.uint8)
    buf = cases.staging_for(chunks)
    with pytest.raises(ValueError):
        oracle.gather(pool, regions, [(tbl, t0, 16, 0)], chunks, buf)


# --- planted mistakes --------------------------------------------------------------

MUTANTS = [
    ("token-major pool order", "(j * P->num_heads + h)", "(h * P->block_size + j)"),
    ("layer/kv swapped in layer-first chunk", "(li * P->num_kv + kv) * T_c", "(kv * P->num_kv + li) * T_c"),
    ("page/layer swapped in page-first chunk", "(pi * CL + li)", "(li * CL + pi)"),
    ("chunk index transposed", "S->first_chunk + lc * n_tc + tc", "S->first_chunk + tc * n_tc + lc"),
    ("last chunk not short", "? CT : S->t_end - S->t_begin - tc * CT", "? CT : CT"),
    ("page-in-chunk ignores the token chunk", "p - (S->t_begin + tc * CT) / bs", "p - S->t_begin / bs"),
    ("ring modulo dropped", "(c % C->n_slots) * C->slot_bytes", "c * C->slot_bytes"),
    ("layer range offset dropped (li)", "li = (l - C->layer_begin) % CL", "li = l % CL"),
    ("layer range offset dropped (lc)", "lc = (l - C->layer_begin) / CL", "lc = l / CL"),
    ("block stride taken as the page size",
     "return b * P->block_stride + ((j * P->num_heads",
     "return b * P->block_size * P->num_heads * P->head_dim * P->elem_bytes + ((j * P->num_heads"),
    ("head-major page read token-major", "((h * P->block_size + j) * P->head_dim",
     "((j * P->num_heads + h) * P->head_dim"),
    ("head-major head stride wrong", "((h * P->block_size + j) * P->head_dim",
     "((h * P->block_size + j) * P->num_heads"),
    ("region index transposed", "bases[l * KV + kv]", "bases[kv * P->num_layers + l]"),
    ("head stride wrong", "* P->head_dim + d) * P->elem_bytes;\n}", "* P->head_dim + d);\n}"),
]


def _pins_pass(lib) -> bool:
    """Run a compact battery of the pins above against an oracle build."""
    for seed in range(60):
        rng = np.random.default_rng(seed)
        pool, spans, chunks = cases.make_case(rng, head_major=None)
        for direction in (oracle.GATHER, oracle.SCATTER):
            try:
                got, exp = _run_pair(direction, pool, spans, chunks, seed * 7 + direction, lib=lib)
            except ValueError:
                return False
            if not np.array_equal(got, exp):
                return False
    return True


def test_pins_pass_on_the_real_oracle():
    assert _pins_pass(oracle._load())


def _battery_in_child(so_path: str) -> int:
    """Run the battery against a build in a child process (a planted mistake may
    write out of bounds); exit code 0 means every pin passed."""
    code = ("import sys; sys.path[:0] = [%r, %r]; import test_oracle, oracle; "
            "sys.exit(0 if test_oracle._pins_pass(oracle.load_library(%r)) else 1)"
            % (os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
               os.path.dirname(os.path.abspath(__file__)), so_path))
    return subprocess.call([sys.executable, "-c", code], stdout=subprocess.DEVNULL,
                           stderr=subprocess.DEVNULL, timeout=300)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    assert src.count(old) == 1, "mutation anchor not unique: %r" % old
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "mut.c")
        so = os.path.join(d, "libmut.so")
        open(c, "w").write(src.replace(old, new))
        subprocess.check_call(["gcc", "-O1", "-fPIC", "-shared", "-fopenmp", c, "-o", so])
        assert _battery_in_child(so) != 0, "planted mistake %r went unnoticed" % name
