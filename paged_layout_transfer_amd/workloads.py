"""Seeded synthetic inputs for the paged-KV transfer workloads.

This module holds the input recipe only -- shapes, seeds, block tables, request
lengths, prefix-hit lengths and random fills -- and none of the transfer's
address arithmetic.  Both the HIP path's tests and the oracle's tests draw their
inputs from here, so the two sides see identical bytes.

The workloads stand in for the long-context serving traffic the Strata guide
("Comprehensive Evaluation Results") and the Tutti summary ("Workload
characterization") evaluate on public suites; only their scale (32K-128K-token
contexts, 16-64-token pages) is taken.  A copy's result does not depend on the
values, so random bytes of the stated element width are used.

Seeds: table/length seed 1000 + k and data seed k for workload k
(tiny 1, llama8b 2, llama70b 3, mixed 4, mla_fp8 5, int8_kv 6, llama8b_hnd 7,
fp8_hnd_d64 8, llama8b_tp8 9, hnd_rows24 10, hnd_h100_r12 11, llama8b_tp2 12, llama8b_tp4 13,
llama8b_hnd_tp4 14).  page_layout (default 0) is the pool's in-page order: 0 token-major
[block_size][H][D], 1 head-major [H][block_size][D].
"""
from __future__ import annotations

import math

import numpy as np

LAYER_FIRST = 0
PAGE_FIRST = 1

# Per-workload recipe.  Shapes follow the model families the workloads are named for;
# pool sizes, chunk shapes and the lognormal sigma are stated readings where the
# workload description leaves them open.
WORKLOADS: dict[str, dict] = {
    # 2 layers x K/V x 2 heads x 64 dims, fp16 random bit patterns, 16-token pages.
    "tiny": dict(k=1, num_layers=2, num_kv=2, num_heads=2, head_dim=64, elem_bytes=2,
                 block_size=16, num_blocks=64, tokens=256, fill="u16_bits",
                 layout=LAYER_FIRST, chunk_layers=2, chunk_tokens=256, staging="hbm"),
    # Llama-3-8B-shaped KV: 32 layers, 8 KV heads, head dim 128, bf16 U[-1,1).
    "llama8b": dict(k=2, num_layers=32, num_kv=2, num_heads=8, head_dim=128, elem_bytes=2,
                    block_size=16, num_blocks=16384, tokens=32768, fill="bf16_uniform",
                    layout=LAYER_FIRST, chunk_layers=32, chunk_tokens=256, staging="hbm"),
    # Llama-3-70B-shaped KV: 80 layers, one 128K-token context, 1 layer x 512 tokens = 2 MiB chunks.
    "llama70b": dict(k=3, num_layers=80, num_kv=2, num_heads=8, head_dim=128, elem_bytes=2,
                     block_size=16, num_blocks=16384, tokens=131072, fill="bf16_uniform",
                     layout=LAYER_FIRST, chunk_layers=1, chunk_tokens=512, staging="host"),
    # Mixed batch: 64 requests, lognormal lengths (median 8K, sigma 1) clipped to [1K, 64K],
    # a U[0, 0.95] prefix-hit fraction floored to whole pages; only the suffix moves.
    "mixed": dict(k=4, num_layers=32, num_kv=2, num_heads=8, head_dim=128, elem_bytes=2,
                  block_size=32, num_blocks=None, n_requests=64, median=8192, sigma=1.0,
                  min_len=1024, max_len=65536, max_hit=0.95, fill="bf16_uniform",
                  layout=LAYER_FIRST, chunk_layers=32, chunk_tokens=256, staging="hbm"),
    # MLA-style latent: one 576-wide fp8 latent per token, 61 layers, page-first chunks.
    "mla_fp8": dict(k=5, num_layers=61, num_kv=1, num_heads=1, head_dim=576, elem_bytes=1,
                    block_size=64, num_blocks=2048, tokens=65536, fill="bytes",
                    layout=PAGE_FIRST, chunk_layers=61, chunk_tokens=64, staging="hbm"),
    # int8 K/V, 8 heads x 128, 61 layers, page-first chunks.
    "int8_kv": dict(k=6, num_layers=61, num_kv=2, num_heads=8, head_dim=128, elem_bytes=1,
                    block_size=64, num_blocks=2048, tokens=65536, fill="bytes",
                    layout=PAGE_FIRST, chunk_layers=61, chunk_tokens=64, staging="hbm"),
    # One GPU's share of the llama8b context under 8-way tensor parallelism: the 8 KV
    # heads split one per GPU, so 16-token pages of 1 head x 128 bf16 = 4 KiB tiles.
    "llama8b_tp8": dict(k=9, num_layers=32, num_kv=2, num_heads=1, head_dim=128, elem_bytes=2,
                        block_size=16, num_blocks=16384, tokens=32768, fill="bf16_uniform",
                        layout=LAYER_FIRST, chunk_layers=32, chunk_tokens=256, staging="hbm"),
    # One GPU's share under 4-way tensor parallelism: 2 KV heads per GPU, 16-token pages
    # of 2 heads x 128 bf16 = 8 KiB tiles.
    "llama8b_tp4": dict(k=13, num_layers=32, num_kv=2, num_heads=2, head_dim=128, elem_bytes=2,
                        block_size=16, num_blocks=16384, tokens=32768, fill="bf16_uniform",
                        layout=LAYER_FIRST, chunk_layers=32, chunk_tokens=256, staging="hbm"),
    # One GPU's share under 2-way tensor parallelism: 4 KV heads per GPU, 16-token pages
    # of 4 heads x 128 bf16 = 16 KiB tiles.
    "llama8b_tp2": dict(k=12, num_layers=32, num_kv=2, num_heads=4, head_dim=128, elem_bytes=2,
                        block_size=16, num_blocks=16384, tokens=32768, fill="bf16_uniform",
                        layout=LAYER_FIRST, chunk_layers=32, chunk_tokens=256, staging="hbm"),
    # One GPU's share under 4-way tensor parallelism with head-major pages: 2 heads of
    # 256-byte rows per 16-token page (8 KiB).
    "llama8b_hnd_tp4": dict(k=14, num_layers=32, num_kv=2, num_heads=2, head_dim=128, elem_bytes=2,
                            block_size=16, num_blocks=16384, tokens=32768, fill="bf16_uniform",
                            layout=LAYER_FIRST, chunk_layers=32, chunk_tokens=256, staging="hbm",
                            page_layout=1),
    # The llama8b shape with head-major pages ([H][16][128] bf16: 256-byte head rows).
    "llama8b_hnd": dict(k=7, num_layers=32, num_kv=2, num_heads=8, head_dim=128, elem_bytes=2,
                        block_size=16, num_blocks=16384, tokens=32768, fill="bf16_uniform",
                        layout=LAYER_FIRST, chunk_layers=32, chunk_tokens=256, staging="hbm",
                        page_layout=1),
    # Head-major fp8 pages with short rows: 8 heads x 64 dims x 1 byte = 64-byte head rows.
    "fp8_hnd_d64": dict(k=8, num_layers=32, num_kv=2, num_heads=8, head_dim=64, elem_bytes=1,
                        block_size=16, num_blocks=16384, tokens=32768, fill="bytes",
                        layout=LAYER_FIRST, chunk_layers=32, chunk_tokens=256, staging="hbm",
                        page_layout=1),
    # Head-major pages whose head rows are not whole 16-byte vectors: 16 heads x 12 bf16
    # dims = 24-byte rows, 64-token pages (24 KiB per layer-page).
    "hnd_rows24": dict(k=10, num_layers=32, num_kv=2, num_heads=16, head_dim=12, elem_bytes=2,
                       block_size=64, num_blocks=4096, tokens=32768, fill="bf16_uniform",
                       layout=LAYER_FIRST, chunk_layers=32, chunk_tokens=256, staging="hbm",
                       page_layout=1),
    # Many heads with short rows of 4-byte words: 100 heads x 6 bf16 dims = 12-byte rows,
    # 16-token pages (a token is 1200 bytes, a page 18.75 KiB per (layer, K/V)).
    "hnd_h100_r12": dict(k=11, num_layers=32, num_kv=2, num_heads=100, head_dim=6, elem_bytes=2,
                         block_size=16, num_blocks=16384, tokens=32768, fill="bf16_uniform",
                         layout=LAYER_FIRST, chunk_layers=32, chunk_tokens=256, staging="hbm",
                         page_layout=1),
}


def token_major_twin(name: str) -> dict:
    """The same workload with token-major pages (page_layout 0): same shape, seeds,
    tables and chunks, so its rate is the reference a head-major pool is judged by."""
    w = dict(WORKLOADS[name])
    w["page_layout"] = 0
    return w


def table_rng(k: int) -> np.random.Generator:
    return np.random.default_rng(1000 + k)


def token_bytes(w: dict) -> int:
    """Bytes of one token of one (layer, K/V): heads x dims x element bytes (a shape, not a layout)."""
    return w["num_heads"] * w["head_dim"] * w["elem_bytes"]


def _draws(w: dict):
    """All table/length draws of a workload, from its one seeded generator."""
    rng = table_rng(w["k"])
    bs = w["block_size"]
    if "n_requests" in w:
        lens = rng.lognormal(mean=math.log(w["median"]), sigma=w["sigma"], size=w["n_requests"])
        lens = np.clip(np.rint(lens), w["min_len"], w["max_len"]).astype(np.int64)
        frac = rng.uniform(0.0, w["max_hit"], size=w["n_requests"])
        # a prefix hit is floored to whole pages: matches end on page boundaries
        hits = (np.floor(frac * lens / bs) * bs).astype(np.int64)
        reqs = [(int(h), int(n)) for h, n in zip(hits, lens)]
    else:
        reqs = [(0, int(w["tokens"]))]
    total_pages = sum(pages_of(t1, bs) for _, t1 in reqs)
    num_blocks = w["num_blocks"] if w.get("num_blocks") else int(math.ceil(1.05 * total_pages))
    if w["k"] == 1:
        # the tiny workload: a seeded choice of distinct ids
        perm = rng.choice(num_blocks, total_pages, replace=False).astype(np.int32)
    else:
        perm = rng.permutation(num_blocks).astype(np.int32)
    return reqs, num_blocks, perm


def pages_of(t_end: int, block_size: int) -> int:
    return -(-int(t_end) // int(block_size))


def resolve(w: dict) -> dict:
    """A workload with its draws filled in: requests [(t_begin, t_end)], num_blocks
    (the mixed pool is 5% over the pages its tables use) and block_tables (one
    global permutation of the pool's ids dealt to the requests in order, one id
    per page of each full context, prefix pages included, so no id repeats)."""
    w = dict(w)
    reqs, num_blocks, perm = _draws(w)
    tables, pos = [], 0
    for _, t1 in reqs:
        n = pages_of(t1, w["block_size"])
        if pos + n > perm.size:
            raise ValueError("pool too small for the requests")
        tables.append(perm[pos:pos + n].copy())
        pos += n
    w.update(requests=reqs, num_blocks=num_blocks, block_tables=tables)
    return w


def staging_plan(w: dict) -> dict:
    """How a resolved workload's requests are staged: every request moves all
    layers, chunk indices are numbered request after request, and each slot
    holds a full chunk (chunk_layers x K/V x chunk_tokens tokens).  Returns
    first_chunk per request, the chunk count and the slot size."""
    bs, CT, CL = w["block_size"], w["chunk_tokens"], w["chunk_layers"]
    per_layer_chunks = w["num_layers"] // CL
    first, c = [], 0
    for t0, t1 in w["requests"]:
        first.append(c)
        c += per_layer_chunks * -(-(t1 - t0) // CT)
    slot = CL * w["num_kv"] * CT * token_bytes(w)
    assert CT % bs == 0
    return dict(first_chunk=first, n_chunks=c, slot_bytes=slot)


def host_fill(nbytes: int, kind: str, seed: int) -> np.ndarray:
    """Seeded random contents as a flat uint8 array.

    u16_bits     : uniformly random 16-bit words (every fp16 bit pattern, NaNs included)
    bf16_uniform : U[-1, 1) rounded to bfloat16 (round to nearest even)
    bytes        : uniformly random bytes (every fp8 / int8 pattern)
    """
    rng = np.random.default_rng(seed)
    if kind == "bytes":
        return rng.integers(0, 256, size=nbytes, dtype=np.uint8)
    if nbytes % 2:
        raise ValueError("16-bit fills need an even byte count")
    if kind == "u16_bits":
        return rng.integers(0, 1 << 16, size=nbytes // 2, dtype=np.uint16).view(np.uint8)
    if kind == "bf16_uniform":
        f = rng.uniform(-1.0, 1.0, size=nbytes // 2).astype(np.float32)
        u = f.view(np.uint32)
        rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
        return rounded.astype(np.uint16).view(np.uint8)
    raise ValueError(kind)


def device_fill_(t, kind: str, seed: int, chunk_bytes: int = 1 << 30) -> None:
    """Seeded random contents for a flat uint8 torch tensor on the GPU, filled in
    slices so no large temporary is needed."""
    import torch

    g = torch.Generator(device=t.device)
    g.manual_seed(seed)
    n = t.numel()
    for off in range(0, n, chunk_bytes):
        sl = t[off:off + chunk_bytes]
        if kind == "bytes" or kind == "u16_bits":
            sl.random_(0, 256, generator=g)
        elif kind == "bf16_uniform":
            v = sl.view(torch.bfloat16)
            v.uniform_(-1.0, 1.0, generator=g)
        else:
            raise ValueError(kind)


SENTINEL = 0xA5
