"""Random small transfer descriptions shared by the oracle pins and the GPU parity tests.

Every case is drawn from a seeded generator and obeys the call's preconditions:
spans start on page boundaries, block ids are distinct across the call (so a
scatter has one writer per pool byte), chunk_layers divides the layer range,
chunk_tokens is a whole number of pages and every chunk owns its own slot.
"""
from __future__ import annotations

import numpy as np

LAYER_FIRST = 0
PAGE_FIRST = 1


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


def slot_capacity(pool: dict, chunks: dict) -> int:
    """Bytes of a full chunk's worth of tokens: chunk_layers x K/V x chunk_tokens
    tokens.  chunk_tokens is a whole number of pages, so every chunk of either
    layout fits; used only to size staging slots."""
    tok = pool["num_heads"] * pool["head_dim"] * pool["elem_bytes"]
    return chunks["chunk_layers"] * pool["num_kv"] * chunks["chunk_tokens"] * tok


def head_rows_ok(row: int, tok: int) -> bool:
    """Head-major pages the library takes: head rows of whole 16-byte vectors, or of
    whole 4-byte words when a token (all heads) is at most 8 KiB."""
    return row % 16 == 0 or (row % 4 == 0 and tok <= 8192)


def make_case(rng: np.random.Generator, *, tok_multiple: int = 1, max_bytes: int = 1 << 20,
              layout: int | None = None, n_spans: int | None = None, medium: bool = False,
              head_major: bool | None = False):
    """A random case: (pool, spans, chunks) with tables as int32 arrays.

    Small cases use tiny heads (tokens of 8-144 bytes, pages of 2-16 tokens);
    medium cases use model-like heads (tokens of 64 B - 4 KiB, pages of 16-64
    tokens) so a page spans several 1 KiB wave copies plus a ragged tail.
    head_major: False = token-major pages, True = head-major, None = either."""
    while True:
        L = int(rng.integers(1, 5 if medium else 4))
        KV = int(rng.integers(1, 3))
        if medium:
            H = int(rng.choice([1, 2, 8]))
            D = int(rng.choice([64, 128, 576]))
            E = int(rng.choice([1, 2]))
        else:
            H = int(rng.integers(1, 4))
            D = int(rng.choice([8, 16, 24]))
            E = int(rng.choice([1, 2]))
        tok = H * D * E
        if tok % tok_multiple:
            continue
        bs = int(rng.choice([16, 32, 64] if medium else [2, 4, 16]))
        tile = bs * tok
        block_stride = tile + int(rng.choice([0, 0, 16, 48]))
        if block_stride % tok_multiple:
            block_stride = tile
        ns = int(n_spans) if n_spans else int(rng.integers(1, 4))
        spans_tok = []
        for _ in range(ns):
            p0 = int(rng.integers(0, 3))
            length = int(rng.integers(1, 4 * bs + 3))
            spans_tok.append((p0 * bs, p0 * bs + length))
        pages = [cdiv(t1, bs) for _, t1 in spans_tok]
        N = sum(pages) + int(rng.integers(0, 6))
        if N * block_stride * L * KV > max_bytes:
            continue
        perm = rng.permutation(N).astype(np.int32)
        tables, pos = [], 0
        for n in pages:
            tables.append(perm[pos:pos + n].copy())
            pos += n
        lb = int(rng.integers(0, L))
        le = int(rng.integers(lb + 1, L + 1))
        divs = [c for c in range(1, le - lb + 1) if (le - lb) % c == 0]
        CL = int(rng.choice(divs))
        CT = bs * int(rng.integers(1, 4))
        lay = int(rng.integers(0, 2)) if layout is None else layout
        page_layout = int(rng.integers(0, 2)) if head_major is None else int(head_major)
        if page_layout == 1 and not head_rows_ok(D * E, tok):
            if head_major:
                continue            # a head-major shape the library refuses: draw again
            page_layout = 0
        pool = dict(num_layers=L, num_kv=KV, num_heads=H, head_dim=D, elem_bytes=E,
                    block_size=bs, num_blocks=N, block_stride=block_stride, page_layout=page_layout)
        chunks = dict(layout=lay, chunk_layers=CL, chunk_tokens=CT, layer_begin=lb,
                      layer_end=le, slot_bytes=0, n_slots=0)
        n_chunks = [((le - lb) // CL) * cdiv(t1 - t0, CT) for t0, t1 in spans_tok]
        total = sum(n_chunks)
        n_slots = total + int(rng.integers(0, 4))
        start = int(rng.integers(0, n_slots))  # may wrap around the ring
        spans, c = [], start
        for (t0, t1), tbl, nc in zip(spans_tok, tables, n_chunks):
            spans.append((tbl, t0, t1, c))
            c += nc
        sb = slot_capacity(pool, chunks) + int(rng.choice([0, 0, 16]))
        if sb % tok_multiple:
            sb += tok_multiple - sb % tok_multiple
        chunks.update(slot_bytes=sb, n_slots=n_slots)
        if sb * n_slots > max_bytes:
            continue
        return pool, spans, chunks


def regions_for(pool: dict, rng: np.random.Generator) -> np.ndarray:
    n = pool["num_layers"] * pool["num_kv"]
    return rng.integers(0, 256, size=(n, pool["num_blocks"] * pool["block_stride"]), dtype=np.uint8)


def staging_for(chunks: dict, fill: int | None = None, rng: np.random.Generator | None = None) -> np.ndarray:
    n = chunks["slot_bytes"] * chunks["n_slots"]
    if rng is not None:
        return rng.integers(0, 256, size=n, dtype=np.uint8)
    return np.full(n, 0xA5 if fill is None else fill, dtype=np.uint8)


# H, D, E, bs: head rows not of whole 16-byte vectors (4-byte words), staged through LDS.
# Pages of at most 8 KiB go in token slabs of a whole page; pages of 8-20 KiB a whole page
# at a time in 16-byte vectors (20 x 12-byte rows, pages of 64; 100 x 12-byte rows,
# pages of 16; 32 x 8-byte rows, pages of 48; 24 x 12-byte rows, pages of 64); larger
# pages in 8 KiB slabs of all heads x tokens, tokens cut to whole pool lines (16 x
# 24-byte rows: 21 fit, 16 taken); too few for a whole line (4 x 100-byte rows: 20 fit,
# 32 would be needed); one token (64 x 100-byte rows).  Where a token slab would split
# pool lines (100 x 12-byte rows in pages of 32: 6 tokens fit, 32 would be needed; 128 x
# 8-byte rows: 8 fit, 16 needed), scatter takes slabs of whole pages of a group of heads
# (20 of 100, 32 of 128), and so does gather where the group's chunk runs are whole lines
# (32 x 8 bytes).
HM_LDS_SHAPES = [(4, 2, 2, 16), (2, 4, 2, 16), (4, 6, 2, 8), (8, 8, 1, 16), (4, 10, 2, 32), (2, 12, 2, 64),
                 (16, 12, 2, 64), (20, 3, 4, 64), (64, 100, 1, 4), (2, 1, 8, 16), (128, 8, 1, 32),
                 (4, 100, 1, 128), (100, 6, 2, 16), (100, 6, 2, 32), (32, 2, 4, 48), (24, 3, 4, 64)]


def head_major_case(rng: np.random.Generator, H: int, D: int, E: int, bs: int):
    """A head-major case of a given head shape: 1-3 layers, K/V or one, 1-2 spans that
    start 0-2 pages in and end in a partial page, chunks of 1-3 pages, either chunk
    layout, all layers per chunk or one."""
    L, KV = int(rng.integers(1, 4)), int(rng.integers(1, 3))
    tok = H * D * E
    spans_tok = [(int(rng.integers(0, 3)) * bs, 0) for _ in range(int(rng.integers(1, 3)))]
    spans_tok = [(t0, t0 + int(rng.integers(1, 6 * bs))) for t0, _ in spans_tok]   # partial last pages
    n_pages = sum(-(-t1 // bs) for _, t1 in spans_tok)
    N = n_pages + 5
    perm = rng.permutation(N).astype(np.int32)
    CT = bs * int(rng.integers(1, 4))
    layout = int(rng.integers(0, 2))
    CL = L if rng.random() < 0.5 else 1
    spans, used, fc, slot = [], 0, 0, 0
    for t0, t1 in spans_tok:
        n = -(-t1 // bs)
        tbl = perm[used:used + n]
        used += n
        n_tc = -(-(t1 - t0) // CT)
        spans.append((tbl, t0, t1, fc))
        fc += (L // CL) * n_tc
    slot = CL * KV * CT * tok
    pool = dict(num_layers=L, num_kv=KV, num_heads=H, head_dim=D, elem_bytes=E, block_size=bs, num_blocks=N,
                block_stride=bs * tok, page_layout=1)
    chunks = dict(layout=layout, chunk_layers=CL, chunk_tokens=CT, layer_begin=0, layer_end=L, slot_bytes=slot,
                  n_slots=fc)
    return pool, spans, chunks


# Shapes on each side of the launch rules, (H, D, E, block_size) -> what the launch does:
# token-major tiles of 4-6 KiB take one wave; 8-14 KiB tiles, and 16-18 KiB scatters, go
# in 4 parts; 16-18 KiB gathers, and non-power-of-two gathers from 64 KiB, walk 32 KiB
# segments (of 2, 4 or 8-vector groups by the pieces they cut); 20-56 KiB scatters, and
# such gathers that are not powers of two, go in 4 KiB parts, 32 KiB gathers whole;
# 64 KiB and larger tiles go in parts (72 KiB gathers in segments), scatters of 80, 96 and
# 144 KiB in 16 KiB parts.  Head-major:
# pages of at most 8 KiB with rows other than the 4 x 4 case through the LDS slabs, the
# 4 x 4 register transpose (scattered in 8 parts from 32 to under 64 KiB), LDS slabs of
# 16 KiB pages and more in 4 parts, and the cursor walk for larger pages of other rows.
RULE_SHAPES = {
    "tm_4k": (0, 1, 128, 2, 16), "tm_6k": (0, 3, 64, 2, 16), "tm_8k": (0, 2, 128, 2, 16),
    "tm_10k": (0, 5, 64, 2, 16), "tm_12k": (0, 3, 128, 2, 16), "tm_14k": (0, 7, 64, 2, 16),
    "tm_16k": (0, 8, 64, 2, 16), "tm_18k": (0, 9, 64, 2, 16), "tm_20k": (0, 5, 128, 2, 16),
    "tm_24k": (0, 3, 128, 2, 32), "tm_28k": (0, 7, 128, 2, 16), "tm_32k": (0, 8, 128, 2, 16),
    "tm_36k": (0, 1, 576, 1, 64), "tm_40k": (0, 5, 128, 2, 32), "tm_48k": (0, 3, 128, 2, 64),
    "tm_64k": (0, 8, 128, 2, 32), "tm_72k": (0, 9, 128, 2, 32), "tm_80k": (0, 5, 128, 2, 64),
    "tm_96k": (0, 3, 128, 2, 128), "tm_144k": (0, 9, 128, 2, 64),
    "hm_8k_2x256": (1, 2, 128, 2, 16), "hm_8k_1x512": (1, 1, 256, 2, 16), "hm_4k_2x128": (1, 2, 64, 2, 16),
    "hm_4k_8x32": (1, 8, 32, 1, 16), "hm_8k_t4": (1, 4, 128, 2, 8), "hm_16k_t4": (1, 4, 128, 2, 16),
    "hm_12k_3x256": (1, 3, 128, 2, 16), "hm_16k_1x256": (1, 1, 128, 2, 64), "hm_24k_3x512": (1, 3, 256, 2, 16),
    "hm_24k_6x256": (1, 6, 128, 2, 16), "hm_32k_t4": (1, 8, 128, 2, 16), "hm_48k_t4": (1, 12, 128, 2, 16),
    "hm_64k_t4": (1, 16, 128, 2, 16), "hm_32k_16x128": (1, 16, 64, 2, 16), "hm_24k_16x24": (1, 16, 12, 2, 64),
}


def rule_case(name: str, layout: int):
    """The call of RULE_SHAPES[name] with the given chunk layout (seeded by both)."""
    page_layout, H, D, E, bs = RULE_SHAPES[name]
    rng = np.random.default_rng(98_000 + 2 * sorted(RULE_SHAPES).index(name) + layout)
    pool, spans, chunks = head_major_case(rng, H, D, E, bs)
    pool["page_layout"] = page_layout
    chunks["layout"] = layout
    return pool, spans, chunks
