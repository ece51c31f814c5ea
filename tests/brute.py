"""Brute-force second formulation of the paged-KV transfer, for pinning the oracle.

The oracle (oracle/oracle.c) walks the pool side and *encodes* each element's
chunk address.  This module goes the other way: it enumerates every byte of
every staging slot, *decodes* the byte's position into chunk coordinates by
repeated div/mod over the chunk's shape, and from those coordinates finds the
pool byte it must hold (or that it is a pad / unused byte).  The two share no
code, so a dropped term, a wrong stride or a transposed axis in either one
shows up as a mismatch.

Definitions follow the Strata guide ("Two-Dimensional Memory Layout
Decoupling": layer-first HBM, page-first host/disk) and the Tutti summary
(Figure 4: one object per (layer, K/V) per block).  Vectorised with numpy over
byte positions; meant for shapes of at most a few MiB.
"""
from __future__ import annotations

import numpy as np


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def slot_map(pool: dict, spans, chunks: dict):
    """For every byte of the staging buffer (n_slots*slot_bytes), the pool region
    index and byte offset it corresponds to, or region -1 when no element maps
    there.  Returns (region[int64], offset[int64])."""
    L, KV, H, D, E = (pool[k] for k in ("num_layers", "num_kv", "num_heads", "head_dim", "elem_bytes"))
    bs, stride = pool["block_size"], pool["block_stride"]
    CL, CT = chunks["chunk_layers"], chunks["chunk_tokens"]
    lb, le = chunks["layer_begin"], chunks["layer_end"]
    SB, NS = chunks["slot_bytes"], chunks["n_slots"]
    n_lc = (le - lb) // CL
    total = SB * NS
    region = np.full(total, -1, dtype=np.int64)
    offset = np.zeros(total, dtype=np.int64)
    owner = {}
    for r, (tbl, t0, t1, fc) in enumerate(spans):
        tbl = np.asarray(tbl, dtype=np.int64)
        n_tc = _cdiv(t1 - t0, CT)
        for lc in range(n_lc):
            for tc in range(n_tc):
                c = fc + lc * n_tc + tc
                s = c % NS
                assert s not in owner, "two chunks share a slot"
                owner[s] = (r, lc, tc)
                first_tok = t0 + tc * CT
                T_c = min(CT, t1 - first_tok)
                o = np.arange(SB, dtype=np.int64)
                q, e = np.divmod(o, E)
                q, d = np.divmod(q, D)
                q, h = np.divmod(q, H)
                if chunks["layout"] == 0:     # [CL][KV][T_c][H][D]
                    q, ti = np.divmod(q, T_c)
                    li, kv = np.divmod(q, KV)
                    ok = li < CL
                    t = first_tok + ti
                else:                          # [P_c][CL][KV][bs][H][D]
                    q, j = np.divmod(q, bs)
                    q, kv = np.divmod(q, KV)
                    pi, li = np.divmod(q, CL)
                    ok = pi < _cdiv(T_c, bs)
                    t = first_tok + pi * bs + j
                    ok &= t < t1
                l = lb + lc * CL + li
                p = np.where(ok, t // bs, 0)
                blk = tbl[p]
                jj = t % bs
                if pool.get("page_layout", 0) == 1:   # [H][bs][D] pages
                    off = blk * stride + ((h * bs + jj) * D + d) * E + e
                else:                                 # [bs][H][D] pages
                    off = blk * stride + ((jj * H + h) * D + d) * E + e
                base = s * SB
                region[base:base + SB] = np.where(ok, l * KV + kv, -1)
                offset[base:base + SB] = np.where(ok, off, 0)
    return region, offset


def gather(pool: dict, regions: np.ndarray, spans, chunks: dict, chunk_buf: np.ndarray) -> np.ndarray:
    """Expected staging buffer after a gather: mapped bytes from the pool, others unchanged."""
    reg, off = slot_map(pool, spans, chunks)
    out = chunk_buf.copy()
    m = reg >= 0
    out[m] = regions[reg[m], off[m]]
    return out


def scatter(pool: dict, regions: np.ndarray, spans, chunks: dict, chunk_buf: np.ndarray) -> np.ndarray:
    """Expected pool after a scatter: mapped pool bytes from the staging buffer, others unchanged."""
    reg, off = slot_map(pool, spans, chunks)
    out = regions.copy()
    m = reg >= 0
    out[reg[m], off[m]] = chunk_buf[m]
    return out
