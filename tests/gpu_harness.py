"""Run one transfer through the C ABI on the GPU, from host (numpy) inputs.

Inputs come from the seeded generators; the oracle gets the same numpy bytes.
Before each launch the case is printed (and flushed) so a failing run names it.
"""
from __future__ import annotations

import numpy as np
import torch

from paged_layout_transfer_amd import kvxfer as K


def hip_runtime():
    """The HIP runtime library this process already uses (the copy torch loaded, which
    the transfer library shares), for direct runtime calls from tests."""
    device()
    return K.hip_runtime()


def device():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm device (torch.cuda.is_available() is False)")
    return torch.device("cuda", 0)


def describe(label, direction, pool, spans, chunks, extra=""):
    sp = [(int(np.asarray(t).size), int(a), int(b), int(c)) for t, a, b, c in spans]
    return "[gpu] %s %s pool=%s chunks=%s spans(len,t0,t1,fc)=%s %s" % (
        label, "gather" if direction == K.KV_GATHER else "scatter", pool, chunks, sp[:6], extra)


def run_transfer(direction: int, pool: dict, spans, chunks: dict, regions_np: np.ndarray,
                 staging_np: np.ndarray, *, ring: bool = False, ring_flags: int = K.KV_RING_COHERENT,
                 max_workgroups: int = 0, flags: int = 0, label: str = "",
                 region_views=None, dma: bool = False):
    """One gather or scatter.  regions_np is [L*KV, bytes] (rows are the regions) or,
    with region_views=(offsets, buffer_bytes), a flat buffer whose regions start at
    the given byte offsets (interleaved pools).  Returns (regions_after,
    staging_after, device_error_bits).  dma=True runs the per-tile copy-engine entry
    points, which take host block tables."""
    dev = device()
    L, KV = pool["num_layers"], pool["num_kv"]
    buf = torch.from_numpy(np.ascontiguousarray(regions_np)).to(dev)
    if region_views is None:
        row = buf.stride(0)
        bases = [buf.data_ptr() + i * row for i in range(L * KV)]
    else:
        bases = [buf.data_ptr() + off for off in region_views]
    tabs = [torch.from_numpy(np.ascontiguousarray(t, dtype=np.int32)).to(dev) for t, _, _, _ in spans]
    nbytes = chunks["slot_bytes"] * chunks["n_slots"]
    assert staging_np.size == nbytes
    ring_h = None
    if ring:
        ring_h = K.kv_ring_create(chunks["slot_bytes"], chunks["n_slots"], ring_flags)
        host = K.ring_host_array(ring_h, nbytes)
        host[:] = staging_np
        base = K.kv_ring_slot(ring_h, 0)[1]
    else:
        stg = torch.from_numpy(np.ascontiguousarray(staging_np)).to(dev)
        base = stg.data_ptr()
    desc = K.make_pool_desc(L, KV, pool["num_heads"], pool["head_dim"], pool["elem_bytes"],
                            pool["block_size"], pool["num_blocks"], pool["block_stride"], bases,
                            pool.get("page_layout", 0))
    host_tabs = [np.ascontiguousarray(t, dtype=np.int32) for t, _, _, _ in spans]
    if dma:
        sp = K.make_spans([(ht.ctypes.data, ht.size, t0, t1, fc)
                           for ht, (_, t0, t1, fc) in zip(host_tabs, spans)])
    else:
        sp = K.make_spans([(tb.data_ptr(), tb.numel(), t0, t1, fc)
                           for tb, (_, t0, t1, fc) in zip(tabs, spans)])
    spec = K.make_chunk_spec(chunks["layout"], chunks["chunk_layers"], chunks["chunk_tokens"],
                             chunks["layer_begin"], chunks["layer_end"], base,
                             chunks["slot_bytes"], chunks["n_slots"], max_workgroups, flags)
    h = K.kv_pool_create(desc)
    try:
        torch.cuda.synchronize()
        print(describe(label, direction, pool, spans, chunks,
                       "ring=%s wg=%d dma=%s" % (ring, max_workgroups, dma)), flush=True)
        stream = torch.cuda.current_stream()
        if dma:
            fn = K.kv_gather_chunks_dma if direction == K.KV_GATHER else K.kv_scatter_chunks_dma
        else:
            fn = K.kv_gather_chunks if direction == K.KV_GATHER else K.kv_scatter_chunks
        fn(h, sp, spec, stream)
        bits = K.kv_pool_get_error(h, stream)
        torch.cuda.synchronize()
        regions_after = buf.cpu().numpy()
        staging_after = host.copy() if ring else stg.cpu().numpy()
    finally:
        K.kv_pool_destroy(h)
        if ring_h is not None:
            K.kv_ring_destroy(ring_h)
    return regions_after, staging_after, bits
