"""Full-size parity: every workload at its stated size, in the launch configuration
bench.py times (default grid, HBM or pinned-host staging as the workload says),
compared with the oracle byte for byte over the whole call: every layer of every
request, both directions.

Gather: the staging buffer starts at the sentinel on the GPU and in the oracle's
copy; the oracle runs over the host copy of the pool, a batch of layers at a time
(so the host holds a bounded slice of the pool), and the whole staging buffer
must then match.  Scatter: the staging buffer holds seeded random bytes and the
pool starts at the sentinel on both sides; for each batch of layers the oracle
scatters into sentinel regions and the GPU's regions of those layers must match
in full, so a byte written where no request names it fails too.

The pinned-host workload (80 layers through a ring of 4-layer windows) is checked
window by window, both directions, every window.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from paged_layout_transfer_amd import kvxfer as K
from paged_layout_transfer_amd import workloads as W

pytestmark = pytest.mark.gpu

SLICE = 1 << 30            # bytes per device-to-host comparison slice
REGION_BUDGET = 24 << 30   # host bytes of pool regions held per oracle batch


def say(*a):
    print("[full]", *a, flush=True)


def resolve(name):
    w = W.resolve(W.WORKLOADS[name])
    tok = W.token_bytes(w)
    pool = {k: w[k] for k in ("num_layers", "num_kv", "num_heads", "head_dim", "elem_bytes",
                              "block_size", "num_blocks")}
    pool["block_stride"] = w["block_size"] * tok
    pool["page_layout"] = w.get("page_layout", 0)
    return w, pool


def to_host(t: torch.Tensor) -> np.ndarray:
    """A flat uint8 device tensor copied to a new host array, a slice at a time."""
    out = np.empty(t.numel(), dtype=np.uint8)
    ho = torch.from_numpy(out)
    for a in range(0, t.numel(), SLICE):
        ho[a:a + SLICE].copy_(t[a:a + SLICE])
    return out


def assert_device_equals(exp: np.ndarray, t: torch.Tensor, what: str):
    """exp (host) == t (device), compared a slice at a time; names the first differing byte."""
    assert exp.size == t.numel()
    for a in range(0, exp.size, SLICE):
        got = t[a:a + SLICE].cpu().numpy()
        e = exp[a:a + SLICE]
        if not np.array_equal(got, e):
            i = int(np.flatnonzero(got != e)[0])
            raise AssertionError("%s: first difference at byte %d (gpu %d, oracle %d)" % (
                what, a + i, got[i], e[i]))


def layer_batches(pool):
    per_layer = pool["num_kv"] * pool["num_blocks"] * pool["block_stride"]
    n = max(1, min(pool["num_layers"], REGION_BUDGET // per_layer))
    return [(l0, min(l0 + n, pool["num_layers"])) for l0 in range(0, pool["num_layers"], n)]


class Setup:
    def __init__(self, name):
        self.dev = torch.device("cuda", 0)
        self.w, self.pool = resolve(name)
        w, pool = self.w, self.pool
        self.plan = W.staging_plan(w)
        L, KV = pool["num_layers"], pool["num_kv"]
        self.L, self.KV = L, KV
        self.row = pool["num_blocks"] * pool["block_stride"]
        self.P = torch.empty((L * KV, self.row), dtype=torch.uint8, device=self.dev)
        bases = [self.P.data_ptr() + i * self.row for i in range(L * KV)]
        self.desc = K.make_pool_desc(L, KV, pool["num_heads"], pool["head_dim"], pool["elem_bytes"],
                                     pool["block_size"], pool["num_blocks"], pool["block_stride"], bases,
                                     pool["page_layout"])
        self.h = K.kv_pool_create(self.desc)
        self.tabs = [torch.from_numpy(t).to(self.dev) for t in w["block_tables"]]
        self.spans_h = [(t, t0, t1, fc) for t, (t0, t1), fc in
                        zip(w["block_tables"], w["requests"], self.plan["first_chunk"])]
        self.spans_d = K.make_spans([(tb, tb.numel(), t0, t1, fc) for tb, (_, t0, t1, fc) in
                                     zip(self.tabs, self.spans_h)])
        self.chunks = dict(layout=w["layout"], chunk_layers=w["chunk_layers"],
                           chunk_tokens=w["chunk_tokens"], layer_begin=0, layer_end=L,
                           slot_bytes=self.plan["slot_bytes"], n_slots=self.plan["n_chunks"])
        self.stream = torch.cuda.current_stream()

    def close(self):
        K.kv_pool_destroy(self.h)
        del self.P, self.tabs
        torch.cuda.empty_cache()

    def host_regions(self, l0, l1, fill=None):
        """Regions list for the oracle: layers [l0, l1) as host arrays (the GPU's bytes,
        or `fill` everywhere), None elsewhere."""
        regs = [None] * (self.L * self.KV)
        for i in range(l0 * self.KV, l1 * self.KV):
            regs[i] = to_host(self.P[i]) if fill is None else np.full(self.row, fill, dtype=np.uint8)
        return regs


HBM_WORKLOADS = ["llama8b", "mixed", "mla_fp8", "int8_kv", "llama8b_hnd", "fp8_hnd_d64", "llama8b_tp8", "llama8b_tp4", "llama8b_tp2", "llama8b_hnd_tp4",
                 "hnd_rows24", "hnd_h100_r12"]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", HBM_WORKLOADS)
def test_full_size_hbm_every_layer(name):
    S = Setup(name)
    try:
        nbytes = S.plan["slot_bytes"] * S.plan["n_chunks"]
        say(name, "pool %.1f GiB, staging %.1f GiB, %d requests, %d oracle threads" % (
            S.P.numel() / 2**30, nbytes / 2**30, len(S.spans_h), oracle.max_threads()))
        W.device_fill_(S.P.view(-1), S.w["fill"], S.w["k"])
        stg = torch.full((nbytes,), W.SENTINEL, dtype=torch.uint8, device=S.dev)
        spec = K.make_chunk_spec(S.chunks["layout"], S.chunks["chunk_layers"], S.chunks["chunk_tokens"],
                                 0, S.L, stg, S.chunks["slot_bytes"], S.chunks["n_slots"])
        say(name, "gather")
        K.kv_gather_chunks(S.h, S.spans_d, spec, S.stream)
        assert K.kv_pool_get_error(S.h, S.stream) == 0
        exp = np.full(nbytes, W.SENTINEL, dtype=np.uint8)
        for l0, l1 in layer_batches(S.pool):
            say(name, "gather oracle layers %d-%d" % (l0, l1 - 1))
            oracle.gather(S.pool, S.host_regions(l0, l1), S.spans_h, S.chunks, exp, only_layers=(l0, l1))
        assert_device_equals(exp, stg, "%s gather" % name)
        del exp

        say(name, "scatter")
        W.device_fill_(stg, "bytes", 200 + S.w["k"])
        src = to_host(stg)
        S.P.fill_(W.SENTINEL)
        K.kv_scatter_chunks(S.h, S.spans_d, spec, S.stream)
        assert K.kv_pool_get_error(S.h, S.stream) == 0
        for l0, l1 in layer_batches(S.pool):
            say(name, "scatter oracle layers %d-%d" % (l0, l1 - 1))
            regs = S.host_regions(l0, l1, fill=W.SENTINEL)
            oracle.scatter(S.pool, regs, S.spans_h, S.chunks, src, only_layers=(l0, l1))
            for i in range(l0 * S.KV, l1 * S.KV):
                assert_device_equals(regs[i], S.P[i], "%s scatter layer %d kv %d" % (name, i // S.KV, i % S.KV))
                regs[i] = None
        del stg, src
    finally:
        S.close()


@pytest.mark.timeout(900)
def test_full_size_llama70b_pinned_ring_every_window():
    """The 128K-token 70B-shaped context through a pinned host ring of 4-layer windows
    (1024 slots of 2 MiB), both directions, every window checked in full."""
    S = Setup("llama70b")
    ring = None
    try:
        w = S.w
        win = 4
        n_tc = -(-w["tokens"] // w["chunk_tokens"])
        slot = S.chunks["slot_bytes"]
        n_slots = win * n_tc
        ring = K.kv_ring_create(slot, n_slots)
        ring_dev = K.kv_ring_slot(ring, 0)[1]
        ring_host = K.ring_host_array(ring, slot * n_slots)
        W.device_fill_(S.P.view(-1), w["fill"], w["k"])
        span = S.spans_h[0]

        def spec(i):
            return K.make_chunk_spec(K.KV_LAYER_FIRST, 1, w["chunk_tokens"], i * win, (i + 1) * win,
                                     ring_dev, slot, n_slots)

        def window_chunks(i):
            return dict(S.chunks, layer_begin=i * win, layer_end=(i + 1) * win, n_slots=n_slots)

        say("llama70b gather through the ring, %d windows" % (S.L // win))
        for i in range(S.L // win):
            ring_host[:] = W.SENTINEL
            K.kv_gather_chunks(S.h, S.spans_d, spec(i), S.stream)
            assert K.kv_pool_get_error(S.h, S.stream) == 0
            exp = np.full(slot * n_slots, W.SENTINEL, dtype=np.uint8)
            oracle.gather(S.pool, S.host_regions(i * win, (i + 1) * win), [span], window_chunks(i), exp,
                          only_layers=(i * win, (i + 1) * win))
            if not np.array_equal(ring_host, exp):
                j = int(np.flatnonzero(ring_host != exp)[0])
                raise AssertionError("ring gather window %d: first difference at byte %d" % (i, j))
            say("gather window %d ok" % i)
        say("llama70b scatter through the ring")
        rnd = torch.empty(slot * n_slots, dtype=torch.uint8, device=S.dev)
        W.device_fill_(rnd, "bytes", 203)
        ring_host[:] = rnd.cpu().numpy()
        del rnd
        S.P.fill_(W.SENTINEL)
        for i in range(S.L // win):
            K.kv_scatter_chunks(S.h, S.spans_d, spec(i), S.stream)
        assert K.kv_pool_get_error(S.h, S.stream) == 0
        src = ring_host.copy()
        for i in range(S.L // win):
            l0, l1 = i * win, (i + 1) * win
            regs = S.host_regions(l0, l1, fill=W.SENTINEL)
            oracle.scatter(S.pool, regs, [span], window_chunks(i), src, only_layers=(l0, l1))
            for r in range(l0 * S.KV, l1 * S.KV):
                assert_device_equals(regs[r], S.P[r], "ring scatter window %d layer %d kv %d" % (
                    i, r // S.KV, r % S.KV))
            say("scatter window %d ok" % i)
    finally:
        if ring is not None:
            K.kv_ring_destroy(ring)
        S.close()
