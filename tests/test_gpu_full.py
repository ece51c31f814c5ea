"""Full-size parity: every workload at its stated size, in the launch configuration
bench.py times (default grid, HBM or pinned-host staging as the workload says),
checked against the oracle on sampled layers and requests.

A sampled check runs the oracle on one request with its chunks numbered from 0
(the same call restricted to that request) and one layer.  The positions the
oracle writes are found by running it over two different initial fills; the GPU
must hold the oracle's bytes there.  For scatter, every byte of the sampled
layer that no request writes must still hold the sentinel.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from paged_layout_transfer_amd import kvxfer as K
from paged_layout_transfer_amd import workloads as W

pytestmark = pytest.mark.gpu


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


def n_chunks_of(w, t0, t1):
    return (w["num_layers"] // w["chunk_layers"]) * -(-(t1 - t0) // w["chunk_tokens"])


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

    def rows_of(self, layer):
        return [self.P[layer * self.KV + k].cpu().numpy() for k in range(self.KV)]

    def sub(self, r):
        """Request r alone, its chunks numbered from 0, and the slice of the full
        staging buffer its chunks occupy."""
        tbl, t0, t1, fc = self.spans_h[r]
        n = n_chunks_of(self.w, t0, t1)
        sb = self.chunks["slot_bytes"]
        return (tbl, t0, t1, 0), dict(self.chunks, n_slots=n), (fc * sb, (fc + n) * sb)


def gather_check(S, stg, layer, requests):
    rows = [None] * (S.L * S.KV)
    for k, r in enumerate(S.rows_of(layer)):
        rows[layer * S.KV + k] = r
    for r in requests:
        span, chunks, (lo, hi) = S.sub(r)
        a = np.zeros(hi - lo, dtype=np.uint8)
        b = np.full(hi - lo, 0xFF, dtype=np.uint8)
        oracle.gather(S.pool, rows, [span], chunks, a, only_layers=(layer, layer + 1))
        oracle.gather(S.pool, rows, [span], chunks, b, only_layers=(layer, layer + 1))
        m = a == b
        assert m.any()
        got = stg[lo:hi].cpu().numpy()
        assert np.array_equal(got[m], a[m]), "gather: request %d layer %d" % (r, layer)


def scatter_check(S, stg, layer, requests):
    """GPU pool started at the sentinel; stg is the staging buffer the scatter read."""
    got = S.rows_of(layer)
    pool, bs, stride = S.pool, S.pool["block_size"], S.pool["block_stride"]
    written = np.zeros(pool["num_blocks"], dtype=bool)
    for tbl, t0, t1, _ in S.spans_h:
        written[tbl[t0 // bs: -(-t1 // bs)]] = True
    for k in range(S.KV):
        blocks = got[k].reshape(pool["num_blocks"], stride)
        assert np.all(blocks[~written] == W.SENTINEL), "scatter wrote a block no request names"
    # the sampled requests own distinct blocks, so one pair of oracle rows serves them all
    ea = [None] * (S.L * S.KV)
    eb = [None] * (S.L * S.KV)
    for k in range(S.KV):
        ea[layer * S.KV + k] = np.zeros(S.row, dtype=np.uint8)
        eb[layer * S.KV + k] = np.full(S.row, 0xFF, dtype=np.uint8)
    own = np.zeros(pool["num_blocks"], dtype=bool)
    for r in requests:
        span, chunks, (lo, hi) = S.sub(r)
        src = stg[lo:hi].cpu().numpy()
        oracle.scatter(S.pool, ea, [span], chunks, src, only_layers=(layer, layer + 1))
        oracle.scatter(S.pool, eb, [span], chunks, src, only_layers=(layer, layer + 1))
        tbl, t0, t1, _ = span
        own[tbl[t0 // bs: -(-t1 // bs)]] = True
    for k in range(S.KV):
        a, b = ea[layer * S.KV + k], eb[layer * S.KV + k]
        m = a == b
        assert m.any()
        assert np.array_equal(got[k][m], a[m]), "scatter: layer %d kv %d" % (layer, k)
        # inside the sampled requests' blocks, bytes no request writes stay at the sentinel
        rest = (~m).reshape(pool["num_blocks"], stride) & own[:, None]
        assert np.all(got[k].reshape(pool["num_blocks"], stride)[rest] == W.SENTINEL)


HBM_CASES = {
    "llama8b": dict(layers=[0, 31], requests=[0]),
    "mixed": dict(layers=[0, 31], requests=[0, 21, 42, 63]),
    "mla_fp8": dict(layers=[0, 60], requests=[0]),
    "int8_kv": dict(layers=[0, 60], requests=[0]),
    "llama8b_hnd": dict(layers=[0, 31], requests=[0]),
    "fp8_hnd_d64": dict(layers=[0, 31], requests=[0]),
    "llama8b_tp8": dict(layers=[0, 31], requests=[0]),
    "hnd_rows24": dict(layers=[0, 31], requests=[0]),
}


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", list(HBM_CASES))
def test_full_size_hbm(name):
    S = Setup(name)
    try:
        c = HBM_CASES[name]
        say(name, "pool %.1f GiB, staging %.1f GiB, %d requests" % (
            S.P.numel() / 2**30, S.plan["slot_bytes"] * S.plan["n_chunks"] / 2**30, len(S.spans_h)))
        W.device_fill_(S.P.view(-1), S.w["fill"], S.w["k"])
        stg = torch.empty(S.plan["slot_bytes"] * S.plan["n_chunks"], dtype=torch.uint8, device=S.dev)
        spec = K.make_chunk_spec(S.chunks["layout"], S.chunks["chunk_layers"], S.chunks["chunk_tokens"],
                                 0, S.L, stg, S.chunks["slot_bytes"], S.chunks["n_slots"])
        say(name, "gather")
        K.kv_gather_chunks(S.h, S.spans_d, spec, S.stream)
        assert K.kv_pool_get_error(S.h, S.stream) == 0
        for layer in c["layers"]:
            gather_check(S, stg, layer, c["requests"])
        say(name, "scatter")
        W.device_fill_(stg, "bytes", 200 + S.w["k"])
        S.P.fill_(W.SENTINEL)
        K.kv_scatter_chunks(S.h, S.spans_d, spec, S.stream)
        assert K.kv_pool_get_error(S.h, S.stream) == 0
        for layer in c["layers"]:
            scatter_check(S, stg, layer, c["requests"])
        del stg
    finally:
        S.close()


@pytest.mark.timeout(600)
def test_full_size_llama70b_pinned_ring():
    """The 128K-token 70B-shaped context through a pinned host ring of 4-layer windows
    (1024 slots of 2 MiB), both directions, every window moved, three checked."""
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
        checked = (0, 10, 19)

        def spec(i):
            return K.make_chunk_spec(K.KV_LAYER_FIRST, 1, w["chunk_tokens"], i * win, (i + 1) * win,
                                     ring_dev, slot, n_slots)

        def window_chunks(i):
            return dict(S.chunks, layer_begin=i * win, layer_end=(i + 1) * win, n_slots=n_slots)

        say("llama70b gather through the ring")
        for i in range(S.L // win):
            K.kv_gather_chunks(S.h, S.spans_d, spec(i), S.stream)
            assert K.kv_pool_get_error(S.h, S.stream) == 0
            if i in checked:
                layer = i * win
                rows = [None] * (S.L * S.KV)
                for k, r in enumerate(S.rows_of(layer)):
                    rows[layer * S.KV + k] = r
                a = np.zeros(slot * n_slots, dtype=np.uint8)
                b = np.full(slot * n_slots, 0xFF, dtype=np.uint8)
                span = S.spans_h[0]
                oracle.gather(S.pool, rows, [span], window_chunks(i), a, only_layers=(layer, layer + 1))
                oracle.gather(S.pool, rows, [span], window_chunks(i), b, only_layers=(layer, layer + 1))
                m = a == b
                assert m.any() and np.array_equal(ring_host[m], a[m]), "ring gather window %d" % i
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
        for i in checked:
            layer = i * win
            got = S.rows_of(layer)
            a = [None] * (S.L * S.KV)
            for k in range(S.KV):
                a[layer * S.KV + k] = np.full(S.row, W.SENTINEL, dtype=np.uint8)
            oracle.scatter(S.pool, a, [S.spans_h[0]], window_chunks(i), src, only_layers=(layer, layer + 1))
            for k in range(S.KV):
                assert np.array_equal(got[k], a[layer * S.KV + k]), "ring scatter window %d kv %d" % (i, k)
    finally:
        if ring is not None:
            K.kv_ring_destroy(ring)
        S.close()
