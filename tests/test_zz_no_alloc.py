"""kv_transfer_chunks_noalloc (static device scratch, no allocation) against the
allocating entry points kv_gather_chunks / kv_scatter_chunks, through the C ABI.

Each case runs the same call both ways on identical device inputs and compares the
whole pool and the whole staging buffer byte for byte (and with the oracle).  Two
noalloc calls are queued back to back on one stream with no synchronisation: the
first with more span records than ride in the kernel arguments (so they go through
the static scratch), the second a smaller call, which reuses the scratch the first
one left behind.  A block id out of range must set the caller's error word.

Under graph capture: a noalloc call whose span records ride in the kernel arguments
is captured and replayed (each replay after another pool's call has rewritten the
device scratch, each checked against the allocating entry point); a noalloc call with
more records, and the allocating entry points with that many records, are refused while
the stream captures; several calls captured into one graph replay in order.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import cases
import oracle
from paged_layout_transfer_amd import kvxfer as K

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        raise RuntimeError("needs a ROCm GPU")
    return torch.device("cuda", 0)


class Call:
    """One case's inputs on the device, twice (one copy per entry point)."""

    def __init__(self, pool, spans, chunks, seed, dev):
        rng = np.random.default_rng(seed)
        self.pool, self.spans, self.chunks = pool, spans, chunks
        self.regions = cases.regions_for(pool, rng)
        self.staging = cases.staging_for(chunks, rng=rng)
        self.tabs = [torch.from_numpy(np.ascontiguousarray(t, dtype=np.int32)).to(dev) for t, _, _, _ in spans]
        self.sp = K.make_spans([(tb.data_ptr(), tb.numel(), t0, t1, fc)
                                for tb, (_, t0, t1, fc) in zip(self.tabs, spans)])
        self.sides = []
        for _ in range(2):
            buf = torch.from_numpy(self.regions.copy()).to(dev)
            stg = torch.from_numpy(self.staging.copy()).to(dev)
            bases = [buf.data_ptr() + i * buf.stride(0) for i in range(buf.shape[0])]
            desc = K.make_pool_desc(pool["num_layers"], pool["num_kv"], pool["num_heads"], pool["head_dim"],
                                    pool["elem_bytes"], pool["block_size"], pool["num_blocks"],
                                    pool["block_stride"], bases, pool.get("page_layout", 0))
            spec = K.make_chunk_spec(chunks["layout"], chunks["chunk_layers"], chunks["chunk_tokens"],
                                     chunks["layer_begin"], chunks["layer_end"], stg, chunks["slot_bytes"],
                                     chunks["n_slots"])
            self.sides.append(dict(buf=buf, stg=stg, h=K.kv_pool_create(desc), spec=spec))

    def close(self):
        for s in self.sides:
            K.kv_pool_destroy(s["h"])

    def results(self):
        return [(s["buf"].cpu().numpy(), s["stg"].cpu().numpy()) for s in self.sides]

    def expected(self, direction):
        regs, stg = self.regions.copy(), self.staging.copy()
        oracle.transfer(direction, self.pool, [regs[i] for i in range(regs.shape[0])], self.spans, self.chunks, stg)
        return regs, stg


def _case(seed, n_spans, medium):
    return cases.make_case(np.random.default_rng(seed), tok_multiple=16, n_spans=n_spans, medium=medium,
                           max_bytes=(32 << 20) if medium else (4 << 20), head_major=None)


@pytest.mark.parametrize("direction", [K.KV_GATHER, K.KV_SCATTER])
def test_noalloc_matches_the_allocating_entry_point_on_two_calls_in_a_row(direction):
    dev = _dev()
    stream = torch.cuda.current_stream()
    big = Call(*_case(81_000 + direction, 40, True), seed=1 + direction, dev=dev)
    small = Call(*_case(82_000 + direction, 3, False), seed=3 + direction, dev=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    fn = K.kv_gather_chunks if direction == K.KV_GATHER else K.kv_scatter_chunks
    try:
        torch.cuda.synchronize()
        print("[noalloc] %s: 40-record call then 3-record call, no sync between" % (
            "gather" if direction == K.KV_GATHER else "scatter"), flush=True)
        for c in (big, small):
            fn(c.sides[0]["h"], c.sp, c.sides[0]["spec"], stream)
        for c in (big, small):
            K.kv_transfer_chunks_noalloc(c.sides[1]["h"], direction, c.sp, c.sides[1]["spec"], err, stream)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert K.kv_pool_get_error(big.sides[0]["h"], stream) == 0
        for c in (big, small):
            (r0, s0), (r1, s1) = c.results()
            assert np.array_equal(s1, s0), "staging differs from the allocating entry point"
            assert np.array_equal(r1, r0), "pool differs from the allocating entry point"
            er, es = c.expected(direction)
            assert np.array_equal(s1, es) and np.array_equal(r1, er), "differs from the oracle"
    finally:
        big.close()
        small.close()


def test_noalloc_reports_a_bad_block_id_in_the_callers_word():
    dev = _dev()
    stream = torch.cuda.current_stream()
    pool, spans, chunks = _case(83_000, 2, False)
    tbl, t0, t1, fc = spans[0]
    bad = tbl.copy()
    bad[t0 // pool["block_size"]] = pool["num_blocks"] + 5
    spans[0] = (bad, t0, t1, fc)
    c = Call(pool, spans, chunks, seed=9, dev=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    try:
        torch.cuda.synchronize()
        print("[noalloc] poisoned block id, both entry points", flush=True)
        K.kv_gather_chunks(c.sides[0]["h"], c.sp, c.sides[0]["spec"], stream)
        K.kv_transfer_chunks_noalloc(c.sides[1]["h"], K.KV_GATHER, c.sp, c.sides[1]["spec"], err, stream)
        torch.cuda.synchronize()
        assert int(err.item()) == K.KV_DEVERR_BLOCK_RANGE
        assert K.kv_pool_get_error(c.sides[0]["h"], stream) == K.KV_DEVERR_BLOCK_RANGE
        (r0, s0), (r1, s1) = c.results()
        assert np.array_equal(s1, s0) and np.array_equal(r1, r0)
    finally:
        c.close()


def test_noalloc_calls_queued_behind_busy_work_keep_their_own_records():
    """Two calls queued behind several milliseconds of other work on the stream, with no
    synchronisation: each call's region table and span records come from the pool's one
    host image, which the second call rewrites as soon as the first returns, so the
    first call's copy must have taken its bytes by then.  Both results must equal the
    allocating entry point's."""
    dev = _dev()
    stream = torch.cuda.current_stream()
    a = Call(*_case(84_000, 40, True), seed=11, dev=dev)
    b = Call(*_case(84_001, 40, True), seed=12, dev=dev)
    busy = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    try:
        torch.cuda.synchronize()
        print("[noalloc] two 40-record scatters queued behind busy work", flush=True)
        for c in (a, b):
            K.kv_scatter_chunks(c.sides[0]["h"], c.sp, c.sides[0]["spec"], stream)
        for _ in range(20):
            busy.fill_(7)                       # ~20 passes over 1 GiB ahead of the calls
        for c in (a, b):
            K.kv_transfer_chunks_noalloc(c.sides[1]["h"], K.KV_SCATTER, c.sp, c.sides[1]["spec"], None, stream)
        torch.cuda.synchronize()
        for c in (a, b):
            (r0, s0), (r1, s1) = c.results()
            assert np.array_equal(r1, r0) and np.array_equal(s1, s0), "a queued call used another call's records"
    finally:
        a.close()
        b.close()
        del busy


@pytest.mark.parametrize("mode", ["global", "relaxed"])
@pytest.mark.parametrize("direction", [K.KV_GATHER, K.KV_SCATTER])
def test_noalloc_call_replays_from_a_captured_graph(direction, mode):
    dev = _dev()
    c = Call(*_case(85_000 + direction, 3, False), seed=21 + direction, dev=dev)
    other = Call(*_case(85_100 + direction, 2, False), seed=31 + direction, dev=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    name = "gather" if direction == K.KV_GATHER else "scatter"
    ref, side = c.sides[0], c.sides[1]
    dst = side["stg"] if direction == K.KV_GATHER else side["buf"]
    start = dst.clone()
    g = None
    try:
        stream = torch.cuda.current_stream()
        fn = K.kv_gather_chunks if direction == K.KV_GATHER else K.kv_scatter_chunks
        fn(ref["h"], c.sp, ref["spec"], stream)
        torch.cuda.synchronize()
        want_buf, want_stg = ref["buf"].cpu().numpy(), ref["stg"].cpu().numpy()
        # one eager call first, so the pool's per-address caches are warm before capture
        K.kv_transfer_chunks_noalloc(side["h"], direction, c.sp, side["spec"], err, stream)
        dst.copy_(start)
        torch.cuda.synchronize()
        print("[noalloc] %s captured in %s mode, replayed 3 times" % (name, mode), flush=True)
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        with torch.cuda.graph(g, stream=cap, capture_error_mode=mode):
            K.kv_transfer_chunks_noalloc(side["h"], direction, c.sp, side["spec"], err, cap)
        torch.cuda.synchronize()
        for rep in range(3):
            # eager work in between: another pool's call leaves its region table in the scratch
            K.kv_transfer_chunks_noalloc(other.sides[1]["h"], direction, other.sp, other.sides[1]["spec"], None,
                                         stream)
            dst.copy_(start)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert int(err.item()) == 0
            assert np.array_equal(side["buf"].cpu().numpy(), want_buf), "replay %d: pool differs" % rep
            assert np.array_equal(side["stg"].cpu().numpy(), want_stg), "replay %d: staging differs" % rep
    finally:
        del g
        c.close()
        other.close()


def test_capture_refuses_calls_that_cannot_replay():
    """While a stream captures: calls with more span records than the kernel arguments
    carry, through the allocating entry points and the noalloc one, return
    KV_ERR_CAPTURE and enqueue nothing; the capture itself stays valid, and the same
    calls made eagerly afterwards match the oracle."""
    dev = _dev()
    c = Call(*_case(87_000, 40, True), seed=51, dev=dev)
    x = torch.zeros(16, device=dev)
    try:
        torch.cuda.synchronize()
        print("[noalloc] refused calls under capture", flush=True)
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        codes = []
        with torch.cuda.graph(g, stream=cap):
            x.add_(1)
            for call in (lambda: K.kv_gather_chunks(c.sides[0]["h"], c.sp, c.sides[0]["spec"], cap),
                         lambda: K.kv_scatter_chunks(c.sides[0]["h"], c.sp, c.sides[0]["spec"], cap),
                         lambda: K.kv_transfer_chunks_noalloc(c.sides[1]["h"], K.KV_GATHER, c.sp,
                                                              c.sides[1]["spec"], None, cap)):
                with pytest.raises(K.KvError) as e:
                    call()
                codes.append(e.value.code)
        torch.cuda.synchronize()
        assert codes == [K.KV_ERR_CAPTURE] * 3
        g.replay()
        torch.cuda.synchronize()
        assert float(x[0]) == 1.0
        (r0, s0), (r1, s1) = c.results()
        assert np.array_equal(r0, c.regions) and np.array_equal(s0, c.staging), "a refused call wrote"
        assert np.array_equal(r1, c.regions) and np.array_equal(s1, c.staging), "a refused call wrote"
        stream = torch.cuda.current_stream()
        K.kv_gather_chunks(c.sides[0]["h"], c.sp, c.sides[0]["spec"], stream)
        K.kv_transfer_chunks_noalloc(c.sides[1]["h"], K.KV_GATHER, c.sp, c.sides[1]["spec"], None, stream)
        torch.cuda.synchronize()
        er, es = c.expected(K.KV_GATHER)
        for r, st in c.results():
            assert np.array_equal(st, es) and np.array_equal(r, er)
    finally:
        c.close()


def test_several_noalloc_calls_in_one_captured_graph():
    """One call per layer chunk of a pool, each into its own staging buffer, captured in
    order on one stream: each carries its own copy of the region table into the shared
    device scratch and the graph's nodes run in capture order, so every replay equals
    the same calls made eagerly through the allocating entry point, buffer for buffer."""
    dev = _dev()
    pool, spans, chunks = _case(88_044, 3, False)
    c = Call(pool, spans, chunks, seed=61, dev=dev)
    ref, side = c.sides[0], c.sides[1]
    CL = chunks["chunk_layers"]
    wins = [(lo, lo + CL) for lo in range(chunks["layer_begin"], chunks["layer_end"], CL)]
    assert len(wins) >= 3
    nbytes = chunks["slot_bytes"] * chunks["n_slots"]
    start = torch.from_numpy(c.staging.copy()).to(dev)
    ref_stg = [start.clone() for _ in wins]
    side_stg = [start.clone() for _ in wins]
    stream = torch.cuda.current_stream()
    g = None

    def spec(buf, lo, hi):
        return K.make_chunk_spec(chunks["layout"], CL, chunks["chunk_tokens"], lo, hi, buf, chunks["slot_bytes"],
                                 chunks["n_slots"])

    try:
        assert start.numel() == nbytes
        for (lo, hi), b in zip(wins, ref_stg):
            K.kv_gather_chunks(ref["h"], c.sp, spec(b, lo, hi), stream)
        for (lo, hi), b in zip(wins, side_stg):  # warm the pool's caches outside capture
            K.kv_transfer_chunks_noalloc(side["h"], K.KV_GATHER, c.sp, spec(b, lo, hi), None, stream)
        torch.cuda.synchronize()
        want = [b.cpu().numpy() for b in ref_stg]
        print("[noalloc] %d gather windows captured in one graph" % len(wins), flush=True)
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        with torch.cuda.graph(g, stream=cap):
            for (lo, hi), b in zip(wins, side_stg):
                K.kv_transfer_chunks_noalloc(side["h"], K.KV_GATHER, c.sp, spec(b, lo, hi), None, cap)
        for rep in range(3):
            for b in side_stg:
                b.copy_(start)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for w, (b, e) in enumerate(zip(side_stg, want)):
                assert np.array_equal(b.cpu().numpy(), e), "replay %d, window %d differs" % (rep, w)
            assert not all(np.array_equal(e, c.staging) for e in want)
    finally:
        del g
        c.close()
