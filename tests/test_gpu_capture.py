"""HIP graph capture of the allocating entry points, kv_gather_chunks and
kv_scatter_chunks, through the C ABI.

A call whose span records ride in the kernel arguments (at most 16 non-empty spans),
on a pool that has made a call before, is captured as its one kernel.  Each replay
must equal the oracle byte for byte, with eager calls on the same pool in between
(they take and recycle the pool's span-record arena, which the captured call does
not use).  Calls a graph could not replay as they stand are refused with
KV_ERR_CAPTURE while the stream captures: more span records, the first call on a pool
(it allocates), KV_FLAG_VALIDATE (it copies tables to the host), and timing on.  A
refused call enqueues nothing and leaves the capture valid.
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


class Setup:
    """One case's pool and staging on the device, with its pool handle."""

    def __init__(self, seed, n_spans, dev, flags=0):
        self.pool, self.spans, self.chunks = cases.make_case(np.random.default_rng(seed), tok_multiple=16,
                                                             n_spans=n_spans, max_bytes=4 << 20,
                                                             head_major=None)
        rng = np.random.default_rng(seed + 1)
        self.regions = cases.regions_for(self.pool, rng)
        self.staging = cases.staging_for(self.chunks, rng=rng)
        p, c = self.pool, self.chunks
        self.tabs = [torch.from_numpy(np.ascontiguousarray(t, dtype=np.int32)).to(dev) for t, _, _, _ in self.spans]
        self.sp = K.make_spans([(tb.data_ptr(), tb.numel(), t0, t1, fc)
                                for tb, (_, t0, t1, fc) in zip(self.tabs, self.spans)])
        self.buf = torch.from_numpy(self.regions.copy()).to(dev)
        self.stg = torch.from_numpy(self.staging.copy()).to(dev)
        bases = [self.buf.data_ptr() + i * self.buf.stride(0) for i in range(self.buf.shape[0])]
        self.h = K.kv_pool_create(K.make_pool_desc(p["num_layers"], p["num_kv"], p["num_heads"], p["head_dim"],
                                                   p["elem_bytes"], p["block_size"], p["num_blocks"],
                                                   p["block_stride"], bases, p.get("page_layout", 0)))
        self.spec = K.make_chunk_spec(c["layout"], c["chunk_layers"], c["chunk_tokens"], c["layer_begin"],
                                      c["layer_end"], self.stg, c["slot_bytes"], c["n_slots"], 0, flags)

    def reset(self):
        self.buf.copy_(torch.from_numpy(self.regions))
        self.stg.copy_(torch.from_numpy(self.staging))

    def expected(self, direction):
        regs, stg = self.regions.copy(), self.staging.copy()
        oracle.transfer(direction, self.pool, [regs[i] for i in range(regs.shape[0])], self.spans, self.chunks, stg)
        return regs, stg

    def check(self, direction, what):
        er, es = self.expected(direction)
        assert np.array_equal(self.stg.cpu().numpy(), es), "%s: staging differs from the oracle" % what
        assert np.array_equal(self.buf.cpu().numpy(), er), "%s: pool differs from the oracle" % what

    def close(self):
        K.kv_pool_destroy(self.h)


def _fn(direction):
    return K.kv_gather_chunks if direction == K.KV_GATHER else K.kv_scatter_chunks


@pytest.mark.parametrize("mode", ["global", "relaxed"])
@pytest.mark.parametrize("direction", [K.KV_GATHER, K.KV_SCATTER])
def test_allocating_call_replays_from_a_captured_graph(direction, mode):
    dev = _dev()
    s = Setup(89_000 + direction, 3, dev)
    fn = _fn(direction)
    name = "gather" if direction == K.KV_GATHER else "scatter"
    g = None
    try:
        stream = torch.cuda.current_stream()
        fn(s.h, s.sp, s.spec, stream)          # the pool's first call, outside the capture
        torch.cuda.synchronize()
        s.check(direction, "eager")
        s.reset()
        torch.cuda.synchronize()
        print("[capture] %s captured in %s mode, replayed 3 times" % (name, mode), flush=True)
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        with torch.cuda.graph(g, stream=cap, capture_error_mode=mode):
            fn(s.h, s.sp, s.spec, cap)
        torch.cuda.synchronize()
        assert np.array_equal(s.stg.cpu().numpy(), s.staging) and np.array_equal(s.buf.cpu().numpy(), s.regions), \
            "capture itself moved bytes"
        for rep in range(3):
            # eager calls on the same pool in between, through its span-record arena
            for _ in range(3):
                fn(s.h, s.sp, s.spec, stream)
            s.reset()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            s.check(direction, "replay %d" % rep)
        assert K.kv_pool_get_error(s.h, stream) == 0
    finally:
        del g
        s.close()


def test_capture_refuses_allocating_calls_that_cannot_replay():
    dev = _dev()
    fresh = Setup(89_100, 3, dev)                 # no call before the capture
    many = Setup(89_200, 40, dev)                 # more records than the kernel arguments carry
    checked = Setup(89_300, 3, dev, flags=K.KV_FLAG_VALIDATE)
    timed = Setup(89_400, 3, dev)
    x = torch.zeros(16, device=dev)
    try:
        stream = torch.cuda.current_stream()
        for s in (many, checked, timed):
            K.kv_gather_chunks(s.h, s.sp, s.spec, stream)
            s.reset()
        K.kv_pool_timing_start(timed.h)
        torch.cuda.synchronize()
        print("[capture] refused allocating calls under capture", flush=True)
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        codes = []
        with torch.cuda.graph(g, stream=cap):
            x.add_(1)
            for s in (fresh, many, checked, timed):
                for fn in (K.kv_gather_chunks, K.kv_scatter_chunks):
                    with pytest.raises(K.KvError) as e:
                        fn(s.h, s.sp, s.spec, cap)
                    codes.append(e.value.code)
        torch.cuda.synchronize()
        assert codes == [K.KV_ERR_CAPTURE] * 8
        g.replay()
        torch.cuda.synchronize()
        assert float(x[0]) == 1.0
        for s in (fresh, many, checked, timed):
            assert np.array_equal(s.stg.cpu().numpy(), s.staging) and np.array_equal(s.buf.cpu().numpy(), s.regions), \
                "a refused call wrote"
        # the same calls made eagerly afterwards match the oracle
        K.kv_pool_timing_read_each(timed.h)
        for s in (fresh, many, checked, timed):
            K.kv_gather_chunks(s.h, s.sp, s.spec, stream)
            torch.cuda.synchronize()
            s.check(K.KV_GATHER, "eager after the capture")
    finally:
        for s in (fresh, many, checked, timed):
            s.close()
