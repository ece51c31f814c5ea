"""A pool in memory mapped through HIP's virtual-memory API.

The regions lie in one reserved address range backed by many physical chunks
(hipMemCreate + hipMemMap, mapped in reverse order), the way allocators with
expandable segments build their memory.  The runtime reports each mapping as an
allocation of its own, so the library's extent check must follow the mappings
across a region instead of refusing it; gather and scatter must then match the
oracle byte for byte, and a pool declared past the end of the mapped range must
still be refused (with block ids that keep the call inside the mapping, so it
would be harmless if launched).
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import gpu_harness as G
import oracle
from paged_layout_transfer_amd import kvxfer as K

pytestmark = pytest.mark.gpu

L, KV, H, D, E, BS, N = 2, 2, 1, 64, 2, 16, 1024
TOK = H * D * E
TILE = BS * TOK
REGION = N * TILE                   # 2 MiB per region
CHUNK = 64 << 10                    # physical chunk: 32 mappings per region


class _Prop(ctypes.Structure):      # hipMemAllocationProp
    _fields_ = [("type", ctypes.c_int), ("handle_type", ctypes.c_int), ("loc_type", ctypes.c_int),
                ("loc_id", ctypes.c_int), ("win32", ctypes.c_void_p), ("compression", ctypes.c_ubyte),
                ("rdma", ctypes.c_ubyte), ("usage", ctypes.c_ushort)]


class _Access(ctypes.Structure):    # hipMemAccessDesc
    _fields_ = [("loc_type", ctypes.c_int), ("loc_id", ctypes.c_int), ("flags", ctypes.c_int)]


class MappedBuffer:
    """total bytes of device memory: CHUNK-sized physical allocations mapped in reverse order."""

    def __init__(self, total: int):
        self.hip = G.hip_runtime()
        # the reservation runs two chunks past the mapped bytes, so the address after
        # the last mapping is never another allocation's
        self.total, self.reserved = total, total + 2 * CHUNK
        self.handles, self.va, self.mapped = [], ctypes.c_void_p(), 0
        dev = ctypes.c_int()
        assert self.hip.hipGetDevice(ctypes.byref(dev)) == 0
        prop = _Prop(type=1, handle_type=0, loc_type=1, loc_id=dev.value)
        gran = ctypes.c_size_t()
        if self.hip.hipMemGetAllocationGranularity(ctypes.byref(gran), ctypes.byref(prop), 0) != 0 \
                or CHUNK % gran.value:
            self.hip.hipGetLastError()
            pytest.skip("virtual-memory mapping at %d-byte chunks is not available" % CHUNK)
        try:
            rc = self.hip.hipMemAddressReserve(ctypes.byref(self.va), ctypes.c_size_t(self.reserved),
                                               ctypes.c_size_t(CHUNK), None, ctypes.c_ulonglong(0))
            assert rc == 0, "hipMemAddressReserve: %d" % rc
            n = total // CHUNK
            for _ in range(n):
                h = ctypes.c_void_p()
                rc = self.hip.hipMemCreate(ctypes.byref(h), ctypes.c_size_t(CHUNK), ctypes.byref(prop),
                                           ctypes.c_ulonglong(0))
                assert rc == 0, "hipMemCreate: %d" % rc
                self.handles.append(h)
            for i in range(n):
                rc = self.hip.hipMemMap(ctypes.c_void_p(self.va.value + i * CHUNK), ctypes.c_size_t(CHUNK),
                                        ctypes.c_size_t(0), self.handles[n - 1 - i], ctypes.c_ulonglong(0))
                assert rc == 0, "hipMemMap: %d" % rc
                self.mapped = (i + 1) * CHUNK
            acc = _Access(loc_type=1, loc_id=dev.value, flags=3)
            rc = self.hip.hipMemSetAccess(self.va, ctypes.c_size_t(total), ctypes.byref(acc), ctypes.c_size_t(1))
            assert rc == 0, "hipMemSetAccess: %d" % rc
        except BaseException:
            self.free()
            raise

    def write(self, data: np.ndarray) -> None:
        assert data.nbytes == self.total
        assert self.hip.hipMemcpy(self.va, data.ctypes.data_as(ctypes.c_void_p), ctypes.c_size_t(self.total), 1) == 0

    def read(self) -> np.ndarray:
        out = np.empty(self.total, dtype=np.uint8)
        assert self.hip.hipMemcpy(out.ctypes.data_as(ctypes.c_void_p), self.va, ctypes.c_size_t(self.total), 2) == 0
        return out

    def free(self) -> None:
        self.hip.hipDeviceSynchronize()
        for off in range(0, self.mapped, CHUNK):
            self.hip.hipMemUnmap(ctypes.c_void_p(self.va.value + off), ctypes.c_size_t(CHUNK))
        for h in self.handles:
            self.hip.hipMemRelease(h)
        if self.va.value:
            self.hip.hipMemAddressFree(self.va, ctypes.c_size_t(self.reserved))
        self.handles, self.mapped, self.va = [], 0, ctypes.c_void_p()


def test_pool_in_mapped_memory_moves_like_the_oracle_and_is_bounded():
    dev = torch.device("cuda", 0)
    rng = np.random.default_rng(77_001)
    buf = MappedBuffer(L * KV * REGION)
    pools = []
    try:
        regions = rng.integers(0, 256, size=(L * KV, REGION), dtype=np.uint8)
        buf.write(regions.reshape(-1))
        bases = [buf.va.value + i * REGION for i in range(L * KV)]
        pool = dict(num_layers=L, num_kv=KV, num_heads=H, head_dim=D, elem_bytes=E, block_size=BS,
                    num_blocks=N, block_stride=TILE)
        T = 500                                          # 32 pages, the last one partial
        table = rng.permutation(N)[:32].astype(np.int32)
        chunks = dict(layout=K.KV_LAYER_FIRST, chunk_layers=L, chunk_tokens=256, layer_begin=0, layer_end=L,
                      slot_bytes=L * KV * 256 * TOK, n_slots=2)
        spans_h = [(table, 0, T, 0)]
        tab_d = torch.from_numpy(table).to(dev)
        spans = K.make_spans([(tab_d, table.size, 0, T, 0)])
        staging = rng.integers(0, 256, size=chunks["slot_bytes"] * 2, dtype=np.uint8)
        stg_d = torch.from_numpy(staging.copy()).to(dev)
        spec = K.make_chunk_spec(K.KV_LAYER_FIRST, L, 256, 0, L, stg_d, chunks["slot_bytes"], 2)
        p = K.kv_pool_create(K.make_pool_desc(L, KV, H, D, E, BS, N, TILE, bases))
        pools.append(p)
        stream = torch.cuda.current_stream()

        print("[vmm] gather from a pool over %d mappings" % (buf.total // CHUNK), flush=True)
        K.kv_gather_chunks(p, spans, spec, stream)
        assert K.kv_pool_get_error(p, stream) == 0
        exp_stg = staging.copy()
        oracle.transfer(K.KV_GATHER, pool, [r.copy() for r in regions], spans_h, chunks, exp_stg)
        assert np.array_equal(stg_d.cpu().numpy(), exp_stg)

        print("[vmm] scatter into it", flush=True)
        staging2 = rng.integers(0, 256, size=staging.size, dtype=np.uint8)
        stg_d.copy_(torch.from_numpy(staging2))
        K.kv_scatter_chunks(p, spans, spec, stream)
        assert K.kv_pool_get_error(p, stream) == 0
        torch.cuda.synchronize()
        exp_regions = [r.copy() for r in regions]
        oracle.transfer(K.KV_SCATTER, pool, exp_regions, spans_h, chunks, staging2.copy())
        assert np.array_equal(buf.read().reshape(L * KV, REGION), np.stack(exp_regions))

        print("[vmm] a pool declared past the mapped range is refused", flush=True)
        low_tab = torch.tensor([0, 1], dtype=torch.int32, device=dev)           # blocks 0 and 1 only
        low = K.make_spans([(low_tab, 2, 0, 2 * BS, 0)])
        # 2^30 blocks = 2 TiB per region: past the mapping, the reservation and any
        # run of allocations that could follow it
        bad = K.kv_pool_create(K.make_pool_desc(L, KV, H, D, E, BS, 1 << 30, TILE, bases))
        pools.append(bad)
        before = buf.read()
        for fn in (K.kv_gather_chunks, K.kv_scatter_chunks):
            with pytest.raises(K.KvError) as e:
                fn(bad, low, spec, stream)
            assert e.value.code == K.KV_ERR_RANGE
        torch.cuda.synchronize()
        assert np.array_equal(buf.read(), before)
    finally:
        torch.cuda.synchronize()
        for p in pools:
            K.kv_pool_destroy(p)
        buf.free()
