// kvxfer.cpp -- host side of the paged-KV transfer library: validation, call
// decomposition into tiles, the block allocator, the pinned staging ring and
// the launch.  The exported functions are declared and documented in
// include/kvxfer.h.
//
// Host work per call is O(n_spans): one descriptor record per span, one small
// stream-ordered upload and one kernel launch, however many pages and layers the
// call moves (the Tutti summary, Q2 "Design 1", cuts CPU work per transfer from
// O(layer x blocks) to O(layer); the Strata guide, "The Mechanics of
// GPU-Assisted I/O", replaces one DMA submission per page with one kernel).
#include "kvxfer.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "kvxfer_host.h"
#include "kvxfer_internal.h"

namespace {

constexpr int64_t kArenaBytes = 4 << 20; // span records of the calls in flight, per pool
constexpr int kInflight = 256;           // calls in flight per pool before the host waits
constexpr int kMaxTimed = 4096;         // launches one timing window can record
constexpr int64_t kMaxU31 = 0x7fffffffLL;

// The last HIP failure seen by this thread, reported by kv_last_hip_error.  The
// runtime's own last-error is consumed on every failure so a stale error never
// leaks into a later status check.
thread_local int g_hip_error = 0;
thread_local const char *g_hip_where = "";

inline bool hip_ok(hipError_t e, const char *where)
{
    if (e == hipSuccess) return true;
    g_hip_error = (int)e;
    g_hip_where = where;
    (void)hipGetLastError();
    return false;
}
#define HIP_OK(call) hip_ok((call), #call)

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct SlotRange {
    int64_t start;  // first slot
    int64_t count;  // chunks
};

// Per-span figures of a validated call.
struct SpanPlan {
    int64_t n_pages, ppc, n_tc, n_chunks, tiles;
};

int check_desc(const kv_pool_desc *d)
{
    if (!d || !d->bases) return KV_ERR_ARG;
    if (d->num_layers < 1 || d->num_kv < 1 || d->num_kv > 2 || d->num_heads < 1 ||
        d->head_dim < 1 || d->block_size < 1)
        return KV_ERR_ARG;
    if (d->elem_bytes != 1 && d->elem_bytes != 2 && d->elem_bytes != 4 && d->elem_bytes != 8)
        return KV_ERR_ARG;
    if (d->num_blocks < 1 || d->num_blocks > kMaxU31) return KV_ERR_ARG;
    if (d->page_layout != KV_PAGE_TOKEN_MAJOR && d->page_layout != KV_PAGE_HEAD_MAJOR)
        return KV_ERR_ARG;
    const int64_t row = (int64_t)d->head_dim * d->elem_bytes;
    const int64_t tok = (int64_t)d->num_heads * row;
    if (tok > kMaxU31 || tok * d->block_size > kMaxU31) return KV_ERR_ARG;
    if (tok % 16 != 0) return KV_ERR_ALIGN;
    // head-major rows: whole 16-byte vectors, or whole 4-byte words with a token
    // (all heads) that fits one wave's LDS slice
    if (d->page_layout == KV_PAGE_HEAD_MAJOR && row % 16 != 0) {
        if (row % 4 != 0) return KV_ERR_ALIGN;
        if (!kvx::hm_lds_ok(KV_PAGE_HEAD_MAJOR, row, tok)) return KV_ERR_ARG;
    }
    const int64_t tile = tok * d->block_size;
    if (d->block_stride < tile) return KV_ERR_ARG;
    if (d->block_stride % 16 != 0) return KV_ERR_ALIGN;
    if (d->block_stride > INT64_MAX / d->num_blocks) return KV_ERR_ARG;
    const int64_t n = (int64_t)d->num_layers * d->num_kv;
    if (n > kMaxU31) return KV_ERR_ARG;
    for (int64_t i = 0; i < n; ++i) {
        if (!d->bases[i]) return KV_ERR_ARG;
        if (!aligned16(d->bases[i])) return KV_ERR_ALIGN;
    }
    return KV_OK;
}

int64_t tok_bytes(const kv_pool_desc *d)
{
    return (int64_t)d->num_heads * d->head_dim * d->elem_bytes;
}

int check_spec(const kv_pool_desc *d, const kv_chunk_spec *s)
{
    if (!s) return KV_ERR_ARG;
    if (s->layout != KV_LAYER_FIRST && s->layout != KV_PAGE_FIRST) return KV_ERR_ARG;
    if (s->layer_begin < 0 || s->layer_end > d->num_layers || s->layer_end <= s->layer_begin)
        return KV_ERR_ARG;
    if (s->chunk_layers < 1 || (s->layer_end - s->layer_begin) % s->chunk_layers != 0)
        return KV_ERR_ARG;
    if (s->chunk_tokens < d->block_size || s->chunk_tokens % d->block_size != 0) return KV_ERR_ARG;
    if (!s->base) return KV_ERR_ARG;
    if (!aligned16(s->base)) return KV_ERR_ALIGN;
    if (s->slot_bytes <= 0 || s->n_slots <= 0) return KV_ERR_ARG;
    if (s->slot_bytes % 16 != 0) return KV_ERR_ALIGN;
    if (s->n_slots > INT64_MAX / s->slot_bytes) return KV_ERR_ARG;
    if (s->max_workgroups < 0) return KV_ERR_ARG;
    if (s->flags & ~(KV_FLAG_VALIDATE | KV_FLAG_DMA_STRIDED | KV_FLAG_CACHED | KV_FLAG_PAGE_RUNS)) return KV_ERR_ARG;
    return KV_OK;
}

int64_t chunk_bytes_for(const kv_pool_desc *d, const kv_chunk_spec *s, int64_t tokens)
{
    const int64_t tok = tok_bytes(d);
    if (s->layout == KV_LAYER_FIRST) return (int64_t)s->chunk_layers * d->num_kv * tokens * tok;
    return cdiv(tokens, d->block_size) * s->chunk_layers * d->num_kv * d->block_size * tok;
}

// Full validation of a call.  plans (n_spans entries) and ranges (n_spans entries)
// are caller-provided scratch so the transfer path allocates nothing.
int validate_call(const kv_pool_desc *d, const kv_span *spans, int32_t n_spans,
                  const kv_chunk_spec *s, kv_transfer_info *info, SpanPlan *plans,
                  SlotRange *ranges)
{
    int rc = check_desc(d);
    if (rc) return rc;
    rc = check_spec(d, s);
    if (rc) return rc;
    if (n_spans < 0 || n_spans > KV_MAX_SPANS) return KV_ERR_ARG;
    if (n_spans > 0 && !spans) return KV_ERR_ARG;

    const int64_t bs = d->block_size;
    const int64_t layers = s->layer_end - s->layer_begin;
    const int64_t n_lc = layers / s->chunk_layers;
    kv_transfer_info acc{0, 0, 0, 0};
    int n_ranges = 0;
    for (int32_t i = 0; i < n_spans; ++i) {
        const kv_span &sp = spans[i];
        if (sp.t_begin < 0 || sp.t_end < sp.t_begin || sp.t_begin % bs != 0) return KV_ERR_ARG;
        if (sp.first_chunk < 0) return KV_ERR_ARG;
        SpanPlan &p = plans[i];
        const int64_t len = sp.t_end - sp.t_begin;
        if (len == 0) {
            p = SpanPlan{0, 0, 0, 0, 0};
            continue;
        }
        if (!sp.block_table) return KV_ERR_ARG;
        if (sp.t_end / bs >= kMaxU31) return KV_ERR_RANGE;
        if (sp.table_len < cdiv(sp.t_end, bs) || sp.table_len > kMaxU31) return KV_ERR_RANGE;
        p.n_pages = cdiv(len, bs);
        p.ppc = std::min<int64_t>(s->chunk_tokens / bs, p.n_pages);
        p.n_tc = cdiv(p.n_pages, p.ppc);
        p.n_chunks = n_lc * p.n_tc;
        p.tiles = layers * d->num_kv * p.n_pages;
        if (p.tiles > kMaxU31) return KV_ERR_RANGE;
        if (sp.first_chunk > INT64_MAX - p.n_chunks) return KV_ERR_ARG;
        const int64_t first_chunk_tokens = std::min(len, p.ppc * bs);
        const int64_t cb = chunk_bytes_for(d, s, first_chunk_tokens);
        if (cb > s->slot_bytes) return KV_ERR_RANGE;
        acc.max_chunk_bytes = std::max(acc.max_chunk_bytes, cb);
        acc.tiles += p.tiles;
        acc.chunks += p.n_chunks;
        acc.payload_bytes += layers * d->num_kv * len * tok_bytes(d);
        ranges[n_ranges++] = SlotRange{sp.first_chunk % s->n_slots, p.n_chunks};
    }
    // Every chunk of the call owns its slot: the chunk ranges, taken mod n_slots,
    // must be disjoint arcs of the ring.
    if (acc.chunks > s->n_slots) return KV_ERR_RING;
    std::sort(ranges, ranges + n_ranges,
              [](const SlotRange &a, const SlotRange &b) { return a.start < b.start; });
    for (int i = 0; i + 1 < n_ranges; ++i)
        if (ranges[i].start + ranges[i].count > ranges[i + 1].start) return KV_ERR_RING;
    if (n_ranges > 1 &&
        ranges[n_ranges - 1].start + ranges[n_ranges - 1].count > ranges[0].start + s->n_slots)
        return KV_ERR_RING;
    if (info) *info = acc;
    return KV_OK;
}

}  // namespace

namespace {

// Validation plus launch-record construction, with caller-provided scratch.
int prepare_with(const kv_pool_desc *d, const kv_span *spans, int32_t n_spans,
                 const kv_chunk_spec *spec, kvx::SpanDev *records, uint32_t *n_records,
                 kvx::Launch *a, kv_transfer_info *info, SpanPlan *plans, SlotRange *ranges)
{
    kv_transfer_info inf;
    int rc = validate_call(d, spans, n_spans, spec, &inf, plans, ranges);
    if (rc) return rc;
    uint32_t n = 0;
    int64_t tile_begin = 0;
    for (int32_t i = 0; i < n_spans; ++i) {
        const SpanPlan &pl = plans[i];
        if (pl.tiles == 0) continue;
        kvx::SpanDev r{};
        r.table = spans[i].block_table;
        r.tile_begin = tile_begin;
        r.t_end = spans[i].t_end;
        r.slot0 = spans[i].first_chunk % spec->n_slots;
        r.first_page = (uint32_t)(spans[i].t_begin / d->block_size);
        r.n_pages = (uint32_t)pl.n_pages;
        r.ppc = (uint32_t)pl.ppc;
        r.n_tc = (uint32_t)pl.n_tc;
        r.per_lc = (uint32_t)((int64_t)spec->chunk_layers * d->num_kv * pl.n_pages);
        r.per_tc = (uint32_t)((int64_t)spec->chunk_layers * d->num_kv * pl.ppc);
        records[n++] = r;
        tile_begin += pl.tiles;
    }
    *n_records = n;
    *a = kvx::Launch{};
    a->chunk_base = static_cast<uint8_t *>(spec->base);
    a->total_tiles = inf.tiles;
    a->block_stride = d->block_stride;
    a->slot_bytes = spec->slot_bytes;
    a->n_slots = spec->n_slots;
    a->tile_bytes = tok_bytes(d) * d->block_size;
    a->num_blocks = (uint32_t)d->num_blocks;
    a->n_spans = n;
    a->num_kv = (uint32_t)d->num_kv;
    a->chunk_layers = (uint32_t)spec->chunk_layers;
    a->layer_begin = (uint32_t)spec->layer_begin;
    a->tok = (uint32_t)tok_bytes(d);
    a->block_size = (uint32_t)d->block_size;
    a->layout = (uint32_t)spec->layout;
    a->page_layout = (uint32_t)d->page_layout;
    a->cached = (spec->flags & KV_FLAG_CACHED) ? 1u : 0u;
    if (d->page_layout == KV_PAGE_HEAD_MAJOR) {
        const int64_t row = (int64_t)d->head_dim * d->elem_bytes;
        const uint32_t H = (uint32_t)d->num_heads;
        a->hm_heads = H;
        a->hm_row = (uint32_t)row;
        if (kvx::hm_lds_use(a->page_layout, row, tok_bytes(d), tok_bytes(d) * d->block_size, H,
                            (uint32_t)d->block_size)) {
            a->hm_lds = 1;
            a->hm_rd = (uint32_t)(row / 4);
            a->hm_tj = kvx::hm_lds_tokens(row, tok_bytes(d), (uint32_t)d->block_size);
            a->hm_m_rd = kvx::magic_u16(a->hm_rd);
            a->hm_m_run = kvx::magic_u16(a->hm_tj * a->hm_rd);
            if (kvx::hm_page_ok(a->page_layout, row, tok_bytes(d), tok_bytes(d) * d->block_size)) {
                a->hm_page = 1;
                a->hm_m_brd = kvx::magic_u16((uint32_t)d->block_size * a->hm_rd);
            }
            for (int dir = 0; dir < 2; ++dir) {
                kvx::hm_lds_head_slab(dir, H, row, tok_bytes(d), (uint32_t)d->block_size, &a->hm_hg[dir],
                                      &a->hm_htj[dir]);
                if (a->hm_hg[dir]) {
                    a->hm_m_hrun[dir] = kvx::magic_u16(a->hm_htj[dir] * a->hm_rd);
                    a->hm_m_hgrp[dir] = kvx::magic_u16(a->hm_hg[dir] * a->hm_rd);
                }
            }
        } else {
            const uint32_t r16 = (uint32_t)(row / 16);
            a->hm_r16 = r16;
            a->hm_bs_r16 = (uint32_t)d->block_size * r16;
            a->hm_dq = 64u % r16;
            a->hm_dh = (64u / r16) % H;
            a->hm_dj = (64u / r16) / H;
            a->hm_t4 = kvx::hm_t4_ok(a->page_layout, r16, H, (uint32_t)d->block_size) ? 1u : 0u;
        }
    }
    if (info) *info = inf;
    return KV_OK;
}

}  // namespace

namespace kvx {

int prepare_call(const kv_pool_desc *d, const kv_span *spans, int32_t n_spans,
                 const kv_chunk_spec *spec, SpanDev *records, uint32_t *n_records, Launch *launch,
                 kv_transfer_info *info)
{
    if (n_spans < 0 || n_spans > KV_MAX_SPANS || !records || !n_records || !launch)
        return KV_ERR_ARG;
    try {
        std::vector<SpanPlan> plans(std::max(1, (int)n_spans));
        std::vector<SlotRange> ranges(std::max(1, (int)n_spans));
        return prepare_with(d, spans, n_spans, spec, records, n_records, launch, info,
                            plans.data(), ranges.data());
    } catch (...) {
        return KV_ERR_OOM;
    }
}

}  // namespace kvx

struct kv_pool {
    kv_pool_desc desc;
    std::vector<void *> bases;
    // allocator: free-block bitmap, lowest ids first
    kvx::BlockBitmap blocks;
    // validation scratch (no allocation on the call path)
    std::vector<SpanPlan> plans;
    std::vector<SlotRange> ranges;
    // host image of the static device scratch (kv_transfer_chunks_noalloc), made at create
    std::vector<uint64_t> scr_image;
    // device state, created on the first transfer
    int device = -1;
    uint8_t **d_regions = nullptr;
    int32_t *d_err = nullptr;
    // Span-record arena: each call takes the next free stretch of a circular buffer
    // (pinned host mirror + device copy) and records an event after its kernel; a
    // stretch is reused once that event has passed.  Allocation is sequential, so
    // the oldest call in flight is always the next one in the way.
    uint8_t *d_arena = nullptr;
    uint8_t *h_arena = nullptr;
    kvx::ArenaRing<kInflight> arena;
    hipEvent_t fl_ev[kInflight] = {};  // one per arena slot
    // staging-memory kind of the last staging base seen
    kvx::StagingKind staging_kind;
    // the declared extents of the regions, staging bases and block tables against
    // the allocations holding them (see check_buffers); the regions are checked until
    // they have passed once
    kvx::ExtentCache extents;
    bool regions_ok = false;
    // timing
    bool timing = false;
    int n_timed = 0;
    std::vector<hipEvent_t> t_ev;
};

struct kv_ring {
    void *host = nullptr;
    void *dev = nullptr;
    int64_t slot_bytes = 0, n_slots = 0;
    // slot fencing: a small pool of events reused round-robin; each slot remembers
    // the event (and that event's generation) of the last work recorded on it.  An
    // event is synchronized before reuse, so a slot whose generation is stale is free.
    std::vector<hipEvent_t> ev;
    std::vector<uint64_t> ev_gen;
    std::vector<int32_t> slot_ev;
    std::vector<uint64_t> slot_gen;
    int next_ev = 0;
};

namespace {

void free_device_state(kv_pool *p)
{
    for (int i = 0; i < kInflight; ++i)
        if (p->fl_ev[i]) (void)hipEventDestroy(p->fl_ev[i]), p->fl_ev[i] = nullptr;
    if (p->h_arena) (void)hipHostFree(p->h_arena), p->h_arena = nullptr;
    if (p->d_arena) (void)hipFree(p->d_arena), p->d_arena = nullptr;
    p->arena.reset();
    if (p->d_err) (void)hipFree(p->d_err), p->d_err = nullptr;
    if (p->d_regions) (void)hipFree(p->d_regions), p->d_regions = nullptr;
    p->device = -1;
}

// Reserve `bytes` of the span-record arena for one call, waiting for the calls
// that still use them (or for the oldest call when kInflight are queued).
int arena_take(kv_pool *p, int64_t bytes, int64_t *off)
{
    return p->arena.take(bytes, off, [p](int i) {
        return HIP_OK(hipEventSynchronize(p->fl_ev[i])) ? 0 : KV_ERR_HIP;
    });
}

// Mark the stretch as used by the work just queued on `stream`.
int arena_commit(kv_pool *p, int64_t off, int64_t bytes, hipStream_t stream)
{
    if (!HIP_OK(hipEventRecord(p->fl_ev[p->arena.next_slot()], stream))) {
        // cannot fence the stretch: wait for the work instead so it is free again
        (void)hipStreamSynchronize(stream);
        return KV_ERR_HIP;
    }
    p->arena.commit(off, bytes);
    return KV_OK;
}

int device_setup(kv_pool *p)
{
    int dev = -1;
    if (!HIP_OK(hipGetDevice(&dev))) return KV_ERR_HIP;
    if (p->device >= 0) return dev == p->device ? KV_OK : KV_ERR_ARG;
    const int64_t n = (int64_t)p->desc.num_layers * p->desc.num_kv;

    if (!HIP_OK(hipMalloc(&p->d_regions, n * sizeof(void *)))) goto fail;
    if (!HIP_OK(hipMemcpy(p->d_regions, p->bases.data(), n * sizeof(void *), hipMemcpyHostToDevice)))
        goto fail;
    if (!HIP_OK(hipMalloc(&p->d_err, sizeof(int32_t)))) goto fail;
    if (!HIP_OK(hipMemset(p->d_err, 0, sizeof(int32_t)))) goto fail;
    if (!HIP_OK(hipMalloc(&p->d_arena, kArenaBytes))) goto fail;
    if (!HIP_OK(hipHostMalloc((void **)&p->h_arena, kArenaBytes, hipHostMallocDefault))) goto fail;
    p->arena.reset();
    p->arena.size = kArenaBytes;
    for (int i = 0; i < kInflight; ++i)
        if (!HIP_OK(hipEventCreateWithFlags(&p->fl_ev[i], hipEventDisableTiming))) goto fail;
    p->device = dev;
    return KV_OK;
fail:
    free_device_state(p);
    return KV_ERR_HIP;
}

void device_teardown(kv_pool *p)
{
    // Every launch that reads the pool's device state (region table, error word,
    // span records) is fenced by its arena event, so waiting for the calls still in
    // flight is enough; other work on the device is left alone.
    if (p->device >= 0)
        for (int k = 0; k < p->arena.count; ++k)
            (void)hipEventSynchronize(p->fl_ev[(p->arena.first + k) % kInflight]);
    free_device_state(p);
    for (hipEvent_t &e : p->t_ev)
        if (e) (void)hipEventDestroy(e), e = nullptr;
}

int validate_tables(kv_pool *p, const kv_span *spans, int32_t n_spans, int direction,
                    hipStream_t stream)
{
    // Host copies of the device tables (debug path; synchronous by design).
    if (!HIP_OK(hipStreamSynchronize(stream))) return KV_ERR_HIP;
    std::vector<std::vector<int32_t>> host(n_spans);
    std::vector<const int32_t *> ptrs(n_spans, nullptr);
    for (int32_t i = 0; i < n_spans; ++i) {
        if (spans[i].t_end == spans[i].t_begin) continue;
        const int64_t n = cdiv(spans[i].t_end, p->desc.block_size);
        host[i].resize(n);
        if (!HIP_OK(hipMemcpy(host[i].data(), spans[i].block_table, n * sizeof(int32_t),
                              hipMemcpyDeviceToHost)))
            return KV_ERR_HIP;
        ptrs[i] = host[i].data();
    }
    std::vector<kv_span> local(spans, spans + n_spans);
    for (int32_t i = 0; i < n_spans; ++i)
        local[i].table_len = (int64_t)host[i].size();
    return kv_validate_targets(&p->desc, local.data(), n_spans, ptrs.data(), direction);
}

// Whether the staging memory is host memory (pinned, mapped): those transfers are
// bound by the host link, which a few workgroups saturate, so by default they get a
// small grid and leave the rest of the chip to compute (Strata guide,
// "Non-Intrusive Resource Sizing").  The answer is kept per staging address and the
// allocation holding it (`alloc`, from the extent check).
bool staging_in_host_memory(kv_pool *p, const void *base, const kvx::AllocRange &alloc)
{
    return p->staging_kind.is_host(base, alloc, [](const void *b) {
        hipPointerAttribute_t attr;
        if (hipPointerGetAttributes(&attr, b) == hipSuccess) return attr.type == hipMemoryTypeHost;
        (void)hipGetLastError();  // unknown to the runtime: treat as device memory
        return false;
    });
}

// The kernels and copies trust the extents a call declares: num_blocks blocks per
// region, n_slots * slot_bytes of staging, table_len entries per block table.  An
// access past the end of an allocation faults the GPU, so where the HIP runtime
// knows the allocation holding a pointer (device memory, hipHostMalloc'd
// or registered host memory) a declared extent that runs past its end is refused
// before anything is enqueued.  Memory the runtime does not know (pageable host
// memory, other allocators) is taken on trust.

// The allocation holding q, or an empty range when the runtime does not know q.
// Memory mapped through the virtual-memory API (hipMemMap) reports each mapping as an
// allocation of its own, which kvx::covered_end walks across.
kvx::AllocRange alloc_range(uintptr_t q)
{
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, reinterpret_cast<hipDeviceptr_t>(q)) != hipSuccess) {
        (void)hipGetLastError();
        return kvx::AllocRange{};
    }
    const uintptr_t b = reinterpret_cast<uintptr_t>(base);
    return kvx::AllocRange{b, b + size};
}

int check_extent(kvx::ExtentCache &c, const void *q, int64_t bytes, kvx::AllocRange *here = nullptr)
{
    return c.covers(q, bytes, alloc_range, here) ? KV_OK : KV_ERR_RANGE;
}

// Extents of a validated call: every region (until they have passed once), the
// staging area, and, when the tables are device memory, each span's block table.
// *staging, if given, receives the allocation holding the staging base.
int check_buffers(kv_pool *p, const kv_span *spans, int32_t n_spans, const kv_chunk_spec *spec,
                  bool device_tables, kvx::AllocRange *staging = nullptr)
{
    const kv_pool_desc &d = p->desc;
    if (!p->regions_ok) {
        const int64_t extent = (int64_t)(d.num_blocks - 1) * d.block_stride + tok_bytes(&d) * d.block_size;
        for (void *b : p->bases)
            if (check_extent(p->extents, b, extent)) return KV_ERR_RANGE;
        p->regions_ok = true;
    }
    if (check_extent(p->extents, spec->base, spec->n_slots * spec->slot_bytes, staging)) return KV_ERR_RANGE;
    if (device_tables) {
        // spans often share one table: a table no longer than the last one checked at
        // the same address needs no second lookup within the call
        const int32_t *last = nullptr;
        int64_t last_len = 0;
        for (int32_t i = 0; i < n_spans; ++i) {
            if (spans[i].t_end == spans[i].t_begin) continue;
            if (spans[i].block_table == last && spans[i].table_len <= last_len) continue;
            if (check_extent(p->extents, spans[i].block_table, spans[i].table_len * (int64_t)sizeof(int32_t)))
                return KV_ERR_RANGE;
            last = spans[i].block_table;
            last_len = spans[i].table_len;
        }
    }
    return KV_OK;
}

// The launch of a prepared call (regions, spans and err set): the split and segment
// choices, the grid (capped by max_workgroups, or small for host staging), the
// workgroup order, and the timing events around the kernel when timing is on.
int launch_prepared(kv_pool *p, kvx::Launch &a, int direction, const kv_chunk_spec *spec,
                    const kvx::AllocRange &staging, hipStream_t stream)
{
    const bool host_staging = staging_in_host_memory(p, spec->base, staging);
    a.split_shift = kvx::launch_split_shift(a, direction);
    a.part_bytes = kvx::part_bytes_for(direction, a, host_staging, (spec->flags & KV_FLAG_PAGE_RUNS) != 0);
    if (a.part_bytes) a.split_shift = 0;
    a.seg_bytes = a.part_bytes ? 0u : kvx::gather_seg_bytes(direction, a.page_layout, a.tile_bytes);
    uint32_t grid = kvx::default_grid(kvx::work_items(a));
    if (spec->max_workgroups > 0) grid = std::min<uint32_t>(grid, (uint32_t)spec->max_workgroups);
    else if (host_staging) grid = std::min<uint32_t>(grid, KVX_HOST_GRID_CAP);
    a.xcd_remap = kvx::xcd_remap_for(direction, a, host_staging);
    a.scatter_buf = kvx::scatter_buffer_form(direction, a, host_staging);
    const bool timed = p->timing && p->n_timed < kMaxTimed;
    if (timed && !HIP_OK(hipEventRecord(p->t_ev[2 * p->n_timed], stream))) return KV_ERR_HIP;
    if (!hip_ok((hipError_t)kvx::launch_tile_copy(direction, a, grid, stream), "hipLaunchKernel(tile_copy)"))
        return KV_ERR_HIP;
    if (timed) {
        if (!HIP_OK(hipEventRecord(p->t_ev[2 * p->n_timed + 1], stream))) return KV_ERR_HIP;
        ++p->n_timed;
    }
    return KV_OK;
}

// The span records a validated call makes: one per non-empty span.
int32_t records_of(const kv_span *spans, int32_t n_spans)
{
    int32_t n = 0;
    for (int32_t i = 0; i < n_spans; ++i) n += spans[i].t_end > spans[i].t_begin;
    return n;
}

// KV_ERR_CAPTURE if `stream` is capturing a graph (or its capture was invalidated),
// KV_OK if not, KV_ERR_HIP if the runtime cannot tell.
int refuse_capture(hipStream_t stream)
{
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (!hip_ok(hipStreamIsCapturing(stream, &st), "hipStreamIsCapturing")) return KV_ERR_HIP;
    return st == hipStreamCaptureStatusNone ? KV_OK : KV_ERR_CAPTURE;
}

int transfer(kv_pool *p, const kv_span *spans, int32_t n_spans, const kv_chunk_spec *spec,
             hipStream_t stream, int direction)
{
    if (!p) return KV_ERR_ARG;
    // Validate first: a rejected call makes no HIP call at all.
    kv_transfer_info info;
    int rc = validate_call(&p->desc, spans, n_spans, spec, &info, p->plans.data(), p->ranges.data());
    if (rc) return rc;
    if (info.tiles == 0) return KV_OK;
    // Under graph capture only a call the graph can replay as it stands is taken: its
    // span records ride in the kernel arguments, the pool's device state exists already
    // (the first call allocates it), and there is no host-side table check and no timing
    // event.  Such a call takes no arena stretch (the arena is recycled under events the
    // host waits on).
    hipStreamCaptureStatus cst = hipStreamCaptureStatusNone;
    if (!hip_ok(hipStreamIsCapturing(stream, &cst), "hipStreamIsCapturing")) return KV_ERR_HIP;
    const bool capturing = cst != hipStreamCaptureStatusNone;
    if (capturing && (cst != hipStreamCaptureStatusActive || records_of(spans, n_spans) > KVX_INLINE_SPANS ||
                      p->device < 0 || (spec->flags & KV_FLAG_VALIDATE) || p->timing))
        return KV_ERR_CAPTURE;
    kvx::AllocRange staging;
    rc = check_buffers(p, spans, n_spans, spec, true, &staging);
    if (rc) return rc;
    rc = device_setup(p);
    if (rc) return rc;
    if (capturing) {
        kvx::SpanDev recs[KVX_INLINE_SPANS];
        kvx::Launch a;
        uint32_t n_rec = 0;
        rc = prepare_with(&p->desc, spans, n_spans, spec, recs, &n_rec, &a, &info, p->plans.data(),
                          p->ranges.data());
        if (rc) return rc;
        std::memcpy(a.inl, recs, n_rec * sizeof(kvx::SpanDev));
        a.regions = p->d_regions;
        a.spans = nullptr;
        a.err = p->d_err;
        return launch_prepared(p, a, direction, spec, staging, stream);
    }
    if (spec->flags & KV_FLAG_VALIDATE) {
        rc = validate_tables(p, spans, n_spans, direction, stream);
        if (rc) return rc;
    }

    // Span records go to a free stretch of the pinned arena, then one stream-ordered
    // copy to the same stretch of the device arena; calls with at most
    // KVX_INLINE_SPANS records pass them in the kernel arguments instead and skip the
    // copy (their stretch still carries the call's fence event).
    const int64_t rec_bytes = ((int64_t)std::max(1, (int)n_spans) * (int64_t)sizeof(kvx::SpanDev) + 255) & ~255LL;
    int64_t off = 0;
    rc = arena_take(p, rec_bytes, &off);
    if (rc) return rc;
    kvx::SpanDev *h = reinterpret_cast<kvx::SpanDev *>(p->h_arena + off);
    kvx::SpanDev *dd = reinterpret_cast<kvx::SpanDev *>(p->d_arena + off);
    kvx::Launch a;
    uint32_t n_rec = 0;
    rc = prepare_with(&p->desc, spans, n_spans, spec, h, &n_rec, &a, &info, p->plans.data(),
                      p->ranges.data());
    if (rc) return rc;
    // a few records ride in the kernel arguments; more go to the device arena
    const bool inline_records = n_rec <= KVX_INLINE_SPANS;
    if (inline_records)
        std::memcpy(a.inl, h, n_rec * sizeof(kvx::SpanDev));
    else if (!HIP_OK(hipMemcpyAsync(dd, h, n_rec * sizeof(kvx::SpanDev), hipMemcpyHostToDevice, stream)))
        return KV_ERR_HIP;
    // From here the copy may be in flight: a failure waits for the stream before
    // returning, so the uncommitted arena stretch is free again.
    auto fail = [stream]() {
        (void)hipStreamSynchronize(stream);
        return KV_ERR_HIP;
    };
    a.regions = p->d_regions;
    a.spans = inline_records ? nullptr : dd;
    a.err = p->d_err;
    if (launch_prepared(p, a, direction, spec, staging, stream)) return fail();
    return arena_commit(p, off, rec_bytes, stream);
}

// The transfer without any allocation: the region table and the span records go to
// the device's static scratch (one stream-ordered copy from the pool's host image of
// it, made at create), the error bits to the caller's word.  Nothing is fenced: calls
// on one stream are ordered, calls that overlap on one device share the scratch.
int transfer_noalloc(kv_pool *p, int direction, const kv_span *spans, int32_t n_spans,
                     const kv_chunk_spec *spec, int32_t *err_word, hipStream_t stream)
{
    if (!p || (direction != KV_GATHER && direction != KV_SCATTER)) return KV_ERR_ARG;
    kv_transfer_info info;
    int rc = validate_call(&p->desc, spans, n_spans, spec, &info, p->plans.data(), p->ranges.data());
    if (rc) return rc;
    if (spec->flags & KV_FLAG_VALIDATE) return KV_ERR_ARG;  // its table check copies to the host
    const int64_t n_regions = (int64_t)p->desc.num_layers * p->desc.num_kv;
    if (n_regions > KVX_SCR_MAX_REGIONS) return KV_ERR_SCRATCH;
    if (err_word && (reinterpret_cast<uintptr_t>(err_word) & 3u)) return KV_ERR_ALIGN;
    if (info.tiles == 0) return KV_OK;
    // Records beyond those the kernel arguments carry are copied from the pool's host
    // image, which a captured copy would read only when the graph runs.
    if (records_of(spans, n_spans) > KVX_INLINE_SPANS) {
        rc = refuse_capture(stream);
        if (rc) return rc;
    }
    kvx::AllocRange staging;
    rc = check_buffers(p, spans, n_spans, spec, true, &staging);
    if (rc) return rc;
    if (err_word && check_extent(p->extents, err_word, sizeof(int32_t))) return KV_ERR_RANGE;
    int dev = -1;
    if (!HIP_OK(hipGetDevice(&dev))) return KV_ERR_HIP;
    int herr = 0;
    uint8_t *scr = static_cast<uint8_t *>(kvx::scratch_address(dev, &herr));
    if (!scr) {
        g_hip_error = herr;
        g_hip_where = "hipGetSymbolAddress(scratch)";
        return KV_ERR_HIP;
    }

    uint8_t *img = reinterpret_cast<uint8_t *>(p->scr_image.data());
    std::memcpy(img + KVX_SCR_REGIONS_OFF, p->bases.data(), (size_t)n_regions * sizeof(void *));
    kvx::SpanDev *h = reinterpret_cast<kvx::SpanDev *>(img + KVX_SCR_RECORDS_OFF);
    kvx::Launch a;
    uint32_t n_rec = 0;
    rc = prepare_with(&p->desc, spans, n_spans, spec, h, &n_rec, &a, &info, p->plans.data(), p->ranges.data());
    if (rc) return rc;
    const bool inline_records = n_rec <= KVX_INLINE_SPANS;
    if (inline_records) std::memcpy(a.inl, h, n_rec * sizeof(kvx::SpanDev));
    const int64_t end = inline_records ? KVX_SCR_REGIONS_OFF + n_regions * (int64_t)sizeof(void *)
                                       : KVX_SCR_RECORDS_OFF + n_rec * (int64_t)sizeof(kvx::SpanDev);
    // The image is pageable host memory: the runtime has taken its bytes when the copy
    // call returns, so the next call may rewrite it.
    if (!HIP_OK(hipMemcpyAsync(scr + KVX_SCR_REGIONS_OFF, img + KVX_SCR_REGIONS_OFF,
                               (size_t)(end - KVX_SCR_REGIONS_OFF), hipMemcpyHostToDevice, stream)))
        return KV_ERR_HIP;
    a.regions = reinterpret_cast<uint8_t *const *>(scr + KVX_SCR_REGIONS_OFF);
    a.spans = inline_records ? nullptr : reinterpret_cast<const kvx::SpanDev *>(scr + KVX_SCR_RECORDS_OFF);
    a.err = err_word ? err_word : reinterpret_cast<int32_t *>(scr);
    return launch_prepared(p, a, direction, spec, staging, stream);
}

// One hipMemcpyAsync per tile, addresses from the same tile resolution the kernel
// uses, block ids from host tables.
int transfer_dma(kv_pool *p, const kv_span *spans, int32_t n_spans, const kv_chunk_spec *spec,
                 hipStream_t stream, int direction)
{
    if (!p) return KV_ERR_ARG;
    kv_transfer_info info;
    int rc = validate_call(&p->desc, spans, n_spans, spec, &info, p->plans.data(), p->ranges.data());
    if (rc) return rc;
    if (info.tiles == 0) return KV_OK;
    rc = check_buffers(p, spans, n_spans, spec, false);
    if (rc) return rc;
    std::vector<const int32_t *> tables(n_spans);
    for (int32_t i = 0; i < n_spans; ++i) tables[i] = spans[i].block_table;
    rc = kv_validate_targets(&p->desc, spans, n_spans, tables.data(), direction);
    if (rc) return rc;
    kvx::Launch a;
    uint32_t n_rec = 0;
    std::vector<kvx::SpanDev> rec(KV_MAX_SPANS);
    rc = prepare_with(&p->desc, spans, n_spans, spec, rec.data(), &n_rec, &a, &info, p->plans.data(),
                      p->ranges.data());
    if (rc) return rc;
    const bool timed = p->timing && p->n_timed < kMaxTimed;
    if (timed && !HIP_OK(hipEventRecord(p->t_ev[2 * p->n_timed], stream))) return KV_ERR_HIP;
    // host block table of each record (records skip empty spans)
    std::vector<const int32_t *> rec_tables;
    rec_tables.reserve(n_rec);
    for (int32_t i = 0; i < n_spans; ++i)
        if (spans[i].t_end > spans[i].t_begin) rec_tables.push_back(spans[i].block_table);
    const int64_t n_regions = (int64_t)p->desc.num_layers * p->desc.num_kv;
    const bool strided = (spec->flags & KV_FLAG_DMA_STRIDED) != 0;
    const int64_t pitch = strided ? kvx::uniform_region_pitch(p->bases.data(), n_regions) : 0;
    const bool gather = direction == KV_GATHER;
    rc = kvx::dma_walk(a, rec.data(), n_rec, rec_tables.data(), p->bases.data(), pitch, strided,
                       [&](const kvx::DmaCopy &c) -> int {
                           void *dst = gather ? (void *)c.chunk : (void *)c.pool;
                           const void *src = gather ? (const void *)c.pool : (const void *)c.chunk;
                           if (c.rows == 1)
                               return HIP_OK(hipMemcpyAsync(dst, src, (size_t)c.width, hipMemcpyDefault,
                                                            stream))
                                          ? 0
                                          : KV_ERR_HIP;
                           const size_t dp = (size_t)(gather ? c.chunk_pitch : c.pool_pitch);
                           const size_t sp = (size_t)(gather ? c.pool_pitch : c.chunk_pitch);
                           return hip_ok(hipMemcpy2DAsync(dst, dp, src, sp, (size_t)c.width,
                                                          (size_t)c.rows, hipMemcpyDefault, stream),
                                         "hipMemcpy2DAsync")
                                      ? 0
                                      : KV_ERR_HIP;
                       });
    if (rc) return rc;
    if (timed) {
        if (!HIP_OK(hipEventRecord(p->t_ev[2 * p->n_timed + 1], stream))) return KV_ERR_HIP;
        ++p->n_timed;
    }
    return KV_OK;
}

}  // namespace

static constexpr int kRingEvents = 64;

static bool ring_range_ok(const kv_ring *r, int64_t first, int64_t count)
{
    return r && first >= 0 && first < r->n_slots && count >= 1 && count <= r->n_slots;
}

template <typename F>
static int ring_for_events(kv_ring *r, int64_t first, int64_t count, F fn)
{
    if (!ring_range_ok(r, first, count)) return KV_ERR_ARG;
    if (r->ev.empty()) return KV_OK;  // nothing recorded yet
    int last = -1;
    for (int64_t i = 0; i < count; ++i) {
        const int64_t sl = (first + i) % r->n_slots;
        const int e = r->slot_ev[sl];
        if (e < 0 || e == last || r->slot_gen[sl] != r->ev_gen[e]) continue;
        int rc = fn(r->ev[e]);
        if (rc) return rc;
        last = e;
    }
    return KV_OK;
}

extern "C" {

int kv_pool_create(const kv_pool_desc *desc, kv_pool **out)
{
    if (!out) return KV_ERR_ARG;
    *out = nullptr;
    int rc = check_desc(desc);
    if (rc) return rc;
    kv_pool *p = new (std::nothrow) kv_pool();
    if (!p) return KV_ERR_OOM;
    try {
        const int64_t n = (int64_t)desc->num_layers * desc->num_kv;
        p->desc = *desc;
        p->bases.assign(desc->bases, desc->bases + n);
        p->desc.bases = p->bases.data();
        p->blocks.init(desc->num_blocks);
        p->plans.resize(KV_MAX_SPANS);
        p->ranges.resize(KV_MAX_SPANS);
        p->scr_image.assign(KVX_SCR_BYTES / sizeof(uint64_t), 0);
    } catch (...) {
        delete p;
        return KV_ERR_OOM;
    }
    *out = p;
    return KV_OK;
}

int kv_pool_destroy(kv_pool *pool)
{
    if (!pool) return KV_OK;
    device_teardown(pool);
    delete pool;
    return KV_OK;
}

int kv_pool_alloc_blocks(kv_pool *p, int32_t n, int32_t *out_ids)
{
    if (!p || n < 0 || (n > 0 && !out_ids)) return KV_ERR_ARG;
    return p->blocks.alloc(n, out_ids);
}

int kv_pool_free_blocks(kv_pool *p, int32_t n, const int32_t *ids)
{
    if (!p || n < 0 || (n > 0 && !ids)) return KV_ERR_ARG;
    return p->blocks.release(n, ids);
}

int kv_pool_free_count(const kv_pool *p, int64_t *out)
{
    if (!p || !out) return KV_ERR_ARG;
    *out = p->blocks.n_free;
    return KV_OK;
}

int kv_check_transfer(const kv_pool_desc *desc, const kv_span *spans, int32_t n_spans,
                      const kv_chunk_spec *spec, kv_transfer_info *info)
{
    if (n_spans < 0 || n_spans > KV_MAX_SPANS) return KV_ERR_ARG;
    try {
        std::vector<SpanPlan> plans(std::max(1, (int)n_spans));
        std::vector<SlotRange> ranges(std::max(1, (int)n_spans));
        return validate_call(desc, spans, n_spans, spec, info, plans.data(), ranges.data());
    } catch (...) {
        return KV_ERR_OOM;
    }
}

int kv_chunk_bytes(const kv_pool_desc *desc, const kv_chunk_spec *spec, int64_t tokens,
                   int64_t *out)
{
    if (!out) return KV_ERR_ARG;
    int rc = check_desc(desc);
    if (rc) return rc;
    if (!spec || (spec->layout != KV_LAYER_FIRST && spec->layout != KV_PAGE_FIRST) ||
        spec->chunk_layers < 1 || spec->chunk_tokens < 1)
        return KV_ERR_ARG;
    if (tokens < 1 || tokens > spec->chunk_tokens) return KV_ERR_ARG;
    *out = chunk_bytes_for(desc, spec, tokens);
    return KV_OK;
}

int kv_validate_targets(const kv_pool_desc *desc, const kv_span *spans, int32_t n_spans,
                        const int32_t *const *host_tables, int32_t direction)
{
    int rc = check_desc(desc);
    if (rc) return rc;
    if (direction != KV_GATHER && direction != KV_SCATTER) return KV_ERR_ARG;
    if (n_spans < 0 || n_spans > KV_MAX_SPANS || (n_spans > 0 && (!spans || !host_tables)))
        return KV_ERR_ARG;
    const int64_t bs = desc->block_size;
    // For scatter, a pool page may be written by one span only, and within a span
    // two logical pages must not share a block.
    std::vector<uint8_t> used;
    try {
        if (direction == KV_SCATTER) used.assign(desc->num_blocks, 0);
    } catch (...) {
        return KV_ERR_OOM;
    }
    for (int32_t i = 0; i < n_spans; ++i) {
        const kv_span &sp = spans[i];
        if (sp.t_end <= sp.t_begin) continue;
        if (!host_tables[i]) return KV_ERR_ARG;
        const int64_t p0 = sp.t_begin / bs, p1 = cdiv(sp.t_end, bs);
        if (sp.table_len < p1) return KV_ERR_RANGE;
        for (int64_t pg = p0; pg < p1; ++pg) {
            const int32_t b = host_tables[i][pg];
            if (b < 0 || b >= desc->num_blocks) return KV_ERR_RANGE;
            if (direction == KV_SCATTER) {
                if (used[b]) return KV_ERR_DUP;
                used[b] = 1;
            }
        }
    }
    return KV_OK;
}

int kv_gather_chunks(kv_pool *pool, const kv_span *spans, int32_t n_spans,
                     const kv_chunk_spec *spec, hipStream_t stream)
{
    return transfer(pool, spans, n_spans, spec, stream, KV_GATHER);
}

int kv_scatter_chunks(kv_pool *pool, const kv_span *spans, int32_t n_spans,
                      const kv_chunk_spec *spec, hipStream_t stream)
{
    return transfer(pool, spans, n_spans, spec, stream, KV_SCATTER);
}

int kv_transfer_chunks_noalloc(kv_pool *pool, int32_t direction, const kv_span *spans, int32_t n_spans,
                               const kv_chunk_spec *spec, int32_t *err_word, hipStream_t stream)
{
    return transfer_noalloc(pool, direction, spans, n_spans, spec, err_word, stream);
}

int kv_gather_chunks_dma(kv_pool *pool, const kv_span *spans, int32_t n_spans,
                         const kv_chunk_spec *spec, hipStream_t stream)
{
    return transfer_dma(pool, spans, n_spans, spec, stream, KV_GATHER);
}

int kv_scatter_chunks_dma(kv_pool *pool, const kv_span *spans, int32_t n_spans,
                          const kv_chunk_spec *spec, hipStream_t stream)
{
    return transfer_dma(pool, spans, n_spans, spec, stream, KV_SCATTER);
}

int kv_pool_get_error(kv_pool *p, hipStream_t stream, int32_t *out_bits)
{
    if (!p || !out_bits) return KV_ERR_ARG;
    *out_bits = 0;
    if (p->device < 0) return KV_OK;
    if (!HIP_OK(hipStreamSynchronize(stream))) return KV_ERR_HIP;
    int32_t v = 0;
    if (!HIP_OK(hipMemcpy(&v, p->d_err, sizeof(v), hipMemcpyDeviceToHost))) return KV_ERR_HIP;
    if (v && !HIP_OK(hipMemset(p->d_err, 0, sizeof(int32_t)))) return KV_ERR_HIP;
    *out_bits = v;
    return v ? KV_ERR_DEVICE : KV_OK;
}

int kv_pool_timing_start(kv_pool *p)
{
    if (!p) return KV_ERR_ARG;
    if (p->t_ev.empty()) {
        try {
            p->t_ev.assign(2 * kMaxTimed, nullptr);
        } catch (...) {
            return KV_ERR_OOM;
        }
        for (auto &e : p->t_ev)
            if (!HIP_OK(hipEventCreate(&e))) return KV_ERR_HIP;
    }
    p->n_timed = 0;
    p->timing = true;
    return KV_OK;
}

int kv_pool_timing_read_each(kv_pool *p, double *ms_each, int64_t cap, int64_t *launches)
{
    if (!p || !launches || cap < 0 || (cap > 0 && !ms_each)) return KV_ERR_ARG;
    for (int i = 0; i < p->n_timed; ++i) {
        if (!HIP_OK(hipEventSynchronize(p->t_ev[2 * i + 1]))) return KV_ERR_HIP;
        float ms = 0.f;
        if (!HIP_OK(hipEventElapsedTime(&ms, p->t_ev[2 * i], p->t_ev[2 * i + 1]))) return KV_ERR_HIP;
        if (i < cap) ms_each[i] = ms;
    }
    *launches = p->n_timed;
    p->timing = false;
    p->n_timed = 0;
    return KV_OK;
}

int kv_pool_timing_read(kv_pool *p, double *total_ms, int64_t *launches)
{
    if (!p || !total_ms || !launches) return KV_ERR_ARG;
    std::vector<double> each;
    try {
        each.resize(std::max(1, p->n_timed));
    } catch (...) {
        return KV_ERR_OOM;
    }
    const int rc = kv_pool_timing_read_each(p, each.data(), (int64_t)each.size(), launches);
    if (rc) return rc;
    double sum = 0.0;
    for (int64_t i = 0; i < *launches; ++i) sum += each[i];
    *total_ms = sum;
    return KV_OK;
}

int kv_ring_create(int64_t slot_bytes, int64_t n_slots, int32_t flags, kv_ring **out)
{
    if (!out) return KV_ERR_ARG;
    *out = nullptr;
    if (slot_bytes <= 0 || n_slots <= 0 || n_slots > INT64_MAX / slot_bytes) return KV_ERR_ARG;
    if (slot_bytes % 16 != 0) return KV_ERR_ALIGN;
    if (flags & ~KV_RING_NONCOHERENT) return KV_ERR_ARG;
    kv_ring *r = new (std::nothrow) kv_ring();
    if (!r) return KV_ERR_OOM;
    const size_t bytes = (size_t)(slot_bytes * n_slots);
    const unsigned hflags = hipHostMallocMapped | hipHostMallocPortable |
                            ((flags & KV_RING_NONCOHERENT) ? hipHostMallocNonCoherent
                                                           : hipHostMallocCoherent);
    if (!HIP_OK(hipHostMalloc(&r->host, bytes, hflags))) {
        delete r;
        return KV_ERR_OOM;
    }
    if (!HIP_OK(hipHostGetDevicePointer(&r->dev, r->host, 0))) {
        (void)hipHostFree(r->host);
        delete r;
        return KV_ERR_HIP;
    }
    std::memset(r->host, 0, bytes);
    r->slot_bytes = slot_bytes;
    r->n_slots = n_slots;
    *out = r;
    return KV_OK;
}

int kv_ring_slot(const kv_ring *r, int64_t i, void **host_ptr, void **dev_ptr)
{
    if (!r || i < 0 || i >= r->n_slots) return KV_ERR_ARG;
    if (host_ptr) *host_ptr = static_cast<uint8_t *>(r->host) + i * r->slot_bytes;
    if (dev_ptr) *dev_ptr = static_cast<uint8_t *>(r->dev) + i * r->slot_bytes;
    return KV_OK;
}

int kv_ring_destroy(kv_ring *r)
{
    if (!r) return KV_OK;
    for (hipEvent_t e : r->ev)
        if (e) (void)hipEventDestroy(e);
    if (r->host) (void)hipHostFree(r->host);
    delete r;
    return KV_OK;
}

int kv_ring_record(kv_ring *r, int64_t first, int64_t count, hipStream_t stream)
{
    if (!ring_range_ok(r, first, count)) return KV_ERR_ARG;
    if (r->ev.empty()) {
        try {
            r->ev.assign(kRingEvents, nullptr);
            r->ev_gen.assign(kRingEvents, 0);
            r->slot_ev.assign(r->n_slots, -1);
            r->slot_gen.assign(r->n_slots, 0);
        } catch (...) {
            return KV_ERR_OOM;
        }
        for (hipEvent_t &e : r->ev)
            if (!HIP_OK(hipEventCreateWithFlags(&e, hipEventDisableTiming))) return KV_ERR_HIP;
    }
    const int e = r->next_ev;
    if (!HIP_OK(hipEventSynchronize(r->ev[e]))) return KV_ERR_HIP;  // its earlier work is done
    if (!HIP_OK(hipEventRecord(r->ev[e], stream))) return KV_ERR_HIP;
    r->next_ev = (e + 1) % kRingEvents;
    const uint64_t g = ++r->ev_gen[e];
    for (int64_t i = 0; i < count; ++i) {
        const int64_t sl = (first + i) % r->n_slots;
        r->slot_ev[sl] = e;
        r->slot_gen[sl] = g;
    }
    return KV_OK;
}

int kv_ring_wait(kv_ring *r, int64_t first, int64_t count)
{
    return ring_for_events(r, first, count, [](hipEvent_t e) {
        return HIP_OK(hipEventSynchronize(e)) ? KV_OK : KV_ERR_HIP;
    });
}

int kv_ring_stream_wait(kv_ring *r, int64_t first, int64_t count, hipStream_t stream)
{
    return ring_for_events(r, first, count, [stream](hipEvent_t e) {
        return HIP_OK(hipStreamWaitEvent(stream, e, 0)) ? KV_OK : KV_ERR_HIP;
    });
}

const char *kv_strerror(int code)
{
    switch (code) {
    case KV_OK: return "ok";
    case KV_ERR_ARG: return "invalid argument";
    case KV_ERR_ALIGN: return "pointer, stride, slot size or token size not 16-byte aligned";
    case KV_ERR_RANGE: return "out of range (table length, slot size, block id, or a buffer past its allocation)";
    case KV_ERR_OOM: return "out of memory or blocks";
    case KV_ERR_RING: return "two chunks of one call share a staging slot";
    case KV_ERR_HIP: return "HIP runtime error";
    case KV_ERR_DEVICE: return "the device reported a block id out of range";
    case KV_ERR_DUP: return "scatter writes one pool page twice";
    case KV_ERR_SCRATCH: return "the call needs more than the static device scratch holds";
    case KV_ERR_CAPTURE: return "the stream is capturing a graph and this call cannot be captured";
    default: return "unknown error";
    }
}

int kv_version(void) { return KV_VERSION; }

int kv_last_hip_error(const char **where)
{
    if (where) *where = g_hip_where;
    return g_hip_error;
}

}  // extern "C"
