// kvxfer_host.h -- host-only bookkeeping of the transfer library (not part of the
// public ABI, never compiled into the kernel): the span-record arena's reservation
// rule and the copy-engine path's plan.  Kept apart from kvxfer_internal.h, which
// holds what the kernel itself runs.
#pragma once
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "kvxfer_internal.h"

namespace kvx {

// ---- declared extents against the runtime's allocations (host) ---------------

// One allocation (or virtual-memory mapping) as the runtime reports it: [base, end).
// end == 0: the runtime does not know the address.
struct AllocRange {
    uintptr_t base = 0, end = 0;
    bool operator==(const AllocRange &o) const { return base == o.base && end == o.end; }
};

// How far from address q the allocations the runtime knows reach without a gap,
// walking from one allocation (or virtual-memory mapping) to the next until `need` is
// covered.  lookup(a) returns the AllocRange holding a.  Returns 0 when q itself is
// unknown, the end of the last adjoining allocation otherwise, and UINTPTR_MAX when
// more than max_pieces would have to be followed (the range is then taken on trust).
// *last, if given, receives the last allocation the walk looked at.
template <class Lookup>
uintptr_t covered_end(uintptr_t q, uintptr_t need, Lookup lookup, int max_pieces = 1 << 16,
                      AllocRange *last = nullptr)
{
    uintptr_t cur = q;
    for (int i = 0; i < max_pieces; ++i) {
        const AllocRange r = lookup(cur);
        if (r.end <= cur) return i == 0 ? 0 : cur;   // unknown memory after known pieces
        if (last) *last = r;
        if (r.end >= need) return r.end;
        cur = r.end;
    }
    return UINTPTR_MAX;
}

// The declared-extent check.  Every call asks the runtime for the allocation holding
// the pointer (one lookup), so an allocation freed and made again at the same address,
// smaller or larger, is always seen as it is now.  Only a range that runs on into
// adjoining allocations (memory mapped in several pieces) needs a longer walk; its
// result is kept in a small direct-mapped table keyed by pointer and reused while the
// allocations holding the first and the last byte the walk reached are unchanged.
struct ExtentCache {
    static constexpr int kEntries = 128;
    const void *key[kEntries] = {};
    AllocRange first[kEntries] = {};  // allocation holding the pointer when the walk ran
    AllocRange last[kEntries] = {};   // last allocation the walk reached
    uintptr_t end[kEntries] = {};     // how far the walk got

    // true when [q, q + bytes) lies inside memory the runtime has allocated or mapped
    // without a gap, or the runtime does not know q.  *here, if given, receives the
    // allocation holding q.
    template <class Lookup>
    bool covers(const void *q, int64_t bytes, Lookup lookup, AllocRange *here = nullptr)
    {
        const uintptr_t a = reinterpret_cast<uintptr_t>(q);
        const uintptr_t need = a + (uintptr_t)bytes;
        const AllocRange r = lookup(a);
        if (here) *here = r;
        if (r.end <= a) return true;      // unknown to the runtime: taken on trust
        if (r.end >= need) return true;   // one allocation holds the whole range
        const int i = (int)(((a >> 9) ^ (a >> 21)) % kEntries);
        if (key[i] == q && first[i] == r && end[i] >= need && lookup(last[i].base) == last[i])
            return true;
        AllocRange l = r;
        const uintptr_t e = covered_end(r.end, need, lookup, 1 << 16, &l);
        const uintptr_t reach = e ? e : r.end;  // nothing adjoins: the first piece's end
        key[i] = q;
        first[i] = r;
        last[i] = l;
        end[i] = reach;
        return reach >= need;
    }
};

// Kind of staging memory (host or device) last seen at one address, remembered
// together with the allocation holding it, so that a new allocation at the same
// address is looked at again.
struct StagingKind {
    const void *base = nullptr;
    AllocRange alloc;
    bool host = false;

    template <class Query>
    bool is_host(const void *b, const AllocRange &r, Query query_host)
    {
        if (b != base || !(r == alloc)) {
            host = query_host(b);
            base = b;
            alloc = r;
        }
        return host;
    }
};

// ---- block allocator (host) --------------------------------------------------

// The free blocks of a pool as a bitmap (bit b of word w: block 64w+b is free).
// Allocation hands out the lowest free ids first, in ascending order, so a request's
// pages sit as close together in each region as the pool's fragmentation allows:
// reloading into nearby pages writes faster than into scattered ones.  Freeing
// checks every id (in range, allocated, not repeated) before freeing any.
struct BlockBitmap {
    std::vector<uint64_t> free_bits;
    int64_t n_blocks = 0, n_free = 0;
    int64_t low_word = 0;  // no free block in the words below this one

    void init(int64_t n)
    {
        n_blocks = n;
        n_free = n;
        low_word = 0;
        free_bits.assign((size_t)((n + 63) / 64), ~0ull);
        if (n % 64) free_bits.back() = (1ull << (n % 64)) - 1;
    }
    bool is_free(int64_t id) const { return (free_bits[(size_t)(id >> 6)] >> (id & 63)) & 1u; }

    int alloc(int32_t n, int32_t *out)
    {
        if (n > n_free) return KV_ERR_OOM;
        int32_t got = 0;
        int64_t w = low_word;
        while (got < n) {
            uint64_t bits = free_bits[(size_t)w];
            while (bits && got < n) {
                const int b = __builtin_ctzll(bits);
                bits &= bits - 1;
                out[got++] = (int32_t)(w * 64 + b);
            }
            free_bits[(size_t)w] = bits;
            if (bits) break;
            ++w;
        }
        low_word = w;
        n_free -= n;
        return KV_OK;
    }

    int release(int32_t n, const int32_t *ids)
    {
        for (int32_t i = 0; i < n; ++i) {
            const int64_t id = ids[i];
            if (id < 0 || id >= n_blocks || is_free(id)) {  // out of range, free, or repeated
                for (int32_t j = 0; j < i; ++j) free_bits[(size_t)(ids[j] >> 6)] &= ~(1ull << (ids[j] & 63));
                return KV_ERR_RANGE;
            }
            free_bits[(size_t)(id >> 6)] |= 1ull << (id & 63);
        }
        for (int32_t i = 0; i < n; ++i) low_word = std::min<int64_t>(low_word, ids[i] >> 6);
        n_free += n;
        return KV_OK;
    }
};

// ---- span-record arena (host bookkeeping) -----------------------------------

// Byte ranges of a circular buffer of `size` bytes reserved by up to N calls in
// flight, oldest first.  Reservations are sequential: a call takes the bytes after
// the previous one, or wraps to offset 0 when they do not fit before the end (the
// skipped tail then counts as taken too).  take() retires, oldest first, every call
// whose bytes the new reservation needs -- and the oldest call whenever N are in
// flight -- by calling wait(slot), which returns nonzero to abort.
template <int N>
struct ArenaRing {
    int64_t size = 0;
    int64_t off[N] = {}, bytes[N] = {};
    int first = 0, count = 0;
    int64_t head = 0;

    void reset() { first = count = 0, head = 0; }

    template <class Wait>
    int take(int64_t b, int64_t *out, Wait wait)
    {
        int64_t start = head;
        bool wrapped = false;
        if (start + b > size) start = 0, wrapped = true;
        while (count > 0) {
            const int i = first;
            // calls at or after the old head precede the wrap: they are the oldest
            const bool in_tail = wrapped && off[i] >= head;
            const bool overlap = off[i] < start + b && start < off[i] + bytes[i];
            if (!in_tail && !overlap && count < N) break;
            if (int rc = wait(i)) return rc;
            first = (i + 1) % N;
            --count;
        }
        *out = start;
        return 0;
    }
    // Slot of the next commit (for the caller's per-call event).
    int next_slot() const { return (first + count) % N; }
    void commit(int64_t o, int64_t b)
    {
        const int i = next_slot();
        off[i] = o;
        bytes[i] = b;
        ++count;
        head = o + b;
    }
};

// ---- the copy-engine path (host) ------------------------------------------

// One copy issued by the host: `rows` rows of `width` bytes; row i lies at
// pool + i*pool_pitch in region `region + i*region_step` and at chunk + i*chunk_pitch.
struct DmaCopy {
    uint8_t *pool;
    uint8_t *chunk;
    int64_t width, rows, pool_pitch, chunk_pitch;
    int64_t region, region_step;
};

// Distance in bytes between consecutive regions when all n are evenly spaced in
// ascending order, else 0.
inline int64_t uniform_region_pitch(void *const *bases, int64_t n)
{
    if (n < 2) return 0;
    const int64_t r = (int64_t)((const uint8_t *)bases[1] - (const uint8_t *)bases[0]);
    if (r <= 0) return 0;
    for (int64_t i = 2; i < n; ++i)
        if ((int64_t)((const uint8_t *)bases[i] - (const uint8_t *)bases[i - 1]) != r) return 0;
    return r;
}

// The copies of one call, in chunk order, handed to emit(const DmaCopy &), which
// returns nonzero to stop the walk (that value is returned).  tables[s] is the host
// block table of record s; ids must already be checked.
//  * token-major pages, per tile: one copy per (layer, kv, page) tile;
//  * token-major pages, strided (region_pitch > 0 and CL*KV > 1): the CL*KV tiles of
//    one page in one chunk -- one per (layer, kv) of the chunk, in region order --
//    become one copy of CL*KV rows: their pool addresses step by region_pitch, their
//    chunk offsets by one (layer, kv) row of the chunk (T_c tokens layer-first, one
//    page page-first);
//  * head-major pages: one copy per (tile, head) of n_tok rows of D*E bytes.
template <class Emit>
int dma_walk(const Launch &a, const SpanDev *rec, uint32_t n_rec, const int32_t *const *tables,
             void *const *bases, int64_t region_pitch, bool strided, Emit emit)
{
    auto tile_ref = [&](const SpanDev &sp, int64_t tile) {
        return a.layout == KV_LAYER_FIRST ? resolve_tile<KV_LAYER_FIRST>(a, sp, tile)
                                          : resolve_tile<KV_PAGE_FIRST>(a, sp, tile);
    };
    auto pool_of = [&](uint32_t s, const TileRef &t) {
        return static_cast<uint8_t *>(bases[t.region]) + (int64_t)tables[s][t.page] * a.block_stride;
    };
    const int64_t rows = (int64_t)a.chunk_layers * a.num_kv;
    if (a.page_layout == KV_PAGE_TOKEN_MAJOR && strided && region_pitch > 0 && rows > 1) {
        for (uint32_t s = 0; s < n_rec; ++s) {
            const SpanDev &sp = rec[s];
            const int64_t span_tiles = (s + 1 < n_rec ? rec[s + 1].tile_begin : a.total_tiles) - sp.tile_begin;
            const int64_t n_lc = span_tiles / sp.per_lc;
            for (int64_t lc = 0; lc < n_lc; ++lc)
                for (uint32_t tc = 0; tc < sp.n_tc; ++tc) {
                    const uint32_t pages_here = min32(sp.ppc, sp.n_pages - tc * sp.ppc);
                    const int64_t base = sp.tile_begin + lc * sp.per_lc + (int64_t)tc * sp.per_tc;
                    for (uint32_t pi = 0; pi < pages_here; ++pi) {
                        // tiles of rows 0 and 1 of this page: the row index is the
                        // slowest digit of a layer-first chunk and the fastest of a
                        // page-first one
                        const int64_t i0 = a.layout == KV_LAYER_FIRST ? base + pi : base + pi * rows;
                        const int64_t i1 = a.layout == KV_LAYER_FIRST ? i0 + pages_here : i0 + 1;
                        const TileRef t0 = tile_ref(sp, i0), t1 = tile_ref(sp, i1);
                        DmaCopy c;
                        c.pool = pool_of(s, t0);
                        c.chunk = a.chunk_base + t0.chunk_off;
                        c.width = t0.nbytes;
                        c.rows = rows;
                        c.pool_pitch = region_pitch;
                        c.chunk_pitch = t1.chunk_off - t0.chunk_off;
                        c.region = t0.region;
                        c.region_step = 1;
                        if (int rc = emit(c)) return rc;
                    }
                }
        }
        return 0;
    }
    uint32_t s = 0;
    for (int64_t tile = 0; tile < a.total_tiles; ++tile) {
        s = find_span(rec, s, n_rec, tile);
        const TileRef t = tile_ref(rec[s], tile);
        DmaCopy c;
        c.pool = pool_of(s, t);
        c.chunk = a.chunk_base + t.chunk_off;
        c.region = t.region;
        c.region_step = 0;
        if (a.page_layout == KV_PAGE_TOKEN_MAJOR) {
            c.width = t.nbytes;
            c.rows = 1;
            c.pool_pitch = c.chunk_pitch = t.nbytes;
            if (int rc = emit(c)) return rc;
            continue;
        }
        const int64_t row = a.hm_row;
        c.width = row;
        c.rows = t.nbytes / a.tok;
        c.pool_pitch = row;
        c.chunk_pitch = (int64_t)a.hm_heads * row;
        uint8_t *pool0 = c.pool, *chunk0 = c.chunk;
        for (uint32_t h = 0; h < a.hm_heads; ++h) {
            c.pool = pool0 + (int64_t)h * a.block_size * row;
            c.chunk = chunk0 + h * row;
            if (int rc = emit(c)) return rc;
        }
    }
    return 0;
}

}  // namespace kvx
