// kernel_emu.cpp -- CPU walk of the tile-copy kernel's grid-stride loop (test only).
//
// Built together with the library's own sources, it runs the library's host
// preparation (kvx::prepare_call) and, for every (workgroup, wave) of the grid the
// library would launch, the same span search and tile resolution the kernel
// runs (kvx::find_span, kvx::resolve_tile), on host buffers.  Every address is
// checked against the buffers it must stay in before anything is copied, and
// every tile must be visited exactly once.  With copy != 0 the tile bytes are
// moved with memcpy so the result can be compared with the oracle.
#include <algorithm>
#include <cstring>
#include <vector>

#include "kvxfer_host.h"
#include "kvxfer_internal.h"

// One wave register of 16-byte values, emulated: each lane holds the index of the
// vector it was loaded from (-1: zero).  The two gfx950 lane swaps the kernel's
// 4x4 transpose uses, with the lane layout measured on the device:
// permlane32_swap(a, b) -> (a lanes 0-31 | b lanes 0-31, a lanes 32-63 | b lanes 32-63);
// permlane16_swap(a, b) -> (a row0, b row0, a row2, b row2 | a row1, b row1, a row3, b row3).
struct EmuReg {
    int64_t v[64];
};
static void emu_p32(EmuReg &a, EmuReg &b)
{
    EmuReg na, nb;
    for (int l = 0; l < 32; ++l) {
        na.v[l] = a.v[l], na.v[32 + l] = b.v[l];
        nb.v[l] = a.v[32 + l], nb.v[32 + l] = b.v[32 + l];
    }
    a = na, b = nb;
}
static void emu_p16(EmuReg &a, EmuReg &b)
{
    EmuReg na, nb;
    for (int l = 0; l < 16; ++l) {
        na.v[l] = a.v[l], na.v[16 + l] = b.v[l], na.v[32 + l] = a.v[32 + l], na.v[48 + l] = b.v[32 + l];
        nb.v[l] = a.v[16 + l], nb.v[16 + l] = b.v[16 + l], nb.v[32 + l] = a.v[48 + l], nb.v[48 + l] = b.v[48 + l];
    }
    a = na, b = nb;
}
static void emu_transpose4(EmuReg *x)
{
    emu_p32(x[0], x[2]);
    emu_p32(x[1], x[3]);
    emu_p16(x[0], x[1]);
    emu_p16(x[2], x[3]);
}

extern "C" int emu_transfer(int direction, const kv_pool_desc *d, const kv_span *spans,
                            int32_t n_spans, const kv_chunk_spec *spec, const int64_t *region_bytes,
                            int64_t staging_bytes, int32_t copy, int64_t *violations,
                            int64_t *tiles_out, int64_t *grid_out)
{
    static kvx::SpanDev records[KV_MAX_SPANS];
    uint32_t n_rec = 0;
    kvx::Launch a;
    kv_transfer_info info;
    int rc = kvx::prepare_call(d, spans, n_spans, spec, records, &n_rec, &a, &info);
    if (rc) return rc;
    *violations = 0;
    *tiles_out = info.tiles;
    if (info.tiles == 0) {
        *grid_out = 0;
        return KV_OK;
    }
    // table length of each record (records skip empty spans)
    std::vector<int64_t> tlen;
    for (int32_t i = 0; i < n_spans; ++i)
        if (spans[i].t_end > spans[i].t_begin) tlen.push_back(spans[i].table_len);

    a.split_shift = kvx::launch_split_shift(a, direction);
    a.part_bytes = kvx::part_bytes_for(direction, a, false,      // staging as if in HBM
                                       (spec->flags & KV_FLAG_PAGE_RUNS) != 0);
    if (a.part_bytes) a.split_shift = 0;
    a.seg_bytes = a.part_bytes ? 0u : kvx::gather_seg_bytes(direction, a.page_layout, a.tile_bytes);
    uint32_t grid = kvx::default_grid(kvx::work_items(a));
    if (spec->max_workgroups > 0 && (uint32_t)spec->max_workgroups < grid)
        grid = (uint32_t)spec->max_workgroups;
    a.xcd_remap = kvx::xcd_remap_for(direction, a, false);   // staging as if in HBM
    *grid_out = grid;
    const int64_t nreg_s = (int64_t)d->num_layers * d->num_kv;
    if (direction == KV_GATHER && a.page_layout == KV_PAGE_TOKEN_MAJOR && a.seg_bytes) {
        // the kernel's segment walk: the pieces of every tile must cover it exactly once
        const int64_t T = a.tile_bytes, total = info.tiles * T, n_seg = kvx::work_items(a);
        struct Piece { int64_t tile, lo, hi; };
        std::vector<Piece> pieces;
        std::vector<uint8_t> seg_seen((size_t)n_seg, 0);
        const int64_t step_s = (int64_t)grid * kvx::kWavesPerBlock;
        for (uint32_t b = 0; b < grid; ++b)
            for (int w = 0; w < kvx::kWavesPerBlock; ++w) {
                uint32_t s = 0;
                for (int64_t seg = (int64_t)b * kvx::kWavesPerBlock + w; seg < n_seg; seg += step_s) {
                    if (seg_seen[seg]++) ++*violations;
                    const int64_t x0 = seg * a.seg_bytes;
                    const int64_t x1 = x0 + a.seg_bytes < total ? x0 + a.seg_bytes : total;
                    for (int64_t tile = x0 / T; tile * T < x1; ++tile) {
                        if (tile >= info.tiles) { ++*violations; break; }
                        s = kvx::find_span(records, s, n_rec, tile);
                        const kvx::SpanDev &sp = records[s];
                        const kvx::TileRef t = a.layout == KV_LAYER_FIRST
                                                   ? kvx::resolve_tile<KV_LAYER_FIRST>(a, sp, tile)
                                                   : kvx::resolve_tile<KV_PAGE_FIRST>(a, sp, tile);
                        int64_t lo, hi;
                        kvx::segment_piece(tile, T, t.nbytes, x0, x1, &lo, &hi);
                        if (hi <= lo) continue;
                        if (lo < 0 || lo % 16 || hi % 16 || hi > (int64_t)t.nbytes) { ++*violations; continue; }
                        pieces.push_back({tile, lo, hi});
                        if ((int64_t)t.page >= tlen[s] || (int64_t)t.region >= nreg_s || t.chunk_off < 0 ||
                            t.chunk_off + hi > staging_bytes) {
                            ++*violations;
                            continue;
                        }
                        const int32_t blk = sp.table[t.page];
                        if (blk < 0 || (uint32_t)blk >= a.num_blocks) continue;  // skipped, as the kernel does
                        const int64_t poff = (int64_t)blk * a.block_stride;
                        if (poff + hi > region_bytes[t.region]) { ++*violations; continue; }
                        if (!copy) continue;
                        uint8_t *pool = static_cast<uint8_t *>(d->bases[t.region]) + poff + lo;
                        std::memcpy(a.chunk_base + t.chunk_off + lo, pool, (size_t)(hi - lo));
                    }
                }
            }
        for (int64_t i = 0; i < n_seg; ++i)
            if (seg_seen[i] != 1) ++*violations;
        // a tile whose block id the kernel skips is still walked, so coverage is complete:
        // sorted by (tile, lo), each tile's pieces must run back to back from 0 to nbytes
        std::sort(pieces.begin(), pieces.end(), [](const Piece &x, const Piece &y) {
            return x.tile != y.tile ? x.tile < y.tile : x.lo < y.lo;
        });
        size_t k = 0;
        for (int64_t i = 0; i < info.tiles; ++i) {
            uint32_t s = kvx::find_span(records, 0, n_rec, i);
            const kvx::TileRef t = a.layout == KV_LAYER_FIRST
                                       ? kvx::resolve_tile<KV_LAYER_FIRST>(a, records[s], i)
                                       : kvx::resolve_tile<KV_PAGE_FIRST>(a, records[s], i);
            int64_t at = 0;
            for (; k < pieces.size() && pieces[k].tile == i; ++k) {
                if (pieces[k].lo != at) ++*violations;
                at = pieces[k].hi;
            }
            if (at != (int64_t)t.nbytes) ++*violations;
        }
        if (k != pieces.size()) ++*violations;
        return KV_OK;
    }
    const uint32_t split = (uint32_t)kvx::parts_per_tile(a);
    const int64_t items = info.tiles * split;
    std::vector<uint8_t> seen((size_t)items, 0);
    // head-major 4x4-block walk: every vector of every tile written once
    const int64_t tvec = a.tile_bytes / 16;
    std::vector<uint64_t> written(a.hm_t4 ? (size_t)((info.tiles * tvec + 63) / 64) : 0, 0);
    // LDS-staged head-major walk: every 4-byte word of every tile written once (words
    // numbered in chunk order), and every slice word read was written in the same slab
    const int64_t twords = a.tile_bytes / 4;
    std::vector<uint64_t> wwritten(a.hm_lds ? (size_t)((info.tiles * twords + 63) / 64) : 0, 0);
    const size_t slice_words = (size_t)std::max(KVX_HM_LDS_SLICE, KVX_HM_PAGE_SLICE) / 4;
    std::vector<uint32_t> slice(slice_words);
    std::vector<int64_t> tag(slice_words, -1);
    int64_t gen = 0;
    const int64_t step = (int64_t)grid * kvx::kWavesPerBlock;
    const int64_t nreg = (int64_t)d->num_layers * d->num_kv;

    for (uint32_t b = 0; b < grid; ++b) {
        const uint32_t block = kvx::launch_block(b, grid, a.xcd_remap);
        for (int w = 0; w < kvx::kWavesPerBlock; ++w) {
            uint32_t s = 0;
            for (int64_t item = (int64_t)block * kvx::kWavesPerBlock + w; item < items; item += step) {
                const int64_t tile = item / split;
                s = kvx::find_span(records, s, n_rec, tile);
                const kvx::SpanDev &sp = records[s];
                if (tile < sp.tile_begin) { ++*violations; continue; }
                const kvx::TileRef t = (a.layout == KV_LAYER_FIRST)
                                           ? kvx::resolve_tile<KV_LAYER_FIRST>(a, sp, tile)
                                           : kvx::resolve_tile<KV_PAGE_FIRST>(a, sp, tile);
                if (seen[item]++) { ++*violations; continue; }
                if ((int64_t)t.page >= tlen[s] || (int64_t)t.region >= nreg || t.nbytes == 0 ||
                    t.nbytes % 16 != 0 || t.chunk_off < 0 ||
                    t.chunk_off + (int64_t)t.nbytes > staging_bytes) {
                    ++*violations;
                    continue;
                }
                const int32_t blk = sp.table[t.page];
                if (blk < 0 || (uint32_t)blk >= a.num_blocks) continue;  // the kernel skips it too
                const int64_t poff = (int64_t)blk * a.block_stride;
                if (poff + (int64_t)t.nbytes > region_bytes[t.region]) {
                    ++*violations;
                    continue;
                }
                uint32_t first, count;
                if (a.page_layout == KV_PAGE_HEAD_MAJOR && a.hm_page) {
                    // the kernel's whole-page walk: 16-byte vectors on both sides, words placed
                    // in the slice by hm_page_slice_words, which is checked against plain division
                    const uint32_t n_tok = t.nbytes / a.tok, H = a.hm_heads, rd = a.hm_rd, bs = a.block_size;
                    const uint32_t page_vec = (uint32_t)(a.tile_bytes / 16), tile_vec = n_tok * a.tok / 16;
                    if (split != 1 || a.tile_bytes > KVX_HM_PAGE_SLICE || a.tile_bytes != (int64_t)H * bs * rd * 4 ||
                        poff + a.tile_bytes > region_bytes[t.region]) {
                        ++*violations;
                        continue;
                    }
                    uint8_t *block = static_cast<uint8_t *>(d->bases[t.region]) + poff;
                    uint8_t *tile_p = a.chunk_base + t.chunk_off;
                    auto mark = [&](int64_t word) {  // chunk-order word of this tile
                        const uint64_t bit = (uint64_t)(tile * twords + word);
                        if (wwritten[bit / 64] >> (bit % 64) & 1u) ++*violations;
                        wwritten[bit / 64] |= 1ull << (bit % 64);
                    };
                    auto words_of = [&](uint32_t v, uint32_t sw[4]) {
                        kvx::hm_page_slice_words(a, v, n_tok, sw);
                        for (uint32_t c = 0; c < 4; ++c) {
                            const uint32_t w = 4 * v + c, h = w / (bs * rd), j = w % (bs * rd) / rd, q = w % rd;
                            const uint32_t want = j < n_tok ? (j * H + h) * rd + q : ~0u;
                            if (sw[c] != want) ++*violations;
                            if (sw[c] != ~0u && (int64_t)sw[c] * 4 >= KVX_HM_PAGE_SLICE) ++*violations;
                        }
                    };
                    ++gen;
                    if (direction == KV_GATHER) {
                        for (uint32_t v = 0; v < page_vec; ++v) {  // pool vectors -> slice
                            uint32_t sw[4];
                            words_of(v, sw);
                            for (int c = 0; c < 4; ++c) {
                                if (sw[c] == ~0u || (int64_t)sw[c] * 4 >= KVX_HM_PAGE_SLICE) continue;
                                if (tag[sw[c]] == gen) ++*violations;  // two words into one place
                                if (copy) std::memcpy(&slice[sw[c]], block + (4ll * v + c) * 4, 4);
                                tag[sw[c]] = gen;
                            }
                        }
                        for (uint32_t v = 0; v < tile_vec; ++v) {  // slice -> chunk vectors
                            if (t.chunk_off + (v + 1) * 16ll > staging_bytes || (v + 1) * 16ll > KVX_HM_PAGE_SLICE) {
                                ++*violations;
                                continue;
                            }
                            bool fresh = true;
                            for (int k = 0; k < 4; ++k) fresh = fresh && tag[4 * v + k] == gen;
                            if (!fresh) { ++*violations; continue; }
                            if (copy) std::memcpy(tile_p + v * 16ll, &slice[4 * v], 16);
                            for (int k = 0; k < 4; ++k) mark(4ll * v + k);
                        }
                    } else {
                        for (uint32_t v = 0; v < tile_vec; ++v) {  // chunk vectors -> slice
                            if (t.chunk_off + (v + 1) * 16ll > staging_bytes || (v + 1) * 16ll > KVX_HM_PAGE_SLICE) {
                                ++*violations;
                                continue;
                            }
                            if (copy) std::memcpy(&slice[4 * v], tile_p + v * 16ll, 16);
                            for (int k = 0; k < 4; ++k) tag[4 * v + k] = gen;
                        }
                        for (uint32_t v = 0; v < page_vec; ++v) {  // slice -> pool, whole or by word
                            uint32_t sw[4];
                            words_of(v, sw);
                            for (int c = 0; c < 4; ++c) {
                                if (sw[c] == ~0u) {
                                    if (n_tok == bs) ++*violations;  // a full page stores every word
                                    continue;
                                }
                                if ((int64_t)sw[c] * 4 >= KVX_HM_PAGE_SLICE || tag[sw[c]] != gen) {
                                    ++*violations;
                                    continue;
                                }
                                if (copy) std::memcpy(block + (4ll * v + c) * 4, &slice[sw[c]], 4);
                                mark(sw[c]);
                            }
                        }
                    }
                    continue;
                }
                if (a.page_layout == KV_PAGE_HEAD_MAJOR && a.hm_lds && a.hm_hg[direction]) {
                    // the kernel's head-group slabs, lane by lane and phase by phase; the
                    // slice holds a slab in pool order, the chunk side is walked in chunk order
                    const uint32_t n_tok = t.nbytes / a.tok, H = a.hm_heads, rd = a.hm_rd, bs = a.block_size;
                    const uint32_t hg = a.hm_hg[direction], tj = a.hm_htj[direction], run = tj * rd, grp = hg * rd;
                    const int64_t page_words = (int64_t)H * bs * rd;
                    if (tj == 0 || H % hg || (int64_t)hg * run * 4 > KVX_HM_LDS_SLICE ||
                        poff + page_words * 4 > region_bytes[t.region]) {
                        ++*violations;
                        continue;
                    }
                    const uint32_t n_tr = (n_tok + tj - 1) / tj;
                    kvx::part_range(kvx::hm_lds_slabs(n_tok, H, hg, tj), (uint32_t)(item % split), split, &first,
                                    &count);
                    uint8_t *block = static_cast<uint8_t *>(d->bases[t.region]) + poff;
                    uint8_t *tile_p = a.chunk_base + t.chunk_off;
                    const uint32_t U = KVX_HM_LDS_UNROLL;
                    auto mark = [&](int64_t word) {  // chunk-order word of this tile
                        const uint64_t bit = (uint64_t)(tile * twords + word);
                        if (wwritten[bit / 64] >> (bit % 64) & 1u) ++*violations;
                        wwritten[bit / 64] |= 1ull << (bit % 64);
                    };
                    for (uint32_t sl = first; sl < first + count; ++sl) {
                        ++gen;
                        const uint32_t gi = sl / n_tr, j0 = (sl - gi * n_tr) * tj, h0 = gi * hg;
                        const uint32_t tt = std::min(tj, n_tok - j0), c_words = tt * grp, p_words = hg * run;
                        // pool side: slice word w <-> pool word ((h0 + hh)*bs + j0)*rd + i
                        auto pool_side = [&](bool load) {
                            for (uint32_t lane = 0; lane < 64; ++lane)
                                for (uint32_t w = lane; w < p_words; w += 64u * U)
                                    for (uint32_t u = 0; u < U; ++u) {
                                        const uint32_t ww = w + 64u * u;
                                        const uint32_t hh = kvx::mdiv(ww, a.hm_m_hrun[direction]);
                                        const uint32_t i = ww - hh * run;
                                        const uint32_t jj = kvx::mdiv(i, a.hm_m_rd);
                                        if (!(ww < p_words && jj < tt)) continue;
                                        if (hh != ww / run || jj != i / rd) { ++*violations; continue; }
                                        const int64_t pw = ((int64_t)(h0 + hh) * bs + j0) * rd + i;
                                        if (pw >= page_words || ww * 4ll >= KVX_HM_LDS_SLICE) { ++*violations; continue; }
                                        if (load) {
                                            if (tag[ww] == gen) ++*violations;
                                            if (copy) std::memcpy(&slice[ww], block + pw * 4, 4);
                                            tag[ww] = gen;
                                        } else {
                                            if (tag[ww] != gen) { ++*violations; continue; }  // stale slice word
                                            if (copy) std::memcpy(block + pw * 4, &slice[ww], 4);
                                            mark(((int64_t)(j0 + jj) * H + h0 + hh) * rd + (i - jj * rd));
                                        }
                                    }
                        };
                        // chunk side: chunk word ((j0 + jj)*H + h0)*rd + rem <-> slice word (hh*tj + jj)*rd + q
                        auto chunk_side = [&](bool load) {
                            for (uint32_t lane = 0; lane < 64; ++lane)
                                for (uint32_t w = lane; w < c_words; w += 64u * U)
                                    for (uint32_t u = 0; u < U; ++u) {
                                        const uint32_t ww = w + 64u * u;
                                        if (ww >= c_words) continue;
                                        const uint32_t jj = kvx::mdiv(ww, a.hm_m_hgrp[direction]);
                                        const uint32_t rem = ww - jj * grp;
                                        const uint32_t hh = kvx::mdiv(rem, a.hm_m_rd);
                                        if (jj != ww / grp || hh != rem / rd) { ++*violations; continue; }
                                        const int64_t cw = ((int64_t)(j0 + jj) * H + h0) * rd + rem;
                                        const int64_t lw = ((int64_t)hh * tj + jj) * rd + (rem - hh * rd);
                                        if (cw * 4 + 4 > (int64_t)t.nbytes || t.chunk_off + cw * 4 + 4 > staging_bytes ||
                                            lw * 4 >= KVX_HM_LDS_SLICE) {
                                            ++*violations;
                                            continue;
                                        }
                                        if (load) {
                                            if (tag[lw] == gen) ++*violations;
                                            if (copy) std::memcpy(&slice[lw], tile_p + cw * 4, 4);
                                            tag[lw] = gen;
                                        } else {
                                            if (tag[lw] != gen) { ++*violations; continue; }
                                            if (copy) std::memcpy(tile_p + cw * 4, &slice[lw], 4);
                                            mark(cw);
                                        }
                                    }
                        };
                        if (direction == KV_GATHER) pool_side(true), chunk_side(false);
                        else chunk_side(true), pool_side(false);
                    }
                    continue;
                }
                if (a.page_layout == KV_PAGE_HEAD_MAJOR && a.hm_lds) {
                    // the kernel's LDS slab walk, lane by lane and phase by phase (lanes
                    // of one phase touch distinct slice words, so their order is free)
                    const uint32_t n_tok = t.nbytes / a.tok, H = a.hm_heads, rd = a.hm_rd, tj = a.hm_tj,
                                   bs = a.block_size;
                    const uint32_t run = tj * rd, words = H * run;
                    const int64_t page_words = (int64_t)H * bs * rd;
                    if (tj == 0 || (int64_t)words * 4 > KVX_HM_LDS_SLICE ||
                        poff + page_words * 4 > region_bytes[t.region]) {
                        ++*violations;
                        continue;
                    }
                    kvx::part_range((n_tok + tj - 1) / tj, (uint32_t)(item % split), split, &first, &count);
                    uint8_t *block = static_cast<uint8_t *>(d->bases[t.region]) + poff;
                    uint8_t *tile_p = a.chunk_base + t.chunk_off;
                    auto mark = [&](int64_t word) {  // chunk-order word of this tile
                        const uint64_t bit = (uint64_t)(tile * twords + word);
                        if (wwritten[bit / 64] >> (bit % 64) & 1u) ++*violations;
                        wwritten[bit / 64] |= 1ull << (bit % 64);
                    };
                    for (uint32_t sl = first; sl < first + count; ++sl) {
                        const uint32_t j0 = sl * tj, tt = std::min(tj, n_tok - j0), nvec = tt * a.tok / 16;
                        const int64_t cs = (int64_t)j0 * a.tok;
                        ++gen;
                        if (direction == KV_SCATTER)
                            for (uint32_t lane = 0; lane < 64; ++lane)
                                for (uint32_t v = lane; v < nvec; v += 64) {
                                    if (v >= 64u * (KVX_HM_LDS_SLICE / 1024) ||
                                        t.chunk_off + cs + (v + 1) * 16ll > staging_bytes) {
                                        ++*violations;
                                        continue;
                                    }
                                    if (copy) std::memcpy(&slice[4 * v], tile_p + cs + v * 16ll, 16);
                                    for (int k = 0; k < 4; ++k) tag[4 * v + k] = gen;
                                }
                        for (uint32_t lane = 0; lane < 64; ++lane)
                            for (uint32_t w = lane; w < words; w += 64u * KVX_HM_LDS_UNROLL)
                                for (uint32_t u = 0; u < KVX_HM_LDS_UNROLL; ++u) {
                                    const uint32_t ww = w + 64u * u;
                                    const uint32_t h = kvx::mdiv(ww, a.hm_m_run);
                                    const uint32_t i = ww - h * run;
                                    const uint32_t jj = kvx::mdiv(i, a.hm_m_rd);
                                    if (!(ww < words && jj < tt)) continue;
                                    if (h != ww / run || jj != i / rd) { ++*violations; continue; }
                                    const uint32_t q = i - jj * rd;
                                    const int64_t pw = ((int64_t)h * bs + j0) * rd + i;
                                    const int64_t lw = ((int64_t)jj * H + h) * rd + q;
                                    if (pw >= page_words || lw * 4 >= KVX_HM_LDS_SLICE) { ++*violations; continue; }
                                    if (direction == KV_GATHER) {
                                        if (tag[lw] == gen) ++*violations;  // two words into one place
                                        if (copy) std::memcpy(&slice[lw], block + pw * 4, 4);
                                        tag[lw] = gen;
                                    } else {
                                        if (tag[lw] != gen) { ++*violations; continue; }  // stale slice word
                                        if (copy) std::memcpy(block + pw * 4, &slice[lw], 4);
                                        mark(((int64_t)(j0 + jj) * H + h) * rd + q);
                                    }
                                }
                        if (direction == KV_GATHER)
                            for (uint32_t lane = 0; lane < 64; ++lane)
                                for (uint32_t v = lane; v < nvec; v += 64) {
                                    if (v >= 64u * (KVX_HM_LDS_SLICE / 1024) ||
                                        t.chunk_off + cs + (v + 1) * 16ll > staging_bytes) {
                                        ++*violations;
                                        continue;
                                    }
                                    bool fresh = true;
                                    for (int k = 0; k < 4; ++k) fresh = fresh && tag[4 * v + k] == gen;
                                    if (!fresh) { ++*violations; continue; }
                                    if (copy) std::memcpy(tile_p + cs + v * 16ll, &slice[4 * v], 16);
                                    for (int k = 0; k < 4; ++k) mark(cs / 4 + 4ll * v + k);
                                }
                    }
                    continue;
                }
                if (a.page_layout == KV_PAGE_HEAD_MAJOR && a.hm_t4) {
                    // the kernel's block walk: loads, the register transpose, stores
                    const uint32_t n_tok = t.nbytes / a.tok, H = a.hm_heads, bs = a.block_size;
                    const int64_t page_vec = (int64_t)H * bs * 16, tile_vec = (int64_t)n_tok * H * 16;
                    if (poff + page_vec * 16 > region_bytes[t.region]) { ++*violations; continue; }
                    kvx::part_range(kvx::hm_t4_units(n_tok, H), (uint32_t)(item % split), split, &first, &count);
                    uint8_t *block = static_cast<uint8_t *>(d->bases[t.region]) + poff;
                    uint8_t *tile_p = a.chunk_base + t.chunk_off;
                    for (uint32_t u = first; u < first + count; ++u) {
                        const uint32_t j0 = (u / (H / 4)) * 4, hb = (u % (H / 4)) * 4;
                        EmuReg x[4];
                        for (int r = 0; r < 4; ++r)
                            for (int l = 0; l < 64; ++l) {
                                if (direction == KV_GATHER) {
                                    const int64_t pv = ((int64_t)(hb + r) * bs + j0) * 16 + l;
                                    if (pv >= page_vec) ++*violations;
                                    x[r].v[l] = pv;
                                } else {
                                    x[r].v[l] = j0 + r < n_tok ? ((int64_t)(j0 + r) * H + hb) * 16 + l : -1;
                                }
                            }
                        emu_transpose4(x);
                        for (int r = 0; r < 4; ++r)
                            for (int l = 0; l < 64; ++l) {
                                int64_t dst, mark;
                                if (direction == KV_GATHER) {
                                    dst = ((int64_t)(j0 + r) * H + hb) * 16 + l;  // chunk vector
                                    if (dst >= tile_vec) continue;                // past the tile: dropped
                                    mark = dst;
                                } else {
                                    if (j0 + (l >> 4) >= n_tok) continue;         // token past the tile
                                    dst = ((int64_t)(hb + r) * bs + j0) * 16 + l;   // pool vector
                                    if (dst >= page_vec) { ++*violations; continue; }
                                    // the pool vector of (head, token, q) is the tile's
                                    // chunk-order vector (token, head, q)
                                    const int64_t hh = dst / (bs * 16), jj = dst / 16 % bs, q = dst % 16;
                                    mark = (jj * H + hh) * 16 + q;
                                }
                                const int64_t src = x[r].v[l];
                                if (src < 0) { ++*violations; continue; }      // would store a zero
                                const uint64_t bit = (uint64_t)(tile * tvec + mark);
                                if (written[bit / 64] >> (bit % 64) & 1u) ++*violations;
                                written[bit / 64] |= 1ull << (bit % 64);
                                if (direction == KV_GATHER) {
                                    if (t.chunk_off + dst * 16 + 16 > staging_bytes) { ++*violations; continue; }
                                    if (copy) std::memcpy(tile_p + dst * 16, block + src * 16, 16);
                                } else {
                                    if (copy) std::memcpy(block + dst * 16, tile_p + src * 16, 16);
                                }
                            }
                    }
                    continue;
                }
                kvx::tile_part(a, t.nbytes >> 4, (uint32_t)(item % split), &first, &count);
                if (first + count > (t.nbytes >> 4)) { ++*violations; continue; }
                if (a.page_layout == KV_PAGE_HEAD_MAJOR) {
                    // each lane's cursor, as the kernel advances it, 64 vectors at a time
                    uint8_t *block = static_cast<uint8_t *>(d->bases[t.region]) + poff;
                    uint8_t *tile = a.chunk_base + t.chunk_off;
                    for (uint32_t lane = 0; lane < 64; ++lane) {
                        kvx::HmCursor c;
                        c.init(first + lane, a);
                        for (uint32_t v = first + lane; v < first + count; v += 64) {
                            const uint32_t pv = c.pool_vec(a);
                            c.advance(a);
                            if ((int64_t)pv * 16 + 16 > (int64_t)a.hm_bs_r16 * a.hm_heads * 16) {
                                ++*violations;  // outside the block's [H][bs][D] page
                                continue;
                            }
                            if (!copy) continue;
                            if (direction == KV_GATHER) std::memcpy(tile + v * 16ull, block + pv * 16ull, 16);
                            else std::memcpy(block + pv * 16ull, tile + v * 16ull, 16);
                        }
                    }
                } else if (copy && count) {
                    uint8_t *pool = static_cast<uint8_t *>(d->bases[t.region]) + poff + first * 16ll;
                    uint8_t *chunk = a.chunk_base + t.chunk_off + first * 16ll;
                    if (direction == KV_GATHER) std::memcpy(chunk, pool, count * 16ull);
                    else std::memcpy(pool, chunk, count * 16ull);
                }
            }
        }
    }
    for (int64_t i = 0; i < items; ++i)
        if (seen[i] != 1) ++*violations;
    if (a.hm_lds) {  // every word of every tile with a valid block id written exactly once
        uint32_t s = 0;
        for (int64_t i = 0; i < info.tiles; ++i) {
            s = kvx::find_span(records, s, n_rec, i);
            const kvx::TileRef t = a.layout == KV_LAYER_FIRST ? kvx::resolve_tile<KV_LAYER_FIRST>(a, records[s], i)
                                                              : kvx::resolve_tile<KV_PAGE_FIRST>(a, records[s], i);
            const int32_t blk = records[s].table[t.page];
            if (blk < 0 || (uint32_t)blk >= a.num_blocks) continue;
            for (int64_t v = 0; v < twords; ++v) {
                const uint64_t bit = (uint64_t)(i * twords + v);
                const bool w = wwritten[bit / 64] >> (bit % 64) & 1u;
                if (w != (v < (int64_t)(t.nbytes / 4))) ++*violations;
            }
        }
    }
    if (a.hm_t4) {  // every vector of every tile with a valid block id written exactly once
        uint32_t s = 0;
        for (int64_t i = 0; i < info.tiles; ++i) {
            s = kvx::find_span(records, s, n_rec, i);
            const kvx::TileRef t = a.layout == KV_LAYER_FIRST ? kvx::resolve_tile<KV_LAYER_FIRST>(a, records[s], i)
                                                              : kvx::resolve_tile<KV_PAGE_FIRST>(a, records[s], i);
            const int32_t blk = records[s].table[t.page];
            if (blk < 0 || (uint32_t)blk >= a.num_blocks) continue;
            for (int64_t v = 0; v < tvec; ++v) {
                const uint64_t bit = (uint64_t)(i * tvec + v);
                const bool w = written[bit / 64] >> (bit % 64) & 1u;
                if (w != (v < (int64_t)(t.nbytes / 16))) ++*violations;
            }
        }
    }
    return KV_OK;
}

// The copy-engine path's plan (kvx::dma_walk, as kv_*_chunks_dma issue it), carried
// out with memcpy on host buffers.  Every row of every copy is checked against the
// region it must lie in and the staging buffer first.  spans[i].block_table are host
// arrays here, as for the _dma entry points.
extern "C" int emu_dma(int direction, const kv_pool_desc *d, const kv_span *spans, int32_t n_spans,
                       const kv_chunk_spec *spec, const int64_t *region_bytes, int64_t staging_bytes,
                       int32_t strided, int64_t *violations, int64_t *copies_out, int64_t *rows_out)
{
    static kvx::SpanDev records[KV_MAX_SPANS];
    uint32_t n_rec = 0;
    kvx::Launch a;
    kv_transfer_info info;
    int rc = kvx::prepare_call(d, spans, n_spans, spec, records, &n_rec, &a, &info);
    if (rc) return rc;
    std::vector<const int32_t *> tables;
    for (int32_t i = 0; i < n_spans; ++i)
        if (spans[i].t_end > spans[i].t_begin) tables.push_back(spans[i].block_table);
    const int64_t nreg = (int64_t)d->num_layers * d->num_kv;
    const int64_t pitch = strided ? kvx::uniform_region_pitch(d->bases, nreg) : 0;
    *violations = 0;
    *copies_out = 0;
    *rows_out = 0;
    uint8_t *stg = static_cast<uint8_t *>(spec->base);
    return kvx::dma_walk(a, records, n_rec, tables.data(), d->bases, pitch, strided != 0,
                         [&](const kvx::DmaCopy &c) -> int {
                             ++*copies_out;
                             for (int64_t i = 0; i < c.rows; ++i) {
                                 const int64_t r = c.region + i * c.region_step;
                                 uint8_t *pool = c.pool + i * c.pool_pitch;
                                 uint8_t *chunk = c.chunk + i * c.chunk_pitch;
                                 uint8_t *rb = static_cast<uint8_t *>(d->bases[r]);
                                 ++*rows_out;
                                 if (r < 0 || r >= nreg || c.width <= 0 || pool < rb ||
                                     pool + c.width > rb + region_bytes[r] || chunk < stg ||
                                     chunk + c.width > stg + staging_bytes) {
                                     ++*violations;
                                     continue;
                                 }
                                 if (direction == KV_GATHER) std::memcpy(chunk, pool, (size_t)c.width);
                                 else std::memcpy(pool, chunk, (size_t)c.width);
                             }
                             return 0;
                         });
}

// The span-record arena's bookkeeping (kvx::ArenaRing) driven by a sequence of call
// sizes, with calls finishing only when the arena waits for them (the slowest
// device) or, with `lag` > 0, also on their own once `lag` newer calls exist.  Every
// reservation must stay inside the arena and must not overlap the bytes of any call
// still in flight; returns the number of violations.
extern "C" int64_t emu_arena(int64_t size, const int64_t *sizes, int64_t n_calls, int32_t lag)
{
    constexpr int N = 256;
    static kvx::ArenaRing<N> ring;
    ring.reset();
    ring.size = size;
    struct Live { int64_t off, bytes, call; };
    std::vector<Live> live;       // calls not yet finished, in call order
    std::vector<int64_t> slot_call(N, -1);
    int64_t violations = 0;
    for (int64_t c = 0; c < n_calls; ++c) {
        if (lag > 0)
            while (!live.empty() && live.front().call + lag <= c) live.erase(live.begin());
        int64_t off = -1;
        ring.take(sizes[c], &off, [&](int slot) {
            // waiting for the call in this slot finishes it (and every older call)
            const int64_t call = slot_call[slot];
            while (!live.empty() && live.front().call <= call) live.erase(live.begin());
            return 0;
        });
        if (off < 0 || off + sizes[c] > size) ++violations;
        for (const Live &l : live)
            if (l.off < off + sizes[c] && off < l.off + l.bytes) ++violations;
        slot_call[ring.next_slot()] = c;
        ring.commit(off, sizes[c]);
        live.push_back({off, sizes[c], c});
        if ((int64_t)live.size() > N) ++violations;  // more than N calls in flight
    }
    return violations;
}

// The launch-shape rules of the library's host preparation, for direct checks.
// The launch decisions for one call: out[0] split shift, out[1] segment bytes, out[2]
// LDS-staged head-major rows, out[3] whole-page head-major path, out[4] 4 x 4 transpose,
// out[5] workgroups remapped per XCD, out[6] scatter through buffer instructions,
// out[7] fixed part bytes of a scatter's tiles (all with the staging in HBM).
extern "C" int emu_launch_rule(int direction, const kv_pool_desc *d, const kv_span *spans, int32_t n_spans,
                               const kv_chunk_spec *spec, int64_t *out)
{
    static kvx::SpanDev records[KV_MAX_SPANS];
    uint32_t n_rec = 0;
    kvx::Launch a;
    kv_transfer_info info;
    const int rc = kvx::prepare_call(d, spans, n_spans, spec, records, &n_rec, &a, &info);
    if (rc) return rc;
    out[0] = kvx::launch_split_shift(a, direction);
    out[2] = a.hm_lds;
    out[3] = a.hm_page;
    out[4] = a.hm_t4;
    out[7] = kvx::part_bytes_for(direction, a, false, (spec->flags & KV_FLAG_PAGE_RUNS) != 0);
    a.split_shift = out[7] ? 0u : (uint32_t)out[0];
    a.part_bytes = (uint32_t)out[7];
    out[0] = a.split_shift;
    out[1] = out[7] ? 0 : kvx::gather_seg_bytes(direction, a.page_layout, a.tile_bytes);
    a.seg_bytes = (uint32_t)out[1];
    out[5] = kvx::xcd_remap_for(direction, a, false);
    out[6] = kvx::scatter_buffer_form(direction, a, false);
    return KV_OK;
}

extern "C" int emu_gather_seg_unroll(int64_t tile_bytes, int64_t seg_bytes)
{
    return kvx::gather_seg_unroll(tile_bytes, seg_bytes);
}
extern "C" int32_t emu_hm_page_ok(int64_t row, int64_t tok, int64_t tile)
{
    return kvx::hm_page_ok(KV_PAGE_HEAD_MAJOR, row, tok, tile) ? 1 : 0;
}

extern "C" uint32_t emu_hm_lds_tokens(int64_t row, int64_t tok, uint32_t block_size)
{
    return kvx::hm_lds_tokens(row, tok, block_size);
}
extern "C" void emu_hm_lds_head_slab(int dir, uint32_t heads, int64_t row, int64_t tok, uint32_t block_size,
                                     uint32_t *hg, uint32_t *tj)
{
    kvx::hm_lds_head_slab(dir, heads, row, tok, block_size, hg, tj);
}

// The declared-extent walk and its cache (kvx::covered_end, kvx::ExtentCache) over a
// fake table of allocations [bases[i], bases[i] + sizes[i]) standing in for the HIP
// runtime's; lookups are counted so a test can see when the cache answers alone.
static std::vector<uint64_t> g_alloc_base, g_alloc_size;
static int64_t g_lookups = 0;
static kvx::ExtentCache g_cache;

static kvx::AllocRange fake_alloc_range(uintptr_t a)
{
    ++g_lookups;
    for (size_t i = 0; i < g_alloc_base.size(); ++i)
        if (a >= g_alloc_base[i] && a - g_alloc_base[i] < g_alloc_size[i])
            return kvx::AllocRange{g_alloc_base[i], g_alloc_base[i] + g_alloc_size[i]};
    return kvx::AllocRange{};
}

extern "C" void emu_set_allocs(const uint64_t *bases, const uint64_t *sizes, int32_t n)
{
    g_alloc_base.assign(bases, bases + n);
    g_alloc_size.assign(sizes, sizes + n);
}

extern "C" uint64_t emu_covered_end(uint64_t q, uint64_t need, int32_t max_pieces)
{
    return kvx::covered_end(q, need, fake_alloc_range, max_pieces);
}

extern "C" void emu_cache_reset() { g_cache = kvx::ExtentCache(); g_lookups = 0; }

extern "C" int32_t emu_cache_covers(uint64_t q, int64_t bytes, int64_t *lookups)
{
    const int64_t before = g_lookups;
    const bool ok = g_cache.covers(reinterpret_cast<const void *>(q), bytes, fake_alloc_range);
    *lookups = g_lookups - before;
    return ok ? 1 : 0;
}

extern "C" uint32_t emu_launch_block(uint32_t b, uint32_t grid, uint32_t remap)
{
    return kvx::launch_block(b, grid, remap);
}
