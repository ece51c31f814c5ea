// kvxfer_internal.h -- launch descriptor and tile addressing shared by the host
// code and the gfx950 kernel (not part of the public ABI).
//
// One call = one kernel launch over "tiles": a tile is the tokens of one page of
// one (layer, kv) region that a span moves.  On both sides a tile is one
// contiguous byte range (tokens are stored token-major, tok bytes each, in the
// pool block and in either chunk layout), so the layout change between pool and
// chunk is only the choice of the two base addresses -- made per tile by the
// wavefront that copies it (Strata guide, "Two-Dimensional Memory Layout
// Decoupling": the target address comes from a little integer arithmetic, and no
// separate transposition pass is needed).
//
// Tiles of a span are numbered in chunk order so that consecutive wavefronts
// walk the contiguous chunk side sequentially, as the printed load kernel walks
// its page-first source linearly (Strata guide, "Step 1: High-Performance
// GPU-Assisted I/O CUDA Kernel"):
//   local tile r = (lc * n_tc + tc) * (tiles of a full chunk) + in-chunk index
//   in-chunk index, layer-first chunk [CL][KV][pages]: (li * KV + kv) * pages_here + pi
//   in-chunk index, page-first chunk  [pages][CL][KV]: (pi * CL + li) * KV + kv
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kvxfer.h"

namespace kvx {

// Launch shape and copy policy; the defaults are the values measured best on MI355X.
#ifndef KVX_WAVES_PER_BLOCK
#define KVX_WAVES_PER_BLOCK 4  // 256-thread workgroups of four 64-lane wavefronts
#endif
#ifndef KVX_GRID_CAP
// Workgroups per launch at most (more work items loop).  At 2^20 every workload here
// gets one work item per wave, so no wave resolves a second tile (span search, record
// and block-id loads) in the middle of its life: measured on MI355X, the 64-request
// mixed gather (1.65 M items, 12.6 per wave at a cap of 32768) +5 to +7 %, the others
// within noise.
#define KVX_GRID_CAP 1048576
#endif
#ifndef KVX_HOST_GRID_CAP
#define KVX_HOST_GRID_CAP 16   // default workgroups when the staging is host memory
#endif
// A tile of at least SPLIT_MIN bytes is shared by 2 or 4 waves (neighbouring waves of
// a workgroup copy neighbouring parts of about PART_BYTES), so the bytes in flight at
// once form longer contiguous runs.  Measured on MI355X: 64 KiB tiles gain 5-12 %,
// splitting 32 KiB tiles loses; PART_BYTES 0 disables the split.
#ifndef KVX_GATHER_SPLIT_MIN
#define KVX_GATHER_SPLIT_MIN 65536
#endif
#ifndef KVX_GATHER_PART_BYTES
#define KVX_GATHER_PART_BYTES 32768
#endif
#ifndef KVX_SCATTER_SPLIT_MIN
#define KVX_SCATTER_SPLIT_MIN 65536
#endif
#ifndef KVX_SCATTER_PART_BYTES
#define KVX_SCATTER_PART_BYTES 16384
#endif
// Token-major tiles of SMALL_SPLIT_MIN bytes up to (not including) SMALL_GATHER_MAX
// (gather) or SMALL_SCATTER_MAX (scatter) are split the same way into parts of about
// SMALL_PART bytes: measured on MI355X, gathers of 8 and 12 KiB tiles gain 4 and 6
// points that way (over one tile or one segment per wave), scatters of 8, 12 and 16 KiB
// tiles 1.1, 1.4 and 2.3 points; a 20 KiB scatter loses 0.9.
#ifndef KVX_SMALL_SPLIT_MIN
#define KVX_SMALL_SPLIT_MIN 8192
#endif
#ifndef KVX_SMALL_GATHER_MAX
#define KVX_SMALL_GATHER_MAX 16384
#endif
#ifndef KVX_SMALL_SCATTER_MAX
#define KVX_SMALL_SCATTER_MAX 20480
#endif
#ifndef KVX_SMALL_PART
#define KVX_SMALL_PART 2048
#endif
// Gather of token-major pages whose tiles are at least SEG_MIN bytes and either not a
// power of two or smaller than a segment runs over the call's tiles laid end to end in
// SEG_BYTES segments, one per wave, instead of one tile per wave: each wave then writes
// one aligned 32 KiB piece of the chunk stream.  Measured on MI355X: 2-9 % faster for
// 24-40 KiB tiles and 4 points for 16 KiB tiles (32 KiB tiles are the two schedules'
// common case; 16, 24 and 48 KiB segments lose).
#ifndef KVX_GATHER_SEG_BYTES
#define KVX_GATHER_SEG_BYTES 32768
#endif
#ifndef KVX_GATHER_SEG_MIN
#define KVX_GATHER_SEG_MIN 16384
#endif
#ifndef KVX_HM_LDS_SPLIT_MIN
// head-major pages staged through LDS slabs (not whole) from this size go in 4 parts:
// measured on MI355X, 24 KiB pages of 24-byte rows gather at 73.5-73.7 % of HBM peak that
// way against 64.7-64.8 % whole (2 parts: 68.6-68.9 %) and scatter at 63.5-63.8 % against
// 61.2-61.3 %
#define KVX_HM_LDS_SPLIT_MIN 16384
#endif
#ifndef KVX_HM_T4_SCATTER_SPLIT_MIN
// head-major pages moved by the 4 x 4 transpose are scattered from this size to under
// twice it in 8 parts (ranges of the page's 4 KiB blocks of 4 tokens x 4 heads), one per
// wave; larger pages follow split_shift_for (not measured split finer): measured on
// MI355X, 32 KiB pages of 256-byte rows scatter at 69.8 % of HBM peak that way against
// 68.4 % whole (8 parts with the per-XCD order 69.4 %, 4 parts with it 67.8 %)
#define KVX_HM_T4_SCATTER_SPLIT_MIN 32768
#endif
#define KVX_HM_T4_SCATTER_SHIFT 3
#ifndef KVX_MAX_SPLIT_SHIFT
#define KVX_MAX_SPLIT_SHIFT 2     // at most 4 waves per tile (other than the case above)
#endif
#ifndef KVX_GATHER_UNROLL
#define KVX_GATHER_UNROLL 8    // 16-byte vectors per lane per group, gather
#endif
#ifndef KVX_GATHER_PIPELINE
#define KVX_GATHER_PIPELINE 1  // next group's loads issued before this group's stores
#endif
#ifndef KVX_SCATTER_UNROLL
#define KVX_SCATTER_UNROLL 16  // 16-byte vectors per lane per group, scatter
#endif
#ifndef KVX_SCATTER_PIPELINE
#define KVX_SCATTER_PIPELINE 0
#endif
#ifndef KVX_HM_UNROLL
#define KVX_HM_UNROLL 8        // vectors per lane per group, head-major pools
#endif
#ifndef KVX_HM_POOL_NT
#define KVX_HM_POOL_NT 1       // nontemporal accesses on the pool side of head-major tiles
#endif
#ifndef KVX_HM_T4_UNITS
#define KVX_HM_T4_UNITS 8      // 4x4 blocks (4 KiB each) in flight per wave, head-major pages
#endif
#ifndef KVX_HM_LDS_SLICE
#define KVX_HM_LDS_SLICE 8192  // LDS bytes per wave, head-major rows staged through LDS (hm_lds_ok)
#endif
#ifndef KVX_HM_PAGE_SLICE
#define KVX_HM_PAGE_SLICE 20480  // LDS bytes per wave, head-major pages of 4-byte-word rows moved whole
#endif
#ifndef KVX_HM_PAGE_GROUP
#define KVX_HM_PAGE_GROUP 8      // 16-byte vectors per lane in flight, same pages
#endif
#ifndef KVX_HM_LDS_POOL_NT
#define KVX_HM_LDS_POOL_NT 1   // nontemporal pool-side words on the LDS-staged head-major paths
#endif
#ifndef KVX_HM_LDS_UNROLL
#define KVX_HM_LDS_UNROLL 8    // 4-byte words per lane in flight, same pages
#endif
#ifndef KVX_TAIL_GROUP
#define KVX_TAIL_GROUP 4       // vectors per lane per group after the full groups
#endif
// Cache-policy bits of a gfx950 buffer load/store (the builtin's last argument).
#define KVX_POL_SC0 1
#define KVX_POL_NT 2
#define KVX_POL_SC1 16
#ifndef KVX_GATHER_POOL_POL
#define KVX_GATHER_POOL_POL KVX_POL_NT                   // gather's loads of pool pages
#endif
#ifndef KVX_SCATTER_SMALL_PART
#define KVX_SCATTER_SMALL_PART 4096    // scatter parts of 20-64 KiB tiles (part_bytes_for)
#endif
#ifndef KVX_GATHER_FIXED_PART
#define KVX_GATHER_FIXED_PART 4096     // gather parts of 20-64 KiB tiles that are not powers of two
#endif
#ifndef KVX_SCATTER_FIXED_PART
#define KVX_SCATTER_FIXED_PART 16384   // scatter parts of larger 16 KiB-multiple tiles
#endif
#ifndef KVX_SCATTER_POOL_POL
#define KVX_SCATTER_POOL_POL (KVX_POL_NT | KVX_POL_SC1)  // buffer-form scatter's pool stores
#endif
#ifndef KVX_GATHER_CHUNK_POL
#define KVX_GATHER_CHUNK_POL (KVX_POL_NT | KVX_POL_SC1)  // gather's stores into the chunk
#endif
// Word 3 of a raw buffer resource: 32-bit data format, no swizzle, no per-lane index
// (the setting untyped dword accesses use on gfx9-family parts).
#define KVX_BUF_WORD3 0x00020000
constexpr int kWavesPerBlock = KVX_WAVES_PER_BLOCK;
constexpr int kThreads = 64 * kWavesPerBlock;

// Per-span launch record, uploaded once per call (64 bytes: one scalar 16-dword load).
// Its alignment is that of its widest field, so the copies of it in the kernel
// arguments (Launch::inl, 8-byte aligned) are properly aligned objects.
struct alignas(8) SpanDev {
    const int32_t *table;  // device block table
    int64_t tile_begin;    // first global tile id of this span
    int64_t t_end;         // one past the last token
    int64_t slot0;         // first_chunk mod n_slots
    uint32_t first_page;   // t_begin / block_size
    uint32_t n_pages;      // pages the span touches (last may be partial)
    uint32_t ppc;          // pages per full chunk (chunk_tokens / block_size, capped at n_pages)
    uint32_t n_tc;         // token chunks of the span
    uint32_t per_lc;       // tiles per layer chunk = CL * KV * n_pages
    uint32_t per_tc;       // tiles per full token chunk = CL * KV * ppc
    uint32_t pad_[2];
};
static_assert(sizeof(SpanDev) == 64, "SpanDev must stay 64 bytes");

// Calls with at most this many span records pass them in the kernel arguments
// (Launch::inl) instead of uploading them to the device arena before the launch.
#ifndef KVX_INLINE_SPANS
#define KVX_INLINE_SPANS 16
#endif

struct Launch {
    uint8_t *const *regions;  // device array [num_layers * num_kv] of region bases
    const SpanDev *spans;     // device array [n_spans]
    uint8_t *chunk_base;      // staging base (HBM or mapped pinned host)
    int32_t *err;             // sticky device error word
    int64_t total_tiles;
    int64_t block_stride;
    int64_t slot_bytes;
    int64_t n_slots;
    int64_t tile_bytes;       // block_size * tok
    uint32_t num_blocks;
    uint32_t n_spans;
    uint32_t num_kv;
    uint32_t chunk_layers;
    uint32_t layer_begin;
    uint32_t tok;             // bytes per token per (layer, kv), multiple of 16
    uint32_t block_size;
    uint32_t layout;          // KV_LAYER_FIRST or KV_PAGE_FIRST
    uint32_t split_shift;     // each tile is copied as 2^split_shift parts by as many waves
    // head-major pools ([H][block_size][D] pages): 16-byte vectors per head row
    // (r16 = D*E/16), per block head (bs_r16 = block_size*r16), and the cursor step
    // for 64 vectors of token-major order (see HmCursor)
    uint32_t page_layout;
    uint32_t hm_heads;
    uint32_t hm_r16;
    uint32_t hm_bs_r16;
    uint32_t hm_dq, hm_dh, hm_dj;
    uint32_t cached;       // 1: plain cached loads and stores (KV_FLAG_CACHED), else nontemporal
    uint32_t seg_bytes;    // > 0: gather in segments of this many bytes (gather_seg_bytes)
    uint32_t hm_t4;        // 1: head-major pages moved in 4-token x 4-head blocks (hm_t4_ok)
    // head-major pages whose rows are staged through LDS (hm_lds_ok): row
    // bytes, 4-byte words per row, tokens per LDS slab (hm_lds_tokens), and the
    // multipliers (magic_u16) that divide by hm_rd and by hm_tj * hm_rd
    uint32_t hm_lds;
    uint32_t hm_row;
    uint32_t hm_rd;
    uint32_t hm_tj;
    uint64_t hm_m_rd;
    uint64_t hm_m_run;
    // where a slab of all heads cannot keep a direction's writes whole lines
    // (hm_lds_head_slab), that direction's slabs of hg heads x tj tokens (hg == 0: the
    // token slabs above), with multipliers dividing by tj * hm_rd and by hg * hm_rd;
    // index 0 gather, 1 scatter
    uint32_t hm_hg[2];
    uint32_t hm_htj[2];
    uint64_t hm_m_hrun[2];
    uint64_t hm_m_hgrp[2];
    // head-major pages of 4-byte-word rows moved a whole page at a time (hm_page_ok), with
    // the multiplier dividing by the words of one head's page (block_size * hm_rd)
    uint32_t hm_page;
    // > 0: each tile is copied as parts of this many bytes (the last one shorter) by as
    // many waves, instead of 2^split_shift equal parts (part_bytes_for)
    uint32_t part_bytes;
    uint64_t hm_m_brd;
    // 1: the workgroups hand each XCD a contiguous eighth of the work items
    // (launch_block, xcd_remap_for)
    uint32_t xcd_remap;
    // 1: token-major scatter tiles split between waves go through buffer instructions,
    // the pool stores with nt + sc1 (scatter_buffer_form; chooses the kernel, host only)
    uint32_t scatter_buf;
    // the span records themselves when n_spans <= KVX_INLINE_SPANS (spans is then
    // unused): 64-byte SpanDev images, read by the kernel from its argument memory
    uint64_t inl[KVX_INLINE_SPANS * sizeof(SpanDev) / sizeof(uint64_t)];
};
static_assert(offsetof(Launch, inl) % alignof(SpanDev) == 0, "inline span records must be aligned SpanDev objects");

// The static device scratch of kv_transfer_chunks_noalloc (kvxfer_kernels.hip):
//   [0, 256)                 a sink for the error bits when the caller passes no error word
//   [KVX_SCR_REGIONS_OFF, +8 * KVX_SCR_MAX_REGIONS)   the call's region table
//   [KVX_SCR_RECORDS_OFF, +64 * KV_MAX_SPANS)         the call's span records (when more
//                                                     than KVX_INLINE_SPANS)
#define KVX_SCR_MAX_REGIONS 1024
#define KVX_SCR_REGIONS_OFF 256
#define KVX_SCR_RECORDS_OFF (KVX_SCR_REGIONS_OFF + 8 * KVX_SCR_MAX_REGIONS)
#define KVX_SCR_BYTES (KVX_SCR_RECORDS_OFF + 64 * KV_MAX_SPANS)
#define KVX_MAX_DEVICES 64

// Kernel-internal page layout values: head-major pages staged through LDS in token
// slabs, in head-group slabs (hm_lds_head_slab), and a whole page at a time (hm_page_ok);
// token-major pages whose split scatter tiles go through buffer instructions
// (scatter_buffer_form), whose tiles go in fixed-size parts (part_bytes_for), and both
// (scatter only).
#define KVX_PAGE_HM_LDS 2
#define KVX_PAGE_HM_LDS_HEADS 3
#define KVX_PAGE_HM_LDS_PAGE 4
#define KVX_PAGE_TM_SCATTER_BUF 5
#define KVX_PAGE_TM_FIXED 6
#define KVX_PAGE_TM_SCATTER_FIXED_BUF 7

// Position of a 16-byte vector of a tile in token-major order -- token j, head h,
// vector q of that head's row -- and its offset (in vectors) inside a head-major
// pool block, [H][block_size][r16].  advance() moves 64 vectors on (one wave
// instruction's worth); each of q and h carries at most once.
struct HmCursor {
    uint32_t j, h, q;
    __host__ __device__ void init(uint32_t v, const Launch &a)
    {
        const uint32_t per_tok = a.hm_heads * a.hm_r16;
        j = v / per_tok;
        const uint32_t rem = v - j * per_tok;
        h = rem / a.hm_r16;
        q = rem - h * a.hm_r16;
    }
    __host__ __device__ uint32_t pool_vec(const Launch &a) const
    {
        return h * a.hm_bs_r16 + j * a.hm_r16 + q;
    }
    __host__ __device__ void advance(const Launch &a)
    {
        q += a.hm_dq;
        if (q >= a.hm_r16) {
            q -= a.hm_r16;
            ++h;
        }
        h += a.hm_dh;
        if (h >= a.hm_heads) {
            h -= a.hm_heads;
            ++j;
        }
        j += a.hm_dj;
    }
};

// Where one tile's bytes live, before the block-table lookup.
struct TileRef {
    uint32_t page;      // index into the span's block table
    uint32_t region;    // layer * num_kv + kv
    uint32_t nbytes;    // n_tok * tok, a multiple of 16
    int64_t chunk_off;  // byte offset of the tile from chunk_base
};

__host__ __device__ inline int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }
__host__ __device__ inline uint32_t min32(uint32_t a, uint32_t b) { return a < b ? a : b; }

// The last span whose first tile is <= tile, searching [lo, n).  Spans is any
// pointer-like type (a constant-space pointer on the device, a plain one on the host).
template <typename SpanPtr>
__host__ __device__ inline uint32_t find_span(SpanPtr spans, uint32_t lo, uint32_t n, int64_t tile)
{
    uint32_t hi = n - 1;
    while (lo < hi) {
        const uint32_t mid = (lo + hi + 1) >> 1;
        if (spans[mid].tile_begin <= tile) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// Decompose a tile of span sp into its page, region, length and chunk offset.
template <int LAYOUT>
__host__ __device__ inline TileRef resolve_tile(const Launch &a, const SpanDev &sp, int64_t tile)
{
    uint32_t r = (uint32_t)(tile - sp.tile_begin);
    const uint32_t lc = r / sp.per_lc;
    r -= lc * sp.per_lc;
    const uint32_t tc = r / sp.per_tc;
    r -= tc * sp.per_tc;
    const uint32_t pages_here = min32(sp.ppc, sp.n_pages - tc * sp.ppc);
    uint32_t li, kv, pi;
    if (LAYOUT == KV_LAYER_FIRST) {  // [CL][KV][pages]
        pi = r % pages_here;
        const uint32_t q = r / pages_here;
        kv = q % a.num_kv;
        li = q / a.num_kv;
    } else {                          // [pages][CL][KV]
        kv = r % a.num_kv;
        const uint32_t q = r / a.num_kv;
        li = q % a.chunk_layers;
        pi = q / a.chunk_layers;
    }
    TileRef t;
    t.page = sp.first_page + tc * sp.ppc + pi;
    t.region = (a.layer_begin + lc * a.chunk_layers + li) * a.num_kv + kv;
    const int64_t first_tok = (int64_t)t.page * a.block_size;
    t.nbytes = (uint32_t)min64((int64_t)a.block_size, sp.t_end - first_tok) * a.tok;

    int64_t slot = sp.slot0 + (int64_t)lc * sp.n_tc + tc;
    if (slot >= a.n_slots) slot -= a.n_slots;
    int64_t coff;
    if (LAYOUT == KV_LAYER_FIRST) {
        const int64_t chunk_tok0 = ((int64_t)sp.first_page + (int64_t)tc * sp.ppc) * a.block_size;
        const int64_t t_c = min64((int64_t)sp.ppc * a.block_size, sp.t_end - chunk_tok0);
        coff = ((int64_t)(li * a.num_kv + kv) * t_c + (int64_t)pi * a.block_size) * a.tok;
    } else {
        coff = ((int64_t)(pi * a.chunk_layers + li) * a.num_kv + kv) * a.tile_bytes;
    }
    t.chunk_off = slot * a.slot_bytes + coff;
    return t;
}

// log2 of the parts a tile of tile_bytes is split into for direction dir.
__host__ __device__ constexpr uint32_t split_shift_for(int dir, int64_t tile_bytes)
{
    const int64_t part = dir == KV_GATHER ? KVX_GATHER_PART_BYTES : KVX_SCATTER_PART_BYTES;
    const int64_t min_tile = dir == KV_GATHER ? KVX_GATHER_SPLIT_MIN : KVX_SCATTER_SPLIT_MIN;
    uint32_t sh = 0;
    if (part > 0 && tile_bytes >= min_tile)
        while (sh < KVX_MAX_SPLIT_SHIFT && tile_bytes >= (part << (sh + 1))) ++sh;
    return sh;
}

// log2 of the parts each tile of a prepared call is split into for direction dir: a
// head-major page moved whole through one wave's slice (hm_page) is never split,
// scatters of 4 x 4-transposed pages of KVX_HM_T4_SCATTER_SPLIT_MIN bytes to under twice
// that go in 8 (ranges of 4 KiB blocks), other LDS-staged head-major pages of KVX_HM_LDS_SPLIT_MIN
// bytes or more in 4 (ranges of slabs), small token-major tiles follow the SMALL_* rule,
// the rest split_shift_for.
__host__ __device__ inline uint32_t launch_split_shift(const Launch &a, int dir)
{
    if (a.hm_page) return 0u;
    if (a.hm_t4 && dir == KV_SCATTER && a.tile_bytes >= KVX_HM_T4_SCATTER_SPLIT_MIN &&
        a.tile_bytes < 2 * KVX_HM_T4_SCATTER_SPLIT_MIN)
        return KVX_HM_T4_SCATTER_SHIFT;
    if (a.hm_lds && a.tile_bytes >= KVX_HM_LDS_SPLIT_MIN) return KVX_MAX_SPLIT_SHIFT;
    const int64_t small_max = dir == KV_GATHER ? KVX_SMALL_GATHER_MAX : KVX_SMALL_SCATTER_MAX;
    if (a.page_layout == KV_PAGE_TOKEN_MAJOR && a.tile_bytes >= KVX_SMALL_SPLIT_MIN && a.tile_bytes < small_max) {
        uint32_t sh = 0;
        while (sh < KVX_MAX_SPLIT_SHIFT && a.tile_bytes >= ((int64_t)KVX_SMALL_PART << (sh + 1))) ++sh;
        return sh;
    }
    return split_shift_for(dir, a.tile_bytes);
}

// Head-major pages whose head rows are 256 bytes (16 vectors, one 16-lane row of a
// wave) with heads and page tokens in multiples of 4 are moved in blocks of 4 tokens x
// 4 heads: four 1 KiB accesses on each side, transposed in registers in between.
__host__ __device__ constexpr bool hm_t4_ok(uint32_t page_layout, uint32_t r16, uint32_t heads,
                                            uint32_t block_size)
{
    return page_layout == KV_PAGE_HEAD_MAJOR && r16 == 16 && heads % 4 == 0 && block_size % 4 == 0;
}

// Blocks of a head-major tile of n_tok tokens: (token group, head group) pairs,
// token-group major.
__host__ __device__ inline uint32_t hm_t4_units(uint32_t n_tok, uint32_t heads)
{
    return ((n_tok + 3) / 4) * (heads / 4);
}

// Head-major pages whose head rows (row = D*E bytes) are not whole 16-byte vectors, or
// are whole vectors but shorter than the 256 bytes of the 4 x 4 register transpose, go
// through a per-wave LDS slice in slabs of whole tokens: rows must be whole 4-byte words
// and one token (all heads) must fit the slice.  For rows of whole vectors the slabs
// replace the per-lane cursor walk (copy_head_major), which measured on MI355X slower
// on almost every such shape: 8 heads x 64-byte rows gather 66 -> 73 %, 8 heads x
// 80-224-byte rows gather +2 to +9 and scatter +15 to +27 points, 16 heads x 32- or
// 64-byte rows scatter +13 to +17; only 128-byte rows in 16-32 KiB pages lose 1-2
// points.  Rows of whole vectors with a token larger than the slice keep the cursor walk.
__host__ __device__ constexpr bool hm_lds_ok(uint32_t page_layout, int64_t row, int64_t tok)
{
    return page_layout == KV_PAGE_HEAD_MAJOR && (row % 16 != 0 || row < 256) && row % 4 == 0 &&
           tok <= KVX_HM_LDS_SLICE;
}

// Whether a head-major pool's pages go through the LDS slabs: the rows hm_lds_ok names,
// and also longer rows of whole vectors (other than the 4 x 4 register-transpose case)
// when the whole page fits one slab: measured on MI355X, 8 KiB pages of 2 x 256-byte or
// 1 x 512-byte rows gather 67 -> 73-74 % that way (scatter -0.7), while 4 and 12 KiB
// pages stay within 1.5 points either way and larger ones lose up to 2.
__host__ __device__ constexpr bool hm_lds_use(uint32_t page_layout, int64_t row, int64_t tok, int64_t tile,
                                              uint32_t heads, uint32_t block_size)
{
    return hm_lds_ok(page_layout, row, tok) ||
           (page_layout == KV_PAGE_HEAD_MAJOR && row % 16 == 0 && tile <= KVX_HM_LDS_SLICE &&
            !hm_t4_ok(page_layout, (uint32_t)(row / 16), heads, block_size));
}

// Head-major pages of LDS-staged rows (hm_lds_ok) whose page is larger than a token slab's slice
// but fits a page slice are moved a whole page at a time: the block is one contiguous
// run of tile_bytes, read or written in 16-byte vectors, and transposed in LDS; so no
// pool line is split between slabs.
__host__ __device__ constexpr bool hm_page_ok(uint32_t page_layout, int64_t row, int64_t tok, int64_t tile)
{
    return hm_lds_ok(page_layout, row, tok) && tile > KVX_HM_LDS_SLICE && tile <= KVX_HM_PAGE_SLICE;
}

// Tokens per LDS slab (a slab is all heads of whole tokens: one contiguous run of the
// chunk, and one run of tj rows per head in the pool block).  As many as the slice
// holds, at most a page; when a slab is less than a page, a multiple of the tokens that
// make a head's run whole 128-byte lines (128 / gcd(row, 128)) if one fits, so no slab
// boundary splits a pool line between two slabs.
__host__ __device__ inline uint32_t hm_lds_tokens(int64_t row, int64_t tok, uint32_t block_size)
{
    const int64_t fit = KVX_HM_LDS_SLICE / tok;
    if (fit >= block_size) return block_size;
    int64_t g = 128, r = row;
    while (r) {
        const int64_t t = g % r;
        g = r;
        r = t;
    }
    const int64_t q = 128 / g;
    return (uint32_t)(fit >= q ? fit - fit % q : fit);
}

// Each direction's slabs should write whole 128-byte lines.  A token slab
// (hm_lds_tokens) writes the chunk in one contiguous run, so gather's writes are whole
// lines, but it covers whole pool lines only when it is a page or its head runs are
// whole lines; otherwise each pool line is split between slabs.  Scatter (which
// writes the pool) then takes slabs of whole pages of a group of heads, one contiguous
// run of the block: the largest divisor of H whose pages fit (all groups equal), or,
// when one head's page does not fit, one head and as many tokens as fit, cut to whole
// lines where possible.  Gather (which then reads split lines twice) takes head-group
// slabs only where their chunk runs, hg*row bytes of each token, are whole lines.
// *hg = 0: keep the token slabs.
__host__ __device__ inline void hm_lds_head_slab(int dir, uint32_t heads, int64_t row, int64_t tok,
                                                 uint32_t block_size, uint32_t *hg, uint32_t *tj)
{
    const uint32_t t0 = hm_lds_tokens(row, tok, block_size);
    *hg = 0;
    *tj = t0;
    if (t0 == block_size || (t0 * row) % 128 == 0) return;
    const int64_t cap = KVX_HM_LDS_SLICE, page_run = (int64_t)block_size * row;
    if (dir == KV_GATHER) {
        if (page_run > cap || tok % 128) return;
        for (uint32_t g = (uint32_t)(cap / page_run < heads ? cap / page_run : heads); g >= 1; --g)
            if (heads % g == 0 && (g * row) % 128 == 0) {
                *hg = g;
                *tj = block_size;
                return;
            }
        return;
    }
    if (page_run <= cap) {
        uint32_t g = (uint32_t)(cap / page_run < heads ? cap / page_run : heads);
        while (heads % g) --g;
        *hg = g;
        *tj = block_size;
    } else {
        *hg = 1;
        *tj = hm_lds_tokens(row, row, block_size);  // tokens of one head that fit
    }
}

// Slabs of a tile of n_tok tokens in head-group slabs: groups x token ranges.
__host__ __device__ inline uint32_t hm_lds_slabs(uint32_t n_tok, uint32_t heads, uint32_t hg, uint32_t tj)
{
    return (heads / hg) * ((n_tok + tj - 1) / tj);
}

// Division by a constant d in [1, 2^16] as a multiply: with m = ceil(2^32 / d),
// (n * m) >> 32 == n / d for every n < 2^16 (m*d - 2^32 < d, so the error term
// n*(m*d - 2^32) / (d*2^32) stays below 1/d, less than the gap from n/d's fraction
// to the next integer).
__host__ __device__ constexpr uint64_t magic_u16(uint32_t d)
{
    return ((1ull << 32) + d - 1) / d;
}
__host__ __device__ inline uint32_t mdiv(uint32_t n, uint64_t m)
{
    return (uint32_t)(((uint64_t)n * m) >> 32);
}

// Slice words of the four 4-byte words of pool vector v of a head-major page moved whole
// (hm_page_ok), ~0u for a word of a token at or past n_tok.  Pool word w = (h*bs + j)*rd
// + q of the block [H][bs][rd] goes to slice word (j*H + h)*rd + q of the tile in chunk
// order [n_tok][H][rd]; the first word's h = w / (bs*rd) and j = (w - h*bs*rd) / rd are
// multiply-high divisions (magic_u16: exact, as w < 2^16), the next three follow by
// carrying q into j and j into h.
__host__ __device__ inline void hm_page_slice_words(const Launch &a, uint32_t v, uint32_t n_tok, uint32_t sw[4])
{
    const uint32_t H = a.hm_heads, rd = a.hm_rd, bs = a.block_size, brd = bs * rd;
    const uint32_t w = 4u * v;
    uint32_t h = mdiv(w, a.hm_m_brd);
    const uint32_t r = w - h * brd;
    uint32_t j = mdiv(r, a.hm_m_rd);
    uint32_t q = r - j * rd;
    for (int c = 0; c < 4; ++c) {
        sw[c] = j < n_tok ? (j * H + h) * rd + q : ~0u;
        if (++q == rd) {
            q = 0;
            if (++j == bs) {
                j = 0;
                ++h;
            }
        }
    }
}

// The gfx950 dispatcher hands a launch's workgroups to its 8 XCDs round robin
// (workgroup b to XCD b % 8).  With remap, workgroup b instead takes the work of
// workgroup (b % 8) * (G8 / 8) + b / 8, G8 = G rounded down to a multiple of 8 (the last
// G % 8 keep their own): each XCD then walks one contiguous eighth of the items instead
// of every eighth workgroup's share.  A permutation of [0, G), so every item is still
// taken exactly once.
__host__ __device__ constexpr uint32_t launch_block(uint32_t b, uint32_t G, uint32_t remap)
{
    return (remap == 0u || b >= (G & ~7u)) ? b : (b & 7u) * ((G & ~7u) >> 3) + (b >> 3);
}

// Whether a launch remaps its workgroups (launch_block), with the staging in HBM:
//  * gathers of tiles walked whole or in parts (not the segment walk), token-major tiles
//    of at least KVX_XCD_REMAP_MIN bytes or head-major pages through the 4 x 4 register
//    transpose.  Measured on MI355X, in interleaved rounds in two processes each: gathers
//    of 8, 32 and 64 KiB token-major tiles and of 32 KiB head-major pages of 256-byte rows
//    gain 0.8-2.4 points of HBM peak; 4 KiB tiles lose 2.5 and the LDS-staged head-major
//    pages 2-3.5, so those keep the plain order;
//  * scatters in 4 KiB parts: 20-56 KiB tiles +2.2 to +6.1 points, the MLA latent's 36 KiB
//    +2.8 to +3.0, page-first 32 KiB +3.6, but 32 KiB tiles with layer-first chunks -0.6
//    to -1.5, which keep the plain order (as do whole and 2^k-part scatter tiles, which
//    show no consistent direction).
#ifndef KVX_XCD_REMAP_MIN
#define KVX_XCD_REMAP_MIN 8192
#endif
__host__ __device__ inline uint32_t xcd_remap_for(int dir, const Launch &a, bool host_staging)
{
    if (dir == KV_SCATTER) {
        // scatters in 4 KiB parts (part_bytes_for), except power-of-two tiles (32 KiB:
        // whole workgroups per tile) with layer-first chunks
        const bool pow2 = (a.tile_bytes & (a.tile_bytes - 1)) == 0;
        return (!host_staging && a.part_bytes == KVX_SCATTER_SMALL_PART && !(pow2 && a.layout == KV_LAYER_FIRST))
                   ? 1u
                   : 0u;
    }
    if (host_staging || a.seg_bytes || a.hm_lds) return 0u;
    if (a.page_layout == KV_PAGE_TOKEN_MAJOR) return a.tile_bytes >= KVX_XCD_REMAP_MIN ? 1u : 0u;
    return a.hm_t4 ? 1u : 0u;
}

// Whether a scatter's token-major tiles go through buffer instructions, the pool stores
// with nt + sc1 (KVX_SCATTER_POOL_POL), instead of global instructions with plain nt:
// tiles split between waves in 2^k parts (8 to under 20 KiB, and from 64 KiB) or in
// 4 KiB parts (part_bytes_for), with the staging in HBM.  Measured on MI355X,
// interleaved rounds in two processes each: the int8_kv scatter (64 KiB tiles, 4 parts)
// gains 4.0-5.4 points of HBM peak, mixed (64 KiB) 0.7-1.0, the TP-2 shard (16 KiB)
// 0.4-0.6, the TP-4 shard (8 KiB) -0.4 to +0.1, and 32 KiB tiles in 4 KiB parts 0.5-0.8
// more than in the global form; whole 32 KiB tiles lose 0.6-0.9, and 16 KiB parts of
// larger tiles do better in the global form.
__host__ __device__ inline uint32_t scatter_buffer_form(int dir, const Launch &a, bool host_staging)
{
    const bool split = a.split_shift > 0 || (a.part_bytes > 0 && a.part_bytes < KVX_SCATTER_FIXED_PART);
    return (dir == KV_SCATTER && a.page_layout == KV_PAGE_TOKEN_MAJOR && split && !host_staging) ? 1u : 0u;
}

// Fixed-size parts for token-major tiles with HBM staging (0: the split_shift rule and,
// for gathers, the segment walk), each part starting at a multiple of its size within
// the tile and copied by its own wave, neighbouring waves taking one tile's parts:
//  * gathers of tiles of 20 KiB to under 64 KiB that are not powers of two: 4 KiB parts
//    (KVX_GATHER_FIXED_PART), in the per-XCD order (xcd_remap_for), instead of the 32 KiB
//    segment walk.  Measured on MI355X in interleaved rounds, two processes: the MLA
//    latent's 36 KiB tiles +3.5 to +3.9 points of HBM peak (71.4 -> 75.3 %), 20-56 KiB
//    tiles with layer-first chunks +1.9 to +4.9, page-first 36 KiB +4.1, page-first 24 and
//    48 KiB -0.8 to 0; 12 KiB parts lose 2, and 32 KiB tiles keep whole (in 4, 8 or 16 KiB
//    parts: -2.4 to -6.6).  Scatters:
//  * tiles of 20 KiB (where the small-tile split ends, KVX_SMALL_SCATTER_MAX) to less
//    than 64 KiB: 4 KiB parts (KVX_SCATTER_SMALL_PART), in the buffer form
//    (scatter_buffer_form).  Measured on MI355X in interleaved rounds, shuffled tables:
//    20-60 KiB tiles +0.6 to +3.7 points of HBM peak against whole tiles, the llama8b
//    call's 32 KiB tiles +1.9 to +3.9 (in a 32 GiB pool; +0.9 in a 16 GiB one, none in an
//    8 GiB one), the MLA latent's 36 KiB tiles +1.4 to +3.1; 32 KiB tiles in 8 KiB parts
//    lose 2, in 2 KiB parts 0.6, 18 KiB tiles 1.1 against their 4 equal parts, and 64 KiB
//    or larger tiles in 4 KiB parts lose 1-8.  Pages in runs of adjacent blocks scatter
//    faster whole (74-77 % against 71-72 % for 32 KiB tiles), which the kernel cannot see
//    from the launch: page_runs (KV_FLAG_PAGE_RUNS, the caller's hint) keeps such tiles
//    whole.
//  * larger tiles that are whole multiples of 16 KiB but not powers of two: 16 KiB parts
//    (KVX_SCATTER_FIXED_PART) in the global form: 80, 96 and 144 KiB tiles +2.3 to +6.5
//    points against 4 equal parts.
__host__ __device__ inline uint32_t part_bytes_for(int dir, const Launch &a, bool host_staging, bool page_runs)
{
    const int64_t T = a.tile_bytes;
    if (a.page_layout != KV_PAGE_TOKEN_MAJOR || host_staging) return 0u;
    if (dir == KV_GATHER)
        return (T >= 20480 && T < 65536 && (T & (T - 1)) != 0) ? (uint32_t)KVX_GATHER_FIXED_PART : 0u;
    if (T >= KVX_SMALL_SCATTER_MAX && T < 65536) return page_runs ? 0u : (uint32_t)KVX_SCATTER_SMALL_PART;
    if (T >= 65536 && T % KVX_SCATTER_FIXED_PART == 0 && (T & (T - 1)) != 0) return (uint32_t)KVX_SCATTER_FIXED_PART;
    return 0u;
}

// Segment size for a gather over tiles of tile_bytes (0: one tile per wave item).
__host__ __device__ constexpr uint32_t gather_seg_bytes(int dir, uint32_t page_layout, int64_t tile_bytes)
{
    return (dir == KV_GATHER && page_layout == KV_PAGE_TOKEN_MAJOR && KVX_GATHER_SEG_BYTES > 0 &&
            tile_bytes >= KVX_GATHER_SEG_MIN &&
            ((tile_bytes & (tile_bytes - 1)) != 0 || tile_bytes < KVX_GATHER_SEG_BYTES))
               ? (uint32_t)KVX_GATHER_SEG_BYTES
               : 0u;
}

// Vectors per lane per group of the segment walk: the pieces a segment cuts from the
// tiles are multiples of gcd(tile_bytes, seg_bytes), and groups that divide them keep
// every piece in whole pipelined groups (a 4 KiB piece in 8 KiB groups is a tail copy
// without overlap): 8 (8 KiB) when that gcd allows, else 4, else 2.
__host__ __device__ inline int gather_seg_unroll(int64_t tile_bytes, int64_t seg_bytes)
{
    int64_t g = seg_bytes, r = tile_bytes;
    while (r) {
        const int64_t t = g % r;
        g = r;
        r = t;
    }
    return g % 8192 == 0 ? 8 : g % 4096 == 0 ? 4 : 2;
}

// Parts of each tile in the tile walk: part_bytes-sized parts, or 2^split_shift.
__host__ __device__ inline int64_t parts_per_tile(const Launch &a)
{
    return a.part_bytes ? (a.tile_bytes + a.part_bytes - 1) / a.part_bytes : (int64_t)1 << a.split_shift;
}

// Work items of a call: segments of the tiles laid end to end at a tile_bytes pitch,
// or tiles times their parts.
__host__ __device__ inline int64_t work_items(const Launch &a)
{
    return a.seg_bytes ? (a.total_tiles * a.tile_bytes + a.seg_bytes - 1) / a.seg_bytes
                       : a.total_tiles * parts_per_tile(a);
}

// The piece [lo, hi) of tile `tile` (bytes from the tile's start) that segment
// [x0, x1) of the end-to-end stream covers; hi <= lo when none.  Tiles shorter than
// tile_bytes (a partial last page) simply end early.
__host__ __device__ inline void segment_piece(int64_t tile, int64_t tile_bytes, uint32_t nbytes, int64_t x0,
                                              int64_t x1, int64_t *lo, int64_t *hi)
{
    const int64_t base = tile * tile_bytes;
    const int64_t end = base + (int64_t)nbytes;
    *lo = (x0 > base ? x0 : base) - base;
    *hi = (x1 < end ? x1 : end) - base;
}

// Part `part` of `split` near-equal parts of nvec 16-byte vectors.
__host__ __device__ inline void part_range(uint32_t nvec, uint32_t part, uint32_t split,
                                           uint32_t *first, uint32_t *count)
{
    const uint32_t lo = (uint32_t)((uint64_t)nvec * part / split);
    const uint32_t hi = (uint32_t)((uint64_t)nvec * (part + 1) / split);
    *first = lo;
    *count = hi - lo;
}

// The vectors [first, first + count) of a token-major tile of nvec vectors that work
// item part `part` copies: a part_bytes-sized part (empty past a partial tile's end),
// or one of the 2^split_shift near-equal parts.
__host__ __device__ inline void tile_part(const Launch &a, uint32_t nvec, uint32_t part, uint32_t *first,
                                          uint32_t *count)
{
    if (a.part_bytes) {
        const uint32_t pv = a.part_bytes >> 4, lo = part * pv;
        *first = lo < nvec ? lo : nvec;
        *count = (lo + pv < nvec ? lo + pv : nvec) - *first;
        return;
    }
    part_range(nvec, part, 1u << a.split_shift, first, count);
}

// Host: validate a call and fill the launch descriptor (all fields but regions,
// spans and err, which hold device addresses) and the span records (records has
// room for KV_MAX_SPANS).  *n_records receives the number of non-empty spans.
int prepare_call(const kv_pool_desc *d, const kv_span *spans, int32_t n_spans,
                 const kv_chunk_spec *spec, SpanDev *records, uint32_t *n_records, Launch *launch,
                 kv_transfer_info *info);

// Kernel launch (kernel file); returns a hipError_t value.
int launch_tile_copy(int direction, const Launch &a, uint32_t grid, hipStream_t stream);

// Default grid for a call of `items` work items (tiles x parts).
uint32_t default_grid(int64_t items);

// Device address of the static scratch on `device` (which must be current), looked up
// once per device; nullptr with *hip_error set if the lookup fails (kernel file).
void *scratch_address(int device, int *hip_error);

}  // namespace kvx
