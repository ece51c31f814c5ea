// kvxfer_kernels.hip -- the gather/scatter tile-copy kernel for gfx950.
//
// One 64-lane wavefront copies one (layer, kv, page) tile -- or one part of a tile
// split between waves (8-20 KiB tiles, scatter tiles of 20 KiB or more, gather tiles of
// 64 KiB or more), or, for a gather over token-major tiles of 16 KiB or more that are
// not whole 32 KiB segments, one 32 KiB segment of the tiles laid end to end -- per
// iteration of a grid-stride loop.  Per
// tile it
//   1. finds the span (binary search over the per-span tile prefix, wave-uniform,
//      so it runs on the scalar unit with scalar loads),
//   2. splits the local tile index into (layer chunk, token chunk, layer, kv, page)
//      in chunk order and loads the block id from the block table once,
//   3. forms both byte addresses -- the layout transform is this address choice
//      (Strata guide, "Two-Dimensional Memory Layout Decoupling"), and
//   4. copies the tile's n_tok*tok contiguous bytes with 16-byte vector loads and
//      stores, 64 lanes x 16 B = 1 KiB per wave instruction, 8-16 vectors in flight
//      per lane, nontemporal on both sides unless the call asks for cached accesses
//      (KV_FLAG_CACHED) (the Strata guide's reload kernel uses
//      cache-streaming stores so a transfer does not evict the working set of
//      concurrent compute kernels: "Non-Intrusive Resource Sizing").  Gather goes
//      through buffer instructions so that its sequential chunk stores can also
//      carry the sc1 bit; scatter through global instructions, except tiles split
//      between waves, whose pool stores carry nt + sc1 through buffer instructions
//      (scatter_buffer_form).
// Gathers of tiles walked whole or in parts hand each XCD a contiguous stretch of the
// work items (launch_block, xcd_remap_for).
// No matrix instructions, and LDS only for head-major pages whose head rows are not
// whole 16-byte vectors (copy_head_major_lds): it is a pure byte copy, bound by HBM
// (both sides in HBM) or by the host link (chunks in pinned host memory).
//
// A block id outside [0, num_blocks) is not followed: lane 0 sets the sticky
// error bit and the wave skips that tile.  All offsets are 64-bit (the printed
// kernel's 32-bit linear index would overflow past 2^31 16-byte items, which a
// 128K-token 70B-shaped transfer exceeds).
#include <hip/hip_runtime.h>

#include <atomic>

#include "kvxfer.h"
#include "kvxfer_internal.h"

// Device memory of kv_transfer_chunks_noalloc, for callers that cannot allocate: the
// region table and span records of one call (layout in kvxfer_internal.h, KVX_SCR_*).
// Each device the library runs on holds its own copy until the process ends; host code
// reaches it only through the address scratch_address() looked up on that device.
static __device__ __align__(256) uint8_t scratch[KVX_SCR_BYTES];

namespace kvx {

void *scratch_address(int device, int *hip_error)
{
    static std::atomic<void *> addr[KVX_MAX_DEVICES];
    if (device < 0 || device >= KVX_MAX_DEVICES) {
        *hip_error = (int)hipErrorInvalidDevice;
        return nullptr;
    }
    void *p = addr[device].load(std::memory_order_acquire);
    if (p) return p;
    // the caller has made `device` current; the symbol resolves to that device's copy
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
        *hip_error = (int)(e != hipSuccess ? e : hipErrorInvalidSymbol);
        (void)hipGetLastError();
        return nullptr;
    }
    addr[device].store(p, std::memory_order_release);
    return p;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Address-space views.  Pointers read out of memory are "generic" to the compiler,
// which then emits flat instructions; the tile data always lives in global memory
// (HBM or mapped host memory), so it is accessed through the global space.  The
// span records, region table and block tables are not written while the kernel
// runs, and a wave reads them at uniform addresses, so they are read through the
// constant space, which lets the compiler use scalar loads.
#define KVX_GLOBAL __attribute__((address_space(1)))
#define KVX_CONST __attribute__((address_space(4)))
typedef KVX_GLOBAL u32x4 gvec;

template <typename T>
__device__ __forceinline__ const KVX_CONST T *as_const(const T *p)
{
    return (const KVX_CONST T *)p;
}
__device__ __forceinline__ gvec *as_global(uint8_t *p) { return (gvec *)p; }

// The call's span records: in the kernel's own argument memory for calls with at
// most KVX_INLINE_SPANS of them (Launch::inl, at its offset in the one explicit
// argument), else in the pool's device arena.  Either way read as constant memory.
__device__ __forceinline__ const KVX_CONST SpanDev *span_records(const Launch &a)
{
    if (a.n_spans <= KVX_INLINE_SPANS)
        return (const KVX_CONST SpanDev *)((const KVX_CONST uint8_t *)__builtin_amdgcn_kernarg_segment_ptr() +
                                           offsetof(Launch, inl));
    return as_const(a.spans);
}

// A span record, read as one 16-dword scalar load: every field arrives with one wait,
// instead of the few separate loads (and waits) the compiler makes of field accesses.
// Measured on MI355X for the tile walk: the int8 page-first gather 73.6 -> 77.3 % of
// HBM peak (the field-by-field form put one more scalar-memory round trip before each
// tile's block-id load), other workloads within 0.3 %.
// A span record read field by field (separate scalar loads as the compiler schedules
// them).  The segment walk, which resolves one or two tile pieces per segment, keeps
// this form: measured on MI355X, the single load below costs its MLA gather 1-1.5 %.
__device__ __forceinline__ SpanDev load_span_fields(const KVX_CONST SpanDev *p)
{
    SpanDev r;
    r.table = p->table;
    r.tile_begin = p->tile_begin;
    r.t_end = p->t_end;
    r.slot0 = p->slot0;
    r.first_page = p->first_page;
    r.n_pages = p->n_pages;
    r.ppc = p->ppc;
    r.n_tc = p->n_tc;
    r.per_lc = p->per_lc;
    r.per_tc = p->per_tc;
    return r;
}
typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ SpanDev load_span(const KVX_CONST SpanDev *p)
{
    const u32x16 w = *(const KVX_CONST u32x16 *)p;
    auto u64 = [&](int i) { return (uint64_t)w[i] | ((uint64_t)w[i + 1] << 32); };
    SpanDev r;
    r.table = (const int32_t *)u64(offsetof(SpanDev, table) / 4);
    r.tile_begin = (int64_t)u64(offsetof(SpanDev, tile_begin) / 4);
    r.t_end = (int64_t)u64(offsetof(SpanDev, t_end) / 4);
    r.slot0 = (int64_t)u64(offsetof(SpanDev, slot0) / 4);
    r.first_page = w[offsetof(SpanDev, first_page) / 4];
    r.n_pages = w[offsetof(SpanDev, n_pages) / 4];
    r.ppc = w[offsetof(SpanDev, ppc) / 4];
    r.n_tc = w[offsetof(SpanDev, n_tc) / 4];
    r.per_lc = w[offsetof(SpanDev, per_lc) / 4];
    r.per_tc = w[offsetof(SpanDev, per_tc) / 4];
    return r;
}

// NT: nontemporal (the default policy) or plain cached accesses (KV_FLAG_CACHED).
template <bool NT>
__device__ __forceinline__ u32x4 ld(const gvec *p)
{
    if (NT) return __builtin_nontemporal_load(p);
    return *p;
}

template <bool NT>
__device__ __forceinline__ void st(gvec *p, u32x4 v)
{
    if (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// One side of a tile copy, addressed in 16-byte vectors from the start of its range.
// PtrSide goes through a global pointer; BufSide through a buffer resource over the
// range, which lets the instruction carry an explicit cache policy (the gfx950 buffer
// instructions' sc0 / nt / sc1 bits, KVX_POL_*) and makes the hardware drop any
// access past the range's end.
template <bool NT>
struct PtrSide {
    gvec *p;
    __device__ __forceinline__ u32x4 load(uint32_t v) const { return ld<NT>(p + v); }
    __device__ __forceinline__ void store(uint32_t v, u32x4 x) const { st<NT>(p + v, x); }
};

// Buffer-instruction policies of gather's two sides, nontemporal or cached.
template <bool NT> constexpr int kGatherPoolPol = NT ? KVX_GATHER_POOL_POL : 0;
template <bool NT> constexpr int kGatherChunkPol = NT ? KVX_GATHER_CHUNK_POL : 0;

template <int POL>
struct BufSide {
    __amdgpu_buffer_rsrc_t r;
    __device__ __forceinline__ BufSide(const uint8_t *base, uint32_t nbytes)
        : r(__builtin_amdgcn_make_buffer_rsrc((void *)base, 0, (int)nbytes, KVX_BUF_WORD3))
    {
    }
    __device__ __forceinline__ u32x4 load(uint32_t v) const
    {
        return __builtin_amdgcn_raw_buffer_load_b128(r, v * 16u, 0, POL);
    }
    __device__ __forceinline__ void store(uint32_t v, u32x4 x) const
    {
        __builtin_amdgcn_raw_buffer_store_b128(x, r, v * 16u, 0, POL);
    }
};

// The remainder after the full groups, in groups of U vectors per lane; within a
// group all loads are issued before the stores (lanes past the end are masked off).
template <int U, class S, class D>
__device__ __forceinline__ void copy_tail(const S &src, const D &dst, uint32_t nvec, uint32_t v)
{
    u32x4 r[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (v + 64u * u < nvec) r[u] = src.load(v + 64u * u);
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (v + 64u * u < nvec) dst.store(v + 64u * u, r[u]);
}

// Copy nvec 16-byte vectors; lane i handles vectors i, i+64, i+128, ...
template <int U, class S, class D>
__device__ __forceinline__ void copy_run(const S &src, const D &dst, uint32_t nvec, uint32_t lane)
{
    uint32_t v = lane;
    for (; v + 64u * (U - 1) < nvec; v += 64u * U) {
        u32x4 r[U];
#pragma unroll
        for (int u = 0; u < U; ++u) r[u] = src.load(v + 64u * u);
#pragma unroll
        for (int u = 0; u < U; ++u) dst.store(v + 64u * u, r[u]);
    }
    for (; v < nvec; v += 64u * KVX_TAIL_GROUP) copy_tail<KVX_TAIL_GROUP>(src, dst, nvec, v);
}

// Software-pipelined variant: the loads of group k+1 are issued before the stores
// of group k, so each lane keeps 2U vectors in flight.
template <int U, class S, class D>
__device__ __forceinline__ void copy_run_pipelined(const S &src, const D &dst, uint32_t nvec,
                                                   uint32_t lane)
{
    constexpr uint32_t G = 64u * U;
    uint32_t v = lane;
    if (v + G - 64u < nvec) {
        u32x4 a[U], b[U];
#pragma unroll
        for (int u = 0; u < U; ++u) a[u] = src.load(v + 64u * u);
        for (;;) {
            if (v + 2 * G - 64u >= nvec) break;
#pragma unroll
            for (int u = 0; u < U; ++u) b[u] = src.load(v + G + 64u * u);
#pragma unroll
            for (int u = 0; u < U; ++u) dst.store(v + 64u * u, a[u]);
            v += G;
            if (v + 2 * G - 64u >= nvec) {
#pragma unroll
                for (int u = 0; u < U; ++u) a[u] = b[u];
                break;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) a[u] = src.load(v + G + 64u * u);
#pragma unroll
            for (int u = 0; u < U; ++u) dst.store(v + 64u * u, b[u]);
            v += G;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) dst.store(v + 64u * u, a[u]);
        v += G;
    }
    for (; v < nvec; v += 64u * KVX_TAIL_GROUP) copy_tail<KVX_TAIL_GROUP>(src, dst, nvec, v);
}

template <int U, class S, class D>
__device__ __forceinline__ void copy_loop(const S &src, const D &dst, uint32_t nvec, uint32_t lane,
                                          bool pipelined)
{
    if (pipelined) copy_run_pipelined<U>(src, dst, nvec, lane);
    else copy_run<U>(src, dst, nvec, lane);
}

// Gather reads scattered pool pages and writes the chunk sequentially.  The chunk
// stores carry nt + sc1: measured on MI355X, sequential stores with that policy
// raise gather by 2-4 % over plain nontemporal stores (the scattered stores of
// scatter show no such gain, so scatter keeps plain nontemporal accesses).
template <bool NT, int U = KVX_GATHER_UNROLL>
__device__ __forceinline__ void gather_tile(const uint8_t *pool, uint8_t *chunk, uint32_t nvec,
                                            uint32_t lane)
{
    copy_loop<U>(BufSide<kGatherPoolPol<NT>>(pool, nvec * 16u),
                                 BufSide<kGatherChunkPol<NT>>(chunk, nvec * 16u), nvec, lane,
                                 KVX_GATHER_PIPELINE);
}

// Scatter reads the chunk sequentially and writes scattered pool pages.  The
// restrict-qualified pointers let the compiler interleave a group's stores with the
// next loads (62 VGPRs, eight waves per SIMD), which measured faster than issuing
// all sixteen loads first.
template <bool NT>
__device__ __forceinline__ void scatter_tile(const gvec *__restrict__ chunk, gvec *__restrict__ pool,
                                             uint32_t nvec, uint32_t lane)
{
    copy_loop<KVX_SCATTER_UNROLL>(PtrSide<NT>{(gvec *)chunk}, PtrSide<NT>{pool}, nvec, lane,
                                  KVX_SCATTER_PIPELINE);
}

// The same copy through buffer instructions, so the pool stores can carry sc1 as well
// as nt (KVX_SCATTER_POOL_POL); taken for tiles split between waves (scatter_buffer_form).
template <bool NT>
__device__ __forceinline__ void scatter_tile_buf(const uint8_t *chunk, const uint8_t *pool, uint32_t nvec,
                                                 uint32_t lane)
{
    copy_loop<KVX_SCATTER_UNROLL>(BufSide<NT ? KVX_POL_NT : 0>(chunk, nvec * 16u),
                                  BufSide<NT ? KVX_SCATTER_POOL_POL : 0>(pool, nvec * 16u), nvec, lane,
                                  KVX_SCATTER_PIPELINE);
}

// The permuted (pool) side of a head-major tile touches each cache line of the block
// from several wave instructions (one per token whose head row shares the line), so
// whether those accesses bypass the caches is a separate choice.
template <bool NT>
__device__ __forceinline__ u32x4 ld_hm_pool(const gvec *p)
{
    return ld<NT && KVX_HM_POOL_NT>(p);
}

template <bool NT>
__device__ __forceinline__ void st_hm_pool(gvec *p, u32x4 v)
{
    st<NT && KVX_HM_POOL_NT>(p, v);
}

// Head-major pool block against a token-major chunk tile: vectors [first, end) of
// the tile in token-major order.  The chunk side is contiguous; on the pool side each
// lane follows a cursor to its vector's place in the block's [H][bs][r16] order, so a
// wave's 1 KiB touches whole D*E-byte head rows.
template <int DIR, int U, bool NT>
__device__ __forceinline__ void copy_head_major(gvec *__restrict__ block, uint8_t *chunk_tile,
                                                uint32_t first, uint32_t end, uint32_t lane,
                                                const Launch &a)
{
    const BufSide<kGatherChunkPol<NT>> out(chunk_tile, end * 16u);
    const PtrSide<NT> in{as_global(chunk_tile)};
    HmCursor c;
    c.init(first + lane, a);
    for (uint32_t v = first + lane; v < end; v += 64u * U) {
        uint32_t pv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            pv[u] = c.pool_vec(a);
            c.advance(a);
        }
        u32x4 r[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // lanes past the end load a valid vector that is not stored (no load behind a
            // lane-dependent branch, which would wait for all earlier loads)
            const bool in_range = v + 64u * u < end;
            r[u] = DIR == KV_GATHER ? ld_hm_pool<NT>(block + (in_range ? pv[u] : 0u))
                                    : in.load(in_range ? v + 64u * u : end - 1u);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (v + 64u * u < end) {
                if (DIR == KV_GATHER) out.store(v + 64u * u, r[u]);
                else st_hm_pool<NT>(block + pv[u], r[u]);
            }
    }
}

// 4x4 transpose of 16-lane rows across four registers: on return, row r of register
// t holds what row t of register r held.  gfx950's permlane32 swap exchanges the upper
// half of one register with the lower half of another, the permlane16 swap the odd
// 16-lane rows of one with the even rows of the other; two of each per dword.
__device__ __forceinline__ void transpose_rows4(u32x4 &A, u32x4 &B, u32x4 &C, u32x4 &D)
{
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const auto ac = __builtin_amdgcn_permlane32_swap(A[c], C[c], false, false);
        const auto bd = __builtin_amdgcn_permlane32_swap(B[c], D[c], false, false);
        const auto ab = __builtin_amdgcn_permlane16_swap(ac[0], bd[0], false, false);
        const auto cd = __builtin_amdgcn_permlane16_swap(ac[1], bd[1], false, false);
        A[c] = ab[0];
        B[c] = ab[1];
        C[c] = cd[0];
        D[c] = cd[1];
    }
}

// Head-major pages with 256-byte head rows (see hm_t4_ok), blocks [u0, u1) of a tile
// of n_tok tokens; block u = (tokens j0..j0+3, heads hb..hb+3).  On the pool side the
// 4 tokens of one head are 1 KiB contiguous, lane = token*16 + vector; on the chunk
// side the 4 heads of one token are, lane = head*16 + vector; so four loads, one
// register transpose and four stores move a block with every access a whole 1 KiB.
// Chunk accesses past the tile's n_tok tokens are dropped by the buffer range (gather)
// or skipped (scatter), and so are pool writes of those tokens.
template <int DIR, bool NT>
__device__ __forceinline__ void copy_head_major_t4(const uint8_t *block, uint8_t *chunk_tile, uint32_t u0,
                                                   uint32_t u1, uint32_t n_tok, uint32_t lane,
                                                   const Launch &a)
{
    constexpr int U = KVX_HM_T4_UNITS;
    const uint32_t H = a.hm_heads, bs = a.block_size, hgroups = H / 4;
    const BufSide<kGatherPoolPol<NT>> pool_in(block, H * bs * 256u);
    const BufSide<kGatherChunkPol<NT>> chunk_out(chunk_tile, n_tok * H * 256u);
    const PtrSide<NT> chunk_in{(gvec *)chunk_tile};
    gvec *const pool_out = (gvec *)block;
    const uint32_t my_tok = lane >> 4;  // this lane's token within a block, pool side
    for (uint32_t u = u0; u < u1; u += U) {
        u32x4 x[U][4];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const uint32_t uu = u + k, j0 = (uu / hgroups) * 4, hb = (uu % hgroups) * 4;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (uu >= u1) continue;
                if (DIR == KV_GATHER) x[k][r] = pool_in.load(((hb + r) * bs + j0) * 16u + lane);
                else if (j0 + r < n_tok) x[k][r] = chunk_in.load(((j0 + r) * H + hb) * 16u + lane);
                else x[k][r] = u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int k = 0; k < U; ++k)
            if (u + k < u1) transpose_rows4(x[k][0], x[k][1], x[k][2], x[k][3]);
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const uint32_t uu = u + k, j0 = (uu / hgroups) * 4, hb = (uu % hgroups) * 4;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (uu >= u1) continue;
                if (DIR == KV_GATHER) chunk_out.store(((j0 + r) * H + hb) * 16u + lane, x[k][r]);
                else if (j0 + my_tok < n_tok) st_hm_pool<NT>(pool_out + ((hb + r) * bs + j0) * 16u + lane, x[k][r]);
            }
        }
    }
}

// 4-byte pool-side words of the LDS-staged head-major path.
typedef KVX_GLOBAL uint32_t gword;
template <bool NT>
__device__ __forceinline__ uint32_t ld_word(const gword *p)
{
    if (NT) return __builtin_nontemporal_load(p);
    return *p;
}
template <bool NT>
__device__ __forceinline__ void st_word(gword *p, uint32_t v)
{
    if (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// Pool-side words of the LDS-staged paths.  A slab boundary can split a pool line
// between two slabs of one wave, so whether those accesses bypass the caches is a
// separate choice (KVX_HM_LDS_POOL_NT).
template <bool NT>
__device__ __forceinline__ uint32_t ld_pool_word(const gword *p)
{
    return ld_word<NT && KVX_HM_LDS_POOL_NT>(p);
}
template <bool NT>
__device__ __forceinline__ void st_pool_word(gword *p, uint32_t v)
{
    st_word<NT && KVX_HM_LDS_POOL_NT>(p, v);
}

// Head-major pages staged through LDS (hm_lds_ok: rows of rd 4-byte words that are not
// whole 16-byte vectors, or are but are shorter than 256 bytes): slabs [s0, s1) of all
// heads x tj tokens (hm_lds_tokens) pass through this
// wave's LDS slice, which holds a slab in chunk (token-major) order, so the chunk side
// moves whole 16-byte vectors of the slab's contiguous run.  The pool side is the
// slab's run of tj rows in each head, moved as 4-byte words with consecutive lanes on
// consecutive words (pool order): pool word w of a slab is head h = w / (tj*rd), row
// jj and word q of i = w - h*tj*rd (jj = i / rd), at pool word (h*bs + j0)*rd + i and
// slice word (jj*H + h)*rd + q, the two divisions done as multiplies (magic_u16).
// Gather fills the slice word by word from the pool and empties it in vectors into
// the chunk; scatter the reverse.  Only this wave uses its slice and a wave's LDS
// accesses complete in order, so the phases need no barrier; wave_barrier only keeps
// the compiler from moving accesses across a phase boundary.
template <int DIR, bool NT>
__device__ __forceinline__ void copy_head_major_lds(uint32_t *lds, uint8_t *block, uint8_t *chunk_tile,
                                                    uint32_t s0, uint32_t s1, uint32_t n_tok, uint32_t lane,
                                                    const Launch &a)
{
    constexpr int U = KVX_HM_LDS_UNROLL;
    constexpr int UV = KVX_HM_LDS_SLICE / 1024;  // chunk vectors per lane in a full slab
    const uint32_t H = a.hm_heads, rd = a.hm_rd, tj = a.hm_tj, bs = a.block_size;
    const uint32_t run = tj * rd, words = H * run;
    gword *const pool = (gword *)block;
    for (uint32_t sl = s0; sl < s1; ++sl) {
        const uint32_t j0 = sl * tj;
        const uint32_t t = min32(tj, n_tok - j0);
        const uint32_t nvec = t * a.tok / 16u;
        uint8_t *const cs = chunk_tile + (uint64_t)j0 * a.tok;
        if (DIR == KV_SCATTER) {  // chunk run -> slice
            const PtrSide<NT> in{as_global(cs)};
            u32x4 x[UV];
#pragma unroll
            for (int k = 0; k < UV; ++k)
                if (lane + 64u * k < nvec) x[k] = in.load(lane + 64u * k);
#pragma unroll
            for (int k = 0; k < UV; ++k)
                if (lane + 64u * k < nvec) *(u32x4 *)(lds + 4u * (lane + 64u * k)) = x[k];
            __builtin_amdgcn_wave_barrier();
        }
        for (uint32_t w = lane; w < words; w += 64u * U) {
            uint32_t pw[U], lw[U], x[U];
            bool ok[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t ww = w + 64u * u;
                const uint32_t h = mdiv(ww, a.hm_m_run);
                const uint32_t i = ww - h * run;
                const uint32_t jj = mdiv(i, a.hm_m_rd);
                ok[u] = ww < words && jj < t;
                pw[u] = (h * bs + j0) * rd + i;
                lw[u] = (jj * H + h) * rd + (i - jj * rd);
            }
            if (DIR == KV_GATHER) {
                // every lane loads (word 0 of the block where it has nothing to move): a
                // load behind a lane-dependent branch would wait for all earlier ones
#pragma unroll
                for (int u = 0; u < U; ++u) x[u] = ld_pool_word<NT>(pool + (ok[u] ? pw[u] : 0u));
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (ok[u]) lds[lw[u]] = x[u];
            } else {
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (ok[u]) x[u] = lds[lw[u]];
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (ok[u]) st_pool_word<NT>(pool + pw[u], x[u]);
            }
        }
        __builtin_amdgcn_wave_barrier();
        if (DIR == KV_GATHER) {  // slice -> chunk run
            const BufSide<kGatherChunkPol<NT>> out(cs, nvec * 16u);
#pragma unroll
            for (int k = 0; k < UV; ++k)
                if (lane + 64u * k < nvec) out.store(lane + 64u * k, *(const u32x4 *)(lds + 4u * (lane + 64u * k)));
            __builtin_amdgcn_wave_barrier();
        }
    }
}

// Scatter of head-major rows of 4-byte words in slabs of hg heads x tj tokens
// (hm_lds_head_slab: whole pages of a head group, where a slab of all heads cannot be
// whole pool lines).  Slab sl is head group g = sl / (token ranges), token range the
// rest.  The chunk's words of the slab, hg*rd per token, are read in chunk order --
// word w is row jj = w / (hg*rd), head hh and word q of the remainder -- into the
// slice in pool order, slice word (hh*tj + jj)*rd + q; the slice is then written out
// along the pool, slice word w to pool word ((h0 + hh)*bs + j0)*rd + i with
// hh = w / (tj*rd), i = w - hh*tj*rd: one contiguous run of the block when tj = bs.
template <bool NT>
__device__ __forceinline__ void hm_lds_scatter_heads(uint32_t *lds, uint8_t *block, const uint8_t *chunk_tile,
                                                     uint32_t s0, uint32_t s1, uint32_t n_tok, uint32_t lane,
                                                     const Launch &a)
{
    constexpr int U = KVX_HM_LDS_UNROLL;
    const uint32_t H = a.hm_heads, rd = a.hm_rd, hg = a.hm_hg[1], tj = a.hm_htj[1], bs = a.block_size;
    const uint32_t run = tj * rd, grp = hg * rd, n_tr = (n_tok + tj - 1) / tj;
    gword *const pool = (gword *)block;
    const gword *const chunk = (const gword *)chunk_tile;
    for (uint32_t sl = s0; sl < s1; ++sl) {
        const uint32_t g = sl / n_tr, j0 = (sl - g * n_tr) * tj, h0 = g * hg;
        const uint32_t t = min32(tj, n_tok - j0);
        const uint32_t in_words = t * grp;
        for (uint32_t w = lane; w < in_words; w += 64u * U) {
            uint32_t cw[U], lw[U], x[U];
            bool ok[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t ww = w + 64u * u;
                const uint32_t jj = mdiv(ww, a.hm_m_hgrp[1]);
                const uint32_t rem = ww - jj * grp;
                const uint32_t hh = mdiv(rem, a.hm_m_rd);
                ok[u] = ww < in_words;
                cw[u] = ((j0 + jj) * H + h0) * rd + rem;
                lw[u] = (hh * tj + jj) * rd + (rem - hh * rd);
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (ok[u]) x[u] = ld_word<NT>(chunk + cw[u]);
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (ok[u]) lds[lw[u]] = x[u];
        }
        __builtin_amdgcn_wave_barrier();
        const uint32_t words = hg * run;
        for (uint32_t w = lane; w < words; w += 64u * U) {
            uint32_t pw[U], x[U];
            bool ok[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t ww = w + 64u * u;
                const uint32_t hh = mdiv(ww, a.hm_m_hrun[1]);
                const uint32_t i = ww - hh * run;
                ok[u] = ww < words && mdiv(i, a.hm_m_rd) < t;
                pw[u] = ((h0 + hh) * bs + j0) * rd + i;
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (ok[u]) x[u] = lds[w + 64u * u];
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (ok[u]) st_pool_word<NT>(pool + pw[u], x[u]);
        }
        __builtin_amdgcn_wave_barrier();
    }
}

// Gather of head-major rows of 4-byte words in slabs of whole pages of hg heads
// (hm_lds_head_slab: where token slabs would split pool lines and a head group's chunk
// runs are whole lines): the group's pages, one contiguous run of the block, are read
// in pool order into the slice (slice word w = pool word ((h0 + hh)*bs + j0)*rd + i,
// hh = w / (tj*rd), i = w - hh*tj*rd); the slice is then written out along the chunk,
// hg*rd words per token -- chunk word w of the slab is row jj = w / (hg*rd), head hh
// and word q of the remainder, from slice word (hh*tj + jj)*rd + q.
template <bool NT>
__device__ __forceinline__ void hm_lds_gather_heads(uint32_t *lds, const uint8_t *block, uint8_t *chunk_tile,
                                                    uint32_t s0, uint32_t s1, uint32_t n_tok, uint32_t lane,
                                                    const Launch &a)
{
    constexpr int U = KVX_HM_LDS_UNROLL;
    const uint32_t H = a.hm_heads, rd = a.hm_rd, hg = a.hm_hg[0], tj = a.hm_htj[0], bs = a.block_size;
    const uint32_t run = tj * rd, grp = hg * rd, n_tr = (n_tok + tj - 1) / tj;
    const gword *const pool = (const gword *)block;
    gword *const chunk = (gword *)chunk_tile;
    for (uint32_t sl = s0; sl < s1; ++sl) {
        const uint32_t g = sl / n_tr, j0 = (sl - g * n_tr) * tj, h0 = g * hg;
        const uint32_t t = min32(tj, n_tok - j0);
        const uint32_t words = hg * run;
        for (uint32_t w = lane; w < words; w += 64u * U) {
            uint32_t pw[U], x[U];
            bool ok[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t ww = w + 64u * u;
                const uint32_t hh = mdiv(ww, a.hm_m_hrun[0]);
                const uint32_t i = ww - hh * run;
                ok[u] = ww < words && mdiv(i, a.hm_m_rd) < t;
                pw[u] = ((h0 + hh) * bs + j0) * rd + i;
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (ok[u]) x[u] = ld_pool_word<NT>(pool + pw[u]);
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (ok[u]) lds[w + 64u * u] = x[u];
        }
        __builtin_amdgcn_wave_barrier();
        const uint32_t out_words = t * grp;
        for (uint32_t w = lane; w < out_words; w += 64u * U) {
            uint32_t cw[U], lw[U], x[U];
            bool ok[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t ww = w + 64u * u;
                const uint32_t jj = mdiv(ww, a.hm_m_hgrp[0]);
                const uint32_t rem = ww - jj * grp;
                const uint32_t hh = mdiv(rem, a.hm_m_rd);
                ok[u] = ww < out_words;
                cw[u] = ((j0 + jj) * H + h0) * rd + rem;
                lw[u] = (hh * tj + jj) * rd + (rem - hh * rd);
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (ok[u]) x[u] = lds[lw[u]];
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (ok[u]) st_word<NT>(chunk + cw[u], x[u]);
        }
        __builtin_amdgcn_wave_barrier();
    }
}

// Head-major pages of 4-byte-word rows moved a whole page at a time (hm_page_ok): the
// block, [H][bs][rd] words, is one contiguous run of tile_bytes, and the tile of n_tok
// tokens one contiguous run of n_tok*H*rd words in the chunk, [n_tok][H][rd].  Both
// runs are moved in 16-byte vectors, KVX_HM_PAGE_GROUP of them per lane in flight, and
// the transposition is done by where each 4-byte word goes in this wave's LDS slice,
// which holds the tile in chunk order (hm_page_slice_words).
// Gather reads the whole block (the buffer range keeps the loads inside it) and drops
// words of tokens past n_tok; scatter writes whole pool vectors when the page is full,
// and single words of the tile's tokens when it is partial.  Only this wave uses its
// slice and a wave's LDS accesses complete in order, so wave_barrier only keeps the
// compiler from moving accesses across a phase boundary.
template <int DIR, bool NT>
__device__ __forceinline__ void copy_head_major_page(uint32_t *lds, uint8_t *block, uint8_t *chunk_tile,
                                                     uint32_t n_tok, uint32_t lane, const Launch &a)
{
    constexpr int G = KVX_HM_PAGE_GROUP;           // 16-byte vectors per lane in flight
    const uint32_t bs = a.block_size;
    const uint32_t page_vec = (uint32_t)(a.tile_bytes >> 4);
    const uint32_t tile_vec = n_tok * a.tok / 16u;
    if (DIR == KV_GATHER) {
        const BufSide<kGatherPoolPol<NT>> in(block, page_vec * 16u);
        const BufSide<kGatherChunkPol<NT>> out(chunk_tile, tile_vec * 16u);
        for (uint32_t v0 = lane; v0 < page_vec; v0 += 64u * G) {
            u32x4 x[G];
#pragma unroll
            for (int k = 0; k < G; ++k) x[k] = in.load(v0 + 64u * k);  // past the block: dropped by the range
#pragma unroll
            for (int k = 0; k < G; ++k) {
                const uint32_t v = v0 + 64u * k;
                if (v < page_vec) {
                    uint32_t sw[4];
                    hm_page_slice_words(a, v, n_tok, sw);
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        if (sw[c] != ~0u) lds[sw[c]] = x[k][c];
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
        for (uint32_t v0 = lane; v0 < tile_vec; v0 += 64u * G)
#pragma unroll
            for (int k = 0; k < G; ++k) {
                const uint32_t v = v0 + 64u * k;
                if (v < tile_vec) out.store(v, *(const u32x4 *)(lds + 4u * v));
            }
        __builtin_amdgcn_wave_barrier();
        return;
    }
    const PtrSide<NT> in{as_global(chunk_tile)};
    for (uint32_t v0 = lane; v0 < tile_vec; v0 += 64u * G) {
        u32x4 x[G];
#pragma unroll
        for (int k = 0; k < G; ++k) {
            const uint32_t v = v0 + 64u * k;
            x[k] = in.load(v < tile_vec ? v : tile_vec - 1u);  // clamped: no load behind a lane-dependent branch
        }
#pragma unroll
        for (int k = 0; k < G; ++k)
            if (v0 + 64u * k < tile_vec) *(u32x4 *)(lds + 4u * (v0 + 64u * k)) = x[k];
    }
    __builtin_amdgcn_wave_barrier();
    if (n_tok == bs) {  // a full page: every pool vector is the tile's
        gvec *const pool = as_global(block);
        for (uint32_t v0 = lane; v0 < page_vec; v0 += 64u * G)
#pragma unroll
            for (int k = 0; k < G; ++k) {
                const uint32_t v = v0 + 64u * k;
                if (v < page_vec) {
                    uint32_t sw[4];
                    hm_page_slice_words(a, v, n_tok, sw);
                    u32x4 y;
#pragma unroll
                    for (int c = 0; c < 4; ++c) y[c] = lds[sw[c]];
                    st<NT>(pool + v, y);
                }
            }
    } else {            // a partial page: only the words of the tile's tokens
        gword *const pool = (gword *)block;
        for (uint32_t v = lane; v < page_vec; v += 64u) {
            uint32_t sw[4];
            hm_page_slice_words(a, v, n_tok, sw);
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (sw[c] != ~0u) st_pool_word<NT>(pool + 4u * v + c, lds[sw[c]]);
        }
    }
    __builtin_amdgcn_wave_barrier();
}

// SEG = 0: the tile walk; SEG = 2, 4 or 8: the segment walk (gather of token-major
// pages), in groups of SEG vectors per lane (gather_seg_unroll).
template <int DIR, int LAYOUT, int PAGE, bool NT, int SEG>
__global__ void __launch_bounds__(kThreads) tile_copy(const Launch a)
{
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t step = (int64_t)gridDim.x * kWavesPerBlock;
    const KVX_CONST SpanDev *spans = span_records(a);
    uint32_t s = 0;

    if (SEG) {  // only instantiated for gather of token-major pages
        // Work item = one segment of the tiles laid end to end: the pieces of the (at
        // most a few) tiles it overlaps, copied in order.
        const int64_t T = a.tile_bytes;
        const int64_t total = a.total_tiles * T;
        const int64_t n_seg = work_items(a);
        for (int64_t seg = (int64_t)blockIdx.x * kWavesPerBlock + wave; seg < n_seg; seg += step) {
            const int64_t x0 = seg * a.seg_bytes;
            const int64_t x1 = x0 + a.seg_bytes < total ? x0 + a.seg_bytes : total;
            for (int64_t tile = x0 / T; tile * T < x1; ++tile) {
                s = find_span(spans, s, a.n_spans, tile);
                const SpanDev sp = load_span_fields(spans + s);
                const TileRef t = resolve_tile<LAYOUT>(a, sp, tile);
                int64_t lo, hi;
                segment_piece(tile, T, t.nbytes, x0, x1, &lo, &hi);
                if (hi <= lo) continue;
                const int32_t blk = as_const(sp.table)[t.page];
                if ((uint32_t)blk >= a.num_blocks) {
                    if (lane == 0) atomicOr(a.err, KV_DEVERR_BLOCK_RANGE);
                    continue;
                }
                const uint8_t *block = as_const(a.regions)[t.region] + (int64_t)blk * a.block_stride;
                gather_tile<NT, (SEG > 0 ? SEG : 1)>(block + lo, a.chunk_base + t.chunk_off + lo,
                                                    (uint32_t)((hi - lo) >> 4), lane);
            }
        }
        return;
    }

    // Work item = one of a tile's parts: 2^split_shift near-equal ones, or, in the
    // fixed-part instantiations only (so the other walks keep the shift arithmetic
    // alone), part_bytes-sized ones.  The waves of a workgroup take consecutive items, so
    // a split tile is copied by neighbouring waves; workgroups take their items in
    // launch_block order (contiguous per XCD when a.xcd_remap).
    constexpr bool FIXED = PAGE == KVX_PAGE_TM_FIXED || PAGE == KVX_PAGE_TM_SCATTER_FIXED_BUF;
    const uint32_t shift = a.split_shift;
    const int64_t ppt = FIXED ? parts_per_tile(a) : (int64_t)1 << shift;
    const int64_t items = a.total_tiles * ppt;
    const uint32_t block = launch_block(blockIdx.x, gridDim.x, a.xcd_remap);
    for (int64_t item = (int64_t)block * kWavesPerBlock + wave; item < items; item += step) {
        const int64_t tile = FIXED ? item / ppt : item >> shift;
        const uint32_t part = FIXED ? (uint32_t)(item - tile * ppt) : (uint32_t)(item & ((1 << shift) - 1));
        // tiles only grow along the loop, so the span search starts at the last span
        s = find_span(spans, s, a.n_spans, tile);
        const SpanDev sp = load_span(spans + s);
        const TileRef t = resolve_tile<LAYOUT>(a, sp, tile);

        const int32_t blk = as_const(sp.table)[t.page];
        if ((uint32_t)blk >= a.num_blocks) {
            if (lane == 0) atomicOr(a.err, KV_DEVERR_BLOCK_RANGE);
            continue;
        }
        uint32_t first, count;
        uint8_t *block = as_const(a.regions)[t.region] + (int64_t)blk * a.block_stride;
        uint8_t *chunk_tile = a.chunk_base + t.chunk_off;
        if constexpr (PAGE == KVX_PAGE_HM_LDS_PAGE) {
            // a whole page per wave (tiles of at most KVX_HM_PAGE_SLICE bytes are never split)
            __shared__ __attribute__((aligned(16))) uint32_t pages[kWavesPerBlock][KVX_HM_PAGE_SLICE / 4];
            copy_head_major_page<DIR, NT>(pages[wave], block, chunk_tile, t.nbytes / a.tok, lane, a);
            continue;
        }
        if constexpr (PAGE == KVX_PAGE_HM_LDS || PAGE == KVX_PAGE_HM_LDS_HEADS) {
            // parts of a split tile are ranges of slabs
            __shared__ __attribute__((aligned(16))) uint32_t slices[kWavesPerBlock][KVX_HM_LDS_SLICE / 4];
            const uint32_t n_tok = t.nbytes / a.tok;
            if (PAGE == KVX_PAGE_HM_LDS_HEADS) {  // head-group slabs
                part_range(hm_lds_slabs(n_tok, a.hm_heads, a.hm_hg[DIR], a.hm_htj[DIR]), part, 1u << shift,
                           &first, &count);
                if (DIR == KV_GATHER)
                    hm_lds_gather_heads<NT>(slices[wave], block, chunk_tile, first, first + count, n_tok, lane, a);
                else
                    hm_lds_scatter_heads<NT>(slices[wave], block, chunk_tile, first, first + count, n_tok, lane, a);
                continue;
            }
            part_range((n_tok + a.hm_tj - 1) / a.hm_tj, part, 1u << shift, &first, &count);
            copy_head_major_lds<DIR, NT>(slices[wave], block, chunk_tile, first, first + count, n_tok, lane, a);
            continue;
        }
        if (PAGE == KV_PAGE_HEAD_MAJOR && a.hm_t4) {
            // parts of a split tile are ranges of 4x4 blocks
            const uint32_t n_tok = t.nbytes / a.tok;
            part_range(hm_t4_units(n_tok, a.hm_heads), part, 1u << shift, &first, &count);
            copy_head_major_t4<DIR, NT>(block, chunk_tile, first, first + count, n_tok, lane, a);
            continue;
        }
        if (FIXED) tile_part(a, t.nbytes >> 4, part, &first, &count);
        else part_range(t.nbytes >> 4, part, 1u << shift, &first, &count);
        if (PAGE == KV_PAGE_HEAD_MAJOR) {
            copy_head_major<DIR, KVX_HM_UNROLL, NT>(as_global(block), chunk_tile, first, first + count,
                                                    lane, a);
        } else {
            uint8_t *pool = block + first * 16ll;
            uint8_t *chunk = chunk_tile + first * 16ll;
            if (DIR == KV_GATHER) gather_tile<NT>(pool, chunk, count, lane);
            else if (PAGE == KVX_PAGE_TM_SCATTER_BUF || PAGE == KVX_PAGE_TM_SCATTER_FIXED_BUF)
                scatter_tile_buf<NT>(chunk, pool, count, lane);
            else scatter_tile<NT>(as_global(chunk), as_global(pool), count, lane);
        }
    }
}

// Segment walks are separate instantiations, one per group size, so that the tile
// walk keeps its own register allocation.
template <int DIR, int LAYOUT, int PAGE, bool NT>
static const void *pick_walk(const Launch &a)
{
    if constexpr (DIR == KV_GATHER && PAGE == KV_PAGE_TOKEN_MAJOR) {
        if (a.seg_bytes) {
            switch (gather_seg_unroll(a.tile_bytes, a.seg_bytes)) {
            case 2: return (const void *)&tile_copy<DIR, LAYOUT, PAGE, NT, 2>;
            case 4: return (const void *)&tile_copy<DIR, LAYOUT, PAGE, NT, 4>;
            default: return (const void *)&tile_copy<DIR, LAYOUT, PAGE, NT, 8>;
            }
        }
    }
    return (const void *)&tile_copy<DIR, LAYOUT, PAGE, NT, 0>;
}

template <int DIR, int LAYOUT, int PAGE>
static const void *pick_policy(const Launch &a)
{
    return a.cached ? pick_walk<DIR, LAYOUT, PAGE, false>(a) : pick_walk<DIR, LAYOUT, PAGE, true>(a);
}

template <int DIR, int LAYOUT>
static const void *pick_page(const Launch &a)
{
    if (a.page_layout == KV_PAGE_HEAD_MAJOR) {
        if (a.hm_page) return pick_policy<DIR, LAYOUT, KVX_PAGE_HM_LDS_PAGE>(a);
        if (a.hm_lds && a.hm_hg[DIR]) return pick_policy<DIR, LAYOUT, KVX_PAGE_HM_LDS_HEADS>(a);
        return a.hm_lds ? pick_policy<DIR, LAYOUT, KVX_PAGE_HM_LDS>(a)
                        : pick_policy<DIR, LAYOUT, KV_PAGE_HEAD_MAJOR>(a);
    }
    if constexpr (DIR == KV_SCATTER) {
        if (a.part_bytes)
            return a.scatter_buf ? pick_policy<DIR, LAYOUT, KVX_PAGE_TM_SCATTER_FIXED_BUF>(a)
                                 : pick_policy<DIR, LAYOUT, KVX_PAGE_TM_FIXED>(a);
        if (a.scatter_buf) return pick_policy<DIR, LAYOUT, KVX_PAGE_TM_SCATTER_BUF>(a);
    } else {
        if (a.part_bytes) return pick_policy<DIR, LAYOUT, KVX_PAGE_TM_FIXED>(a);
    }
    return pick_policy<DIR, LAYOUT, KV_PAGE_TOKEN_MAJOR>(a);
}

int launch_tile_copy(int direction, const Launch &a, uint32_t grid, hipStream_t stream)
{
    const void *fn;
    if (direction == KV_GATHER)
        fn = a.layout == KV_LAYER_FIRST ? pick_page<KV_GATHER, KV_LAYER_FIRST>(a)
                                        : pick_page<KV_GATHER, KV_PAGE_FIRST>(a);
    else
        fn = a.layout == KV_LAYER_FIRST ? pick_page<KV_SCATTER, KV_LAYER_FIRST>(a)
                                        : pick_page<KV_SCATTER, KV_PAGE_FIRST>(a);
    Launch arg = a;
    void *args[] = {&arg};
    // hipLaunchKernel reports this launch's own status (not a stale runtime error).
    return (int)hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, 0, stream);
}

uint32_t default_grid(int64_t items)
{
    const int64_t need = (items + kWavesPerBlock - 1) / kWavesPerBlock;
    return (uint32_t)(need < KVX_GRID_CAP ? need : KVX_GRID_CAP);
}

}  // namespace kvx
