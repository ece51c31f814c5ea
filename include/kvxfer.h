/*
 * kvxfer.h -- paged KV-cache gather/scatter for AMD Instinct MI355X (gfx950).
 *
 * The library moves a request's KV pages between a paged pool (per-layer K/V
 * regions addressed through a block table) and large contiguous transfer
 * chunks, in either direction, with one kernel launch per call:
 *
 *   gather  (offload): pool pages  -> chunks   (Strata guide, "Implementation"
 *                      lifecycle figure, step 6: background eviction of cold
 *                      pages to host memory with a one-block kernel)
 *   scatter (reload) : chunks      -> pool pages (same figure, step 3, and
 *                      "Step 1: High-Performance GPU-Assisted I/O CUDA Kernel")
 *
 * Chunks may sit in HBM or in pinned host memory that the kernel reads and
 * writes directly with ordinary loads and stores, instead of one DMA per page
 * (Strata guide, "The Mechanics of GPU-Assisted I/O").  The layout change
 * between the pool (layer-first) and the chunk (layer-first or page-first) is
 * done by address arithmetic during the copy (Strata guide, "Two-Dimensional
 * Memory Layout Decoupling").  Host work per call is proportional to the number
 * of spans, not to pages x layers (Tutti summary, Q2 "Design 1": CPU work drops
 * from O(layer x blocks) to O(layer)).
 *
 * ---------------------------------------------------------------------------
 * Data model
 * ---------------------------------------------------------------------------
 * Pool.  For layer l < num_layers and kv < num_kv (2 = K and V, 1 = a single
 * latent) the caller provides one device region, bases[l*num_kv + kv].  Block
 * b of that region starts at bases[l*num_kv+kv] + b*block_stride and holds
 * block_size tokens, token-major ([block_size][H][D]) or, with page_layout
 * KV_PAGE_HEAD_MAJOR, head-major ([H][block_size][D]); a token is num_heads x
 * head_dim elements of elem_bytes bytes: tok = num_heads*head_dim*elem_bytes.  One
 * block id names the same page in every (layer, kv) region.  K and V are
 * separate objects per layer, as in the Tutti summary's Figure 4 (2L objects
 * per block).  block_stride >= block_size*tok; block_stride == block_size*tok
 * gives a vLLM-style [num_blocks][block_size][H][D] region, block_stride ==
 * num_kv*block_size*tok with bases offset by kv*block_size*tok gives a per-layer
 * [num_blocks][num_kv][block_size][H][D] pool.
 * Placement (measured on MI355X, not part of the contract): scattered page writes
 * into a pool whose regions all lie in one 64 GiB window of one plain allocation run
 * at about 68 % of HBM peak, and at about 80 % when the regions span two windows
 * (gathers lose 1-3 points there).  What decides is the physical memory behind the
 * addresses, which the library cannot see: the caller chooses where regions live,
 * and a pool larger than 64 GiB spans windows by its size alone.
 *
 * Span.  (block_table, t_begin, t_end, first_chunk): tokens [t_begin, t_end)
 * of one request, whose token t lives at slot t % block_size of block
 * block_table[t / block_size].  t_begin must be a multiple of block_size
 * (prefix matches end on page boundaries: Strata guide, "The Conflict Between
 * PagedAttention and Transfer Efficiency"); t_end is arbitrary, so the last
 * page may be partial.
 *
 * Chunks.  A call moves layers [layer_begin, layer_end).  Each span splits into
 * chunks of chunk_layers layers x chunk_tokens tokens, layer-chunk major:
 *     c = first_chunk + lc*n_tc + tc,  lc = (l - layer_begin) / chunk_layers,
 *     tc = (t - t_begin) / chunk_tokens,  n_tc = ceil((t_end - t_begin) / chunk_tokens)
 * and chunk c occupies slot (c mod n_slots), at base + (c mod n_slots)*slot_bytes.
 * With li = (l - layer_begin) % chunk_layers, a chunk is laid out as
 *     KV_LAYER_FIRST: [chunk_layers][num_kv][T_c][H][D], T_c = tokens in the
 *                     chunk (the span's last chunk may be short, and is dense)
 *     KV_PAGE_FIRST : [P_c][chunk_layers][num_kv][block_size][H][D], P_c = pages
 *                     in the chunk; a partial last page leaves pad bytes that
 *                     are neither written (gather) nor read (scatter).
 * The page-first order is the Strata guide's host-side [P, L, H, D] tensor
 * ("Two-Dimensional Memory Layout Decoupling", item 2); layer-first matches its
 * HBM-side [L, P, H, D] tensor (item 1).  Chunks are token-major in both; a
 * head-major pool is transposed to token-major on the way out and back on the way in.
 *
 * Nothing outside the referenced pool tokens and the chunk bytes is written.
 *
 * ---------------------------------------------------------------------------
 * Conventions
 * ---------------------------------------------------------------------------
 * Every function returns KV_OK (0) or a negative KV_ERR_* code; no exception
 * crosses the ABI.  A call that returns an error has launched nothing and
 * changed no state.
 * Pointers named "device" must be valid on the device current when the call
 * is made (HBM, or mapped pinned host memory from kv_ring_create / hipHostMalloc).
 * All device and chunk pointers, block_stride, slot_bytes and tok must be
 * multiples of 16 bytes (16-byte vector loads and stores).
 * Transfers are asynchronous on the given stream (0 = the null stream): the
 * caller keeps every buffer alive and unmodified until the stream has passed
 * the call.  Handles are not thread-safe.
 * The caller's buffers must hold what the call declares: each region
 * (num_blocks - 1) * block_stride + block_size * tok bytes, the staging area
 * n_slots * slot_bytes, each device block table table_len entries.  Where the
 * HIP runtime knows the allocation holding such a pointer (hipMalloc'd device
 * memory, hipHostMalloc'd or registered host memory, virtual-memory mappings),
 * a transfer whose declared extent runs past the end of that allocation and
 * any allocations adjoining it without a gap is refused with KV_ERR_RANGE
 * before anything is enqueued (an access past mapped memory would fault the
 * GPU); memory the runtime does not know is taken on trust.  A sub-allocator's
 * block (e.g. a torch tensor) is checked against the runtime allocation it lies
 * in, not against its own size.
 */
#ifndef KVXFER_H
#define KVXFER_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KV_API __attribute__((visibility("default")))

/* ---- error codes ------------------------------------------------------- */
#define KV_OK 0
#define KV_ERR_ARG (-1)    /* null pointer, bad shape, empty or inverted range */
#define KV_ERR_ALIGN (-2)  /* pointer, stride, slot size or token size not a multiple of 16 */
#define KV_ERR_RANGE (-3)  /* span past its block table, slot too small, block id out of range, buffer past its allocation */
#define KV_ERR_OOM (-4)    /* allocator exhausted, or a host/device allocation failed */
#define KV_ERR_RING (-5)   /* two chunks of one call share a staging slot */
#define KV_ERR_HIP (-6)    /* a HIP runtime call failed (no device, launch failure, ...) */
#define KV_ERR_DEVICE (-7) /* kv_pool_get_error: the device reported a bad block id */
#define KV_ERR_DUP (-8)    /* KV_FLAG_VALIDATE: a scatter writes one pool page twice */
#define KV_ERR_SCRATCH (-9) /* kv_transfer_chunks_noalloc: more regions than its static scratch holds */
#define KV_ERR_CAPTURE (-10) /* the stream is capturing a graph and this call cannot be captured */

/* ---- chunk layouts, in-page layouts, directions, flags ----------------- */
#define KV_LAYER_FIRST 0
#define KV_PAGE_FIRST 1

/* kv_pool_desc.page_layout: how a pool block orders its tokens and heads */
#define KV_PAGE_TOKEN_MAJOR 0 /* [block_size][H][D] (vLLM-style NHD) */
#define KV_PAGE_HEAD_MAJOR 1  /* [H][block_size][D] (HND); chunks stay token-major */

#define KV_GATHER 0  /* pool -> chunks (offload) */
#define KV_SCATTER 1 /* chunks -> pool (reload)  */

/* kv_chunk_spec.flags */
#define KV_FLAG_VALIDATE 0x1 /* copy the block tables to the host (synchronously) and check
                                ids in range and, for scatter, one writer per pool page */
#define KV_FLAG_DMA_STRIDED 0x2 /* read by the _dma entry points only: where the regions are
                                   evenly spaced, one strided copy per (chunk, page) covers
                                   the page's chunk_layers*num_kv tiles */
#define KV_FLAG_CACHED 0x4 /* kernel entry points: plain cached loads and stores instead of the
                              default nontemporal ones (same bytes, same result).  The default
                              keeps a transfer from evicting the working set of kernels that
                              run beside it (Strata guide, "Non-Intrusive Resource Sizing");
                              this flag is for callers that touch the moved bytes right after */
#define KV_FLAG_PAGE_RUNS 0x8 /* kernel scatters: a hint that the call's pages lie mostly in
                                 runs of adjacent block ids (as kv_pool_alloc_blocks hands them
                                 out on an unfragmented pool), so token-major tiles of 20 KiB
                                 to under 64 KiB are copied whole, one wave each, instead of in
                                 4 KiB parts by several.  Same bytes, same result; measured on
                                 MI355X with 32 KiB tiles: runs of adjacent blocks scatter at
                                 74-77 % of HBM peak whole against 71-72 % in parts, shuffled
                                 blocks at 68-69 % whole against 70-72 % in parts.  No passage:
                                 a performance hint of this library. */

/* device error bits reported through kv_pool_get_error */
#define KV_DEVERR_BLOCK_RANGE 0x1 /* a block table held an id outside [0, num_blocks); that
                                     (layer, kv, page) tile was skipped */

/* kv_ring_create flags */
#define KV_RING_COHERENT 0x0     /* hipHostMalloc coherent mapped memory (default) */
#define KV_RING_NONCOHERENT 0x1  /* hipHostMallocNonCoherent: the GPU may cache it */

/* Limits of one call. */
#define KV_MAX_SPANS 4096

typedef struct kv_pool kv_pool; /* opaque, owned by the library */
typedef struct kv_ring kv_ring; /* opaque, owned by the library */

typedef struct {
    int32_t num_layers;   /* L >= 1 */
    int32_t num_kv;       /* 1 or 2 */
    int32_t num_heads;    /* H >= 1 */
    int32_t head_dim;     /* D >= 1 */
    int32_t elem_bytes;   /* 1, 2, 4 or 8 (the payload is moved as opaque bytes) */
    int32_t block_size;   /* tokens per page, >= 1 */
    int32_t page_layout;  /* KV_PAGE_TOKEN_MAJOR or KV_PAGE_HEAD_MAJOR; a head-major row,
                             head_dim*elem_bytes bytes, must be a multiple of 16 bytes, or a
                             multiple of 4 with tok <= 8192 (such rows are transposed
                             through LDS); other rows: KV_ERR_ALIGN, too large a token for
                             4-byte rows: KV_ERR_ARG */
    int64_t num_blocks;   /* blocks per (layer, kv) region, 1 .. 2^31-1 */
    int64_t block_stride; /* bytes between consecutive blocks of one region */
    void *const *bases;   /* host array of num_layers*num_kv device pointers; the
                             library copies it, the regions stay caller-owned */
} kv_pool_desc;

typedef struct {
    const int32_t *block_table; /* device array (host array for kv_validate_targets) */
    int64_t table_len;          /* entries in block_table; >= ceil(t_end / block_size), < 2^31 */
    int64_t t_begin;            /* first token, a multiple of block_size, >= 0 */
    int64_t t_end;              /* one past the last token, >= t_begin (an empty span moves nothing) */
    int64_t first_chunk;        /* chunk index of the span's first chunk, >= 0 */
} kv_span;

typedef struct {
    int32_t layout;        /* KV_LAYER_FIRST or KV_PAGE_FIRST */
    int32_t chunk_layers;  /* CL, divides layer_end - layer_begin */
    int64_t chunk_tokens;  /* CT, a multiple of block_size */
    int32_t layer_begin;   /* first layer moved */
    int32_t layer_end;     /* one past the last layer moved (<= num_layers) */
    void *base;            /* device-visible staging: HBM or mapped pinned host memory */
    int64_t slot_bytes;    /* bytes per staging slot, >= the largest chunk of the call */
    int64_t n_slots;       /* slots at base; chunk c uses slot c mod n_slots */
    int32_t max_workgroups;/* 0 = library default grid: the whole chip when base is device
                              memory, 16 workgroups of 256 threads when it is host memory
                              (a host-link-bound copy needs few: Strata guide,
                              "Non-Intrusive Resource Sizing"); the kind of memory is
                              looked up with hipPointerGetAttributes and remembered for
                              the last base the pool saw.  > 0 caps the grid.  A reload
                              and an offload over the host link at the same time do
                              best with smaller grids than either alone: 6 workgroups
                              for the scatter and 2 for the gather measured 95 GB/s
                              combined on MI355X (98 % of the link's two-way rate),
                              the default 16 each 71 GB/s */
    int32_t flags;         /* KV_FLAG_* */
} kv_chunk_spec;

/* Sizes of one call, as kv_check_transfer reports them. */
typedef struct {
    int64_t tiles;          /* (layer, kv, page) tiles the kernel copies */
    int64_t chunks;         /* chunks the call touches */
    int64_t payload_bytes;  /* bytes copied (each read once and written once) */
    int64_t max_chunk_bytes;/* largest chunk of the call */
} kv_transfer_info;

/* ---- pool ------------------------------------------------------------------ */

/* Validates desc and creates a pool handle with a host bitmap of free blocks (one
 * bit per block, all free).  Device-side state (a region
 * table, an error word, a 4 MiB span-record arena with its pinned mirror and 256
 * events) is created on the first transfer, on the device current then; later
 * transfers must run with the same device current.  Errors: KV_ERR_ARG,
 * KV_ERR_ALIGN (a base, block_stride or tok not 16-byte aligned, or a head-major
 * row neither 16- nor 4-byte aligned), KV_ERR_OOM. */
KV_API int kv_pool_create(const kv_pool_desc *desc, kv_pool **out);

/* Frees the handle and its device state, after waiting for the transfers it
 * queued that are still in flight (their fence events; other device work is not
 * waited for, nor are replays of calls captured into graphs: those must have finished,
 * and such graphs must not run again).  The caller's regions are untouched.  NULL is
 * accepted.
 * No passage: library infrastructure (the handle's lifetime). */
KV_API int kv_pool_destroy(kv_pool *pool);

/* Block allocator (a host bitmap of free blocks, preallocated at create time, no
 * allocation on the call path: Tutti summary, "Key implementation details", item 1).
 * alloc: writes the n lowest free ids to out_ids in ascending order (so a request's
 * pages lie as close together as the pool's fragmentation allows, which makes
 * reloading them faster), or fails with KV_ERR_OOM and allocates nothing.
 * free: ids must be currently allocated and distinct, else KV_ERR_RANGE and
 * nothing is freed. */
KV_API int kv_pool_alloc_blocks(kv_pool *pool, int32_t n, int32_t *out_ids);
KV_API int kv_pool_free_blocks(kv_pool *pool, int32_t n, const int32_t *ids);
/* Free blocks left in the allocator (same source as the two calls above). */
KV_API int kv_pool_free_count(const kv_pool *pool, int64_t *out);

/* ---- calls -------------------------------------------------------------------- */

/* Host-only dry run: validates a prospective call exactly as kv_gather_chunks /
 * kv_scatter_chunks do (shapes, alignment, span ranges, slot sizes, one slot per
 * chunk) and reports its sizes.  Makes no HIP call, so the allocation-extent
 * checks (Conventions above) are left to the transfer itself; info may be NULL.
 * No passage of its own: it is the host-side part of the transfer calls below
 * (their call decomposition, Tutti summary, Q2 "Design 1"), run without a launch. */
KV_API int kv_check_transfer(const kv_pool_desc *desc, const kv_span *spans, int32_t n_spans,
                      const kv_chunk_spec *spec, kv_transfer_info *info);

/* Bytes of a chunk holding `tokens` tokens (1 <= tokens <= chunk_tokens) in the
 * spec's layout (the two chunk layouts of the Data model above: Strata guide,
 * "Two-Dimensional Memory Layout Decoupling", items 1 and 2), so a caller can size
 * staging slots. */
KV_API int kv_chunk_bytes(const kv_pool_desc *desc, const kv_chunk_spec *spec, int64_t tokens,
                   int64_t *out);

/* Host-side check of the block tables of a call, given host copies of them
 * (host_tables[i] holds spans[i].table_len ids): every id of every referenced
 * page lies in [0, num_blocks) (else KV_ERR_RANGE) and, for KV_SCATTER, no pool
 * page receives two writers (else KV_ERR_DUP).  Gather may read a page twice.
 * No passage: the pages are silent on duplicate targets; this checks the
 * precondition the library states for scatter (one writer per pool page). */
KV_API int kv_validate_targets(const kv_pool_desc *desc, const kv_span *spans, int32_t n_spans,
                        const int32_t *const *host_tables, int32_t direction);

/* Gather (offload): for every span, layer in [layer_begin, layer_end), kv and
 * token, copies the pool token into its chunk position.  One kernel launch on
 * `stream`, preceded by one small stream-ordered descriptor upload.  spans is a
 * host array of n_spans (1 .. KV_MAX_SPANS) entries; each block_table is a
 * device pointer.  n_spans == 0, or spans that are all empty, is a no-op.  Loads
 * and stores are nontemporal.  Returns after enqueueing.
 * Under HIP graph capture (the same holds for kv_scatter_chunks): a call is captured as
 * its one kernel, every replay repeating the call, when its span records ride in the
 * kernel arguments (at most 16 non-empty spans), the pool has made a call outside the
 * capture before (the first call allocates the pool's device state), KV_FLAG_VALIDATE
 * is not set (its table check copies to the host) and the pool's timing is off.  Any
 * other call is refused with KV_ERR_CAPTURE and enqueues nothing (more records go
 * through the pool's arena, which is recycled under events the host waits on).  A
 * replay reads the pool's region table and writes its error word (kv_pool_get_error),
 * so the pool must outlive the graph, and kv_pool_destroy must not be called while a
 * replay may still run (it waits only for calls made outside a graph). */
KV_API int kv_gather_chunks(kv_pool *pool, const kv_span *spans, int32_t n_spans,
                     const kv_chunk_spec *spec, hipStream_t stream);

/* Scatter (reload): the inverse move, chunk positions -> pool tokens.  The
 * spans of one call must not write one pool page twice (checked only with
 * KV_FLAG_VALIDATE); then every written byte has exactly one writer. */
KV_API int kv_scatter_chunks(kv_pool *pool, const kv_span *spans, int32_t n_spans,
                      const kv_chunk_spec *spec, hipStream_t stream);

/* For callers that cannot allocate (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): kv_gather_chunks (direction KV_GATHER) or
 * kv_scatter_chunks (KV_SCATTER) with the same data model, validation, kernels and
 * results, but no allocation of any kind on any call, the first included.  The call's
 * region table and span records go to a static device array of 264.25 KiB that each
 * device the library runs on holds until the process ends (one stream-ordered
 * host-to-device copy per call from a host image the pool made at kv_pool_create; the
 * copy has taken the image's bytes when the call returns), instead of the pool's
 * arena.  Limits beyond the other entry points': num_layers*num_kv <= 1024 (else
 * KV_ERR_SCRATCH), and KV_FLAG_VALIDATE is refused (KV_ERR_ARG: its table check
 * copies to the host).  Every call on one device shares that device's array, which
 * keeps the last call's contents: calls that overlap on one device (different
 * streams, or other threads, with no ordering between them) race and must not be
 * made; calls on one stream are ordered and safe.  A block id out of range is
 * skipped, as in the other entry points, and its KV_DEVERR_* bit OR-ed into
 * *err_word, a caller-owned device int32 (4-byte aligned) that the caller clears
 * and reads; err_word may be NULL to ignore such ids.  kv_pool_get_error does not
 * see these calls.  Returns after enqueueing.
 * Under HIP graph capture: a call with at most 16 non-empty spans carries its span
 * records in the kernel arguments, and is captured as the copy of the pool's region
 * table (which the graph reads from the pool's host image each time it runs, so the
 * pool must outlive the graph) followed by the kernel; every replay repeats the
 * call.  A call with more non-empty spans is refused with KV_ERR_CAPTURE while
 * `stream` is capturing: the graph would read its records from the host image when
 * it runs, after later calls have rewritten them.  Replays share the device's static
 * array like any other call: a replay must not overlap another call on the device. */
KV_API int kv_transfer_chunks_noalloc(kv_pool *pool, int32_t direction, const kv_span *spans,
                                      int32_t n_spans, const kv_chunk_spec *spec, int32_t *err_word,
                                      hipStream_t stream);

/* The conventional engine, for comparison: the same transfer done by the copy
 * engine as one hipMemcpyAsync per (layer, kv, page) tile, issued from the host on
 * `stream` -- the per-page DMA loop whose submission overhead the Strata guide
 * measures ("The Conflict Between PagedAttention and Transfer Efficiency",
 * paged-fragmentation figure, and the framework comparison table).  Same data
 * model, validation and results as kv_gather_chunks / kv_scatter_chunks, except
 * that each spans[i].block_table is a HOST array (the host issues the copies), and
 * every block id of the call is checked on the host before any copy is issued
 * (KV_ERR_RANGE; for scatter also KV_ERR_DUP).  Host work is O(tiles).  The tables
 * are read during the call only.  A head-major pool takes one hipMemcpy2DAsync per
 * (tile, head) instead.  With KV_FLAG_DMA_STRIDED and token-major pages whose
 * regions are evenly spaced (bases[i+1] - bases[i] the same positive value for all
 * i), the tiles of one page in one chunk -- one per (layer, kv) of the chunk --
 * go as one hipMemcpy2DAsync of chunk_layers*num_kv rows (the "where strides allow"
 * variant of the conventional engine); otherwise the flag changes nothing. */
KV_API int kv_gather_chunks_dma(kv_pool *pool, const kv_span *spans, int32_t n_spans,
                                const kv_chunk_spec *spec, hipStream_t stream);
KV_API int kv_scatter_chunks_dma(kv_pool *pool, const kv_span *spans, int32_t n_spans,
                                 const kv_chunk_spec *spec, hipStream_t stream);

/* Synchronizes `stream`, then reads and clears the pool's sticky device error
 * word.  *out_bits receives KV_DEVERR_* bits (0 if none); the return value is
 * KV_ERR_DEVICE when any bit was set, else KV_OK.
 * No passage: library infrastructure (failure detection: how a bad block id the
 * kernel skipped is reported to the caller). */
KV_API int kv_pool_get_error(kv_pool *pool, hipStream_t stream, int32_t *out_bits);

/* Kernel timing.  After kv_pool_timing_start, every transfer records a HIP
 * event pair around its kernel launch on its stream (up to 4096 launches).
 * kv_pool_timing_read synchronizes those events, writes the summed kernel time
 * in milliseconds and the number of launches timed, and stops timing.
 * kv_pool_timing_read_each does the same but writes each launch's time, in launch
 * order, to ms_each[0 .. min(cap, *launches)) (caller-owned; may be null when cap
 * is 0). */
/* No passage: library infrastructure (measurement of the kernel alone, as the
 * pages' bandwidth figures are rates of the transfer itself). */
KV_API int kv_pool_timing_start(kv_pool *pool);
KV_API int kv_pool_timing_read(kv_pool *pool, double *total_ms, int64_t *launches);
KV_API int kv_pool_timing_read_each(kv_pool *pool, double *ms_each, int64_t cap, int64_t *launches);

/* ---- pinned-host staging ring ------------------------------------------------ */

/* Allocates and pins n_slots*slot_bytes bytes of host memory once, mapped into
 * the device address space of the current device (hipHostMalloc; pinning is done
 * up front, never on the transfer path: Strata guide, "Production Cluster Sizing
 * and Configuration Guidelines", item 2).  slot_bytes must be a multiple of 16.
 * The memory is zero-filled.  Use kv_ring_slot's device pointer as
 * kv_chunk_spec.base. */
KV_API int kv_ring_create(int64_t slot_bytes, int64_t n_slots, int32_t flags, kv_ring **out);

/* Host and device addresses of slot i (0 <= i < n_slots); either out may be NULL.
 * Same source as kv_ring_create. */
KV_API int kv_ring_slot(const kv_ring *ring, int64_t i, void **host_ptr, void **dev_ptr);

/* Frees the pinned memory; the caller must have synchronized every transfer
 * that uses it.  NULL is accepted.  No passage: library infrastructure (the
 * ring's lifetime). */
KV_API int kv_ring_destroy(kv_ring *ring);

/* Slot fencing, for using the ring as a queue between the GPU and the host (slot
 * reuse across calls is fenced by events, as the Tutti summary's GPU io_uring
 * orders its I/O with events, Figure 5).  kv_ring_record marks slots
 * [first, first+count) (taken mod n_slots) as used by the work enqueued so far on
 * `stream` (one event per call).  kv_ring_wait blocks the host until the last work
 * recorded on every slot of the range has finished -- e.g. before the host reads
 * slots an offload wrote, or refills slots a reload read.  kv_ring_stream_wait
 * makes `stream` wait for that work instead.  A slot never recorded is free.
 * 1 <= count <= n_slots, 0 <= first < n_slots, else KV_ERR_ARG.  Not thread-safe. */
KV_API int kv_ring_record(kv_ring *ring, int64_t first, int64_t count, hipStream_t stream);
KV_API int kv_ring_wait(kv_ring *ring, int64_t first, int64_t count);
KV_API int kv_ring_stream_wait(kv_ring *ring, int64_t first, int64_t count, hipStream_t stream);

/* ---- misc ------------------------------------------------------------------------ */

/* Static description of a KV_* return code.  No passage: library infrastructure
 * (error reporting). */
KV_API const char *kv_strerror(int code);

/* Library version: major*10000 + minor*100 + patch (KV_VERSION of the header the
 * library was built with).  No passage: library infrastructure. */
#define KV_VERSION 200
KV_API int kv_version(void);

/* The hipError_t of the last HIP runtime call that failed inside the library on
 * the calling thread (0 if none), and in *where (if not NULL) the call's text.
 * Lets a caller that got KV_ERR_HIP see which call failed and why.  No passage:
 * library infrastructure (failure detection). */
KV_API int kv_last_hip_error(const char **where);

#ifdef __cplusplus
}
#endif

#endif /* KVXFER_H */
