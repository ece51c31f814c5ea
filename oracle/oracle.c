/*
 * oracle.c -- plain, slow CPU reference for paged-KV gather (offload) and
 * scatter (reload).
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load or call this file's library. It shares no source,
 * header, table or helper with the HIP library; it takes the same descriptor
 * values, in structs of its own.
 *
 * What is computed (a pure byte copy, so the result is exact):
 *
 *   Pool. For every layer l and K/V index kv there is one pool region; block b
 *   of it starts at bases[l*KV + kv] + b*block_stride and holds the page's
 *   tokens token-major, each token as [H][D] elements of E bytes -- or, for a
 *   head-major pool, the page as [H][bs][D] (chunks stay token-major, so such a
 *   pool is transposed on the way in and out).  A block id
 *   names the same page in every (layer, K/V) region, as the page index array
 *   does for all layers in the transfer kernel of the Strata guide
 *   ("Step 1: High-Performance GPU-Assisted I/O CUDA Kernel"); the HBM side is
 *   layer-first, the [L, P, H, D] tensor of the Strata guide,
 *   "Two-Dimensional Memory Layout Decoupling", item 1.  K and V are separate
 *   objects per layer, as the Tutti summary's Figure 4 (2L objects per block)
 *   describes.
 *
 *   Block table. Token t of a span lives on logical page p = t / bs at slot
 *   j = t % bs of block table[p] (vLLM-style page blocks of 16-64 tokens,
 *   Tutti summary, "Memory management").
 *
 *   Spans and chunks. A span is (table, t_begin, t_end, first_chunk) with
 *   t_begin <= t_end (an empty span moves nothing) and t_begin on a page
 *   boundary (prefix matches end at page boundaries, Strata guide, "The
 *   Conflict Between PagedAttention and Transfer Efficiency").  The
 *   call moves layers [layer_begin, layer_end).  A span splits into chunks of
 *   chunk_layers layers x chunk_tokens tokens, layer-chunk major:
 *       c = first_chunk + lc*n_tc + tc,  lc = (l-layer_begin)/CL,
 *       tc = (t-t_begin)/CT,  n_tc = ceil((t_end-t_begin)/CT),
 *   and chunk c occupies slot (c mod n_slots) at chunk_base + slot*slot_bytes.
 *   Inside a chunk, with li = (l-layer_begin) % CL and ti = (t-t_begin) % CT:
 *     layer-first  [CL][KV][T_c][H][D], T_c = min(CT, t_end-t_begin-tc*CT)
 *     page-first   [P_c][CL][KV][bs][H][D], pi = p - (t_begin+tc*CT)/bs
 *   The page-first order is the host-side [P, L, H, D] tensor of the Strata
 *   guide ("Two-Dimensional Memory Layout Decoupling", item 2, and its
 *   register-transposition figure); a page-first chunk is padded to whole
 *   pages and its pad bytes are neither written nor read.
 *
 *   gather : CHUNK(...) := POOL(...)      (offload, pool -> chunks)
 *   scatter: POOL(...)  := CHUNK(...)     (reload,  chunks -> pool)
 *   Nothing else is written.
 *
 * The loops run span -> layer -> kv -> token -> head -> dim and copy E bytes
 * per element, exactly as the definition reads.  Optional [only_l0, only_l1)
 * evaluates just the layers in that range (same layout, fewer layers), so a
 * large transfer can be checked slice by slice.
 *
 * Threads.  Built with OpenMP, the (span, layer) pairs are shared out between
 * threads; everything inside a pair runs exactly as above.  The pairs write
 * disjoint bytes whenever the call meets the definition's preconditions: on
 * gather, a pair writes its own layer's slice of its own span's chunks (chunks
 * of different spans are distinct, and so are their staging slots); on
 * scatter, it writes its own layer's regions at its own span's blocks (the
 * spans of one scatter name distinct blocks).  A call that breaks those
 * preconditions (two writers of one byte) has no unique result in any case.
 * orc_set_threads(1) gives the single-threaded run.
 */
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int64_t num_layers, num_kv, num_heads, head_dim, elem_bytes;
    int64_t block_size, num_blocks, block_stride;
    int64_t page_layout; /* 0 = token-major pages [bs][H][D], 1 = head-major [H][bs][D] */
} orc_pool;

typedef struct {
    const int32_t *block_table; /* host array, ceil(t_end / block_size) ids */
    int64_t t_begin, t_end, first_chunk;
} orc_span;

typedef struct {
    int64_t layout; /* 0 = layer-first chunks, 1 = page-first chunks */
    int64_t chunk_layers, chunk_tokens;
    int64_t layer_begin, layer_end;
    int64_t slot_bytes, n_slots;
} orc_chunks;

#define ORC_GATHER 0
#define ORC_SCATTER 1

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

/* Byte offset, inside its pool region, of element (block b, slot j, head h, dim d). */
static int64_t pool_offset(const orc_pool *P, int64_t b, int64_t j, int64_t h, int64_t d)
{
    if (P->page_layout == 1)
        return b * P->block_stride + ((h * P->block_size + j) * P->head_dim + d) * P->elem_bytes;
    return b * P->block_stride + ((j * P->num_heads + h) * P->head_dim + d) * P->elem_bytes;
}

/* Byte offset, inside its chunk, of element (li, kv, ti, h, d) of a layer-first chunk with T_c tokens. */
static int64_t lf_offset(const orc_pool *P, int64_t li, int64_t kv, int64_t T_c, int64_t ti,
                         int64_t h, int64_t d)
{
    return ((((li * P->num_kv + kv) * T_c + ti) * P->num_heads + h) * P->head_dim + d) *
           P->elem_bytes;
}

/* Byte offset, inside its chunk, of element (pi, li, kv, j, h, d) of a page-first chunk. */
static int64_t pf_offset(const orc_pool *P, int64_t CL, int64_t pi, int64_t li, int64_t kv,
                         int64_t j, int64_t h, int64_t d)
{
    return (((((pi * CL + li) * P->num_kv + kv) * P->block_size + j) * P->num_heads + h) *
                P->head_dim + d) * P->elem_bytes;
}

/* Threads the next orc_transfer calls may use (n >= 1); without OpenMP, 1. */
void orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Threads orc_transfer uses now. */
int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * One span S and one layer l of a call: every kv, token, head and dim, in that
 * order.  Returns the number of bytes copied, or -1 if the span breaks a
 * precondition the copy needs to stay in bounds.
 */
static int64_t span_layer(int dir, const orc_pool *P, uint8_t *const *bases, const orc_span *S,
                          const orc_chunks *C, uint8_t *chunk_base, int64_t l)
{
    const int64_t KV = P->num_kv, H = P->num_heads, D = P->head_dim, E = P->elem_bytes;
    const int64_t bs = P->block_size, CL = C->chunk_layers, CT = C->chunk_tokens;
    const int64_t n_tc = ceil_div(S->t_end - S->t_begin, CT);
    const int64_t lc = (l - C->layer_begin) / CL;
    const int64_t li = (l - C->layer_begin) % CL;
    int64_t copied = 0;

    for (int64_t kv = 0; kv < KV; ++kv) {
        uint8_t *region = bases[l * KV + kv];

        for (int64_t t = S->t_begin; t < S->t_end; ++t) {
            const int64_t p = t / bs, j = t % bs;
            const int64_t b = S->block_table[p];
            if (b < 0 || b >= P->num_blocks) return -1;
            const int64_t tc = (t - S->t_begin) / CT;
            const int64_t ti = (t - S->t_begin) % CT;
            const int64_t T_c = (CT < S->t_end - S->t_begin - tc * CT)
                                    ? CT : S->t_end - S->t_begin - tc * CT;
            const int64_t c = S->first_chunk + lc * n_tc + tc;
            if (c < 0) return -1;
            uint8_t *slot = chunk_base + (c % C->n_slots) * C->slot_bytes;
            const int64_t pi = p - (S->t_begin + tc * CT) / bs;

            for (int64_t h = 0; h < H; ++h) {
                for (int64_t d = 0; d < D; ++d) {
                    uint8_t *pool_el = region + pool_offset(P, b, j, h, d);
                    int64_t co = (C->layout == 0)
                                     ? lf_offset(P, li, kv, T_c, ti, h, d)
                                     : pf_offset(P, CL, pi, li, kv, j, h, d);
                    if (co + E > C->slot_bytes) return -1;
                    uint8_t *chunk_el = slot + co;
                    if (dir == ORC_GATHER)
                        memcpy(chunk_el, pool_el, (size_t)E);
                    else
                        memcpy(pool_el, chunk_el, (size_t)E);
                    copied += E;
                }
            }
        }
    }
    return copied;
}

/*
 * Returns the number of bytes copied, or -1 if the call breaks a precondition
 * of the definition (the oracle checks only what it needs to stay in bounds).
 */
int64_t orc_transfer(int dir, const orc_pool *P, uint8_t *const *bases, const orc_span *spans,
                     int64_t n_spans, const orc_chunks *C, uint8_t *chunk_base,
                     int64_t only_l0, int64_t only_l1)
{
    const int64_t bs = P->block_size, CL = C->chunk_layers, CT = C->chunk_tokens;
    int64_t copied = 0, bad = 0;

    if (dir != ORC_GATHER && dir != ORC_SCATTER) return -1;
    if (P->page_layout != 0 && P->page_layout != 1) return -1;
    if (CL <= 0 || CT <= 0 || CT % bs != 0 || C->n_slots <= 0) return -1;
    if (C->layer_begin < 0 || C->layer_end > P->num_layers || C->layer_end <= C->layer_begin)
        return -1;
    if ((C->layer_end - C->layer_begin) % CL != 0) return -1;
    for (int64_t r = 0; r < n_spans; ++r) {
        const orc_span *S = &spans[r];
        if (S->t_begin < 0 || S->t_end < S->t_begin || S->t_begin % bs != 0) return -1;
    }

    /* span -> layer, as one loop over the (span, layer) pairs */
    const int64_t n_l = C->layer_end - C->layer_begin;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : copied, bad)
    for (int64_t it = 0; it < n_spans * n_l; ++it) {
        const int64_t r = it / n_l, l = C->layer_begin + it % n_l;
        if (l < only_l0 || l >= only_l1) continue;
        const int64_t n = span_layer(dir, P, bases, &spans[r], C, chunk_base, l);
        if (n < 0) bad += 1;
        else copied += n;
    }
    return bad ? -1 : copied;
}
