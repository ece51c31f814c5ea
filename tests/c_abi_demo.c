/* c_abi_demo.c -- the C ABI used from plain C (no Python, no PyTorch): a test.
 *
 * Allocates one pool of 3 layers x K/V with hipMalloc, fills it with a byte
 * pattern, gathers two requests (one with a partial last page) into layer-first
 * chunks in device memory, scatters them into a second, sentinel-filled pool, and
 * checks both results byte for byte against the CPU oracle (oracle/oracle.c, linked
 * in: tests may use it).  Also drives the allocator and the pinned ring once.
 * Prints one line per step and "c_abi_demo ok" at the end; exits non-zero on any
 * mismatch or error.
 */
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kvxfer.h"

/* the oracle's interface (oracle/oracle.c) */
typedef struct {
    int64_t num_layers, num_kv, num_heads, head_dim, elem_bytes;
    int64_t block_size, num_blocks, block_stride;
    int64_t page_layout;
} orc_pool;
typedef struct {
    const int32_t *block_table;
    int64_t t_begin, t_end, first_chunk;
} orc_span;
typedef struct {
    int64_t layout, chunk_layers, chunk_tokens, layer_begin, layer_end, slot_bytes, n_slots;
} orc_chunks;
int64_t orc_transfer(int dir, const orc_pool *P, uint8_t *const *bases, const orc_span *spans,
                     int64_t n_spans, const orc_chunks *C, uint8_t *chunk_base, int64_t only_l0,
                     int64_t only_l1);

#define CHECK_HIP(x)                                                                    \
    do {                                                                                \
        hipError_t e_ = (x);                                                            \
        if (e_ != hipSuccess) {                                                         \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
            return 1;                                                                   \
        }                                                                               \
    } while (0)
#define CHECK_KV(x)                                                                          \
    do {                                                                                     \
        int r_ = (x);                                                                        \
        if (r_ != KV_OK) {                                                                   \
            fprintf(stderr, "%s:%d: %s (%d)\n", __FILE__, __LINE__, kv_strerror(r_), r_); \
            return 1;                                                                        \
        }                                                                                    \
    } while (0)

enum { L = 3, KV = 2, H = 2, D = 64, E = 2, BS = 16, NB = 96, CT = 64 };

int main(void)
{
    const int64_t tok = H * D * E, page = BS * tok, region = (int64_t)NB * page;
    const int64_t n_reg = L * KV;
    /* two requests: 200 tokens (13 pages, the last partial) and 96 tokens (6 pages) */
    const int64_t t_end[2] = {200, 96};
    int32_t tables[2][13];
    int used = 0;
    for (int r = 0; r < 2; ++r)
        for (int p = 0; p < 13; ++p) tables[r][p] = (int32_t)((used++ * 37) % NB); /* distinct ids */
    const int64_t n_tc[2] = {(t_end[0] + CT - 1) / CT, (t_end[1] + CT - 1) / CT};
    const int64_t first_chunk[2] = {0, n_tc[0]}; /* one layer chunk of all 3 layers */
    const int64_t slot = (int64_t)L * KV * CT * tok, n_slots = n_tc[0] + n_tc[1];

    uint8_t *h_pool = malloc(n_reg * region), *h_stg = malloc(slot * n_slots);
    uint8_t *e_pool = malloc(n_reg * region), *e_stg = malloc(slot * n_slots);
    uint8_t *g_pool = malloc(n_reg * region), *g_stg = malloc(slot * n_slots);
    if (!h_pool || !h_stg || !e_pool || !e_stg || !g_pool || !g_stg) return 1;
    for (int64_t i = 0; i < n_reg * region; ++i) h_pool[i] = (uint8_t)(i * 131 + (i >> 9));
    memset(h_stg, 0xA5, slot * n_slots);

    uint8_t *d_pool, *d_pool2, *d_stg;
    int32_t *d_tab;
    CHECK_HIP(hipMalloc((void **)&d_pool, n_reg * region));
    CHECK_HIP(hipMalloc((void **)&d_pool2, n_reg * region));
    CHECK_HIP(hipMalloc((void **)&d_stg, slot * n_slots));
    CHECK_HIP(hipMalloc((void **)&d_tab, sizeof(tables)));
    CHECK_HIP(hipMemcpy(d_pool, h_pool, n_reg * region, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemset(d_pool2, 0xA5, n_reg * region));
    CHECK_HIP(hipMemcpy(d_stg, h_stg, slot * n_slots, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_tab, tables, sizeof(tables), hipMemcpyHostToDevice));

    void *bases[L * KV], *bases2[L * KV];
    uint8_t *h_bases[L * KV], *e_bases[L * KV];
    for (int i = 0; i < n_reg; ++i) {
        bases[i] = d_pool + i * region;
        bases2[i] = d_pool2 + i * region;
        h_bases[i] = h_pool + i * region;
        e_bases[i] = e_pool + i * region;
    }
    kv_pool_desc desc = {L, KV, H, D, E, BS, KV_PAGE_TOKEN_MAJOR, NB, page, bases};
    kv_pool_desc desc2 = desc;
    desc2.bases = bases2;
    kv_pool *pool, *pool2;
    CHECK_KV(kv_pool_create(&desc, &pool));
    CHECK_KV(kv_pool_create(&desc2, &pool2));

    kv_span spans[2];
    orc_span ospans[2];
    for (int r = 0; r < 2; ++r) {
        spans[r] = (kv_span){d_tab + 13 * r, 13, 0, t_end[r], first_chunk[r]};
        ospans[r] = (orc_span){tables[r], 0, t_end[r], first_chunk[r]};
    }
    kv_chunk_spec spec = {KV_LAYER_FIRST, L, CT, 0, L, d_stg, slot, n_slots, 0, 0};
    kv_transfer_info info;
    CHECK_KV(kv_check_transfer(&desc, spans, 2, &spec, &info));
    printf("c_abi_demo: %lld tiles, %lld chunks, %lld payload bytes\n", (long long)info.tiles,
           (long long)info.chunks, (long long)info.payload_bytes);

    /* gather, then compare the staging buffer with the oracle's */
    CHECK_KV(kv_gather_chunks(pool, spans, 2, &spec, 0));
    int32_t bits = 0;
    CHECK_KV(kv_pool_get_error(pool, 0, &bits));
    CHECK_HIP(hipMemcpy(g_stg, d_stg, slot * n_slots, hipMemcpyDeviceToHost));
    const orc_pool op = {L, KV, H, D, E, BS, NB, page, 0};
    const orc_chunks oc = {0, L, CT, 0, L, slot, n_slots};
    memcpy(e_stg, h_stg, slot * n_slots);
    if (orc_transfer(0, &op, h_bases, ospans, 2, &oc, e_stg, 0, L) != info.payload_bytes) return 1;
    if (memcmp(g_stg, e_stg, slot * n_slots) != 0) {
        fprintf(stderr, "gather differs from the oracle\n");
        return 1;
    }
    printf("c_abi_demo: gather matches the oracle\n");

    /* scatter the gathered chunks into the sentinel pool */
    CHECK_KV(kv_scatter_chunks(pool2, spans, 2, &spec, 0));
    CHECK_KV(kv_pool_get_error(pool2, 0, &bits));
    CHECK_HIP(hipMemcpy(g_pool, d_pool2, n_reg * region, hipMemcpyDeviceToHost));
    memset(e_pool, 0xA5, n_reg * region);
    if (orc_transfer(1, &op, e_bases, ospans, 2, &oc, e_stg, 0, L) != info.payload_bytes) return 1;
    if (memcmp(g_pool, e_pool, n_reg * region) != 0) {
        fprintf(stderr, "scatter differs from the oracle\n");
        return 1;
    }
    printf("c_abi_demo: scatter matches the oracle\n");

    /* the allocator and a pinned ring, once each */
    int32_t ids[4];
    int64_t free_n = 0;
    CHECK_KV(kv_pool_alloc_blocks(pool, 4, ids));
    CHECK_KV(kv_pool_free_count(pool, &free_n));
    if (free_n != NB - 4) return 1;
    CHECK_KV(kv_pool_free_blocks(pool, 4, ids));
    kv_ring *ring;
    void *ring_host, *ring_dev;
    CHECK_KV(kv_ring_create(slot, n_slots, KV_RING_COHERENT, &ring));
    CHECK_KV(kv_ring_slot(ring, 0, &ring_host, &ring_dev));
    spec.base = ring_dev;
    CHECK_KV(kv_gather_chunks(pool, spans, 2, &spec, 0));
    CHECK_KV(kv_ring_record(ring, 0, n_slots, 0));
    CHECK_KV(kv_ring_wait(ring, 0, n_slots));
    /* bytes the gather writes are those where the oracle's result differs from the
       0xA5 fill, plus any payload byte that happens to be 0xA5: compare where written */
    for (int64_t i = 0; i < slot * n_slots; ++i)
        if (e_stg[i] != 0xA5 && ((uint8_t *)ring_host)[i] != e_stg[i]) {
            fprintf(stderr, "ring gather differs at %lld\n", (long long)i);
            return 1;
        }
    printf("c_abi_demo: pinned-ring gather matches the oracle\n");
    CHECK_KV(kv_ring_destroy(ring));

    CHECK_KV(kv_pool_destroy(pool));
    CHECK_KV(kv_pool_destroy(pool2));
    CHECK_HIP(hipFree(d_pool));
    CHECK_HIP(hipFree(d_pool2));
    CHECK_HIP(hipFree(d_stg));
    CHECK_HIP(hipFree(d_tab));
    free(h_pool), free(h_stg), free(e_pool), free(e_stg), free(g_pool), free(g_stg);
    printf("c_abi_demo ok\n");
    return 0;
}
