/*
 * The library's C ABI used from plain C99 (no HIP, no GPU): descriptor
 * creation and rejection, block-table preparation, slot checks, workspace
 * sizing, and the argument checks that reject a call before anything is
 * submitted.  Device pointers here are stand-in addresses that no call in
 * this program dereferences: every call below either validates host-side
 * data only or is rejected before a launch.  Prints "ok" and exits 0 when
 * every check holds.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kvp.h"

#define CHECK(cond)                                                                            \
    do {                                                                                       \
        if (!(cond)) {                                                                         \
            fprintf(stderr, "FAIL line %d: %s (last error: %s)\n", __LINE__, #cond, kvp_last_error()); \
            return 1;                                                                          \
        }                                                                                      \
    } while (0)

static kvp_pool_desc desc(int64_t num_blocks, int32_t hkv, int32_t dh, uintptr_t k, uintptr_t v, int64_t sk,
                          int64_t sv)
{
    kvp_pool_desc d;
    memset(&d, 0, sizeof d);
    d.num_blocks = num_blocks;
    d.block_size = KVP_BLOCK_SIZE;
    d.num_kv_heads = hkv;
    d.head_dim = dh;
    d.k_cache = (void *)k;
    d.v_cache = (void *)v;
    d.k_block_stride = sk;
    d.v_block_stride = sv;
    return d;
}

int main(void)
{
    const int64_t page = 2 * 16 * 128; /* one block's K (or V) pages, Hkv 2, Dh 128, in elements */
    kvp_pool *pool = NULL;
    kvp_pool_desc d;
    int64_t span = 0;
    size_t ws = 0, ws_wide = 0;

    CHECK(strncmp(kvp_version(), "kvp", 3) == 0);

    /* separate pools */
    d = desc(64, 2, 128, 0x10000000u, 0x20000000u, page, page);
    CHECK(kv_pool_create(&d, &pool) == KVP_OK && pool != NULL);
    CHECK(kvp_last_error()[0] == '\0');
    CHECK(kv_pool_span_bytes(pool, &span) == KVP_OK);
    CHECK(span == 0x10000000 + 64 * page * 2);

    /* rejections: head_dim, block_size, misaligned, overlapping K/V pages */
    {
        kvp_pool *p = NULL;
        kvp_pool_desc bad = desc(64, 2, 64, 0x10000000u, 0x20000000u, page, page);
        CHECK(kv_pool_create(&bad, &p) == KVP_ERR_UNSUPPORTED && kvp_last_error()[0] != '\0');
        bad = desc(64, 2, 128, 0x10000000u, 0x20000000u, page, page);
        bad.block_size = 32;
        CHECK(kv_pool_create(&bad, &p) == KVP_ERR_UNSUPPORTED);
        bad = desc(64, 2, 128, 0x10000002u, 0x20000000u, page, page);
        CHECK(kv_pool_create(&bad, &p) == KVP_ERR_INVALID_ARGUMENT);
        bad = desc(64, 2, 128, 0x10000000u, 0x10000000u + 64, page, page);
        CHECK(kv_pool_create(&bad, &p) == KVP_ERR_INVALID_ARGUMENT);
        bad = desc(64, 2, 128, 0x10000000u, 0x10000000u + 4 * page, 2 * page, 3 * page);
        CHECK(kv_pool_create(&bad, &p) == KVP_ERR_INVALID_ARGUMENT);
        CHECK(kv_pool_create(NULL, &p) == KVP_ERR_INVALID_ARGUMENT);
    }

    /* interleaved pool: each block holds its K pages, then its V pages */
    {
        kvp_pool *p = NULL;
        kvp_pool_desc il = desc(1000, 2, 128, 0x10000000u, 0x10000000u + 2 * page, 2 * page, 2 * page);
        CHECK(kv_pool_create(&il, &p) == KVP_OK);
        CHECK(kv_pool_destroy(p) == KVP_OK);
    }

    /* block tables: rows padded to whole 8-column tiles, unused columns
     * replaced by the row's last page (block 0 for a row without pages) */
    {
        const int32_t bt[2 * 3] = {5, 7, -1, 9, 1, 2};
        const int32_t seq[2] = {20, 48};
        int32_t out[2 * 8];
        const int32_t want[2 * 8] = {5, 7, 7, 7, 7, 7, 7, 7, 9, 1, 2, 2, 2, 2, 2, 2};
        CHECK(kvp_padded_width(3) == 8 && kvp_padded_width(8) == 8 && kvp_padded_width(9) == 16);
        CHECK(kv_prepare_block_tables(pool, bt, 2, 3, seq, out) == KVP_OK);
        CHECK(memcmp(out, want, sizeof want) == 0);
        {
            const int32_t seq_long[2] = {20, 49}; /* four pages in a three-column row */
            CHECK(kv_prepare_block_tables(pool, bt, 2, 3, seq_long, out) == KVP_ERR_INVALID_ARGUMENT);
        }
        {
            const int32_t bt_bad[3] = {5, 64, 0}; /* block 64 is outside a 64-block pool */
            const int32_t seq1[1] = {20};
            CHECK(kv_prepare_block_tables(pool, bt_bad, 1, 3, seq1, out) == KVP_ERR_INVALID_ARGUMENT);
        }
    }

    /* slot checks: negative skipped, beyond the pool or shared rejected */
    {
        const int64_t ok_slots[4] = {0, 17, -1, 1023};
        const int64_t dup[3] = {3, 5, 3};
        const int64_t far[2] = {0, 1024};
        CHECK(kvp_check_slot_mapping(pool, ok_slots, 4) == KVP_OK);
        CHECK(kvp_check_slot_mapping(pool, dup, 3) == KVP_ERR_INVALID_ARGUMENT);
        CHECK(kvp_check_slot_mapping(pool, far, 2) == KVP_ERR_INVALID_ARGUMENT);
    }

    /* workspace sizes grow with the split width */
    CHECK(kvp_workspace_bytes(pool, 8, 4, 7168, &ws) == KVP_OK && ws > 0);
    CHECK(kvp_workspace_bytes_split(pool, 8, 4, 7168, 512, &ws_wide) == KVP_OK && ws_wide > ws);
    CHECK(kvp_workspace_bytes_split(pool, 8, 4, 7168, 24, &ws_wide) == KVP_ERR_INVALID_ARGUMENT);

    /* calls rejected before any submission (stand-in device addresses) */
    {
        void *q = (void *)(uintptr_t)0x30000000u, *o = (void *)(uintptr_t)0x40000000u;
        const int32_t *bt = (const int32_t *)(uintptr_t)0x50000000u;
        const int32_t *sl = (const int32_t *)(uintptr_t)0x60000000u, *qsl = (const int32_t *)(uintptr_t)0x70000000u;
        void *w = (void *)(uintptr_t)0x80000000u;
        const int64_t row = 8 * 128;
        CHECK(paged_attention(NULL, q, row, o, row, 8, 4, bt, 448, sl, qsl, 1, 7168, 0.088f, 1, w, ws, NULL) ==
              KVP_ERR_INVALID_ARGUMENT);
        CHECK(paged_attention(pool, q, row, o, row, 8, 4, bt, 448, sl, qsl, 1, 7168, -1.f, 1, w, ws, NULL) ==
              KVP_ERR_INVALID_ARGUMENT);
        CHECK(paged_attention(pool, q, row, o, row, 5, 4, bt, 448, sl, qsl, 1, 7168, 0.088f, 1, w, ws, NULL) ==
              KVP_ERR_UNSUPPORTED); /* 5 query heads over 2 kv heads */
        CHECK(paged_attention(pool, q, 34 * 128, o, 34 * 128, 34, 4, bt, 448, sl, qsl, 1, 7168, 0.088f, 1, w, ws,
                              NULL) == KVP_ERR_UNSUPPORTED); /* group of 17 */
        CHECK(paged_attention(pool, q, row, o, row, 8, 4, bt, 447, sl, qsl, 1, 7168, 0.088f, 1, w, ws, NULL) ==
              KVP_ERR_INVALID_ARGUMENT);
        CHECK(paged_attention(pool, q, row, o, row, 8, 4, bt, 448, sl, qsl, 1, 7168, 0.088f, 1, w, ws - 16, NULL) ==
              KVP_ERR_WORKSPACE_TOO_SMALL);
        CHECK(paged_attention(pool, q, row, o, row, 8, 0, bt, 448, sl, qsl, 1, 7168, 0.088f, 1, NULL, 0, NULL) ==
              KVP_OK); /* nothing to do */
        CHECK(kvp_merge_attention(q, NULL, o, NULL, o, NULL, 4, 8, 128, NULL) == KVP_ERR_INVALID_ARGUMENT);
    }

    {
        kvp_counters c;
        CHECK(kvp_reset_counters() == KVP_OK);
        CHECK(kvp_get_counters(&c) == KVP_OK);
        CHECK(c.split_kv_launches == 0 && c.prefill_launches == 0 && c.reshape_and_cache_launches == 0);
    }
    CHECK(kv_pool_destroy(pool) == KVP_OK);
    puts("ok");
    return 0;
}
