/*
 * The composition driven from C through the library's C ABI, as a serving
 * engine written in C would call it: device buffers from hipMalloc, a HIP
 * stream, plain pointers.  Built as a shared library whose one entry point
 * the GPU test calls in its own process (no child process).  TEST
 * INFRASTRUCTURE: it links the CPU oracle to check the results.
 *
 * kvp_c_e2e(head_dim, msg, msg_len) -> 0 when every check holds, else 1
 * with the reason in msg:
 *   1. reshape_and_cache of every token of three sequences into shuffled
 *      pages of a NaN-poisoned pool: the pool equals the oracle's bit for bit
 *      ("test(rocm): ReshapeAndCache->PagedAttention composition at real
 *      dims", What changed);
 *   2. causal prefill of the three sequences through their block tables:
 *      within tolerance of the oracle (max |err| <= 2e-2, RMS of the error
 *      <= 1e-2 of the RMS of the reference);
 *   3. decode of each sequence's last token: bitwise the prefill's last row
 *      ("fix(rocm): stabilize direct paged CK attention for bitwise R/R",
 *      intro and Additional checks);
 *   4. the dispatch counters show both paths ran.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kvp.h"

/* the CPU oracle (oracle/kvp_oracle.c) */
int oracle_reshape_and_cache(uint16_t *k_pool, uint16_t *v_pool, int64_t num_blocks, int Hkv, int D,
                             int64_t k_block_stride, int64_t v_block_stride, const uint16_t *k, const uint16_t *v,
                             int64_t T, int64_t k_token_stride, int64_t v_token_stride, const int64_t *slot_mapping);
int oracle_paged_attention(float *out, const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                           int64_t num_blocks, int64_t k_block_stride, int64_t v_block_stride,
                           const int32_t *block_tables, int B, int W, const int32_t *seq_lens,
                           const int32_t *query_start_loc, int Hq, int Hkv, int D, float scale, int causal,
                           const int64_t *rows, int64_t n_rows, float *lse);

enum { B = 3, HQ = 8, HKV = 2, NBLK = 96 };
static const int32_t LENS[B] = {130, 257, 64};

static uint64_t rng_state;
static double uniform(void) /* 64-bit LCG, top 53 bits */
{
    rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(rng_state >> 11) / 9007199254740992.0;
}
static uint16_t bf16_bits(float f) /* round to nearest even */
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
static float bf16_value(uint16_t b)
{
    const uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

#define FAIL(...)                                  \
    do {                                           \
        snprintf(msg, (size_t)msg_len, __VA_ARGS__); \
        rc = 1;                                    \
        goto done;                                 \
    } while (0)
#define HIPCHECK(x)                                                                        \
    do {                                                                                   \
        const hipError_t e_ = (x);                                                         \
        if (e_ != hipSuccess)                                                              \
            FAIL("%s: %s", #x, hipGetErrorString(e_));                                     \
    } while (0)
#define KVPCHECK(x)                                                                        \
    do {                                                                                   \
        const int r_ = (x);                                                                \
        if (r_ != KVP_OK)                                                                  \
            FAIL("%s -> %d: %s", #x, r_, kvp_last_error());                                \
    } while (0)

int kvp_c_e2e(int D, char *msg, int msg_len)
{
    int rc = 0;
    const int64_t page = (int64_t)HKV * KVP_BLOCK_SIZE * D; /* one block's K (or V) pages, elements */
    const int64_t pool_elems = NBLK * page;
    const float scale = (float)(1.0 / sqrt((double)D));
    int64_t T = 0;
    int32_t qsl[B + 1], W = 0;
    uint16_t *h_k = NULL, *h_v = NULL, *h_q = NULL, *ref_kp = NULL, *ref_vp = NULL, *got_kp = NULL, *got_vp = NULL;
    uint16_t *h_out = NULL, *h_dec = NULL, *h_qd = NULL;
    int64_t *slots = NULL;
    int32_t *bt = NULL, *btp = NULL, perm[NBLK];
    float *ref = NULL;
    void *d_kp = NULL, *d_vp = NULL, *d_k = NULL, *d_v = NULL, *d_q = NULL, *d_out = NULL, *d_bt = NULL;
    void *d_sl = NULL, *d_qsl = NULL, *d_slots = NULL, *d_ws = NULL, *d_qd = NULL, *d_dec = NULL, *d_qsld = NULL;
    hipStream_t s = NULL;
    kvp_pool *pool = NULL;
    kvp_counters c0, c1;
    size_t ws_bytes = 0;
    int32_t wp = 0;

    if (D != 128 && D != 256 && D != 512)
        FAIL("head_dim %d", D);
    rng_state = 0x9E3779B97F4A7C15ull ^ (uint64_t)D;
    qsl[0] = 0;
    for (int b = 0; b < B; ++b) {
        qsl[b + 1] = qsl[b] + LENS[b];
        W += (LENS[b] + KVP_BLOCK_SIZE - 1) / KVP_BLOCK_SIZE;
    }
    T = qsl[B];
    /* block tables: the pool's blocks in shuffled order, row after row */
    for (int i = 0; i < NBLK; ++i)
        perm[i] = i;
    for (int i = NBLK - 1; i > 0; --i) {
        const int j = (int)(uniform() * (i + 1));
        const int32_t t = perm[i];
        perm[i] = perm[j];
        perm[j] = t;
    }
    bt = calloc((size_t)B * W, sizeof *bt);
    slots = malloc((size_t)T * sizeof *slots);
    h_k = malloc((size_t)T * HKV * D * 2);
    h_v = malloc((size_t)T * HKV * D * 2);
    h_q = malloc((size_t)T * HQ * D * 2);
    ref_kp = malloc((size_t)pool_elems * 2);
    ref_vp = malloc((size_t)pool_elems * 2);
    got_kp = malloc((size_t)pool_elems * 2);
    got_vp = malloc((size_t)pool_elems * 2);
    h_out = malloc((size_t)T * HQ * D * 2);
    ref = malloc((size_t)T * HQ * D * sizeof *ref);
    h_qd = malloc((size_t)B * HQ * D * 2);
    h_dec = malloc((size_t)B * HQ * D * 2);
    if (!bt || !slots || !h_k || !h_v || !h_q || !ref_kp || !ref_vp || !got_kp || !got_vp || !h_out || !ref ||
        !h_qd || !h_dec)
        FAIL("host allocation");
    {
        int used = 0;
        for (int b = 0; b < B; ++b) {
            const int np = (LENS[b] + KVP_BLOCK_SIZE - 1) / KVP_BLOCK_SIZE;
            for (int c = 0; c < np; ++c)
                bt[(int64_t)b * W + c] = perm[used++];
            for (int i = 0; i < LENS[b]; ++i)
                slots[qsl[b] + i] = (int64_t)bt[(int64_t)b * W + i / KVP_BLOCK_SIZE] * KVP_BLOCK_SIZE + i % KVP_BLOCK_SIZE;
        }
    }
    for (int64_t i = 0; i < T * HKV * D; ++i) {
        h_k[i] = bf16_bits((float)(uniform() - 0.5));
        h_v[i] = bf16_bits((float)(uniform() - 0.5));
    }
    for (int64_t i = 0; i < T * HQ * D; ++i)
        h_q[i] = bf16_bits((float)(2.0 * uniform() - 1.0));
    for (int64_t i = 0; i < pool_elems; ++i)
        ref_kp[i] = ref_vp[i] = 0x7FC1; /* NaN poison in every unwritten slot */

    /* device side */
    HIPCHECK(hipStreamCreate(&s));
    HIPCHECK(hipMalloc(&d_kp, (size_t)pool_elems * 2));
    HIPCHECK(hipMalloc(&d_vp, (size_t)pool_elems * 2));
    HIPCHECK(hipMemcpy(d_kp, ref_kp, (size_t)pool_elems * 2, hipMemcpyHostToDevice));
    HIPCHECK(hipMemcpy(d_vp, ref_vp, (size_t)pool_elems * 2, hipMemcpyHostToDevice));
    HIPCHECK(hipMalloc(&d_k, (size_t)T * HKV * D * 2));
    HIPCHECK(hipMalloc(&d_v, (size_t)T * HKV * D * 2));
    HIPCHECK(hipMalloc(&d_q, (size_t)T * HQ * D * 2));
    HIPCHECK(hipMalloc(&d_out, (size_t)T * HQ * D * 2));
    HIPCHECK(hipMalloc(&d_slots, (size_t)T * sizeof *slots));
    HIPCHECK(hipMemcpy(d_k, h_k, (size_t)T * HKV * D * 2, hipMemcpyHostToDevice));
    HIPCHECK(hipMemcpy(d_v, h_v, (size_t)T * HKV * D * 2, hipMemcpyHostToDevice));
    HIPCHECK(hipMemcpy(d_q, h_q, (size_t)T * HQ * D * 2, hipMemcpyHostToDevice));
    HIPCHECK(hipMemcpy(d_slots, slots, (size_t)T * sizeof *slots, hipMemcpyHostToDevice));
    {
        kvp_pool_desc d;
        memset(&d, 0, sizeof d);
        d.num_blocks = NBLK;
        d.block_size = KVP_BLOCK_SIZE;
        d.num_kv_heads = HKV;
        d.head_dim = D;
        d.k_cache = d_kp;
        d.v_cache = d_vp;
        d.k_block_stride = d.v_block_stride = page;
        KVPCHECK(kv_pool_create(&d, &pool));
    }
    KVPCHECK(kvp_get_counters(&c0));

    /* 1. the cache write, bit for bit */
    KVPCHECK(reshape_and_cache(pool, d_k, d_v, T, (int64_t)HKV * D, (int64_t)HKV * D, d_slots, s));
    if (oracle_reshape_and_cache(ref_kp, ref_vp, NBLK, HKV, D, page, page, h_k, h_v, T, (int64_t)HKV * D,
                                 (int64_t)HKV * D, slots) != 0)
        FAIL("oracle_reshape_and_cache rejected the slots");
    HIPCHECK(hipStreamSynchronize(s));
    HIPCHECK(hipMemcpy(got_kp, d_kp, (size_t)pool_elems * 2, hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(got_vp, d_vp, (size_t)pool_elems * 2, hipMemcpyDeviceToHost));
    if (memcmp(got_kp, ref_kp, (size_t)pool_elems * 2) != 0 || memcmp(got_vp, ref_vp, (size_t)pool_elems * 2) != 0)
        FAIL("D %d: pool after reshape_and_cache differs from the oracle's", D);

    /* 2. causal prefill of every token */
    wp = kvp_padded_width(W);
    btp = malloc((size_t)B * wp * sizeof *btp);
    if (!btp)
        FAIL("host allocation");
    KVPCHECK(kv_prepare_block_tables(pool, bt, B, W, LENS, btp));
    HIPCHECK(hipMalloc(&d_bt, (size_t)B * wp * sizeof *btp));
    HIPCHECK(hipMalloc(&d_sl, sizeof LENS));
    HIPCHECK(hipMalloc(&d_qsl, sizeof qsl));
    HIPCHECK(hipMemcpy(d_bt, btp, (size_t)B * wp * sizeof *btp, hipMemcpyHostToDevice));
    HIPCHECK(hipMemcpy(d_sl, LENS, sizeof LENS, hipMemcpyHostToDevice));
    HIPCHECK(hipMemcpy(d_qsl, qsl, sizeof qsl, hipMemcpyHostToDevice));
    {
        int32_t maxl = 0;
        for (int b = 0; b < B; ++b)
            maxl = LENS[b] > maxl ? LENS[b] : maxl;
        KVPCHECK(paged_attention(pool, d_q, (int64_t)HQ * D, d_out, (int64_t)HQ * D, HQ, B, (const int32_t *)d_bt, wp,
                                 (const int32_t *)d_sl, (const int32_t *)d_qsl, maxl, maxl, scale, 1, NULL, 0, s));
        HIPCHECK(hipStreamSynchronize(s));
        HIPCHECK(hipMemcpy(h_out, d_out, (size_t)T * HQ * D * 2, hipMemcpyDeviceToHost));
        if (oracle_paged_attention(ref, h_q, ref_kp, ref_vp, NBLK, page, page, btp, B, wp, LENS, qsl, HQ, HKV, D, scale,
                                   1, NULL, 0, NULL) != 0)
            FAIL("oracle_paged_attention rejected the metadata");
        {
            double max_err = 0, se = 0, sr = 0;
            for (int64_t i = 0; i < T * HQ * D; ++i) {
                const double g = bf16_value(h_out[i]), r = ref[i], e = fabs(g - r);
                if (!(e <= max_err))
                    max_err = isnan(e) ? INFINITY : (e > max_err ? e : max_err);
                se += e * e;
                sr += r * r;
            }
            if (!(max_err <= 2e-2) || !(sqrt(se) <= 1e-2 * sqrt(sr)))
                FAIL("D %d prefill: max |err| %.3g, relative RMS %.3g", D, max_err, sqrt(se / (sr > 0 ? sr : 1)));
        }

        /* 3. decode of each row's last token: the prefill's last row, bit for bit */
        {
            int32_t qsld[B + 1];
            for (int b = 0; b < B; ++b)
                memcpy(h_qd + (int64_t)b * HQ * D, h_q + (int64_t)(qsl[b + 1] - 1) * HQ * D, (size_t)HQ * D * 2);
            for (int b = 0; b <= B; ++b)
                qsld[b] = b;
            KVPCHECK(kvp_workspace_bytes(pool, HQ, B, maxl, &ws_bytes));
            HIPCHECK(hipMalloc(&d_ws, ws_bytes));
            HIPCHECK(hipMalloc(&d_qd, (size_t)B * HQ * D * 2));
            HIPCHECK(hipMalloc(&d_dec, (size_t)B * HQ * D * 2));
            HIPCHECK(hipMalloc(&d_qsld, sizeof qsld));
            HIPCHECK(hipMemcpy(d_qd, h_qd, (size_t)B * HQ * D * 2, hipMemcpyHostToDevice));
            HIPCHECK(hipMemcpy(d_qsld, qsld, sizeof qsld, hipMemcpyHostToDevice));
            KVPCHECK(paged_attention(pool, d_qd, (int64_t)HQ * D, d_dec, (int64_t)HQ * D, HQ, B, (const int32_t *)d_bt,
                                     wp, (const int32_t *)d_sl, (const int32_t *)d_qsld, 1, maxl, scale, 1, d_ws,
                                     ws_bytes, s));
            HIPCHECK(hipStreamSynchronize(s));
            HIPCHECK(hipMemcpy(h_dec, d_dec, (size_t)B * HQ * D * 2, hipMemcpyDeviceToHost));
            for (int b = 0; b < B; ++b)
                if (memcmp(h_dec + (int64_t)b * HQ * D, h_out + (int64_t)(qsl[b + 1] - 1) * HQ * D, (size_t)HQ * D * 2))
                    FAIL("D %d: decode of row %d differs from the prefill's last row", D, b);
        }
    }

    /* 4. both paths ran */
    KVPCHECK(kvp_get_counters(&c1));
    if (c1.reshape_and_cache_launches <= c0.reshape_and_cache_launches || c1.prefill_launches <= c0.prefill_launches ||
        c1.split_kv_launches <= c0.split_kv_launches)
        FAIL("D %d: dispatch counters did not move", D);
    snprintf(msg, (size_t)msg_len, "ok");

done:
    if (s)
        hipStreamSynchronize(s);
    if (pool)
        kv_pool_destroy(pool);
    {
        void *dev[] = {d_kp, d_vp, d_k, d_v, d_q, d_out, d_bt, d_sl, d_qsl, d_slots, d_ws, d_qd, d_dec, d_qsld};
        for (size_t i = 0; i < sizeof dev / sizeof dev[0]; ++i)
            if (dev[i])
                hipFree(dev[i]);
    }
    if (s)
        hipStreamDestroy(s);
    free(bt);
    free(btp);
    free(slots);
    free(h_k);
    free(h_v);
    free(h_q);
    free(ref_kp);
    free(ref_vp);
    free(got_kp);
    free(got_vp);
    free(h_out);
    free(ref);
    free(h_qd);
    free(h_dec);
    return rc;
}
