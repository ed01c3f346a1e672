/*
 * kvp_oracle.c -- plain, slow, obviously-correct CPU reference for the paged
 * BF16 KV-cache composition (cache scatter, then paged GQA attention).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant
 * with the HIP library; the pool layout below is written out again here
 * from its definition.
 *
 * Sources (web pages; cited by title and section):
 *   [Composition]  "test(rocm): ReshapeAndCache->PagedAttention composition
 *                   at real dims" -- What changed; review thread (slot of a
 *                   logical token = block_table[i / BS] * BS + i % BS, and
 *                   the worked example with table {3,1,2,0}).
 *   [Bitwise R/R]  "fix(rocm): stabilize direct paged CK attention for
 *                   bitwise R/R" -- Changes (padded, sanitised tail page
 *                   tables; decode request-to-query mapping), Additional
 *                   checks (full/suffix queries, tails 128/17/1).
 *
 * Numerics: the attention is the textbook definition evaluated on the
 * logically reassembled sequence, accumulated in FP32 (d ascending for the
 * dot products, keys ascending for the sums), with expf.  Parallelism is
 * only across independent (query row, head) outputs, so results do not
 * depend on the number of threads.
 *
 * Pool layout (a format both sides must agree on; restated, not shared):
 *   block b, kv head h, token t (0..15), dim d:
 *     K element at k_pool[b*k_block_stride + h*16*D + (d/8)*128 + t*8 + d%8]
 *     V element at v_pool[b*v_block_stride + h*16*D + d*16 + t]
 *   i.e. a K page is [D/8][16 tokens][8 dims] and a V page is [D][16 tokens].
 *
 * LSE (log-sum-exp) output [Bitwise R/R, Additional checks: the causal
 * and LSE results are compared with decode]: the pages name the quantity
 * only; it is read here as the natural-log log-sum-exp of the scaled scores
 * a query row sees, lse = m + log(l) with m and l of the softmax below.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - GQA: query head h uses kv head h / (Hq/Hkv).
 *   - Suffix queries are bottom-right aligned: query r of a row with q_len
 *     queries and seq_len keys sits at position seq_len - q_len + r.
 *   - Negative slots are skipped; duplicate or out-of-range slots are errors.
 *   - Unused block-table columns are replaced by the row's last valid block
 *     (block 0 for a row with no blocks); tables are padded to a multiple of
 *     8 columns (one 128-token KV tile of 16-token pages).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_BS 16

static float bf16_to_f32(uint16_t b)
{
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Element offsets of the layout described in the header. */
static int64_t k_off(int64_t block, int64_t k_block_stride, int h, int t, int d, int D)
{
    return block * k_block_stride + (int64_t)h * ORACLE_BS * D
         + (int64_t)(d / 8) * (ORACLE_BS * 8) + (int64_t)t * 8 + (d % 8);
}

static int64_t v_off(int64_t block, int64_t v_block_stride, int h, int t, int d, int D)
{
    return block * v_block_stride + (int64_t)h * ORACLE_BS * D + (int64_t)d * ORACLE_BS + t;
}

/*
 * Cache scatter [Composition, What changed]: for every token i with
 * slot s = slot_mapping[i] >= 0, copy the bits of k[i][h][:] and v[i][h][:]
 * into block s / 16, offset s % 16.  Every other element is left unchanged.
 * Returns 0, or -1 (nothing written) for an out-of-range or duplicated slot.
 */
int oracle_reshape_and_cache(uint16_t *k_pool, uint16_t *v_pool, int64_t num_blocks,
                             int Hkv, int D, int64_t k_block_stride, int64_t v_block_stride,
                             const uint16_t *k, const uint16_t *v, int64_t T,
                             int64_t k_token_stride, int64_t v_token_stride,
                             const int64_t *slot_mapping)
{
    int64_t nslots = num_blocks * ORACLE_BS;
    /* validate first so that a rejected call leaves the pool untouched */
    for (int64_t i = 0; i < T; ++i) {
        int64_t s = slot_mapping[i];
        if (s >= nslots)
            return -1;
        if (s < 0)
            continue;
        for (int64_t j = 0; j < i; ++j)
            if (slot_mapping[j] == s)
                return -1;
    }
    for (int64_t i = 0; i < T; ++i) {
        int64_t s = slot_mapping[i];
        if (s < 0)
            continue;
        int64_t block = s / ORACLE_BS;
        int t = (int)(s % ORACLE_BS);
        for (int h = 0; h < Hkv; ++h)
            for (int d = 0; d < D; ++d) {
                k_pool[k_off(block, k_block_stride, h, t, d, D)] = k[i * k_token_stride + (int64_t)h * D + d];
                v_pool[v_off(block, v_block_stride, h, t, d, D)] = v[i * v_token_stride + (int64_t)h * D + d];
            }
    }
    return 0;
}

/* Reads logical token j of a sequence through its block-table row
 * [Composition, review thread]: physical block row[j / 16], offset j % 16. */
static float k_logical(const uint16_t *k_pool, int64_t k_block_stride, const int32_t *row,
                       int h, int64_t j, int d, int D)
{
    int64_t block = row[j / ORACLE_BS];
    return bf16_to_f32(k_pool[k_off(block, k_block_stride, h, (int)(j % ORACLE_BS), d, D)]);
}

static float v_logical(const uint16_t *v_pool, int64_t v_block_stride, const int32_t *row,
                       int h, int64_t j, int d, int D)
{
    int64_t block = row[j / ORACLE_BS];
    return bf16_to_f32(v_pool[v_off(block, v_block_stride, h, (int)(j % ORACLE_BS), d, D)]);
}

/*
 * One query row of paged attention, one query head h.  b is the sequence, r
 * the query index within that sequence's queries.  Writes out[h][D] (FP32)
 * and lse[h].  Returns the number of keys the row attended to.
 */
static int64_t attend_row(float *out, const uint16_t *qrow, const uint16_t *k_pool,
                          const uint16_t *v_pool, int64_t k_block_stride, int64_t v_block_stride,
                          const int32_t *bt_row, int64_t seq_len, int64_t q_len, int64_t r,
                          int Hq, int Hkv, int D, float scale, int causal,
                          float *lse /* [Hq] or NULL */, float *s /* scratch [seq_len] */, int h)
{
    int G = Hq / Hkv;
    int64_t pos = seq_len - q_len + r;               /* bottom-right alignment */
    int64_t nkeys = causal ? pos + 1 : seq_len;      /* keys 0 .. nkeys-1 visible */
    int g = h / G;
    const uint16_t *qh = qrow + (int64_t)h * D;
    /* scores: s_j = scale * sum_d q[d] * K_j[d], FP32, d ascending */
    float m = -INFINITY;
    for (int64_t j = 0; j < nkeys; ++j) {
        float dot = 0.0f;
        for (int d = 0; d < D; ++d)
            dot += bf16_to_f32(qh[d]) * k_logical(k_pool, k_block_stride, bt_row, g, j, d, D);
        s[j] = scale * dot;
        if (s[j] > m)
            m = s[j];
    }
    /* softmax weights and their sum, keys ascending */
    float l = 0.0f;
    for (int64_t j = 0; j < nkeys; ++j) {
        s[j] = expf(s[j] - m);
        l += s[j];
    }
    /* weighted sum of V rows, keys ascending, then normalise */
    for (int d = 0; d < D; ++d) {
        float acc = 0.0f;
        for (int64_t j = 0; j < nkeys; ++j)
            acc += s[j] * v_logical(v_pool, v_block_stride, bt_row, g, j, d, D);
        out[(int64_t)h * D + d] = acc / l;
    }
    /* log-sum-exp of the scaled scores: log(sum_j exp(s_j)) = m + log(l) */
    if (lse)
        lse[h] = m + logf(l);
    return nkeys;
}

/*
 * Paged attention over a ragged batch.
 *   q:  [Tq][Hq][D] BF16 bits, Tq = query_start_loc[B]
 *   block_tables: [B][W] int32, seq_lens: [B], query_start_loc: [B+1]
 *   rows: optional list of n_rows query-row indices in [0, Tq) to compute;
 *         NULL computes every row.  out is [n_rows or Tq][Hq][D] FP32.
 * Returns 0, or -1 for inconsistent metadata.
 */
int oracle_paged_attention(float *out, const uint16_t *q, const uint16_t *k_pool,
                           const uint16_t *v_pool, int64_t num_blocks, int64_t k_block_stride,
                           int64_t v_block_stride, const int32_t *block_tables, int B, int W,
                           const int32_t *seq_lens, const int32_t *query_start_loc, int Hq,
                           int Hkv, int D, float scale, int causal, const int64_t *rows,
                           int64_t n_rows, float *lse /* [n_rows or Tq][Hq] or NULL */)
{
    if (Hkv <= 0 || Hq % Hkv != 0)
        return -1;
    for (int b = 0; b < B; ++b) {
        int64_t q_len = (int64_t)query_start_loc[b + 1] - query_start_loc[b];
        if (q_len < 0 || q_len > seq_lens[b])
            return -1;
        int64_t npages = (seq_lens[b] + ORACLE_BS - 1) / ORACLE_BS;
        if (npages > W)
            return -1;
        for (int64_t c = 0; c < npages; ++c) {
            int32_t blk = block_tables[(int64_t)b * W + c];
            if (blk < 0 || blk >= num_blocks)
                return -1;
        }
    }
    int64_t Tq = query_start_loc[B];
    int64_t count = rows ? n_rows : Tq;
    for (int64_t i = 0; i < count; ++i)
        if (rows && (rows[i] < 0 || rows[i] >= Tq))
            return -1;
    int64_t max_len = 1;
    for (int b = 0; b < B; ++b)
        if (seq_lens[b] > max_len)
            max_len = seq_lens[b];

    int failed = 0;
#pragma omp parallel
    {
        float *s = (float *)malloc(sizeof(float) * (size_t)max_len);
        if (!s) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t ih = 0; ih < count * Hq; ++ih) {
            if (!s)
                continue;
            int64_t i = ih / Hq;
            int h = (int)(ih % Hq);
            int64_t row = rows ? rows[i] : i;
            int b = 0;
            while (!(row >= query_start_loc[b] && row < query_start_loc[b + 1]))
                ++b;
            int64_t q_len = (int64_t)query_start_loc[b + 1] - query_start_loc[b];
            attend_row(out + i * (int64_t)Hq * D, q + row * (int64_t)Hq * D, k_pool, v_pool,
                       k_block_stride, v_block_stride, block_tables + (int64_t)b * W,
                       seq_lens[b], q_len, row - query_start_loc[b], Hq, Hkv, D, scale,
                       causal, lse ? lse + i * (int64_t)Hq : NULL, s, h);
        }
        free(s);
    }
    return failed ? -1 : 0;
}

/*
 * Merge of two attention results over disjoint key sets of the same query
 * rows, each given as (output, LSE) [Bitwise R/R, Additional checks: LSE
 * results].  With M = max(lse_a, lse_b) and weights w = exp(lse - M), the
 * softmax over the union of the key sets gives
 *   out = (w_a * out_a + w_b * out_b) / (w_a + w_b),
 *   lse = M + log(w_a + w_b),
 * because each side's output is its own exp-weighted mean of V and its LSE
 * the log of its weight total.  A side with lse = -inf has no keys and
 * contributes nothing (its output is not read); both empty gives out = 0,
 * lse = -inf.  FP64 throughout.  Arrays are [n][D] and [n] (n = rows x heads).
 */
void oracle_merge_states(double *out, double *lse, const double *out_a, const double *lse_a,
                         const double *out_b, const double *lse_b, int64_t n, int D)
{
    for (int64_t i = 0; i < n; ++i) {
        double la = lse_a[i], lb = lse_b[i];
        double M = la > lb ? la : lb;
        if (M == -INFINITY) {
            for (int d = 0; d < D; ++d)
                out[i * D + d] = 0.0;
            lse[i] = -INFINITY;
            continue;
        }
        double wa = la == -INFINITY ? 0.0 : exp(la - M);
        double wb = lb == -INFINITY ? 0.0 : exp(lb - M);
        double w = wa + wb;
        for (int d = 0; d < D; ++d) {
            double x = 0.0;
            if (wa != 0.0)
                x += wa * out_a[i * D + d];
            if (wb != 0.0)
                x += wb * out_b[i * D + d];
            out[i * D + d] = x / w;
        }
        lse[i] = M + log(w);
    }
}

/*
 * Page-table preparation [Bitwise R/R, Changes]: pad every row to
 * W_pad = ceil(W / 8) * 8 columns (whole 128-token tiles of 16-token pages)
 * and sanitise every column at or beyond ceil(seq_len / 16) -- including all
 * columns of rows with seq_len == 0 -- to the row's last valid block, or to
 * block 0 when the row has none.  Active entries must lie in
 * [0, num_blocks).  Returns 0, or -1 (out untouched) on invalid input.
 */
int oracle_prepare_block_tables(int32_t *out, const int32_t *block_tables, int B, int W,
                                const int32_t *seq_lens, int64_t num_blocks)
{
    int W_pad = (W + 7) / 8 * 8;
    for (int b = 0; b < B; ++b) {
        if (seq_lens[b] < 0)
            return -1;
        int64_t npages = ((int64_t)seq_lens[b] + ORACLE_BS - 1) / ORACLE_BS;
        if (npages > W)
            return -1;
        for (int64_t c = 0; c < npages; ++c) {
            int32_t blk = block_tables[(int64_t)b * W + c];
            if (blk < 0 || blk >= num_blocks)
                return -1;
        }
    }
    for (int b = 0; b < B; ++b) {
        int64_t npages = ((int64_t)seq_lens[b] + ORACLE_BS - 1) / ORACLE_BS;
        int32_t fill = npages > 0 ? block_tables[(int64_t)b * W + npages - 1] : 0;
        for (int c = 0; c < W_pad; ++c)
            out[(int64_t)b * W_pad + c] = c < npages ? block_tables[(int64_t)b * W + c] : fill;
    }
    return 0;
}
