/*
 * kvp.h -- C ABI of the MI355X (gfx950) paged BF16 KV-cache library.
 *
 * The library implements the composition described on the pages
 *   "test(rocm): ReshapeAndCache->PagedAttention composition at real dims"
 *     (What changed; review thread: the slot of logical token i of a
 *     sequence is block_table[i / 16] * 16 + i % 16) and
 *   "fix(rocm): stabilize direct paged CK attention for bitwise R/R"
 *     (Changes: one fixed arithmetic schedule so that prefill and decode give
 *     the same BF16 bits; padded and sanitised tail page tables; 64-bit
 *     addressing for pools over 2 GB; no dense KV materialisation),
 * i.e. a cache scatter (reshape_and_cache) followed by GQA attention that
 * reads K/V in place through per-sequence block tables (paged_attention),
 * for causal prefill, suffix prefill and single-query decode.
 *
 * Conventions shared by every entry point
 *   - Every function returns an int: KVP_OK (0) or a negative KVP_ERR_*.
 *     All argument checks run before anything is submitted to the GPU; a
 *     call that returns an error has queued no work, written no memory and
 *     left the current HIP device unchanged.  kvp_last_error() then
 *     describes the failure (thread-local, valid until the next call on the
 *     same thread).  After submission a HIP failure returns KVP_ERR_HIP; it
 *     is never retried and no other path is tried instead.
 *   - Device buffers (pool, q, k, v, out, tables, workspace) are owned by the
 *     caller.  The library owns only the small host-side pool descriptor and
 *     never allocates device memory; its one device-resident object is the
 *     fixed scratch array of paged_attention_noalloc, part of its code
 *     object (KVP_SCRATCH_BYTES per device, held until the process ends).
 *   - Work is queued on the caller's stream (a hipStream_t passed as void*;
 *     NULL is the default stream).  No entry point synchronises the host.
 *   - Every launching entry point may be captured into a HIP graph: none
 *     allocates, synchronises or issues a memset, and the launch shapes
 *     depend only on host arguments (num_seqs, max_query_len, max_seq_len,
 *     num_tokens).  A captured call replays with changed device metadata;
 *     a row leaves a captured batch by getting seq_len 0 and no queries (its
 *     table row sanitised by kv_prepare_block_tables), and its output rows
 *     are then not written ("fix(rocm): stabilize direct paged CK attention
 *     for bitwise R/R", Changes: inactive graph rows; Additional checks:
 *     graph batches shrinking 4 -> 3 -> 2 -> 1).
 *   - BF16 values are passed as raw 16-bit patterns (uint16_t storage).
 *   - No C++ exception crosses this interface.
 */
#ifndef KVP_H
#define KVP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVP_BLOCK_SIZE 16           /* tokens per page (block) */

enum {
    KVP_OK = 0,
    KVP_ERR_INVALID_ARGUMENT = -1,  /* null pointer, bad size, inconsistent metadata */
    KVP_ERR_UNSUPPORTED = -2,       /* head_dim not 128/256/512, block_size != 16, Hq % Hkv != 0, G > 16 */
    KVP_ERR_WORKSPACE_TOO_SMALL = -3,
    KVP_ERR_HIP = -4                /* a HIP call failed after validation */
};

/*
 * KV pool layout (one page = 16 tokens of one kv head of one block):
 *   K page: [head_dim / 8][16 tokens][8 dims]  BF16  (16-byte dim groups, token-major inside)
 *   V page: [head_dim][16 tokens]              BF16  (dim-major: each dim's 16 tokens contiguous)
 *   element (block b, kv head h, token t, dim d):
 *     K: k_cache[b * k_block_stride + h * 16 * head_dim + (d / 8) * 128 + t * 8 + d % 8]
 *     V: v_cache[b * v_block_stride + h * 16 * head_dim + d * 16 + t]
 * Strides are in elements and must be >= num_kv_heads * 16 * head_dim.
 * Separate pools: k_cache, v_cache distinct; both strides = Hkv * 16 * head_dim.
 * Interleaved pool: one allocation, v_cache = k_cache + Hkv * 16 * head_dim,
 * both strides = 2 * Hkv * 16 * head_dim (each block: K pages then V pages).
 * Block addresses are always formed in 64-bit arithmetic, so pools larger
 * than 2 GB (or 4 GB) are addressed correctly.  Pointers must be 16-byte
 * aligned.
 */
typedef struct {
    int64_t num_blocks;
    int32_t block_size;             /* must be KVP_BLOCK_SIZE */
    int32_t num_kv_heads;
    int32_t head_dim;               /* 128, 256 or 512 */
    int32_t reserved;
    void *k_cache;                  /* device, caller-owned */
    void *v_cache;                  /* device, caller-owned */
    int64_t k_block_stride;         /* elements */
    int64_t v_block_stride;         /* elements */
} kvp_pool_desc;

typedef struct kvp_pool kvp_pool;   /* opaque host-side descriptor */

/* kv_pool_create -- validate desc and create a host-side descriptor over
 * the caller's pool memory ("fix(rocm): stabilize direct paged CK attention
 * for bitwise R/R", Changes: the attention consumes the serving engine's KV
 * cache directly, and 64-bit addressing is kept when a K/V view spans more
 * than 2 GB; Operator benchmarks: separate and interleaved pools, small and
 * over 2 GB).  Validation happens here once, before any work is submitted
 * ("ROCm: harden compact peer-local KV prefill for Gemma-4", Required
 * hardening: invalid metadata and byte budgets are covered before
 * submission).  *out receives the handle; the library reads `desc` only
 * during this call.  The K/V overlap check is constant-time when the two
 * block strides are equal or the K and V spans are apart, and walks the
 * blocks once otherwise.
 * Errors: INVALID_ARGUMENT (null, non-positive sizes, short strides,
 * misaligned pointers, overlapping K/V pages), UNSUPPORTED (head_dim,
 * block_size). */
int kv_pool_create(const kvp_pool_desc *desc, kvp_pool **out);

/* Release a descriptor (the caller's device memory is untouched): the
 * teardown half of the descriptor lifecycle ("ROCm: harden compact
 * peer-local KV prefill for Gemma-4", Required hardening: persistent
 * resource lifecycle, no progressive host-RAM growth). */
int kv_pool_destroy(kvp_pool *pool);

/* Total bytes spanned by the pool from its lowest to highest page byte:
 * what decides whether 32-bit offsets would overflow ("fix(rocm): stabilize
 * direct paged CK attention for bitwise R/R", Changes: 64-bit addressing
 * when a K/V view spans more than 2 GB; every kernel here always forms block
 * addresses in 64 bits, so this is informational). */
int kv_pool_span_bytes(const kvp_pool *pool, int64_t *bytes);

/*
 * reshape_and_cache -- scatter new K/V rows into the pool
 * ("test(rocm): ReshapeAndCache->PagedAttention composition at real dims",
 * What changed).  For each token i in [0, num_tokens) with
 * s = slot_mapping[i] >= 0, copies the bits of k[i][h][:] and v[i][h][:]
 * (h < num_kv_heads) into block s / 16, token s % 16.  Nothing else in the
 * pool changes.  Negative slots are skipped.
 *   k, v          device, [num_tokens][num_kv_heads][head_dim] BF16 with
 *                 token strides k_token_stride / v_token_stride (elements,
 *                 >= num_kv_heads * head_dim); heads and dims contiguous.
 *   slot_mapping  device, [num_tokens] int64.
 * Preconditions not checked on the device: no two tokens share a slot (the
 * result would be one of them), every slot < num_blocks * 16 (larger slots
 * are skipped by the kernel).
 */
int reshape_and_cache(const kvp_pool *pool, const void *k, const void *v, int64_t num_tokens,
                      int64_t k_token_stride, int64_t v_token_stride,
                      const int64_t *slot_mapping, void *stream);

/*
 * kvp_check_slot_mapping -- host-side check of a slot mapping (a debug aid
 * for the preconditions reshape_and_cache does not check on the device;
 * "test(rocm): ReshapeAndCache->PagedAttention composition at real dims",
 * review thread: the slot of token i is block_table[i / 16] * 16 + i % 16,
 * so a valid mapping names each slot at most once):
 * every slot is < num_blocks * 16 and no two tokens share a slot; negative
 * slots are allowed (skipped by the scatter).
 *   slots  host, [num_tokens] int64.
 * Errors: INVALID_ARGUMENT, naming the first offending token in
 * kvp_last_error().
 */
int kvp_check_slot_mapping(const kvp_pool *pool, const int64_t *slots, int64_t num_tokens);

/*
 * kv_prepare_block_tables -- page-table metadata prep on the host
 * ("fix(rocm): stabilize direct paged CK attention for bitwise R/R",
 * Changes: pad page tables to complete KV tiles and sanitise unused
 * columns of active and inactive rows).
 *   block_tables  host, [num_seqs][width] int32 (raw; columns past a row's
 *                 last page may hold anything)
 *   seq_lens      host, [num_seqs] int32, >= 0 (0 = inactive row)
 *   out           host, [num_seqs][kvp_padded_width(width)] int32
 * Columns < ceil(seq_len / 16) must name blocks in [0, num_blocks); they are
 * copied.  Every other column becomes the row's last valid block, or 0 for a
 * row without pages.  The caller copies `out` to the device and passes it to
 * paged_attention with stride kvp_padded_width(width).
 * Errors: INVALID_ARGUMENT (a row needs more than `width` pages, an active
 * entry is out of range, negative seq_len); `out` is then untouched.
 */
int kv_prepare_block_tables(const kvp_pool *pool, const int32_t *block_tables, int32_t num_seqs,
                            int32_t width, const int32_t *seq_lens, int32_t *out);

/*
 * kv_prepare_block_tables_device -- the same preparation for a table that
 * is already in device memory, on `stream`, with no host copy and no
 * synchronisation, so a captured graph can replay it with new tables
 * ("fix(rocm): stabilize direct paged CK attention for bitwise R/R",
 * Changes: pad page tables to complete KV tiles, sanitise unused columns of
 * active and inactive rows, inactive graph rows).
 *   block_tables  device, [num_seqs][width] int32 (row stride `width`)
 *   seq_lens      device, [num_seqs] int32
 *   out           device, [num_seqs][kvp_padded_width(width)] int32; must
 *                 not overlap block_tables
 *   status        device int32 or NULL.  The checks of the host version
 *                 cannot fail the call here; instead the kernel ORs bits
 *                 into *status for rows the host version would reject
 *                 (1: negative seq_len, read as 0; 2: more than `width`
 *                 pages, the extra ones dropped; 4: a kept entry outside
 *                 [0, num_blocks), written as block 0), so every later
 *                 kernel stays inside the pool.  The caller clears *status
 *                 beforehand and reads it whenever it synchronises.
 * For every table the host version accepts, `out` receives exactly the
 * host version's values.
 * Errors: INVALID_ARGUMENT (null pointer, negative size, overlapping
 * buffers), HIP (launch failure).
 */
int kv_prepare_block_tables_device(const kvp_pool *pool, const int32_t *block_tables, int32_t num_seqs,
                                   int32_t width, const int32_t *seq_lens, int32_t *out, int32_t *status,
                                   void *stream);

/* Width a prepared table has: width rounded up to a multiple of 8 pages,
 * i.e. whole 128-token KV tiles ("fix(rocm): stabilize direct paged CK
 * attention for bitwise R/R", Changes: pad page tables to complete KV
 * tiles). */
int32_t kvp_padded_width(int32_t width);

/*
 * Bytes of device workspace paged_attention needs for these bounds: the
 * per-tile partial softmax states (m, l, acc) of the split-KV (decode) path.
 * No passage of the pages defines this call: the split-KV decode (one
 * workgroup per KV tile, then a fold of the tile states in tile order) is
 * this library's design for spreading a decode row over the chip under the
 * fixed schedule of "fix(rocm): stabilize direct paged CK attention for
 * bitwise R/R" (Changes).  The caller owns the buffer, so the library itself
 * allocates nothing ("ROCm: harden compact peer-local KV prefill for
 * Gemma-4", Required hardening: no progressive VRAM growth).
 * Every call writes the partials it reads before reading them, so the
 * workspace needs no initialisation and one workspace sized for the largest
 * bounds serves calls of any smaller batch or length.  One workspace must
 * not be used by two calls that can run at the same time.
 */
int kvp_workspace_bytes(const kvp_pool *pool, int32_t num_q_heads, int32_t num_seqs,
                        int32_t max_seq_len, size_t *bytes);

/*
 * Bytes of a workspace that also lets the rows of a mixed batch with up to
 * split_cols columns (q_len * G <= split_cols; split_cols a multiple of 16
 * in [16, 1024]) take the split-KV path: their KV tiles are spread over the
 * chip (one workgroup per tile and group of up to eight 16-column blocks,
 * the tile staged in LDS once for all of them) and their tile states folded
 * in tile order, instead of streaming every tile through
 * one prefill workgroup.  Same bits either way (the fixed schedule of
 * "fix(rocm): stabilize direct paged CK attention for bitwise R/R",
 * Changes); faster when the batch's long-query rows leave the GPU idle and
 * its medium rows have long KV (the ragged batches of that page's
 * Additional checks: tails of 128 and 17 queries on 4096/4171 keys).  The
 * partials take split_cols * (head_dim + 2) * 4 bytes per (row, kv head,
 * KV tile).  paged_attention picks the widest limit (a multiple of 16, at
 * most max_query_len * G rounded up, at most 1024) whose partials fit the
 * workspace it is given.
 */
int kvp_workspace_bytes_split(const kvp_pool *pool, int32_t num_q_heads, int32_t num_seqs,
                              int32_t max_seq_len, int32_t split_cols, size_t *bytes);

/* Zero-fill a workspace on `stream` with a fill kernel (optional; useful to
 * make a fresh buffer's contents defined).  No passage of the pages defines
 * it; it is a fill kernel rather than a memset so that it may be captured
 * into a HIP graph. */
int kvp_workspace_init(void *workspace, size_t workspace_bytes, void *stream);

/*
 * paged_attention -- GQA attention reading K/V in place through block tables
 * ("fix(rocm): stabilize direct paged CK attention for bitwise R/R",
 * Changes and Additional checks; the decode request-to-query mapping uses
 * one query per row).
 *   q     device, [total_q][num_q_heads][head_dim] BF16, token stride
 *         q_token_stride (elements); total_q = query_start_loc[num_seqs].
 *   out   device, same shape, token stride out_token_stride.
 *   block_tables     device, 32-byte aligned, [num_seqs][block_table_stride]
 *                    int32, as made by kv_prepare_block_tables
 *                    (block_table_stride a multiple of 8, >= ceil(max_seq_len
 *                    / 16); whole 128-token tiles of a row are read at once).
 *   seq_lens         device, [num_seqs] int32: KV length of each row.
 *   query_start_loc  device, [num_seqs + 1] int32: row b's queries are
 *                    q[query_start_loc[b] .. query_start_loc[b+1]); they sit
 *                    at the last q_len positions of the row (bottom-right).
 *   max_query_len, max_seq_len  host bounds of the device metadata (no sync).
 *   scale            softmax scale applied to q.k; positive and finite
 *                    (the kernels take the max of the unscaled scores).
 *   causal           1: query at position p sees keys 0..p; 0: all keys.
 * Query head h reads kv head h / (num_q_heads / num_kv_heads).
 * Rows with q_len == 0 are skipped; rows that violate 0 <= q_len <=
 * seq_len <= max_seq_len produce no output and no memory access.
 *   workspace        device, kvp_workspace_bytes(pool, num_q_heads, num_seqs,
 *                    max_seq_len) bytes, 16-byte aligned.  Required when
 *                    max_query_len * G <= 16 (decode).  Otherwise optional:
 *                    given (large enough) with num_seqs > 1, rows whose
 *                    q_len * G <= 16 take the split-KV decode path and the
 *                    others the prefill path, in two launches on `stream`;
 *                    a workspace of kvp_workspace_bytes_split(..., S) bytes
 *                    moves the rows with q_len * G <= S to the split-KV
 *                    path as well.
 *                    The host cannot see the query lengths, so a batch
 *                    given a workspace launches the split-KV kernels even
 *                    when none of its rows is short (they then only read
 *                    the row metadata); a caller that knows its batch has
 *                    no short row passes no workspace.
 * Numerics: one fixed arithmetic schedule (KV tiles and their softmax folds
 * at fixed absolute positions), so an output row's bits do not depend on
 * the batch, the other rows, the query count or the kernel chosen: a decode
 * call gives bitwise the same row as the prefill that ends at that token.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED, WORKSPACE_TOO_SMALL, HIP.
 */
int paged_attention(const kvp_pool *pool, const void *q, int64_t q_token_stride, void *out,
                    int64_t out_token_stride, int32_t num_q_heads, int32_t num_seqs,
                    const int32_t *block_tables, int32_t block_table_stride,
                    const int32_t *seq_lens, const int32_t *query_start_loc,
                    int32_t max_query_len, int32_t max_seq_len, float scale, int causal,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * paged_attention_lse -- paged_attention that also writes, for every query
 * row and head it computes, the natural-log log-sum-exp of that row's scaled
 * scores, lse = log(sum_j exp(scale * q.k_j)) over the keys the row sees
 * ("fix(rocm): stabilize direct paged CK attention for bitwise R/R",
 * Additional checks: LSE results compared with decode).
 *   lse   device, FP32, [total_q][num_q_heads] with token stride
 *         lse_token_stride (elements, >= num_q_heads), 4-byte aligned.
 * Every other argument, check and result is paged_attention's.  The lse of a
 * decode row equals bitwise the lse of the prefill row that ends at the same
 * token.  With kvp_merge_attention, results over disjoint key ranges (for
 * example a prefix and a new chunk) combine into the result over both.
 * Errors: those of paged_attention; INVALID_ARGUMENT for a null or
 * misaligned lse or a short lse_token_stride (nothing submitted).
 */
int paged_attention_lse(const kvp_pool *pool, const void *q, int64_t q_token_stride, void *out,
                        int64_t out_token_stride, float *lse, int64_t lse_token_stride, int32_t num_q_heads,
                        int32_t num_seqs, const int32_t *block_tables, int32_t block_table_stride,
                        const int32_t *seq_lens, const int32_t *query_start_loc, int32_t max_query_len,
                        int32_t max_seq_len, float scale, int causal, void *workspace, size_t workspace_bytes,
                        void *stream);

/*
 * kvp_merge_attention -- combine two attention results of the same query
 * rows over disjoint key sets into the result over their union, by the
 * log-sum-exp identity (the LSE results of "fix(rocm): stabilize direct
 * paged CK attention for bitwise R/R", Additional checks):
 *   M = max(lse_a, lse_b), w = exp(lse - M),
 *   out = (w_a out_a + w_b out_b) / (w_a + w_b),  lse = M + log(w_a + w_b).
 *   out_a, out_b, out  device, BF16, [num_tokens][num_heads][head_dim]
 *                      contiguous, 16-byte aligned.
 *   lse_a, lse_b       device, FP32, [num_tokens][num_heads] contiguous.
 *   lse                device, same shape, or NULL (not written).
 * head_dim: a multiple of 8 in [8, 512].  FP32 arithmetic, BF16 RNE output.
 * A side with lse = -inf has no keys and is ignored (its output row is not
 * used); both -inf gives out = 0 and lse = -inf.  lse values must not be
 * NaN or +inf.  out may be out_a or out_b exactly and lse may be lse_a or
 * lse_b exactly (in-place merge); any other overlap is rejected.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED (head_dim), HIP.
 */
int kvp_merge_attention(const void *out_a, const float *lse_a, const void *out_b, const float *lse_b, void *out,
                        float *lse, int64_t num_tokens, int32_t num_heads, int32_t head_dim, void *stream);

/*
 * kvp_decode_step -- reshape_and_cache followed by paged_attention
 * ("test(rocm): ReshapeAndCache->PagedAttention composition at real dims",
 * What changed: the cache write and the attention that reads it), with the
 * same arguments, checks and results as the two calls in that order on
 * `stream` (the pool ends up with the same bits, `out` gets the same bits).
 * When only the split-KV path runs (max_query_len * G <= 16) and num_tokens
 * <= 64, both happen in the split-KV partial launch: the partial kernel
 * scatters the new rows into the pool and, for keys whose slot is written by
 * this call, reads the new rows instead of the pool.  Otherwise the cache
 * kernel runs first.  Duplicate slots and slots beyond the pool follow
 * reshape_and_cache's rules.
 */
int kvp_decode_step(const kvp_pool *pool, const void *k, const void *v, int64_t num_tokens,
                    int64_t k_token_stride, int64_t v_token_stride, const int64_t *slot_mapping,
                    const void *q, int64_t q_token_stride, void *out, int64_t out_token_stride,
                    int32_t num_q_heads, int32_t num_seqs, const int32_t *block_tables,
                    int32_t block_table_stride, const int32_t *seq_lens, const int32_t *query_start_loc,
                    int32_t max_query_len, int32_t max_seq_len, float scale, int causal,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * paged_attention_noalloc -- paged_attention for callers that cannot
 * allocate device memory or pass a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments (minus the workspace), checks, kernels and bits as
 * paged_attention; the split-KV partials go to a library-owned scratch
 * array of KVP_SCRATCH_BYTES in device memory (a static __device__ array:
 * each GPU the library runs on holds its own copy from module load until
 * the process ends).  Nothing is allocated or freed by the call.
 *   - A call that needs the split-KV path alone (max_query_len * G <= 16,
 *     decode) and whose partials exceed KVP_SCRATCH_BYTES is rejected with
 *     KVP_ERR_WORKSPACE_TOO_SMALL before anything is queued; the bytes a call
 *     needs are kvp_workspace_bytes(pool, num_q_heads, num_seqs,
 *     max_seq_len).  Other calls whose partials would not fit run every row
 *     through the prefill kernels (same bits).
 *   - Every call on one GPU uses that GPU's one array.  The array keeps the
 *     last call's contents; every call writes the partials it reads before
 *     reading them, so nothing needs clearing.  Two calls that can overlap
 *     on one GPU (different streams, or different host threads) race on
 *     the array: serialise them.
 * Errors: those of paged_attention; KVP_ERR_HIP if the scratch address
 * cannot be obtained (nothing queued).
 */
#define KVP_SCRATCH_BYTES (32u << 20)

int paged_attention_noalloc(const kvp_pool *pool, const void *q, int64_t q_token_stride, void *out,
                            int64_t out_token_stride, int32_t num_q_heads, int32_t num_seqs,
                            const int32_t *block_tables, int32_t block_table_stride,
                            const int32_t *seq_lens, const int32_t *query_start_loc,
                            int32_t max_query_len, int32_t max_seq_len, float scale, int causal,
                            void *stream);

/* Dispatch counters: evidence of which kernel actually ran ("ROCm: harden
 * compact peer-local KV prefill for Gemma-4", Required hardening: positive
 * execution breadcrumb/counters, a dispatch miss invalidates a measurement;
 * "fix(rocm): stabilize direct paged CK attention for bitwise R/R",
 * Changes: report the entrypoint actually selected).  Process-wide,
 * updated atomically by every launching call after a successful launch. */
typedef struct {
    uint64_t reshape_and_cache_launches;
    uint64_t split_kv_launches;        /* decode / short-query kernel */
    uint64_t prefill_launches;         /* streaming prefill kernel */
    uint64_t workspace_init_launches;
    uint64_t last_grid_blocks;         /* workgroups of the most recent launch */
    uint64_t fused_decode_steps;       /* kvp_decode_step calls done in one partial launch */
    uint64_t merge_launches;           /* kvp_merge_attention kernels */
} kvp_counters;

int kvp_get_counters(kvp_counters *out);
/* Zero the dispatch counters (same passages as kvp_get_counters). */
int kvp_reset_counters(void);

/* Thread-local description of the last error ("" after success), so that a
 * failure before submission is reported with its reason and leaves nothing
 * behind, and a failure after submission is reported, not retried ("ROCm:
 * harden compact peer-local KV prefill for Gemma-4", Required hardening:
 * pre-submit failures leave state unchanged; after any submission a failure
 * is fatal, never double-submitted). */
const char *kvp_last_error(void);

/* Library version string (no passage of the pages; identifies the build). */
const char *kvp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVP_H */
