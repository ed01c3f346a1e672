// C-ABI entry points: argument validation, page-table preparation, workspace
// sizing, kernel dispatch and dispatch counters.  Every check runs before the
// first launch, so a rejected call queues nothing and writes nothing; the
// library never changes the current HIP device and never allocates device
// memory.  The error policy follows "ROCm: harden compact peer-local KV
// prefill for Gemma-4" (Required hardening: failures before submission leave
// state unchanged; after submission a failure is reported, never retried or
// routed elsewhere).
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <unordered_map>

#include "kvp_internal.h"

// Scratch of paged_attention_noalloc: the split-KV partials of calls that
// bring no workspace.  One copy per device (loaded with the code object);
// host code never names it except to look up that device's address.
static __device__ __align__(256) char scratch[KVP_SCRATCH_BYTES];

namespace {

thread_local char g_err[512];      // fixed storage: setting it cannot throw

std::atomic<uint64_t> g_cache_launches{0}, g_split_launches{0}, g_prefill_launches{0},
    g_init_launches{0}, g_last_grid{0}, g_fused_steps{0}, g_merge_launches{0};

int fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok()
{
    g_err[0] = '\0';
    return KVP_OK;
}

int hip_fail(hipError_t e, const char *what)
{
    return fail(KVP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int64_t page_elems(const kvp_pool_desc &d) { return (int64_t)d.num_kv_heads * KVP_BLOCK_SIZE * d.head_dim; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Whether some K page and some V page of the pool share an element (each
// page is pg elements; K page i starts at element i * k_block_stride of
// k_cache, V page j at j * v_block_stride of v_cache; the pointers are
// 16-byte aligned, so their distance is a whole number of elements).
bool kv_pages_overlap(const kvp_pool_desc &d, int64_t pg)
{
    const int64_t n = d.num_blocks, sk = d.k_block_stride, sv = d.v_block_stride;
    const int64_t x0 = ((const char *)d.v_cache - (const char *)d.k_cache) / 2;   // V page 0, in K elements
    // spans apart: no page of one reaches the other
    if (x0 >= (n - 1) * sk + pg || x0 + (n - 1) * sv + pg <= 0)
        return false;
    if (sk == sv) {
        // two lattices of one step: apart iff every V page sits in a gap
        int64_t r = x0 % sk;
        if (r < 0)
            r += sk;
        return r < pg || sk - r < pg;
    }
    // V page j starting at K element x meets K page i iff x - pg < i * sk <
    // x + pg; with sk >= pg only i = floor(x / sk) and the next one can
    for (int64_t j = 0; j < n; ++j) {
        const int64_t x = x0 + j * sv;
        const int64_t i0 = x >= 0 ? x / sk : -((-x + sk - 1) / sk);
        for (int64_t i = i0; i <= i0 + 1; ++i)
            if (i >= 0 && i < n && x - i * sk < pg && i * sk - x < pg)
                return true;
    }
    return false;
}

// ---- reshape_and_cache: checks (nothing submitted) and launch
int prepare_cache(const kvp_pool *pool, const void *k, const void *v, int64_t num_tokens, int64_t k_token_stride,
                  int64_t v_token_stride, const int64_t *slot_mapping, kvp::CacheArgs &a)
{
    if (!pool)
        return fail(KVP_ERR_INVALID_ARGUMENT, "reshape_and_cache: null pool");
    const kvp_pool_desc &d = pool->d;
    if (num_tokens < 0)
        return fail(KVP_ERR_INVALID_ARGUMENT, "reshape_and_cache: negative num_tokens");
    if (num_tokens == 0)
        return KVP_OK;
    if (!k || !v || !slot_mapping)
        return fail(KVP_ERR_INVALID_ARGUMENT, "reshape_and_cache: null pointer");
    if (!aligned16(k) || !aligned16(v))
        return fail(KVP_ERR_INVALID_ARGUMENT, "reshape_and_cache: k and v must be 16-byte aligned");
    const int64_t row = (int64_t)d.num_kv_heads * d.head_dim;
    if (k_token_stride < row || v_token_stride < row || k_token_stride % 8 || v_token_stride % 8)
        return fail(KVP_ERR_INVALID_ARGUMENT,
                    "reshape_and_cache: token strides must be >= %lld and multiples of 8", (long long)row);
    if (num_tokens > ((int64_t)1 << 40) / row)
        return fail(KVP_ERR_INVALID_ARGUMENT, "reshape_and_cache: num_tokens too large");
    a.k = (const uint16_t *)k;
    a.v = (const uint16_t *)v;
    a.num_tokens = num_tokens;
    a.k_token_stride = k_token_stride;
    a.v_token_stride = v_token_stride;
    a.slot_mapping = slot_mapping;
    a.k_cache = (uint16_t *)d.k_cache;
    a.v_cache = (uint16_t *)d.v_cache;
    a.k_block_stride = d.k_block_stride;
    a.v_block_stride = d.v_block_stride;
    a.num_blocks = d.num_blocks;
    a.num_kv_heads = d.num_kv_heads;
    a.head_dim = d.head_dim;
    return KVP_OK;
}

int launch_cache(const kvp::CacheArgs &a, void *stream)
{
    uint64_t blocks = 0;
    hipError_t e = kvp::launch_reshape_and_cache(a, (hipStream_t)stream, &blocks);
    if (e != hipSuccess)
        return hip_fail(e, "reshape_and_cache launch");
    g_cache_launches++;
    g_last_grid = blocks;
    return ok();
}

// ---- paged_attention: checks and path choice (nothing submitted), launch
struct AttnPlan {
    bool noop, split, prefill;
    int D, max_query_len;
};

int prepare_attention(const kvp_pool *pool, const void *q, int64_t q_token_stride, void *out,
                      int64_t out_token_stride, int32_t num_q_heads, int32_t num_seqs,
                      const int32_t *block_tables, int32_t block_table_stride, const int32_t *seq_lens,
                      const int32_t *query_start_loc, int32_t max_query_len, int32_t max_seq_len, float scale,
                      int causal, void *workspace, size_t workspace_bytes, kvp::AttnArgs &a, AttnPlan &plan)
{
    plan.noop = true;
    plan.split = plan.prefill = false;
    if (!pool)
        return fail(KVP_ERR_INVALID_ARGUMENT, "paged_attention: null pool");
    const kvp_pool_desc &d = pool->d;
    const int D = d.head_dim;
    if (num_q_heads <= 0 || num_q_heads % d.num_kv_heads)
        return fail(KVP_ERR_UNSUPPORTED, "paged_attention: num_q_heads %d not a multiple of num_kv_heads %d",
                    num_q_heads, d.num_kv_heads);
    const int G = num_q_heads / d.num_kv_heads;
    if (G > kvp::kSplitCols)
        return fail(KVP_ERR_UNSUPPORTED, "paged_attention: group size %d > %d", G, kvp::kSplitCols);
    if (num_seqs < 0 || max_query_len < 0 || max_seq_len < 0)
        return fail(KVP_ERR_INVALID_ARGUMENT, "paged_attention: negative size");
    if (max_query_len > max_seq_len)
        return fail(KVP_ERR_INVALID_ARGUMENT, "paged_attention: max_query_len %d > max_seq_len %d", max_query_len,
                    max_seq_len);
    if (causal != 0 && causal != 1)
        return fail(KVP_ERR_INVALID_ARGUMENT, "paged_attention: causal must be 0 or 1");
    if (!std::isfinite(scale) || !(scale > 0.f) || !std::isfinite(scale * 1.44269504088896340736f))
        return fail(KVP_ERR_INVALID_ARGUMENT, "paged_attention: scale must be positive and finite");
    if (num_seqs == 0 || max_query_len == 0)
        return KVP_OK;
    if (!q || !out || !block_tables || !seq_lens || !query_start_loc)
        return fail(KVP_ERR_INVALID_ARGUMENT, "paged_attention: null pointer");
    if (!aligned16(q) || !aligned16(out))
        return fail(KVP_ERR_INVALID_ARGUMENT, "paged_attention: q and out must be 16-byte aligned");
    const int64_t row = (int64_t)num_q_heads * D;
    if (q_token_stride < row || out_token_stride < row || q_token_stride % 8 || out_token_stride % 8)
        return fail(KVP_ERR_INVALID_ARGUMENT, "paged_attention: token strides must be >= %lld and multiples of 8",
                    (long long)row);
    if (block_table_stride < cdiv(max_seq_len, KVP_BLOCK_SIZE) || block_table_stride % 8)
        return fail(KVP_ERR_INVALID_ARGUMENT,
                    "paged_attention: block_table_stride %d must be a multiple of 8 and >= %lld pages",
                    block_table_stride, (long long)cdiv(max_seq_len, KVP_BLOCK_SIZE));
    if (((uintptr_t)block_tables & 31u) != 0)
        return fail(KVP_ERR_INVALID_ARGUMENT, "paged_attention: block_tables must be 32-byte aligned");

    const int T = kvp::tile_tokens(D);
    a.q = (const uint16_t *)q;
    a.out = (uint16_t *)out;
    a.k_cache = (const uint16_t *)d.k_cache;
    a.v_cache = (const uint16_t *)d.v_cache;
    a.k_block_stride = d.k_block_stride;
    a.v_block_stride = d.v_block_stride;
    a.num_blocks = d.num_blocks;
    a.q_token_stride = q_token_stride;
    a.out_token_stride = out_token_stride;
    a.block_tables = block_tables;
    a.bt_stride = block_table_stride;
    a.seq_lens = seq_lens;
    a.qsl = query_start_loc;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = d.num_kv_heads;
    a.group = G;
    a.max_seq_len = max_seq_len;
    a.max_tiles = (int32_t)cdiv(max_seq_len, T);
    a.col_groups = 0;
    a.scale_log2 = scale * 1.44269504088896340736f;
    a.causal = causal;
    a.ws_acc = a.ws_m = a.ws_l = nullptr;
    a.lse = nullptr;
    a.lse_token_stride = 0;
    a.split_cols = 0;
    a.new_k = a.new_v = nullptr;
    a.new_k_stride = a.new_v_stride = 0;
    a.new_slots = nullptr;
    a.num_new = 0;

    // Rows with q_len * G <= 16 (decode, short suffixes) take the split-KV
    // path, which spreads their KV tiles over the chip; the rest stream
    // through a prefill kernel.  A call with only such rows needs the
    // workspace; a mixed batch of several rows uses both paths when a large
    // enough workspace is given (both paths give the same bits per row).  A
    // mixed batch whose workspace holds the partials of wider rows sends the
    // rows with up to that many columns (a multiple of 16, at most
    // kMaxSplitCols) to the split-KV path as well: the widest limit that fits.
    const bool split_only = (int64_t)max_query_len * G <= kvp::kSplitCols;
    // launch grids: rows in gridDim.z, kv heads x column-block groups in gridDim.y
    constexpr int kMaxGroups = (kvp::kMaxSplitCols / 16 + kvp::kTileWaves - 1) / kvp::kTileWaves;
    if (num_seqs > 65535 || (int64_t)d.num_kv_heads * kMaxGroups > 65535)
        return fail(KVP_ERR_UNSUPPORTED, "paged_attention: num_seqs must be <= 65535 and num_kv_heads <= %d",
                    65535 / kMaxGroups);
    kvp::Workspace w = kvp::workspace_layout(num_seqs, d.num_kv_heads, a.max_tiles, D, kvp::kSplitCols);
    const bool ws_ok = workspace && aligned16(workspace) && workspace_bytes >= w.total;
    if (split_only) {
        if (!workspace || !aligned16(workspace))
            return fail(KVP_ERR_INVALID_ARGUMENT, "paged_attention: decode needs a 16-byte aligned workspace");
        if (workspace_bytes < w.total)
            return fail(KVP_ERR_WORKSPACE_TOO_SMALL, "paged_attention: workspace %zu < %zu bytes", workspace_bytes,
                        w.total);
    }
    const bool use_split = split_only || (num_seqs > 1 && ws_ok);
    int split_cols = kvp::kSplitCols;
    if (use_split && !split_only) {
        const int64_t widest = std::min<int64_t>(((int64_t)max_query_len * G + 15) / 16 * 16, kvp::kMaxSplitCols);
        for (int64_t sc = widest; sc > kvp::kSplitCols; sc -= 16) {
            const kvp::Workspace wsc = kvp::workspace_layout(num_seqs, d.num_kv_heads, a.max_tiles, D, sc);
            if (workspace_bytes >= wsc.total) {
                split_cols = (int)sc;
                w = wsc;
                break;
            }
        }
    }
    if (use_split) {
        char *base = (char *)workspace;
        a.ws_acc = (float *)(base + w.acc_off);
        a.ws_m = (float *)(base + w.m_off);
        a.ws_l = (float *)(base + w.l_off);
        a.split_cols = split_cols;
    }
    plan.noop = false;
    plan.split = use_split;
    plan.prefill = !split_only;
    plan.D = D;
    plan.max_query_len = max_query_len;
    return KVP_OK;
}

int launch_attention(kvp::AttnArgs a, const AttnPlan &plan, void *stream)
{
    if (plan.split) {
        uint64_t blocks = 0;
        hipError_t e = a.num_new > 0 ? kvp::launch_split_kv_fused(a, plan.D, plan.max_query_len, (hipStream_t)stream, &blocks)
                                     : kvp::launch_split_kv(a, plan.D, plan.max_query_len, (hipStream_t)stream, &blocks);
        if (e != hipSuccess)
            return hip_fail(e, "paged_attention split-KV launch");
        g_split_launches++;
        if (a.num_new > 0)
            g_fused_steps++;
        g_last_grid = blocks;
    }
    if (plan.prefill) {
        uint64_t blocks = 0;
        hipError_t e = kvp::launch_prefill(a, plan.D, plan.max_query_len, (hipStream_t)stream, &blocks);
        if (e != hipSuccess)
            return hip_fail(e, "paged_attention prefill launch");
        g_prefill_launches++;
        g_last_grid = blocks;
    }
    return ok();
}

// Device address of `scratch` on the current device, looked up once per
// device with that device current (each device holds its own copy).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

int scratch_address(void **ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "paged_attention_noalloc: hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(KVP_ERR_UNSUPPORTED, "paged_attention_noalloc: device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return hip_fail(e, "paged_attention_noalloc: hipGetSymbolAddress(scratch)");
        if (!p)
            return fail(KVP_ERR_HIP, "paged_attention_noalloc: null scratch address");
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return KVP_OK;
}

}  // namespace

extern "C" {

int kv_pool_create(const kvp_pool_desc *desc, kvp_pool **out)
{
    if (!desc || !out)
        return fail(KVP_ERR_INVALID_ARGUMENT, "kv_pool_create: null argument");
    const kvp_pool_desc &d = *desc;
    if (d.block_size != KVP_BLOCK_SIZE)
        return fail(KVP_ERR_UNSUPPORTED, "kv_pool_create: block_size %d (only %d)", d.block_size, KVP_BLOCK_SIZE);
    if (d.head_dim != 128 && d.head_dim != 256 && d.head_dim != 512)
        return fail(KVP_ERR_UNSUPPORTED, "kv_pool_create: head_dim %d (128, 256, 512)", d.head_dim);
    if (d.num_blocks <= 0 || d.num_kv_heads <= 0)
        return fail(KVP_ERR_INVALID_ARGUMENT, "kv_pool_create: num_blocks and num_kv_heads must be positive");
    if (!d.k_cache || !d.v_cache)
        return fail(KVP_ERR_INVALID_ARGUMENT, "kv_pool_create: null cache pointer");
    if (!aligned16(d.k_cache) || !aligned16(d.v_cache))
        return fail(KVP_ERR_INVALID_ARGUMENT, "kv_pool_create: cache pointers must be 16-byte aligned");
    const int64_t pg = page_elems(d);
    if (d.k_block_stride < pg || d.v_block_stride < pg)
        return fail(KVP_ERR_INVALID_ARGUMENT, "kv_pool_create: block strides must be >= %lld elements", (long long)pg);
    if (d.k_block_stride % 8 || d.v_block_stride % 8)
        return fail(KVP_ERR_INVALID_ARGUMENT, "kv_pool_create: block strides must be multiples of 8 elements");
    if (kv_pages_overlap(d, pg))
        return fail(KVP_ERR_INVALID_ARGUMENT, "kv_pool_create: K and V pages overlap");
    kvp_pool *p = new (std::nothrow) kvp_pool;
    if (!p)
        return fail(KVP_ERR_INVALID_ARGUMENT, "kv_pool_create: out of host memory");
    p->d = d;
    *out = p;
    return ok();
}

int kv_pool_destroy(kvp_pool *pool)
{
    delete pool;
    return ok();
}

int kv_pool_span_bytes(const kvp_pool *pool, int64_t *bytes)
{
    if (!pool || !bytes)
        return fail(KVP_ERR_INVALID_ARGUMENT, "kv_pool_span_bytes: null argument");
    const kvp_pool_desc &d = pool->d;
    const int64_t pg = page_elems(d);
    const char *k0 = (const char *)d.k_cache, *v0 = (const char *)d.v_cache;
    const char *k1 = k0 + 2 * ((d.num_blocks - 1) * d.k_block_stride + pg);
    const char *v1 = v0 + 2 * ((d.num_blocks - 1) * d.v_block_stride + pg);
    const char *lo = k0 < v0 ? k0 : v0;
    const char *hi = k1 > v1 ? k1 : v1;
    *bytes = (int64_t)(hi - lo);
    return ok();
}

int reshape_and_cache(const kvp_pool *pool, const void *k, const void *v, int64_t num_tokens,
                      int64_t k_token_stride, int64_t v_token_stride, const int64_t *slot_mapping,
                      void *stream)
{
    kvp::CacheArgs a;
    const int rc = prepare_cache(pool, k, v, num_tokens, k_token_stride, v_token_stride, slot_mapping, a);
    if (rc != KVP_OK || num_tokens == 0)
        return rc == KVP_OK ? ok() : rc;
    return launch_cache(a, stream);
}

int kv_prepare_block_tables_device(const kvp_pool *pool, const int32_t *block_tables, int32_t num_seqs,
                                   int32_t width, const int32_t *seq_lens, int32_t *out, int32_t *status,
                                   void *stream)
{
    if (!pool)
        return fail(KVP_ERR_INVALID_ARGUMENT, "kv_prepare_block_tables_device: null pool");
    if (num_seqs < 0 || width < 0)
        return fail(KVP_ERR_INVALID_ARGUMENT, "kv_prepare_block_tables_device: negative size");
    if (num_seqs == 0)
        return ok();
    if (!seq_lens || !out || (width > 0 && !block_tables))
        return fail(KVP_ERR_INVALID_ARGUMENT, "kv_prepare_block_tables_device: null argument");
    const int32_t wp = kvp_padded_width(width);
    if (width > 0) {
        const uintptr_t i0 = (uintptr_t)block_tables, i1 = i0 + (uintptr_t)num_seqs * width * 4;
        const uintptr_t o0 = (uintptr_t)out, o1 = o0 + (uintptr_t)num_seqs * wp * 4;
        if (i0 < o1 && o0 < i1)
            return fail(KVP_ERR_INVALID_ARGUMENT, "kv_prepare_block_tables_device: out overlaps block_tables");
    }
    kvp::TableArgs a{block_tables, seq_lens, out, status, num_seqs, width, wp, pool->d.num_blocks};
    uint64_t blocks = 0;
    hipError_t e = kvp::launch_prepare_tables(a, (hipStream_t)stream, &blocks);
    if (e != hipSuccess)
        return hip_fail(e, "kv_prepare_block_tables_device launch");
    g_last_grid = blocks;
    return ok();
}

int32_t kvp_padded_width(int32_t width)
{
    if (width <= 0)
        return 8;
    return (int32_t)(cdiv(width, 8) * 8);
}

int kvp_check_slot_mapping(const kvp_pool *pool, const int64_t *slots, int64_t num_tokens)
{
    if (!pool || num_tokens < 0 || (num_tokens > 0 && !slots))
        return fail(KVP_ERR_INVALID_ARGUMENT, "kvp_check_slot_mapping: null pool or slots, or negative count");
    const int64_t nslots = pool->d.num_blocks * KVP_BLOCK_SIZE;
    try {
        std::unordered_map<int64_t, int64_t> first;
        first.reserve((size_t)num_tokens);
        for (int64_t i = 0; i < num_tokens; ++i) {
            const int64_t s = slots[i];
            if (s < 0)
                continue;
            if (s >= nslots)
                return fail(KVP_ERR_INVALID_ARGUMENT,
                            "kvp_check_slot_mapping: token %lld has slot %lld beyond the pool (%lld)", (long long)i,
                            (long long)s, (long long)nslots);
            const auto r = first.emplace(s, i);
            if (!r.second)
                return fail(KVP_ERR_INVALID_ARGUMENT, "kvp_check_slot_mapping: tokens %lld and %lld share slot %lld",
                            (long long)r.first->second, (long long)i, (long long)s);
        }
    } catch (...) {     // allocation failure: no exception crosses the C ABI
        return fail(KVP_ERR_INVALID_ARGUMENT, "kvp_check_slot_mapping: out of host memory");
    }
    return ok();
}

int kv_prepare_block_tables(const kvp_pool *pool, const int32_t *block_tables, int32_t num_seqs,
                            int32_t width, const int32_t *seq_lens, int32_t *out)
{
    if (!pool || !seq_lens || !out || (num_seqs > 0 && width > 0 && !block_tables))
        return fail(KVP_ERR_INVALID_ARGUMENT, "kv_prepare_block_tables: null argument");
    if (num_seqs < 0 || width < 0)
        return fail(KVP_ERR_INVALID_ARGUMENT, "kv_prepare_block_tables: negative size");
    const int64_t nb = pool->d.num_blocks;
    for (int32_t b = 0; b < num_seqs; ++b) {
        if (seq_lens[b] < 0)
            return fail(KVP_ERR_INVALID_ARGUMENT, "kv_prepare_block_tables: seq_lens[%d] < 0", b);
        const int64_t np = cdiv(seq_lens[b], KVP_BLOCK_SIZE);
        if (np > width)
            return fail(KVP_ERR_INVALID_ARGUMENT, "kv_prepare_block_tables: row %d needs %lld pages > width %d", b,
                        (long long)np, width);
        for (int64_t c = 0; c < np; ++c) {
            const int32_t blk = block_tables[(int64_t)b * width + c];
            if (blk < 0 || blk >= nb)
                return fail(KVP_ERR_INVALID_ARGUMENT, "kv_prepare_block_tables: block %d at [%d][%lld] outside pool",
                            blk, b, (long long)c);
        }
    }
    const int32_t wp = kvp_padded_width(width);
    for (int32_t b = 0; b < num_seqs; ++b) {
        const int64_t np = cdiv(seq_lens[b], KVP_BLOCK_SIZE);
        const int32_t *src = block_tables + (int64_t)b * width;
        const int32_t fill = np > 0 ? src[np - 1] : 0;
        int32_t *dst = out + (int64_t)b * wp;
        for (int32_t c = 0; c < wp; ++c)
            dst[c] = c < np ? src[c] : fill;
    }
    return ok();
}

int kvp_workspace_bytes(const kvp_pool *pool, int32_t num_q_heads, int32_t num_seqs, int32_t max_seq_len,
                        size_t *bytes)
{
    if (!pool || !bytes)
        return fail(KVP_ERR_INVALID_ARGUMENT, "kvp_workspace_bytes: null argument");
    if (num_q_heads <= 0 || num_seqs < 0 || max_seq_len < 0)
        return fail(KVP_ERR_INVALID_ARGUMENT, "kvp_workspace_bytes: bad sizes");
    const int T = kvp::tile_tokens(pool->d.head_dim);
    const kvp::Workspace w = kvp::workspace_layout(num_seqs, pool->d.num_kv_heads, cdiv(max_seq_len, T),
                                                   pool->d.head_dim, kvp::kSplitCols);
    *bytes = w.total;
    return ok();
}

int kvp_workspace_bytes_split(const kvp_pool *pool, int32_t num_q_heads, int32_t num_seqs, int32_t max_seq_len,
                              int32_t split_cols, size_t *bytes)
{
    if (!pool || !bytes)
        return fail(KVP_ERR_INVALID_ARGUMENT, "kvp_workspace_bytes_split: null argument");
    if (num_q_heads <= 0 || num_seqs < 0 || max_seq_len < 0)
        return fail(KVP_ERR_INVALID_ARGUMENT, "kvp_workspace_bytes_split: bad sizes");
    if (split_cols < kvp::kSplitCols || split_cols > kvp::kMaxSplitCols || split_cols % 16)
        return fail(KVP_ERR_INVALID_ARGUMENT, "kvp_workspace_bytes_split: split_cols %d must be a multiple of 16 in "
                                              "[%d, %d]", split_cols, kvp::kSplitCols, kvp::kMaxSplitCols);
    const int T = kvp::tile_tokens(pool->d.head_dim);
    const kvp::Workspace w = kvp::workspace_layout(num_seqs, pool->d.num_kv_heads, cdiv(max_seq_len, T),
                                                   pool->d.head_dim, split_cols);
    *bytes = w.total;
    return ok();
}

int kvp_workspace_init(void *workspace, size_t workspace_bytes, void *stream)
{
    if (!workspace || !aligned16(workspace) || workspace_bytes % 16)
        return fail(KVP_ERR_INVALID_ARGUMENT, "kvp_workspace_init: workspace must be 16-byte aligned and sized");
    uint64_t blocks = 0;
    hipError_t e = kvp::launch_fill_zero(workspace, workspace_bytes, (hipStream_t)stream, &blocks);
    if (e != hipSuccess)
        return hip_fail(e, "kvp_workspace_init launch");
    g_init_launches++;
    g_last_grid = blocks;
    return ok();
}

int paged_attention(const kvp_pool *pool, const void *q, int64_t q_token_stride, void *out,
                    int64_t out_token_stride, int32_t num_q_heads, int32_t num_seqs,
                    const int32_t *block_tables, int32_t block_table_stride, const int32_t *seq_lens,
                    const int32_t *query_start_loc, int32_t max_query_len, int32_t max_seq_len, float scale,
                    int causal, void *workspace, size_t workspace_bytes, void *stream)
{
    kvp::AttnArgs a{};
    AttnPlan plan;
    const int rc = prepare_attention(pool, q, q_token_stride, out, out_token_stride, num_q_heads, num_seqs,
                                     block_tables, block_table_stride, seq_lens, query_start_loc, max_query_len,
                                     max_seq_len, scale, causal, workspace, workspace_bytes, a, plan);
    if (rc != KVP_OK)
        return rc;
    if (plan.noop)
        return ok();
    return launch_attention(a, plan, stream);
}

int paged_attention_noalloc(const kvp_pool *pool, const void *q, int64_t q_token_stride, void *out,
                            int64_t out_token_stride, int32_t num_q_heads, int32_t num_seqs,
                            const int32_t *block_tables, int32_t block_table_stride, const int32_t *seq_lens,
                            const int32_t *query_start_loc, int32_t max_query_len, int32_t max_seq_len, float scale,
                            int causal, void *stream)
{
    void *ws = nullptr;
    int rc = scratch_address(&ws);
    if (rc != KVP_OK)
        return rc;
    kvp::AttnArgs a{};
    AttnPlan plan;
    rc = prepare_attention(pool, q, q_token_stride, out, out_token_stride, num_q_heads, num_seqs, block_tables,
                           block_table_stride, seq_lens, query_start_loc, max_query_len, max_seq_len, scale, causal,
                           ws, KVP_SCRATCH_BYTES, a, plan);
    if (rc == KVP_ERR_WORKSPACE_TOO_SMALL) {
        char why[sizeof g_err];
        snprintf(why, sizeof why, "%s", g_err);
        return fail(rc, "paged_attention_noalloc: the split-KV partials of this call exceed the %u-byte scratch (%s)",
                    (unsigned)KVP_SCRATCH_BYTES, why);
    }
    if (rc != KVP_OK)
        return rc;
    if (plan.noop)
        return ok();
    return launch_attention(a, plan, stream);
}

int paged_attention_lse(const kvp_pool *pool, const void *q, int64_t q_token_stride, void *out,
                        int64_t out_token_stride, float *lse, int64_t lse_token_stride, int32_t num_q_heads,
                        int32_t num_seqs, const int32_t *block_tables, int32_t block_table_stride,
                        const int32_t *seq_lens, const int32_t *query_start_loc, int32_t max_query_len,
                        int32_t max_seq_len, float scale, int causal, void *workspace, size_t workspace_bytes,
                        void *stream)
{
    kvp::AttnArgs a{};
    AttnPlan plan;
    const int rc = prepare_attention(pool, q, q_token_stride, out, out_token_stride, num_q_heads, num_seqs,
                                     block_tables, block_table_stride, seq_lens, query_start_loc, max_query_len,
                                     max_seq_len, scale, causal, workspace, workspace_bytes, a, plan);
    if (rc != KVP_OK)
        return rc;
    if (plan.noop)
        return ok();
    if (!lse || ((uintptr_t)lse & 3u) != 0)
        return fail(KVP_ERR_INVALID_ARGUMENT, "paged_attention_lse: lse must be a non-null, 4-byte aligned pointer");
    if (lse_token_stride < num_q_heads)
        return fail(KVP_ERR_INVALID_ARGUMENT, "paged_attention_lse: lse_token_stride %lld < num_q_heads %d",
                    (long long)lse_token_stride, num_q_heads);
    a.lse = lse;
    a.lse_token_stride = lse_token_stride;
    return launch_attention(a, plan, stream);
}

int kvp_merge_attention(const void *out_a, const float *lse_a, const void *out_b, const float *lse_b, void *out,
                        float *lse, int64_t num_tokens, int32_t num_heads, int32_t head_dim, void *stream)
{
    if (num_tokens < 0 || num_heads <= 0)
        return fail(KVP_ERR_INVALID_ARGUMENT, "kvp_merge_attention: negative token count or no heads");
    if (head_dim < 8 || head_dim > 512 || head_dim % 8)
        return fail(KVP_ERR_UNSUPPORTED, "kvp_merge_attention: head_dim %d must be a multiple of 8 in [8, 512]",
                    head_dim);
    if (num_tokens == 0)
        return ok();
    if (!out_a || !out_b || !out || !lse_a || !lse_b)
        return fail(KVP_ERR_INVALID_ARGUMENT, "kvp_merge_attention: null pointer");
    if (!aligned16(out_a) || !aligned16(out_b) || !aligned16(out))
        return fail(KVP_ERR_INVALID_ARGUMENT, "kvp_merge_attention: outputs must be 16-byte aligned");
    if (((uintptr_t)lse_a | (uintptr_t)lse_b | (uintptr_t)lse) & 3u)
        return fail(KVP_ERR_INVALID_ARGUMENT, "kvp_merge_attention: lse arrays must be 4-byte aligned");
    const int64_t pairs = num_tokens * num_heads;
    const int64_t per_block = 4 * (64 / (head_dim / 8));
    if ((pairs + per_block - 1) / per_block > 0x7fffffff)
        return fail(KVP_ERR_UNSUPPORTED, "kvp_merge_attention: too many rows");
    // an output may be one of the inputs exactly, or apart from both
    auto partial_overlap = [](const void *x, const void *y, int64_t bytes) {
        const uintptr_t a = (uintptr_t)x, b = (uintptr_t)y;
        return a != b && a < b + (uintptr_t)bytes && b < a + (uintptr_t)bytes;
    };
    const int64_t row_bytes = pairs * head_dim * 2, lse_bytes = pairs * 4;
    if (partial_overlap(out, out_a, row_bytes) || partial_overlap(out, out_b, row_bytes))
        return fail(KVP_ERR_INVALID_ARGUMENT, "kvp_merge_attention: out partially overlaps an input");
    if (lse && (partial_overlap(lse, lse_a, lse_bytes) || partial_overlap(lse, lse_b, lse_bytes)))
        return fail(KVP_ERR_INVALID_ARGUMENT, "kvp_merge_attention: lse partially overlaps an input");
    kvp::MergeArgs m;
    m.out_a = (const uint16_t *)out_a;
    m.out_b = (const uint16_t *)out_b;
    m.lse_a = lse_a;
    m.lse_b = lse_b;
    m.out = (uint16_t *)out;
    m.lse = lse;
    m.pairs = pairs;
    m.head_dim = head_dim;
    uint64_t blocks = 0;
    const hipError_t e = kvp::launch_merge(m, (hipStream_t)stream, &blocks);
    if (e != hipSuccess)
        return hip_fail(e, "kvp_merge_attention launch");
    g_merge_launches++;
    g_last_grid = blocks;
    return ok();
}

int kvp_decode_step(const kvp_pool *pool, const void *k, const void *v, int64_t num_tokens, int64_t k_token_stride,
                    int64_t v_token_stride, const int64_t *slot_mapping, const void *q, int64_t q_token_stride,
                    void *out, int64_t out_token_stride, int32_t num_q_heads, int32_t num_seqs,
                    const int32_t *block_tables, int32_t block_table_stride, const int32_t *seq_lens,
                    const int32_t *query_start_loc, int32_t max_query_len, int32_t max_seq_len, float scale,
                    int causal, void *workspace, size_t workspace_bytes, void *stream)
{
    kvp::CacheArgs ca;
    int rc = prepare_cache(pool, k, v, num_tokens, k_token_stride, v_token_stride, slot_mapping, ca);
    if (rc != KVP_OK)
        return rc;
    kvp::AttnArgs a{};
    AttnPlan plan;
    rc = prepare_attention(pool, q, q_token_stride, out, out_token_stride, num_q_heads, num_seqs, block_tables,
                           block_table_stride, seq_lens, query_start_loc, max_query_len, max_seq_len, scale, causal,
                           workspace, workspace_bytes, a, plan);
    if (rc != KVP_OK)
        return rc;
    // one launch when only the split-KV path runs and the new tokens fit a wave
    if (!plan.noop && plan.split && !plan.prefill && num_tokens > 0 && num_tokens <= kvp::kMaxFusedTokens) {
        a.new_k = (const uint16_t *)k;
        a.new_v = (const uint16_t *)v;
        a.new_k_stride = k_token_stride;
        a.new_v_stride = v_token_stride;
        a.new_slots = slot_mapping;
        a.num_new = (int32_t)num_tokens;
        return launch_attention(a, plan, stream);
    }
    if (num_tokens > 0) {
        rc = launch_cache(ca, stream);
        if (rc != KVP_OK)
            return rc;
    }
    if (plan.noop)
        return ok();
    return launch_attention(a, plan, stream);
}

int kvp_get_counters(kvp_counters *out)
{
    if (!out)
        return fail(KVP_ERR_INVALID_ARGUMENT, "kvp_get_counters: null argument");
    out->reshape_and_cache_launches = g_cache_launches.load();
    out->split_kv_launches = g_split_launches.load();
    out->prefill_launches = g_prefill_launches.load();
    out->workspace_init_launches = g_init_launches.load();
    out->last_grid_blocks = g_last_grid.load();
    out->fused_decode_steps = g_fused_steps.load();
    out->merge_launches = g_merge_launches.load();
    return ok();
}

int kvp_reset_counters(void)
{
    g_cache_launches = 0;
    g_split_launches = 0;
    g_prefill_launches = 0;
    g_fused_steps = 0;
    g_merge_launches = 0;
    g_init_launches = 0;
    g_last_grid = 0;
    return ok();
}

const char *kvp_last_error(void) { return g_err; }

const char *kvp_version(void) { return "kvp 0.1 gfx950"; }

}  // extern "C"
