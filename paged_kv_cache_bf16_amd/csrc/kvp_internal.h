// Internal declarations shared by the host entry points (kvp_api.cpp) and the
// kernel launchers (cache_kernel.hip, attn_kernel.hip).  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/kvp.h"

struct kvp_pool {
    kvp_pool_desc d;
};

namespace kvp {

// KV tile (keys per softmax tile) for each head size.  Part of the numeric
// contract: tile boundaries sit at multiples of this many absolute positions.
constexpr int tile_tokens(int head_dim) { return head_dim == 128 ? 128 : 64; }

// Columns (query position x head-in-group pairs) of one MFMA column block:
// rows with at most this many columns always take the split-KV path.
constexpr int kSplitCols = 16;
// A larger workspace lets rows with up to kMaxSplitCols columns take the
// split-KV path too: their partial workgroups stage one KV tile in LDS and
// run kTileWaves column blocks against it, one per wave.
constexpr int kMaxSplitCols = 1024;
constexpr int kTileWaves = 8;

struct CacheArgs {
    const uint16_t *k, *v;
    int64_t num_tokens, k_token_stride, v_token_stride;
    const int64_t *slot_mapping;
    uint16_t *k_cache, *v_cache;
    int64_t k_block_stride, v_block_stride, num_blocks;
    int32_t num_kv_heads, head_dim;
};

struct AttnArgs {
    const uint16_t *q;
    uint16_t *out;
    const uint16_t *k_cache, *v_cache;
    int64_t k_block_stride, v_block_stride, num_blocks;
    int64_t q_token_stride, out_token_stride;
    const int32_t *block_tables;
    int32_t bt_stride;
    const int32_t *seq_lens, *qsl;
    int32_t num_seqs, num_q_heads, num_kv_heads, group;
    int32_t max_seq_len, max_tiles, col_groups;
    float scale_log2;          // softmax scale * log2(e), rounded once on the host
    int32_t causal;
    int32_t split_cols;        // rows with q_len * G <= split_cols take the split-KV path (prefill kernels
                               // skip them); 0 when it does not run.  Also the workspace's columns per slot.
    // optional log-sum-exp output [total_q][num_q_heads] (token stride below)
    float *lse;
    int64_t lse_token_stride;
    // split-KV workspace
    float *ws_acc;             // [B][Hkv][max_tiles][split_cols][D]
    float *ws_m, *ws_l;        // [B][Hkv][max_tiles][split_cols]
    // new tokens written into the pool by the same launch (decode step):
    // token i's K/V rows, its slot (< 0: none); keys in those slots are read
    // from these rows, not from the pool
    const uint16_t *new_k, *new_v;
    int64_t new_k_stride, new_v_stride;
    const int64_t *new_slots;
    int32_t num_new;
};

// Most new tokens one fused decode step takes (one per lane of a wave).
constexpr int kMaxFusedTokens = 64;

struct Workspace {
    size_t acc_off, m_off, l_off, total;
};

Workspace workspace_layout(int64_t num_seqs, int64_t num_kv_heads, int64_t max_tiles, int64_t head_dim,
                           int64_t split_cols);

hipError_t launch_reshape_and_cache(const CacheArgs &a, hipStream_t s, uint64_t *blocks);
// Split-KV path: per-tile partial kernel, then the fold kernel.
hipError_t launch_split_kv(const AttnArgs &a, int head_dim, int max_query_len, hipStream_t s, uint64_t *blocks);
// The same with a.num_new (<= kMaxFusedTokens) tokens scattered into the pool
// by the partial kernel itself.
hipError_t launch_split_kv_fused(const AttnArgs &a, int head_dim, int max_query_len, hipStream_t s, uint64_t *blocks);
hipError_t launch_prefill(const AttnArgs &a, int head_dim, int max_query_len, hipStream_t s, uint64_t *blocks);
hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t s, uint64_t *blocks);

// Block-table preparation on the device (kv_prepare_block_tables_device).
struct TableArgs {
    const int32_t *block_tables, *seq_lens;
    int32_t *out, *status;
    int32_t num_seqs, width, padded_width;
    int64_t num_blocks;
};
hipError_t launch_prepare_tables(const TableArgs &a, hipStream_t s, uint64_t *blocks);

// Merge of two (output, lse) results over disjoint key sets; rows are
// [pairs][head_dim] BF16, lse [pairs] FP32 (lse may be null).
struct MergeArgs {
    const uint16_t *out_a, *out_b;
    const float *lse_a, *lse_b;
    uint16_t *out;
    float *lse;
    int64_t pairs;
    int32_t head_dim;          // multiple of 8, 8..512
};
hipError_t launch_merge(const MergeArgs &m, hipStream_t s, uint64_t *blocks);

}  // namespace kvp
