// reshape_and_cache on gfx950: scatter new K/V rows into the paged pool.
//
// Operation ("test(rocm): ReshapeAndCache->PagedAttention composition at
// real dims", What changed): token i with slot s >= 0 lands in block s / 16,
// token s % 16, for every kv head; the copy is bit-exact and touches nothing
// else.  The pool's page layout is
//   K page [D/8][16 tokens][8]  -> one token's 8-dim group is a 16-byte unit,
//   V page [D][16 tokens]       -> one token's value of dim d is 2 bytes at d*32.
//
// The work is HBM-bound (read + write of 2 * T * Hkv * D * 2 bytes).
//   K: one lane per 16-byte unit; reads are contiguous across lanes and each
//      store is a whole 16-byte unit.
//   V: lanes walk consecutive tokens of one (head, 8-dim group), so the 2-byte
//      stores of neighbouring lanes fall next to each other inside a page row
//      whenever consecutive tokens occupy consecutive slots (the usual case);
//      arbitrary slot mappings stay correct, only less coalesced.
// Block addresses are computed in 64-bit (pools beyond 2 GB).
#include "kvp_internal.h"

namespace kvp {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void cache_k(const CacheArgs &a, int64_t blk_id)
{
    const int units_per_head = a.head_dim / 8;
    const int64_t units = a.num_tokens * a.num_kv_heads * units_per_head;
    const int64_t u = blk_id * blockDim.x + threadIdx.x;
    if (u >= units)
        return;
    const int du = (int)(u % units_per_head);
    const int64_t th = u / units_per_head;
    const int h = (int)(th % a.num_kv_heads);
    const int64_t i = th / a.num_kv_heads;
    const int64_t s = a.slot_mapping[i];
    if (s < 0 || s >= a.num_blocks * KVP_BLOCK_SIZE)
        return;
    const int64_t blk = s / KVP_BLOCK_SIZE;
    const int t = (int)(s % KVP_BLOCK_SIZE);
    const u32x4 val = *reinterpret_cast<const u32x4 *>(a.k + i * a.k_token_stride + (int64_t)h * a.head_dim + du * 8);
    uint16_t *dst = a.k_cache + blk * a.k_block_stride + (int64_t)h * KVP_BLOCK_SIZE * a.head_dim
                  + du * (KVP_BLOCK_SIZE * 8) + t * 8;
    *reinterpret_cast<u32x4 *>(dst) = val;
}

// Waves cover (head, dim-group) x token-chunks of 64; lane = token in chunk.
__device__ __forceinline__ void cache_v(const CacheArgs &a, int64_t blk_id)
{
    const int units_per_head = a.head_dim / 8;
    const int64_t chunks = (a.num_tokens + 63) / 64;
    const int64_t w = (blk_id * blockDim.x + threadIdx.x) / 64;   // wave id
    const int lane = threadIdx.x % 64;
    const int64_t per_token_units = (int64_t)a.num_kv_heads * units_per_head;
    if (w >= chunks * per_token_units)
        return;
    const int64_t hu = w % per_token_units;          // (head, dim group)
    const int64_t i = (w / per_token_units) * 64 + lane;
    if (i >= a.num_tokens)
        return;
    const int h = (int)(hu / units_per_head);
    const int du = (int)(hu % units_per_head);
    const int64_t s = a.slot_mapping[i];
    if (s < 0 || s >= a.num_blocks * KVP_BLOCK_SIZE)
        return;
    const int64_t blk = s / KVP_BLOCK_SIZE;
    const int t = (int)(s % KVP_BLOCK_SIZE);
    const u32x4 val = *reinterpret_cast<const u32x4 *>(a.v + i * a.v_token_stride + (int64_t)h * a.head_dim + du * 8);
    uint16_t *dst = a.v_cache + blk * a.v_block_stride + (int64_t)h * KVP_BLOCK_SIZE * a.head_dim
                  + (int64_t)(du * 8) * KVP_BLOCK_SIZE + t;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        dst[(2 * j) * KVP_BLOCK_SIZE] = (uint16_t)(val[j] & 0xFFFFu);
        dst[(2 * j + 1) * KVP_BLOCK_SIZE] = (uint16_t)(val[j] >> 16);
    }
}

// One launch for both halves: workgroups [0, k_blocks) copy K, the rest V.
__global__ __launch_bounds__(256) void cache_kernel(CacheArgs a, int64_t k_blocks)
{
    const int64_t bid = blockIdx.x;
    if (bid < k_blocks)
        cache_k(a, bid);
    else
        cache_v(a, bid - k_blocks);
}

__global__ __launch_bounds__(256) void fill_zero_kernel(u32x4 *p, int64_t n16)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n16)
        p[i] = u32x4{0u, 0u, 0u, 0u};
}

}  // namespace

hipError_t launch_reshape_and_cache(const CacheArgs &a, hipStream_t s, uint64_t *blocks)
{
    const int64_t units = a.num_tokens * a.num_kv_heads * (a.head_dim / 8);
    const int64_t gk = (units + 255) / 256;
    const int64_t waves = ((a.num_tokens + 63) / 64) * a.num_kv_heads * (a.head_dim / 8);
    const int64_t gv = (waves + 3) / 4;
    if (gk + gv > 0x7fffffff)
        return hipErrorInvalidValue;
    if (gk + gv > 0)
        hipLaunchKernelGGL(cache_kernel, dim3((unsigned)(gk + gv)), dim3(256), 0, s, a, gk);
    *blocks = (uint64_t)(gk + gv);
    return hipGetLastError();
}

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t s, uint64_t *blocks)
{
    const int64_t n16 = (int64_t)(bytes / 16);
    const int64_t g = (n16 + 255) / 256;
    if (g > 0)
        hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)g), dim3(256), 0, s, (u32x4 *)p, n16);
    *blocks = (uint64_t)g;
    return hipGetLastError();
}

}  // namespace kvp
