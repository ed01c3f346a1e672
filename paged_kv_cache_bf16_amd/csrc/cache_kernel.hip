// reshape_and_cache on gfx950: scatter new K/V rows into the paged pool.
//
// Operation ("test(rocm): ReshapeAndCache->PagedAttention composition at
// real dims", What changed): token i with slot s >= 0 lands in block s / 16,
// token s % 16, for every kv head; the copy is bit-exact and touches nothing
// else.  The pool's page layout is
//   K page [D/8][16 tokens][8]  -> one token's 8-dim group is a 16-byte unit,
//   V page [D][16 tokens]       -> one token's value of dim d is 2 bytes at d*32.
//
// The work is HBM-bound (read + write of 2 * T * Hkv * D * 2 bytes).  One
// workgroup takes 16 consecutive tokens of one kv head: their K and V rows
// are read whole (each token's head_dim values are contiguous) into LDS, then
// written out in the page layouts:
//   K: 16-byte units (dim group, token), token fastest across lanes, so a
//      page's run of tokens is one contiguous stretch per dim group;
//   V: 16-byte units of 8 tokens of one dim when those 8 tokens sit in 8
//      consecutive slots starting at a multiple of 8 (a run inside one page,
//      the usual case), otherwise one 2-byte store per token, so arbitrary
//      slot mappings stay exact.
// Block addresses are computed in 64-bit (pools beyond 2 GB).
#include "kvp_internal.h"

namespace kvp {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 16;          // tokens per workgroup
constexpr int kCacheThreads = 256;

template <int D>
__global__ __launch_bounds__(kCacheThreads) void cache_kernel(CacheArgs a)
{
    constexpr int UPT = D / 8;                          // 16-byte units per token row
    constexpr int UNITS = kChunk * UPT;                 // per chunk, for K (and for V)
    static_assert(UNITS % kCacheThreads == 0, "whole units per thread");
    __shared__ __attribute__((aligned(16))) uint16_t kl[kChunk][D];
    __shared__ __attribute__((aligned(16))) uint16_t vl[kChunk][D];
    __shared__ int64_t sl[kChunk];

    const int64_t chunk = blockIdx.x / a.num_kv_heads;
    const int h = (int)(blockIdx.x % a.num_kv_heads);
    const int64_t i0 = chunk * kChunk;
    const int nt = (int)min((int64_t)kChunk, a.num_tokens - i0);
    const int th = threadIdx.x;
    const int64_t nslots = a.num_blocks * KVP_BLOCK_SIZE;

    if (th < kChunk) {
        const int64_t s = th < nt ? a.slot_mapping[i0 + th] : -1;
        sl[th] = (s >= 0 && s < nslots) ? s : -1;       // slots beyond the pool are skipped
    }
#pragma unroll
    for (int r = 0; r < UNITS / kCacheThreads; ++r) {
        const int u = th + r * kCacheThreads;
        const int tok = u / UPT, du = u % UPT;
        if (tok < nt) {
            const int64_t i = i0 + tok;
            *reinterpret_cast<u32x4 *>(&kl[tok][8 * du]) =
                __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(a.k + i * a.k_token_stride + (int64_t)h * D + 8 * du));
            *reinterpret_cast<u32x4 *>(&vl[tok][8 * du]) =
                __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(a.v + i * a.v_token_stride + (int64_t)h * D + 8 * du));
        }
    }
    __syncthreads();

    const int64_t hoff = (int64_t)h * KVP_BLOCK_SIZE * D;
    // K: unit (du, tok), token fastest
#pragma unroll
    for (int r = 0; r < UNITS / kCacheThreads; ++r) {
        const int u = th + r * kCacheThreads;
        const int tok = u % kChunk, du = u / kChunk;
        const int64_t s = sl[tok];
        if (tok < nt && s >= 0) {
            uint16_t *dst = a.k_cache + (s / KVP_BLOCK_SIZE) * a.k_block_stride + hoff + du * (KVP_BLOCK_SIZE * 8)
                          + (s % KVP_BLOCK_SIZE) * 8;
            *reinterpret_cast<u32x4 *>(dst) = *reinterpret_cast<const u32x4 *>(&kl[tok][8 * du]);
        }
    }
    // V: unit (dim d, half of the chunk's tokens)
#pragma unroll
    for (int r = 0; r < UNITS / kCacheThreads; ++r) {
        const int u = th + r * kCacheThreads;
        const int half = u % 2, d = u / 2;
        const int t0 = 8 * half;
        const int64_t s0 = sl[t0];
        bool run = t0 + 8 <= nt && s0 >= 0 && (s0 % 8) == 0;
#pragma unroll
        for (int k = 1; k < 8; ++k)
            run = run && sl[t0 + k] == s0 + k;
        uint16_t *vbase = a.v_cache + hoff + (int64_t)d * KVP_BLOCK_SIZE;
        if (run) {
            u32x4 val;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                val[j] = (uint32_t)vl[t0 + 2 * j][d] | ((uint32_t)vl[t0 + 2 * j + 1][d] << 16);
            *reinterpret_cast<u32x4 *>(vbase + (s0 / KVP_BLOCK_SIZE) * a.v_block_stride + s0 % KVP_BLOCK_SIZE) = val;
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int64_t s = sl[t0 + k];
                if (t0 + k < nt && s >= 0)
                    vbase[(s / KVP_BLOCK_SIZE) * a.v_block_stride + s % KVP_BLOCK_SIZE] = vl[t0 + k][d];
            }
        }
    }
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
    const int64_t grid = (a.num_tokens + kChunk - 1) / kChunk * a.num_kv_heads;
    *blocks = 0;
    if (grid <= 0)
        return hipSuccess;
    if (grid > 0x7fffffff)
        return hipErrorInvalidValue;
    switch (a.head_dim) {
    case 128: hipLaunchKernelGGL(cache_kernel<128>, dim3((unsigned)grid), dim3(kCacheThreads), 0, s, a); break;
    case 256: hipLaunchKernelGGL(cache_kernel<256>, dim3((unsigned)grid), dim3(kCacheThreads), 0, s, a); break;
    case 512: hipLaunchKernelGGL(cache_kernel<512>, dim3((unsigned)grid), dim3(kCacheThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    *blocks = (uint64_t)grid;
    return hipGetLastError();
}

// Block-table preparation on the device: one thread per output entry of the
// padded table.  Row b keeps its first ceil(seq_len / 16) entries and repeats
// its last kept entry in every later column (0 for a row without pages);
// entries outside the pool become block 0.  Rows the host preparation would
// reject set bits in *status (1: negative seq_len, read as 0; 2: more pages
// than the row has columns, the extra ones dropped; 4: a kept entry outside
// the pool).
__global__ __launch_bounds__(256) void table_kernel(TableArgs a)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)a.num_seqs * a.padded_width)
        return;
    const int b = (int)(i / a.padded_width);
    const int c = (int)(i % a.padded_width);
    int64_t sl = a.seq_lens[b];
    int flags = 0;
    if (sl < 0) {
        flags |= 1;
        sl = 0;
    }
    int64_t np = (sl + KVP_BLOCK_SIZE - 1) / KVP_BLOCK_SIZE;
    if (np > a.width) {
        flags |= 2;
        np = a.width;
    }
    const int32_t *src = a.block_tables + (int64_t)b * a.width;
    int32_t v = 0;
    if (np > 0) {
        const int32_t id = src[c < np ? c : np - 1];
        const bool bad = id < 0 || (int64_t)id >= a.num_blocks;
        if (bad && c < np)
            flags |= 4;
        v = bad ? 0 : id;
    }
    a.out[i] = v;
    if (flags && a.status)
        atomicOr(a.status, flags);
}

hipError_t launch_prepare_tables(const TableArgs &a, hipStream_t s, uint64_t *blocks)
{
    const int64_t n = (int64_t)a.num_seqs * a.padded_width;
    const int64_t g = (n + 255) / 256;
    *blocks = 0;
    if (g <= 0)
        return hipSuccess;
    if (g > 0x7fffffff)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(table_kernel, dim3((unsigned)g), dim3(256), 0, s, a);
    *blocks = (uint64_t)g;
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
