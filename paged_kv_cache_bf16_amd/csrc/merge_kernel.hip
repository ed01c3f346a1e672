// Merge of two attention results over disjoint key sets on gfx950.
//
// Operation (the LSE results that "fix(rocm): stabilize direct paged CK
// attention for bitwise R/R" compares in its Additional checks): each
// (token, head) pair carries an output row o (BF16, head_dim values) and the
// natural-log log-sum-exp lse of the scores behind it.  Over the union of
// the two key sets the softmax gives, with M = max(lse_a, lse_b) and
// w = exp(lse - M),
//   o   = (w_a o_a + w_b o_b) / (w_a + w_b),
//   lse = M + log(w_a + w_b).
// A side with lse = -inf has no keys: its weight is 0 and its output row is
// not used (even if it holds NaN); both sides empty give o = 0, lse = -inf.
//
// HBM-bound: 3 * head_dim * 2 bytes of rows + 12 bytes of lse per pair.
// One pair takes head_dim / 8 consecutive lanes of one wave (16 bytes each),
// so a wave reads and writes whole consecutive rows, and every lane of a
// pair reads its lse values before the pair's lse is stored (in-place
// merges, out == out_a and lse == lse_a, are safe).  Rows are read and
// written with non-temporal accesses: each byte is touched once.
#include "kvp_internal.h"

namespace kvp {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMergeThreads = 256;

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
}

__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeArgs m)
{
    const int lpp = m.head_dim / 8;                  // lanes per pair
    const int ppw = 64 / lpp;                        // pairs per wave
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int sub = lane / lpp, chunk = lane % lpp;
    if (sub >= ppw)
        return;
    const int64_t pair = ((int64_t)blockIdx.x * (kMergeThreads / 64) + w) * ppw + sub;
    if (pair >= m.pairs)
        return;
    const int64_t off = pair * m.head_dim + chunk * 8;
    const float la = m.lse_a[pair], lb = m.lse_b[pair];
    const u32x4 ra = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(m.out_a + off));
    const u32x4 rb = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(m.out_b + off));

    const float M = la > lb ? la : lb;
    u32x4 r = {0u, 0u, 0u, 0u};
    float lse = -INFINITY;
    if (M != -INFINITY) {
        const float log2e = 1.44269504088896340736f;
        const float wa = la == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(__fmul_rn(__fsub_rn(la, M), log2e));
        const float wb = lb == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(__fmul_rn(__fsub_rn(lb, M), log2e));
        const float wt = __fadd_rn(wa, wb);
        const float inv = 1.0f / wt;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float x0 = 0.f, x1 = 0.f;
            if (wa != 0.f) {
                x0 = __fmul_rn(wa, bf16_lo(ra[j]));
                x1 = __fmul_rn(wa, bf16_hi(ra[j]));
            }
            if (wb != 0.f) {
                x0 = __builtin_fmaf(wb, bf16_lo(rb[j]), x0);
                x1 = __builtin_fmaf(wb, bf16_hi(rb[j]), x1);
            }
            r[j] = pack_bf16(__fmul_rn(x0, inv), __fmul_rn(x1, inv));
        }
        lse = __builtin_fmaf(__builtin_amdgcn_logf(wt), 0.693147180559945309f, M);
    }
    __builtin_nontemporal_store(r, reinterpret_cast<u32x4 *>(m.out + off));
    if (m.lse && chunk == 0)
        m.lse[pair] = lse;
}

}  // namespace

hipError_t launch_merge(const MergeArgs &m, hipStream_t s, uint64_t *blocks)
{
    const int64_t per_block = (int64_t)(kMergeThreads / 64) * (64 / (m.head_dim / 8));
    const int64_t grid = (m.pairs + per_block - 1) / per_block;
    *blocks = (uint64_t)grid;
    hipLaunchKernelGGL(merge_kernel, dim3((uint32_t)grid), dim3(kMergeThreads), 0, s, m);
    return hipGetLastError();
}

}  // namespace kvp
