// Paged GQA attention on gfx950 (CDNA4): causal / suffix prefill and decode.
//
// Operation ("fix(rocm): stabilize direct paged CK attention for bitwise
// R/R", Changes; "test(rocm): ReshapeAndCache->PagedAttention composition at
// real dims", What changed): for every query row of sequence b at position p
// and every query head h, softmax(scale * q . K_j) over the visible keys j of
// kv head h / G, applied to V_j, where key j of sequence b lives in page
// block_tables[b][j / 16], token j % 16.  K/V are read in place from the pool.
//
// Fixed arithmetic schedule (the same for every kernel and launch shape):
//   * Keys are cut into tiles of T tokens at absolute positions (T = 128 for
//     head_dim 128, 64 otherwise).  For one query column and one tile:
//       S = K . q with BF16 MFMA (v_mfma_f32_16x16x32_bf16), FP32 accumulate,
//           the head dimension walked in 32-wide steps in ascending order;
//       S = -inf for keys the column does not see;
//       m = max(S) * c with c = scale * log2 e (c > 0, so the max of the
//           scaled scores);  p = exp2(fma(S, c, -m)) (v_exp_f32);
//       l = sum p in a fixed tree;
//       acc = P . V with P = bf16(p), MFMA over the tile's keys in 32-key
//           steps in ascending order.
//   * Tiles are folded into the running (R, L, ACC) in ascending order, from
//     (-inf, 0, 0); R is the running max rounded up to a multiple of 16:
//       R' = max(R, ref(m));  gs = R' > R ? exp2(R - R') : 1;
//       h = exp2(m - R') (0 for an empty tile);
//       ACC = fma(acc, h, ACC * gs);  L = fma(l, h, L * gs);  R = R'.
//     The output is bf16(ACC * (1 / L) + 0).
//   * No implicit FMA contraction (the library is built -ffp-contract=off);
//     every FMA above is written explicitly.
// Who computes a tile (a streaming prefill workgroup, or one split-KV
// workgroup per tile whose partial a fold kernel combines) never changes
// these operations, so decode and prefill rows agree bit for bit.
//
// MFMA operand plumbing.  With S^T = K . Q^T the score tile comes out with
// the keys along the accumulator's row axis and query columns along lanes,
// which is exactly the B-operand layout P^T needs for O^T = V^T . P^T, so
// probabilities never leave registers.  The 16 rows of key block kb = 2s+e
// hold keys 32s + 8(r/4) + 4e + r%4, so that each lane group g owns eight
// consecutive keys 32s + 8g .. 32s + 8g + 7 of PV step s; V is stored
// dim-major in its pages ([d][16 tokens]), so those eight keys of one dim
// are one 16-byte LDS read.
//
// LDS: the K and V pages of a tile are staged (one kv head), with a
// 16-byte-unit XOR swizzle that keeps the MFMA operand reads free of bank
// conflicts.  V of keys at or beyond seq_len is zeroed and their scores are
// -inf, so padded or poisoned page tails never reach the arithmetic.
#include "kvp_internal.h"

namespace kvp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BS = KVP_BLOCK_SIZE;
constexpr int NT = 256;          // threads per workgroup (4 waves)
constexpr int NW = NT / 64;

template <int D>
struct Geo {
    static constexpr int T = tile_tokens(D);     // keys per tile
    static constexpr int NKB = T / 16;           // MFMA key blocks per tile (= pages per tile)
    static constexpr int NKS = T / 32;           // PV k-steps per tile
    static constexpr int NDS = D / 32;           // QK k-steps
    static constexpr int NDB = D / 16;           // PV output d-blocks
    static constexpr int PAGE = BS * D * 2;      // bytes of one kv head's page
    static constexpr int UPP = PAGE / 16;        // 16-byte units per page
    static constexpr int LDS = 2 * NKB * PAGE;   // K tile + V tile
};

__device__ __forceinline__ int ksw(int tok, int page)
{
    return tok ^ ((((tok >> 3) ^ page) & 1) << 2);
}

// LDS slot (16-byte unit) of V unit (dim d, token half) inside a staged page:
// each 1 KB chunk holds 32 dims, half 0 of all 32 then half 1, so the 16
// lanes of one P.V operand read (16 consecutive dims, one half) touch 256
// contiguous bytes (no bank conflicts), and chunk i of the page still comes
// from source bytes [i KB, (i+1) KB) of the pool's [Dh][16 tokens] page.
__device__ __forceinline__ int vslot(int d, int half)
{
    return (d >> 5) * 64 + half * 32 + (d & 31);
}

// IEEE 754-2019 maximum (v_maximum3_f32 for nested uses; unlike fmaxf it
// needs no quieting step on operands such as MFMA results).  Maxima are
// exact in any order and -0 < +0, so every kernel gets the same bits.
__device__ __forceinline__ float fmax2(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Cross-lane steps of the softmax reductions, lane l combined with lane
// l ^ 16, then with lane l ^ 32, using the gfx950 row / half swaps (VALU, no
// LDS round trip).  With both operands the same register, the two halves of
// the swap result hold x[l] and x[l ^ 16] (resp. x[l ^ 32]) in some order on
// every lane, and both combining operations are commutative, so every lane
// gets the same bits as x[l] op x[l ^ k].
__device__ __forceinline__ float sum_xor16(float v)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __fadd_rn(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __fadd_rn(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor16(float v)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmax2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmax2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Max of N values in three-input steps (v_maximum3_f32): exact in any order,
// so the reduction shape is free; this one needs about N / 2 instructions.
template <int N>
__device__ __forceinline__ float max_reduce(const float (&v)[N])
{
    if constexpr (N == 1) {
        return v[0];
    } else if constexpr (N == 2) {
        return fmax2(v[0], v[1]);
    } else {
        constexpr int M = (N + 2) / 3;
        float r[M];
#pragma unroll
        for (int i = 0; i < M; ++i) {
            const int a = 3 * i;
            if (a + 2 < N)
                r[i] = fmax2(fmax2(v[a], v[a + 1]), v[a + 2]);
            else if (a + 1 < N)
                r[i] = fmax2(v[a], v[a + 1]);
            else
                r[i] = v[a];
        }
        return max_reduce<M>(r);
    }
}

// ---------------------------------------------------------------- staging

// Block ids of the NKB pages of tile `tile` (wave-uniform), as one vector
// value (never an indexable array, so lane-dependent choices between two ids
// stay register selects).  Rows are padded to a multiple of 8 pages (checked
// on the host), so the whole tile's entries are in the row: one aligned
// load.  Entries past the row's last page may hold anything and ids outside
// the pool become 0, so every later load is in bounds; data of keys >=
// seq_len is discarded by the callers (V zeroed, scores masked).
template <int NKB>
using ids_t = int32_t __attribute__((ext_vector_type(NKB)));

template <int NKB>
__device__ __forceinline__ ids_t<NKB> tile_blocks(const AttnArgs &a, const int32_t *bt_row, int tile)
{
    ids_t<NKB> ids = *reinterpret_cast<const ids_t<NKB> *>(bt_row + tile * NKB);
#pragma unroll
    for (int i = 0; i < NKB; ++i)
        ids[i] = (ids[i] < 0 || (int64_t)ids[i] >= a.num_blocks) ? 0 : ids[i];
    return ids;
}

// Zero the BF16 elements j of v whose token tok0 + j is >= valid.
__device__ __forceinline__ u32x4 mask_tokens(u32x4 v, int tok0, int valid)
{
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t lo = (tok0 + 2 * j < valid) ? 0x0000FFFFu : 0u;
        const uint32_t hi = (tok0 + 2 * j + 1 < valid) ? 0xFFFF0000u : 0u;
        v[j] &= (lo | hi);
    }
    return v;
}

// ---------------------------------------------------------------- tile step

// Per-lane view of one 16-column block: lane (g = lane/16, c = lane%16) owns
// column c.  Holds the Q fragments and the column's key limit.
template <int D>
struct Cols {
    bf16x8 qf[Geo<D>::NDS];
    int lim;         // keys < lim are visible (0: column inactive)
};

// Running softmax state of one column (lane-replicated over g).  ACC and L
// are kept relative to the reference R: the running maximum rounded up to a
// multiple of kRefStep (log2 units).  R changes only when the running
// maximum crosses such a multiple, so nearly every tile folds with one FMA
// per value and no rescaling of ACC.
template <int D>
struct State {
    float R, L;
    f32x4 acc[Geo<D>::NDB];
};

template <int D>
__device__ __forceinline__ void state_init(State<D> &st)
{
    st.R = -INFINITY;
    st.L = 0.f;
#pragma unroll
    for (int db = 0; db < Geo<D>::NDB; ++db)
        st.acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
}

constexpr float kRefStep = 16.f;

// Reference of a maximum: m rounded up to a multiple of kRefStep (exact;
// monotone, so the reference of a running max is the max of the references).
__device__ __forceinline__ float ref_of(float m)
{
    return __fmul_rn(__builtin_ceilf(__fmul_rn(m, 1.f / kRefStep)), kRefStep);
}

// Factors for folding a tile with max m (log2 units, -inf when empty) into
// a state with reference R.  Rn = max(R, ref(m)); gs = exp2(R - Rn) when
// Rn > R (rescales the state), else 1; h = exp2(m - Rn) scales the tile,
// 0 for an empty tile.
struct FoldF {
    float gs, h, Rn;
    bool up;
};

__device__ __forceinline__ FoldF fold_factors(float R, float m)
{
    FoldF f;
    f.Rn = fmax2(R, ref_of(m));
    f.up = f.Rn > R;
    f.gs = f.up ? __builtin_amdgcn_exp2f(__fsub_rn(R, f.Rn)) : 1.f;
    f.h = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(__fsub_rn(m, f.Rn));
    return f;
}

// ACC' = fma(tile, h, ACC * gs).  ACC * 1 is exact, so a state whose
// reference did not move may skip the product: the result is the same.
__device__ __forceinline__ float fold1v(float acc, float tile, float gs, float h)
{
    return __builtin_fmaf(tile, h, __fmul_rn(acc, gs));
}

// (R, L) after the fold; L follows the same rule as ACC.
__device__ __forceinline__ void fold_stats(float &R, float &L, float l, const FoldF &f)
{
    L = fold1v(L, l, f.gs, f.h);
    R = f.Rn;
}

// bf16 output of one dim: RNE of acc * (1 / L), signed zero made +0
__device__ __forceinline__ uint16_t finish1(float acc, float inv)
{
    const __bf16 r = (__bf16)__fadd_rn(__fmul_rn(acc, inv), 0.f);
    return __builtin_bit_cast(uint16_t, r);
}

// bf16 output of 4 consecutive dims
__device__ __forceinline__ u32x2 finish4(const f32x4 &acc, float inv)
{
    u32x2 r;
#pragma unroll
    for (int j = 0; j < 2; ++j)
        r[j] = (uint32_t)finish1(acc[2 * j], inv) | ((uint32_t)finish1(acc[2 * j + 1], inv) << 16);
    return r;
}

// Column bookkeeping: column index -> (query row, head, key limit).
struct ColInfo {
    int64_t row, row0;   // the column's query row; the sequence's first query row
    int head;
    int lim;
};

__device__ __forceinline__ ColInfo col_info(const AttnArgs &a, int col, int kvh, int q0, int q_len, int seq_len)
{
    ColInfo ci;
    const int pr = col / a.group;
    ci.head = kvh * a.group + col % a.group;
    ci.row = (int64_t)q0 + pr;
    ci.row0 = q0;
    ci.head = col < q_len * a.group ? ci.head : kvh * a.group;
    const int pos = seq_len - q_len + pr;
    ci.lim = col < q_len * a.group ? (a.causal ? pos + 1 : seq_len) : 0;
    return ci;
}

template <int D>
__device__ __forceinline__ void load_q(Cols<D> &cf, const AttnArgs &a, const ColInfo &ci)
{
    const int g = (threadIdx.x & 63) >> 4;
    // Inactive columns (lim == 0) read the sequence's first query row, which
    // always exists; every key is masked for them, so their values never
    // reach a probability.
    const uint16_t *src = a.q + (ci.lim > 0 ? ci.row : ci.row0) * a.q_token_stride + (int64_t)ci.head * D + 8 * g;
#pragma unroll
    for (int ds = 0; ds < Geo<D>::NDS; ++ds)
        cf.qf[ds] = *reinterpret_cast<const bf16x8 *>(src + 32 * ds);
    cf.lim = ci.lim;
}

// Natural-log log-sum-exp of a column's scaled scores from its final state:
// sum_j exp2(S_j * scale * log2 e) = 2^R * L, so lse = (R + log2 L) * ln 2.
// Decode and prefill reach the same (R, L) bits, hence the same lse bits.
__device__ __forceinline__ float lse_of(float R, float L)
{
    return __fmul_rn(__fadd_rn(R, __builtin_amdgcn_logf(L)), 0.693147180559945309f);
}

template <int D>
__device__ __forceinline__ void store_out(const AttnArgs &a, const ColInfo &ci, const State<D> &st)
{
    const int g = (threadIdx.x & 63) >> 4;
    if (a.lse && g == 0)
        a.lse[ci.row * a.lse_token_stride + ci.head] = lse_of(st.R, st.L);
    const float inv = 1.0f / st.L;
    uint16_t *dst = a.out + ci.row * a.out_token_stride + (int64_t)ci.head * D + 4 * g;
#pragma unroll
    for (int db = 0; db < Geo<D>::NDB; ++db)
        *reinterpret_cast<u32x2 *>(dst + 16 * db) = finish4(st.acc[db], inv);
}

// Rows that violate 0 < q_len <= seq_len <= max_seq_len are skipped.
__device__ __forceinline__ bool row_ok(const AttnArgs &a, int b, int &q0, int &q_len, int &seq_len)
{
    q0 = a.qsl[b];
    q_len = a.qsl[b + 1] - q0;
    seq_len = a.seq_lens[b];
    return q_len > 0 && q_len <= seq_len && seq_len <= a.max_seq_len && q0 >= 0;
}

// Prefill workgroup -> (sequence b, kv head, column-group index cgi; cgi 0 is
// the row's heaviest (latest) column group).  Workgroups go to the 8 XCDs
// round-robin (XCD = blockIdx.x % 8), and one XCD's workgroups share its L2.
// When the rows' column groups fit in one XCD's share of the grid, each XCD
// takes a contiguous run of (row, column group) pairs, so a row's tiles are
// read through one L2.  When a row has more column groups than that share
// (few rows, long causal rows), a contiguous run would give some XCDs only
// the heavy column groups and others only the light ones, so the pairs are
// dealt out column group by column group instead: XCD x takes every 8th
// pair, heaviest first, and with a row count dividing 8 it stays on one row.
// Returns false for the grid's padding workgroups.
__device__ __forceinline__ bool wg_slot(const AttnArgs &a, int &b, int &kvh, int &cgi)
{
    const int rows = a.num_seqs * a.num_kv_heads;
    const int n = rows * a.col_groups;
    const int per = (n + 7) / 8;
    int r;
    if (a.col_groups > per) {
        const int j = (int)blockIdx.x;
        if (j >= n)
            return false;
        r = j % rows;
        cgi = j / rows;
    } else {
        const int j = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
        if (j >= n)
            return false;
        r = j / a.col_groups;
        cgi = j % a.col_groups;
    }
    kvh = r % a.num_kv_heads;
    b = r / a.num_kv_heads;
    return true;
}

// ---------------------------------------------------------------- joint tile step (prefill)

// P.V for every 16-dim block of CB column blocks, each result folded into
// its state with fma(tile, h, ACC) (the states were rescaled by gs first
// where needed).  The V fragments of block db+1 are read while the MFMAs of
// block db run, and block db is folded after the MFMAs of block db+1 are
// issued, so neither the LDS latency nor the MFMA latency is exposed.
// Hook of the QK and P.V loops below: called after each step's MFMAs with
// the step's index (a compile-time value once the loop is unrolled), so that
// a caller can spread other instructions (tile transfers) over the MFMA
// loop.  The default does nothing.
struct NoHook {
    __device__ __forceinline__ void operator()(int) const {}
};

template <int D, int CB, class Hook = NoHook>
__device__ __forceinline__ void prefill_pv(const char *vl, const bf16x8 (&pf)[CB][Geo<D>::NKS],
                                           const FoldF (&f)[CB], State<D> (&st)[CB], Hook hook = Hook{})
{
    using G = Geo<D>;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, c = lane & 15;
    auto vaddr = [&](int db) -> const char * {
        const int d = 16 * db + c;
        return vl + (g >> 1) * G::PAGE + vslot(d, g & 1) * 16;
    };
    bf16x8 vf[G::NKS], vn[G::NKS];
    {
        const char *p0 = vaddr(0);
#pragma unroll
        for (int stp = 0; stp < G::NKS; ++stp)
            vf[stp] = *reinterpret_cast<const bf16x8 *>(p0 + 2 * stp * G::PAGE);
    }
    f32x4 prev[CB];
#pragma unroll
    for (int db = 0; db < G::NDB; ++db) {
        if (db + 1 < G::NDB) {
            const char *pn = vaddr(db + 1);
#pragma unroll
            for (int stp = 0; stp < G::NKS; ++stp)
                vn[stp] = *reinterpret_cast<const bf16x8 *>(pn + 2 * stp * G::PAGE);
        }
        f32x4 acc[CB];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
            acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int stp = 0; stp < G::NKS; ++stp)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
                acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[stp], pf[cb][stp], acc[cb], 0, 0, 0);
        if (db > 0) {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    st[cb].acc[db - 1][i] = __builtin_fmaf(prev[cb][i], f[cb].h, st[cb].acc[db - 1][i]);
        }
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
            prev[cb] = acc[cb];
#pragma unroll
        for (int stp = 0; stp < G::NKS; ++stp)
            vf[stp] = vn[stp];
        if (db + 1 < G::NDB)
            __builtin_amdgcn_sched_group_barrier(0x100, G::NKS, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, G::NKS * CB, 0);
        __builtin_amdgcn_sched_barrier(0);
        hook(db);
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            st[cb].acc[G::NDB - 1][i] = __builtin_fmaf(prev[cb][i], f[cb].h, st[cb].acc[G::NDB - 1][i]);
}

// Phase 1 of the tile step: S^T = K . Q^T for every column block.
template <int D, int CB, class Hook = NoHook>
__device__ __forceinline__ void prefill_qk(const char *kl, const Cols<D> (&cols)[CB], f32x4 (&s)[CB][Geo<D>::NKB],
                                           Hook hook = Hook{})
{
    using G = Geo<D>;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, c = lane & 15;
    auto kaddr = [&](int kb) -> const char * {
        const int stp = kb >> 1, e = kb & 1;
        const int page = 2 * stp + (c >> 3);
        const int tok = ((c >> 2) & 1) * 8 + e * 4 + (c & 3);
        return kl + page * G::PAGE + ksw(tok, page) * 16 + g * 256;
    };
    bf16x8 kf[G::NDS], kn[G::NDS];
    {
        const char *p0 = kaddr(0);
#pragma unroll
        for (int ds = 0; ds < G::NDS; ++ds)
            kf[ds] = *reinterpret_cast<const bf16x8 *>(p0 + ds * 1024);
    }
#pragma unroll
    for (int kb = 0; kb < G::NKB; ++kb) {
        if (kb + 1 < G::NKB) {
            const char *pn = kaddr(kb + 1);
#pragma unroll
            for (int ds = 0; ds < G::NDS; ++ds)
                kn[ds] = *reinterpret_cast<const bf16x8 *>(pn + ds * 1024);
        }
        f32x4 acc[CB];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
            acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < G::NDS; ++ds)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
                acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ds], cols[cb].qf[ds], acc[cb], 0, 0, 0);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
            s[cb][kb] = acc[cb];
#pragma unroll
        for (int ds = 0; ds < G::NDS; ++ds)
            kf[ds] = kn[ds];
        // the next block's fragment reads go out before this block's MFMAs
        if (kb + 1 < G::NKB)
            __builtin_amdgcn_sched_group_barrier(0x100, G::NDS, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, G::NDS * CB, 0);
        __builtin_amdgcn_sched_barrier(0);
        hook(kb);
    }
}

// Phase 1 for wide heads (many 32-dim steps) and single-column-block waves:
// the same MFMA chains (one per (column block, key block), head dim
// ascending from zero), walked with the head-dim step outermost; the K
// fragments are read through a ring of RD register sets, each reloaded
// with the fragment RD positions ahead as soon as its MFMA is issued.
template <int D, int CB, int RD = 6, class Hook = NoHook>
__device__ __forceinline__ void prefill_qk_wide(const char *kl, const Cols<D> (&cols)[CB],
                                                f32x4 (&s)[CB][Geo<D>::NKB], Hook hook = Hook{})
{
    using G = Geo<D>;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, c = lane & 15;
    auto kaddr = [&](int kb) -> const char * {
        const int stp = kb >> 1, e = kb & 1;
        const int page = 2 * stp + (c >> 3);
        const int tok = ((c >> 2) & 1) * 8 + e * 4 + (c & 3);
        return kl + page * G::PAGE + ksw(tok, page) * 16 + g * 256;
    };
    const char *base[G::NKB];
#pragma unroll
    for (int kb = 0; kb < G::NKB; ++kb)
        base[kb] = kaddr(kb);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int kb = 0; kb < G::NKB; ++kb)
            s[cb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // fragment j = (dim step j / NKB, key block j % NKB)
    constexpr int N = G::NDS * G::NKB;
    static_assert(RD >= 1 && RD <= N, "ring depth");
    auto frag = [&](int j) { return *reinterpret_cast<const bf16x8 *>(base[j % G::NKB] + (j / G::NKB) * 1024); };
    bf16x8 ring[RD];
#pragma unroll
    for (int j = 0; j < RD; ++j)
        ring[j] = frag(j);
#pragma unroll
    for (int j = 0; j < N; ++j) {
        const int ds = j / G::NKB, kb = j % G::NKB;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
            s[cb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ring[j % RD], cols[cb].qf[ds], s[cb][kb], 0, 0, 0);
        if (j + RD < N)
            ring[j % RD] = frag(j + RD);
        __builtin_amdgcn_sched_group_barrier(0x008, CB, 0);
        if (j + RD < N)
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_barrier(0);
        hook(j);
    }
}

// Phase 2: softmax statistics and BF16 P^T of the tile, the fold factors
// and the (R, L) fold; returns whether some column's reference moved (its
// ACC must then be rescaled by gs before this tile's P.V is added).
// The tile's statistics: mx = the scaled max of the scores each column sees
// (-inf if none), lsum = the sum tree of p = exp2(fma(S, scale_log2, -mx)),
// and P^T in BF16 (the same values the split-KV partial kernel stores).
template <int D, int CB, bool MASK>
__device__ __forceinline__ void tile_stats(f32x4 (&s)[CB][Geo<D>::NKB], const Cols<D> (&cols)[CB], int tile,
                                           float scale_log2, float (&mx)[CB], float (&lsum)[CB],
                                           bf16x8 (&pf)[CB][Geo<D>::NKS])
{
    using G = Geo<D>;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;
    // ---- softmax statistics and P^T, each step for all column blocks.
    // The max runs over raw scores (scale_log2 > 0, so max(S) * scale_log2
    // is the max of the scaled scores); p = exp2(fma(S, scale_log2, -m)).
    const int key0 = tile * G::T;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        float vals[4 * G::NKB];
#pragma unroll
        for (int kb = 0; kb < G::NKB; ++kb) {
            if (MASK) {
                const int stp = kb >> 1, e = kb & 1;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = key0 + 32 * stp + 8 * g + 4 * e + i;
                    s[cb][kb][i] = key < cols[cb].lim ? s[cb][kb][i] : -INFINITY;
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                vals[4 * kb + i] = s[cb][kb][i];
        }
        mx[cb] = max_reduce<4 * G::NKB>(vals);
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
        mx[cb] = __fmul_rn(max_xor32(max_xor16(mx[cb])), scale_log2);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const float nmu = mx[cb] == -INFINITY ? 0.f : -mx[cb];
        float part[G::NKB];
#pragma unroll
        for (int kb = 0; kb < G::NKB; ++kb) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                s[cb][kb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[cb][kb][i], scale_log2, nmu));
            part[kb] = __fadd_rn(__fadd_rn(s[cb][kb][0], s[cb][kb][1]), __fadd_rn(s[cb][kb][2], s[cb][kb][3]));
        }
#pragma unroll
        for (int w = 1; w < G::NKB; w *= 2)
#pragma unroll
            for (int kb = 0; kb < G::NKB; kb += 2 * w)
                part[kb] = __fadd_rn(part[kb], part[kb + w]);
        lsum[cb] = part[0];
#pragma unroll
        for (int stp = 0; stp < G::NKS; ++stp)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pf[cb][stp][i] = (__bf16)s[cb][2 * stp][i];
                pf[cb][stp][4 + i] = (__bf16)s[cb][2 * stp + 1][i];
            }
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
        lsum[cb] = sum_xor32(sum_xor16(lsum[cb]));
}

template <int D, int CB, bool MASK>
__device__ __forceinline__ bool prefill_softmax_stats(f32x4 (&s)[CB][Geo<D>::NKB], const Cols<D> (&cols)[CB],
                                                      int tile, float scale_log2, State<D> (&st)[CB],
                                                      bf16x8 (&pf)[CB][Geo<D>::NKS], FoldF (&f)[CB])
{
    float mx[CB], lsum[CB];
    tile_stats<D, CB, MASK>(s, cols, tile, scale_log2, mx, lsum, pf);

    // ---- fold factors; one wave-uniform choice of fold sequence per tile
    bool any_up = false;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        f[cb] = fold_factors(st[cb].R, mx[cb]);
        any_up |= __ballot(f[cb].up) != 0;
    }

#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
        fold_stats(st[cb].R, st[cb].L, lsum[cb], f[cb]);
    return any_up;
}

// States whose reference moved are rescaled before P.V adds into them
// (ACC * 1 is exact, so every column of the wave may take the product).
template <int D, int CB>
__device__ __forceinline__ void rescale_states(State<D> (&st)[CB], const FoldF (&f)[CB])
{
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int db = 0; db < Geo<D>::NDB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                st[cb].acc[db][i] = __fmul_rn(st[cb].acc[db][i], f[cb].gs);
}

template <int D, int CB, bool MASK>
__device__ __forceinline__ void prefill_softmax(f32x4 (&s)[CB][Geo<D>::NKB], const Cols<D> (&cols)[CB], int tile,
                                                float scale_log2, State<D> (&st)[CB],
                                                bf16x8 (&pf)[CB][Geo<D>::NKS], FoldF (&f)[CB])
{
    if (prefill_softmax_stats<D, CB, MASK>(s, cols, tile, scale_log2, st, pf, f))
        rescale_states<D, CB>(st, f);
}

// P.V with DG 16-dim blocks in flight at once (independent MFMA chains for
// waves that have their SIMD to themselves): per block the same chain (32-key
// steps ascending from zero) and the same fold fma(tile, h, ACC) as
// prefill_pv.
template <int D, int CB, int DG, bool RS = false, class Hook = NoHook>
__device__ __forceinline__ void prefill_pv_grp(const char *vl, const bf16x8 (&pf)[CB][Geo<D>::NKS],
                                               const FoldF (&f)[CB], State<D> (&st)[CB], Hook hook = Hook{})
{
    using G = Geo<D>;
    static_assert(G::NDB % DG == 0, "whole groups");
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, c = lane & 15;
    auto vaddr = [&](int db, int stp) -> const char * {
        const int d = 16 * db + c;
        return vl + (g >> 1) * G::PAGE + vslot(d, g & 1) * 16 + 2 * stp * G::PAGE;
    };
#pragma unroll
    for (int db0 = 0; db0 < G::NDB; db0 += DG) {
        f32x4 o[CB][DG];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int d = 0; d < DG; ++d)
                o[cb][d] = f32x4{0.f, 0.f, 0.f, 0.f};
        bf16x8 vf[DG], vn[DG];
#pragma unroll
        for (int d = 0; d < DG; ++d)
            vf[d] = *reinterpret_cast<const bf16x8 *>(vaddr(db0 + d, 0));
#pragma unroll
        for (int stp = 0; stp < G::NKS; ++stp) {
            if (stp + 1 < G::NKS) {
#pragma unroll
                for (int d = 0; d < DG; ++d)
                    vn[d] = *reinterpret_cast<const bf16x8 *>(vaddr(db0 + d, stp + 1));
            }
#pragma unroll
            for (int d = 0; d < DG; ++d)
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
                    o[cb][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[d], pf[cb][stp], o[cb][d], 0, 0, 0);
#pragma unroll
            for (int d = 0; d < DG; ++d)
                vf[d] = vn[d];
            if (stp + 1 < G::NKS)
                __builtin_amdgcn_sched_group_barrier(0x100, DG, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, DG * CB, 0);
            __builtin_amdgcn_sched_barrier(0);
            hook((db0 / DG) * G::NKS + stp);
        }
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int d = 0; d < DG; ++d)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    st[cb].acc[db0 + d][i] = __builtin_fmaf(o[cb][d][i], f[cb].h,
                                                            RS ? __fmul_rn(st[cb].acc[db0 + d][i], f[cb].gs)
                                                               : st[cb].acc[db0 + d][i]);
    }
}

// The tile step's QK and P.V for a wave: single-column-block waves (which
// often have their SIMD to themselves) take the variants with several
// independent MFMA chains in flight.
template <int D, int CB>
__device__ __forceinline__ void tile_qk(const char *kl, const Cols<D> (&cols)[CB], f32x4 (&s)[CB][Geo<D>::NKB])
{
    if (CB == 1 || Geo<D>::NDS > 4)
        prefill_qk_wide<D, CB>(kl, cols, s);
    else
        prefill_qk<D, CB>(kl, cols, s);
}

template <int D, int CB>
__device__ __forceinline__ void tile_pv(const char *vl, const bf16x8 (&pf)[CB][Geo<D>::NKS], const FoldF (&f)[CB],
                                        State<D> (&st)[CB])
{
    if (CB == 1)
        prefill_pv_grp<D, CB, (D == 128 ? 8 : 4)>(vl, pf, f, st);
    else
        prefill_pv<D, CB>(vl, pf, f, st);
}

// ---------------------------------------------------------------- split-KV (decode)

// Partial kernel.  Workgroup = (tile, kv head, sequence) for rows whose
// q_len * G <= 16 (one 16-column block).  The four waves split the tile:
// wave w owns key blocks [w*KPW, (w+1)*KPW) for S and dim blocks
// [w*DPW, (w+1)*DPW) for P.V.  K and V fragments are loaded from the pool
// straight into MFMA operand registers.  The softmax statistics are combined
// across waves through LDS in exactly the order the single-wave tile step
// uses (max is exact; the sum tree's first levels are the per-wave sums), so
// the tile's (m, l, acc) are bitwise those of the prefill tile step.
// Scatter of the new tokens' kv head kvh into the pool (the decode step's
// cache write, done by workgroup (max_tiles, kvh, 0) of the partial launch):
// the same bit copy as the cache kernel, slots < 0 or beyond the pool skipped.
template <int D>
__device__ __forceinline__ void scatter_new_tokens(const AttnArgs &a, int kvh)
{
    uint16_t *kc = const_cast<uint16_t *>(a.k_cache), *vc = const_cast<uint16_t *>(a.v_cache);
    const int64_t hoff = (int64_t)kvh * BS * D;
    for (int u = threadIdx.x; u < a.num_new * (D / 8); u += NT) {
        const int i = u / (D / 8), du = u % (D / 8);
        const int64_t sl = a.new_slots[i];
        if (sl < 0 || sl >= a.num_blocks * BS)
            continue;
        const u32x4 val = *reinterpret_cast<const u32x4 *>(a.new_k + i * a.new_k_stride + (int64_t)kvh * D + du * 8);
        *reinterpret_cast<u32x4 *>(kc + (sl / BS) * a.k_block_stride + hoff + du * (BS * 8) + (sl % BS) * 8) = val;
    }
    for (int u = threadIdx.x; u < a.num_new * D; u += NT) {
        const int i = u / D, d = u % D;
        const int64_t sl = a.new_slots[i];
        if (sl < 0 || sl >= a.num_blocks * BS)
            continue;
        vc[(sl / BS) * a.v_block_stride + hoff + (int64_t)d * BS + sl % BS] = a.new_v[i * a.new_v_stride + (int64_t)kvh * D + d];
    }
}

template <int D, bool FUSE>
__global__ __launch_bounds__(NT) void split_partial_kernel(AttnArgs a)
{
    using G = Geo<D>;
    constexpr int KPW = G::NKB / NW;   // key blocks per wave
    constexpr int DPW = G::NDB / NW;   // dim blocks per wave
    static_assert(KPW == 1 || KPW == 2, "tile shape");
    // head_dim 512: the Q fragments go through LDS (each wave loads a quarter
    // of the dim steps), so the tile's K and V fit in registers with room for
    // three workgroups per CU
    constexpr bool QL = D == 512;
    __shared__ float smax[NW][16];
    __shared__ float ssum[NW][64];
    __shared__ uint32_t spf[NW][2 * KPW][64];
    __shared__ bf16x8 sq[QL ? G::NDS : 1][64];

    const int tile = blockIdx.x;
    const int kvh = blockIdx.y;
    const int b = blockIdx.z;
    if (FUSE && tile == a.max_tiles) {
        // the extra column of workgroups writes the new tokens (kv head kvh)
        if (b == 0)
            scatter_new_tokens<D>(a, kvh);
        return;
    }
    // new token slots, one per lane (FUSE; num_new >= 1), loaded with the
    // block ids, before anything waits
    int64_t my_new = -1;
    if (FUSE) {
        const int ln = (int)(threadIdx.x & 63);
        const int64_t sl = a.new_slots[min(ln, a.num_new - 1)];
        my_new = ln < a.num_new ? sl : -1;
    }
    // The tile's block-table entries are always inside the padded row
    // (tile < max_tiles), so they are fetched together with the row's
    // metadata instead of after it: the four loads are issued at once and
    // the empty asm statement, which takes all of them as inputs, keeps the
    // compiler from sinking the block-id load below the row checks or
    // ordering the metadata loads one after another (it computes nothing).
    const int32_t *bt_row = a.block_tables + (int64_t)b * a.bt_stride;
    const ids_t<G::NKB> raw = *reinterpret_cast<const ids_t<G::NKB> *>(bt_row + tile * G::NKB);
    const int r_q0 = a.qsl[b], r_q1 = a.qsl[b + 1], r_sl = a.seq_lens[b];
    asm volatile("" ::"s"(raw[0]), "s"(raw[G::NKB - 1]), "s"(r_q0), "s"(r_q1), "s"(r_sl));
    ids_t<G::NKB> blk;
#pragma unroll
    for (int i = 0; i < G::NKB; ++i)
        blk[i] = (raw[i] < 0 || (int64_t)raw[i] >= a.num_blocks) ? 0 : raw[i];
    const int q0 = r_q0, q_len = r_q1 - r_q0, seq_len = r_sl;
    if (!(q_len > 0 && q_len <= seq_len && seq_len <= a.max_seq_len && q0 >= 0))    // as row_ok
        return;
    const int ncols = q_len * a.group;
    if (ncols > a.split_cols)
        return;
    const int n_tiles = (seq_len + G::T - 1) / G::T;
    if (tile >= n_tiles)
        return;
    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, c = lane & 15;
    const int64_t hoff = (int64_t)kvh * BS * D;


    // ---- issue every load of this workgroup up front (non-temporal: each
    // K/V byte is read once per call, so the lines need not stay cached)
    Cols<D> cols;
    const ColInfo ci = col_info(a, c, kvh, q0, q_len, seq_len);
    constexpr int QPW = G::NDS / NW;               // dim steps of Q each wave stages (QL)
    bf16x8 qpart[QL ? QPW : 1];
    if (QL) {
        const uint16_t *src = a.q + (ci.lim > 0 ? ci.row : ci.row0) * a.q_token_stride + (int64_t)ci.head * D + 8 * g;
#pragma unroll
        for (int k = 0; k < QPW; ++k)
            qpart[k] = *reinterpret_cast<const bf16x8 *>(src + 32 * (w * QPW + k));
        cols.lim = ci.lim;
    } else {
        load_q<D>(cols, a, ci);
    }
    bf16x8 kf[KPW][G::NDS];
#pragma unroll
    for (int kl = 0; kl < KPW; ++kl) {
        const int kb = w * KPW + kl;
        const int st = kb >> 1, e = kb & 1;
        const int tok = ((c >> 2) & 1) * 8 + e * 4 + (c & 3);
        const int64_t bk = (c >> 3) ? (int64_t)blk[2 * st + 1] : (int64_t)blk[2 * st];
        const uint16_t *pg = a.k_cache + bk * a.k_block_stride + hoff + tok * 8 + g * 128;
#pragma unroll
        for (int ds = 0; ds < G::NDS; ++ds)
            kf[kl][ds] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8 *>(pg + ds * 512));
    }
    u32x4 vraw[DPW][G::NKS];
#pragma unroll
    for (int st = 0; st < G::NKS; ++st) {
        const int64_t bv = (g >> 1) ? (int64_t)blk[2 * st + 1] : (int64_t)blk[2 * st];
        const uint16_t *pg = a.v_cache + bv * a.v_block_stride + hoff + 8 * (g & 1) + c * 16;
#pragma unroll
        for (int dl = 0; dl < DPW; ++dl)
            vraw[dl][st] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(pg + (16 * (w * DPW + dl)) * 16));
    }
    // keep every load above ahead of the first use of any of them
    __builtin_amdgcn_sched_barrier(0);
    if (QL) {
#pragma unroll
        for (int k = 0; k < QPW; ++k)
            sq[w * QPW + k][lane] = qpart[k];
        __syncthreads();
    }

    // ---- new tokens of this launch whose slots fall in this tile (FUSE):
    // their keys and values come from the new rows, not from the pool.  A
    // lane's K fragment is one token, so at most one new token replaces it;
    // a lane's V fragment holds 8 consecutive tokens of one dim, any number
    // of which may be new (consecutive positions of one sequence), so each of
    // the 8 elements records its own token (8-bit field: index + 1, 0 =
    // none).  The pool load of a fragment may race with this launch's scatter
    // of the new tokens, but only in elements that are replaced here; the
    // other elements are never written by the launch.
    if (FUSE) {
        int knew[KPW];
        uint64_t vidx[G::NKS];
#pragma unroll
        for (int kl = 0; kl < KPW; ++kl)
            knew[kl] = -1;
#pragma unroll
        for (int st = 0; st < G::NKS; ++st)
            vidx[st] = 0;
        for (int jn = a.num_new - 1; jn >= 0; --jn) {       // for a shared slot, the first token wins
            const int64_t sj = ((int64_t)__builtin_amdgcn_readlane((int)(my_new >> 32), jn) << 32) |
                               (uint32_t)__builtin_amdgcn_readlane((int)my_new, jn);
            if (sj < 0 || sj >= a.num_blocks * BS)
                continue;
            const int64_t bj = sj / BS;
            const int tj = (int)(sj % BS);
#pragma unroll
            for (int kl = 0; kl < KPW; ++kl) {
                const int kb = w * KPW + kl;
                const int st = kb >> 1, e = kb & 1;
                const int tok = ((c >> 2) & 1) * 8 + e * 4 + (c & 3);
                const int64_t bk = (c >> 3) ? (int64_t)blk[2 * st + 1] : (int64_t)blk[2 * st];
                knew[kl] = (bk == bj && tok == tj) ? jn : knew[kl];
            }
            const int sh = 8 * (tj & 7);
#pragma unroll
            for (int st = 0; st < G::NKS; ++st) {
                const int64_t bv = (g >> 1) ? (int64_t)blk[2 * st + 1] : (int64_t)blk[2 * st];
                const bool hit = bv == bj && (tj >> 3) == (g & 1);
                vidx[st] = hit ? (vidx[st] & ~(0xFFull << sh)) | ((uint64_t)(jn + 1) << sh) : vidx[st];
            }
        }
#pragma unroll
        for (int kl = 0; kl < KPW; ++kl) {
            if (knew[kl] >= 0) {
                const uint16_t *row = a.new_k + knew[kl] * a.new_k_stride + (int64_t)kvh * D + g * 8;
#pragma unroll
                for (int ds = 0; ds < G::NDS; ++ds)
                    kf[kl][ds] = *reinterpret_cast<const bf16x8 *>(row + ds * 32);
            }
        }
        bool vhit = false;
#pragma unroll
        for (int st = 0; st < G::NKS; ++st)
            vhit |= vidx[st] != 0;
        if (__builtin_amdgcn_ballot_w64(vhit) != 0) {      // wave-uniform: only waves holding a new value
            const uint16_t *vrow = a.new_v + (int64_t)kvh * D + 16 * (w * DPW) + c;
            // one round per (step, element) that some lane of the wave replaces
            // (a decode step with one new token per sequence: one round)
#pragma unroll
            for (int st = 0; st < G::NKS; ++st) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int id = (int)((vidx[st] >> (8 * e)) & 0xFF);
                    if (__builtin_amdgcn_ballot_w64(id != 0) == 0)
                        continue;
                    if (id != 0) {
                        const uint32_t keep = (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
#pragma unroll
                        for (int dl = 0; dl < DPW; ++dl) {
                            const uint32_t x = vrow[(int64_t)(id - 1) * a.new_v_stride + 16 * dl];
                            vraw[dl][st][e >> 1] = (vraw[dl][st][e >> 1] & keep) | (x << (16 * (e & 1)));
                        }
                    }
                }
            }
        }
    }
    // V of keys >= seq_len is zeroed; only the tile holding key seq_len - 1
    // has such keys (a wave-uniform branch, so full tiles skip the masks)
    bf16x8 vf[DPW][G::NKS];
    if ((tile + 1) * G::T > seq_len) {
#pragma unroll
        for (int st = 0; st < G::NKS; ++st) {
            const int valid = seq_len - (tile * G::NKB + 2 * st + (g >> 1)) * BS;
#pragma unroll
            for (int dl = 0; dl < DPW; ++dl)
                vf[dl][st] = __builtin_bit_cast(bf16x8, valid >= BS ? vraw[dl][st]
                                                                    : mask_tokens(vraw[dl][st], 8 * (g & 1), valid));
        }
    } else {
#pragma unroll
        for (int st = 0; st < G::NKS; ++st)
#pragma unroll
            for (int dl = 0; dl < DPW; ++dl)
                vf[dl][st] = __builtin_bit_cast(bf16x8, vraw[dl][st]);
    }

    // ---- S for this wave's key blocks; scale, mask, wave max.  Scores are
    // masked only in a tile that reaches past the smallest key limit of the
    // row's columns (the first query's); a column past ncols is never
    // stored, and no column's output depends on another column's scores.
    const int lim_min = a.causal ? seq_len - q_len + 1 : seq_len;
    const bool smask = (tile + 1) * G::T > lim_min;
    f32x4 s[KPW];
    float mx = -INFINITY;
#pragma unroll
    for (int kl = 0; kl < KPW; ++kl) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < G::NDS; ++ds)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kl][ds], QL ? sq[ds][lane] : cols.qf[QL ? 0 : ds], acc,
                                                          0, 0, 0);
        const int kb = w * KPW + kl;
        const int st = kb >> 1, e = kb & 1;
        s[kl] = acc;
        if (smask) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = tile * G::T + 32 * st + 8 * g + 4 * e + i;
                s[kl][i] = key < cols.lim ? acc[i] : -INFINITY;
            }
        }
        mx = fmax2(mx, fmax2(fmax2(s[kl][0], s[kl][1]), fmax2(s[kl][2], s[kl][3])));
    }
    mx = max_xor32(max_xor16(mx));
    if (g == 0)
        smax[w][c] = mx;
    __syncthreads();
    mx = __fmul_rn(fmax2(fmax2(smax[0][c], smax[1][c]), fmax2(smax[2][c], smax[3][c])), a.scale_log2);
    const float nmu = mx == -INFINITY ? 0.f : -mx;

    // ---- p, this wave's level of the sum tree, P^T values to LDS
    float part[KPW];
#pragma unroll
    for (int kl = 0; kl < KPW; ++kl) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            s[kl][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kl][i], a.scale_log2, nmu));
        part[kl] = __fadd_rn(__fadd_rn(s[kl][0], s[kl][1]), __fadd_rn(s[kl][2], s[kl][3]));
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const __bf16 lo = (__bf16)s[kl][2 * h], hi = (__bf16)s[kl][2 * h + 1];
            spf[w][2 * kl + h][lane] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                                       ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
    }
    ssum[w][lane] = KPW == 2 ? __fadd_rn(part[0], part[KPW - 1]) : part[0];
    __syncthreads();

    // ---- l: remaining levels of the tree, then across lanes
    float l = __fadd_rn(__fadd_rn(ssum[0][lane], ssum[1][lane]), __fadd_rn(ssum[2][lane], ssum[3][lane]));
    l = sum_xor32(sum_xor16(l));

    // ---- P^T operands of every 32-key step, then P.V for this wave's dims
    bf16x8 pf[G::NKS];
#pragma unroll
    for (int st = 0; st < G::NKS; ++st) {
        u32x4 u;
        if (KPW == 2) {
            u = u32x4{spf[st][0][lane], spf[st][1][lane], spf[st][2][lane], spf[st][3][lane]};
        } else {
            u = u32x4{spf[2 * st][0][lane], spf[2 * st][1][lane], spf[2 * st + 1][0][lane], spf[2 * st + 1][1][lane]};
        }
        pf[st] = __builtin_bit_cast(bf16x8, u);
    }
    const int64_t slot = ((int64_t)b * a.num_kv_heads + kvh) * a.max_tiles + tile;
    float *accp = a.ws_acc + (slot * a.split_cols + c) * D + 4 * g;
#pragma unroll
    for (int dl = 0; dl < DPW; ++dl) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < G::NKS; ++st)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dl][st], pf[st], acc, 0, 0, 0);
        if (c < ncols) {
            // head_dim 512: 16 KB of partials per tile (an eighth of the tile's
            // K/V bytes) stream out during the kernel instead of leaving the
            // L2 dirty for its end
            if (D == 512)
                __builtin_nontemporal_store(acc, reinterpret_cast<f32x4 *>(accp + 16 * (w * DPW + dl)));
            else
                *reinterpret_cast<f32x4 *>(accp + 16 * (w * DPW + dl)) = acc;
        }
    }
    if (w == 0 && g == 0 && c < ncols) {
        a.ws_m[slot * a.split_cols + c] = mx;
        a.ws_l[slot * a.split_cols + c] = l;
    }
}

// Fold kernel.  Workgroup = (32 consecutive dims of one column, kv head,
// sequence).  All waves stage the column's per-tile partials into LDS, with
// every load of a round issued before any is used (the first round is
// fetched before the row's length is even known: the workspace holds
// max_tiles slots).  The fold factor of tile t depends only on the running
// max before t -- the max of the earlier tile maxima, exact in any order,
// whose reference is the state's reference -- so all factors come from one
// prefix-max scan, stored per tile as one (gs, h) pair; then wave 0 runs
// the dependent ACC chain (one dim per lane, half the wave) and wave 1 the L chain, each in
// ascending tile order, and wave 0 writes the BF16 output.
constexpr int kFoldSlice = 32;
constexpr int kFoldTiles = 192;
constexpr int kFoldUnits = kFoldTiles * (kFoldSlice / 4) / NT;   // 16-byte loads per thread per round

// One round of the fold's inputs: the (acc, m, l) partials of tiles
// t0 .. t0+nt-1 for one column and one 32-dim slice.  fold_load issues the
// (m, l) loads first, then the acc loads (rounds of whole workgroups past
// the last tile issue none); the max scan reads the m values from the
// registers of the threads that loaded them while the acc partials are still
// in flight, and fold_store waits for those and writes them to LDS.
struct FoldRound {
    f32x4 v[kFoldUnits];
    float m, l;
};

template <int D>
__device__ __forceinline__ void fold_load(const AttnArgs &a, int64_t slot0, int col, int d0, int t0, int nt,
                                          FoldRound &fr)
{
    const int th = threadIdx.x;
    fr.m = 0.f;
    fr.l = 0.f;
    if (th < nt) {                           // nt <= kFoldTiles: one tile per thread
        const int64_t si = (slot0 + t0 + th) * a.split_cols + col;
        fr.m = a.ws_m[si];
        fr.l = a.ws_l[si];
    }
#pragma unroll
    for (int r = 0; r < kFoldUnits; ++r) {
        if (r * NT >= nt * (kFoldSlice / 4))
            break;
        const int u = th + r * NT;
        const int tt = min(u / (kFoldSlice / 4), nt - 1);
        const int q = u % (kFoldSlice / 4);
        const int64_t si = (slot0 + t0 + tt) * a.split_cols + col;
        fr.v[r] = *reinterpret_cast<const f32x4 *>(a.ws_acc + si * D + d0 + 4 * q);
    }
}

__device__ __forceinline__ void fold_store(const FoldRound &fr, int nt, float (*stage)[kFoldSlice])
{
    const int th = threadIdx.x;
#pragma unroll
    for (int r = 0; r < kFoldUnits; ++r) {
        if (r * NT >= nt * (kFoldSlice / 4))
            break;
        const int u = th + r * NT;
        const int tt = u / (kFoldSlice / 4);
        if (tt < nt)
            *reinterpret_cast<f32x4 *>(&stage[tt][4 * (u % (kFoldSlice / 4))]) = fr.v[r];
    }
}


template <int D>
__global__ __launch_bounds__(NT) void split_fold_kernel(AttnArgs a)
{
    using G = Geo<D>;
    constexpr int NSL = D / kFoldSlice;
    __shared__ float stage[kFoldTiles][kFoldSlice];
    __shared__ float sl[kFoldTiles];
    __shared__ float2 sgh[kFoldTiles];         // (gs, h) of each tile: one LDS read per tile in the chains
    __shared__ float wmax[NW], sL;

    const int slice = blockIdx.x % NSL;
    const int col = blockIdx.x / NSL;
    const int kvh = blockIdx.y;
    const int b = blockIdx.z;
    const int64_t slot0 = ((int64_t)b * a.num_kv_heads + kvh) * a.max_tiles;
    const int d0 = slice * kFoldSlice;
    const int th = threadIdx.x, lane = th & 63, w = th >> 6;

    // the first round's loads are issued speculatively for min(max_tiles,
    // kFoldTiles) tiles, then the row's metadata; the metadata is waited for
    // (and the workgroup may leave) while the partials are still in flight
    const int nt0 = min(kFoldTiles, a.max_tiles);
    FoldRound fr;
    fold_load<D>(a, slot0, col, d0, 0, nt0, fr);
    int q0, q_len, seq_len;
    if (!row_ok(a, b, q0, q_len, seq_len))
        return;
    const int ncols = q_len * a.group;
    if (ncols > a.split_cols || col >= ncols)
        return;
    const int n_tiles = (seq_len + G::T - 1) / G::T;

    float M = -INFINITY, L = 0.f, acc = 0.f;
    for (int t0 = 0; t0 < n_tiles; t0 += kFoldTiles) {
        const int nt = min(kFoldTiles, n_tiles - t0);
        if (t0 > 0) {
            fold_load<D>(a, slot0, col, d0, t0, nt, fr);
            __syncthreads();
        }
        // running max before each tile: inclusive wave scans, then wave
        // totals; thread t holds tile t's max in a register (this waits for
        // the (m, l) loads only)
        const float mt = th < nt ? fr.m : -INFINITY;
        float v = mt;
#pragma unroll
        for (int off = 1; off < 64; off *= 2) {
            const float o = __shfl_up(v, off, 64);
            v = lane >= off ? fmax2(v, o) : v;
        }
        if (lane == 63)
            wmax[w] = v;
        __syncthreads();
        float pre = M, total = M;
        for (int k = 0; k < NW; ++k) {
            pre = k < w ? fmax2(pre, wmax[k]) : pre;
            total = fmax2(total, wmax[k]);
        }
        const float incl = fmax2(pre, v);
        float excl = __shfl_up(incl, 1, 64);
        excl = lane == 0 ? pre : excl;
        if (th < nt) {
            const FoldF f = fold_factors(ref_of(excl), mt);
            sgh[th] = make_float2(f.gs, f.h);
            sl[th] = fr.l;
        }
        fold_store(fr, nt, stage);          // the partials, needed only by the chains
        __syncthreads();
        // wave 0 folds ACC (one dim per lane), wave 1 folds L, side by side;
        // every thread carries M (the next round's scan starts from it)
        if (w == 0 && th < kFoldSlice) {
#pragma unroll 8
            for (int tt = 0; tt < nt; ++tt) {
                const float2 gh = sgh[tt];
                acc = fold1v(acc, stage[tt][th], gh.x, gh.y);
            }
        } else if (w == 1) {
#pragma unroll 8
            for (int tt = 0; tt < nt; ++tt) {
                const float2 gh = sgh[tt];
                L = fold1v(L, sl[tt], gh.x, gh.y);
            }
        }
        M = total;
    }
    if (th == 64)
        sL = L;
    __syncthreads();
    L = sL;
    if (th < kFoldSlice) {
        const ColInfo ci = col_info(a, col, kvh, q0, q_len, seq_len);
        a.out[ci.row * a.out_token_stride + (int64_t)ci.head * D + d0 + th] = finish1(acc, 1.0f / L);
        if (a.lse && slice == 0 && th == 0)
            a.lse[ci.row * a.lse_token_stride + ci.head] = lse_of(ref_of(M), L);
    }
}

// Register fold of NU (column, 64-dim slice) units of one row by one wave,
// one dim per lane.  In rounds of up to 64 tiles: lane t loads a unit's
// (m, l) of tile t and every lane loads its dim's acc partials of the round
// into registers (all units' loads issued before any is used); the wave scans
// the running max over the lanes (the prefix max of split_fold_kernel) and
// each lane derives its tile's fold factors; then every lane runs its dim's
// ACC chain and the column's L chain in tile order, taking tile tt's factors
// from lane tt (readlane).  Same factors and the same FMA order as
// split_fold_kernel, so the same bits; no LDS and no barrier.  on[j] is
// wave-uniform (a unit past the row's columns is skipped).
constexpr int kFoldWideTiles = 64;

template <int D, int NU>
__device__ __forceinline__ void fold_units(const AttnArgs &a, int b, int kvh, int q0, int q_len, int seq_len,
                                           const int (&col)[NU], const int (&slice)[NU], const bool (&on)[NU])
{
    using G = Geo<D>;
    const int lane = threadIdx.x & 63;
    const int n_tiles = (seq_len + G::T - 1) / G::T;
    const int64_t slot0 = ((int64_t)b * a.num_kv_heads + kvh) * a.max_tiles;
    float M[NU], L[NU], acc[NU];
#pragma unroll
    for (int j = 0; j < NU; ++j) {
        M[j] = -INFINITY;
        L[j] = 0.f;
        acc[j] = 0.f;
    }
    for (int t0 = 0; t0 < n_tiles; t0 += kFoldWideTiles) {
        const int nt = min(kFoldWideTiles, n_tiles - t0);
        float mt[NU], lt[NU], v[NU][kFoldWideTiles];
#pragma unroll
        for (int j = 0; j < NU; ++j) {
            mt[j] = -INFINITY;
            lt[j] = 0.f;
            if (on[j] && lane < nt) {
                const int64_t si = (slot0 + t0 + lane) * a.split_cols + col[j];
                mt[j] = a.ws_m[si];
                lt[j] = a.ws_l[si];
            }
        }
#pragma unroll
        for (int j = 0; j < NU; ++j) {
            const float *src = a.ws_acc + ((slot0 + t0) * a.split_cols + col[j]) * D + slice[j] * 64 + lane;
#pragma unroll
            for (int tt = 0; tt < kFoldWideTiles; ++tt)
                v[j][tt] = on[j] && tt < nt ? src[(int64_t)tt * a.split_cols * D] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < NU; ++j) {
            // running max before each tile (lane = tile), from the running max M of earlier rounds
            float incl = mt[j];
#pragma unroll
            for (int off = 1; off < 64; off *= 2) {
                const float o = __shfl_up(incl, off, 64);
                incl = lane >= off ? fmax2(incl, o) : incl;
            }
            incl = fmax2(incl, M[j]);
            float excl = __shfl_up(incl, 1, 64);
            excl = lane == 0 ? M[j] : excl;
            const FoldF f = fold_factors(ref_of(excl), mt[j]);
            M[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(incl), 63));
#pragma unroll
            for (int tt = 0; tt < kFoldWideTiles; ++tt) {
                if (tt < nt) {
                    const float gs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f.gs), tt));
                    const float h = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f.h), tt));
                    const float l = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lt[j]), tt));
                    acc[j] = fold1v(acc[j], v[j][tt], gs, h);
                    L[j] = fold1v(L[j], l, gs, h);
                }
            }
        }
    }
#pragma unroll
    for (int j = 0; j < NU; ++j) {
        if (!on[j])
            continue;
        const ColInfo ci = col_info(a, col[j], kvh, q0, q_len, seq_len);
        a.out[ci.row * a.out_token_stride + (int64_t)ci.head * D + slice[j] * 64 + lane] = finish1(acc[j], 1.0f / L[j]);
        if (a.lse && slice[j] == 0 && lane == 0)
            a.lse[ci.row * a.lse_token_stride + ci.head] = lse_of(ref_of(M[j]), L[j]);
    }
}

// Fold kernel for rows with many columns (split_cols > 16).  Workgroup =
// (kFoldWideCols consecutive columns, 64-dim slice, kv head, sequence), one
// wave per column: the register fold above, one unit per wave.
constexpr int kFoldWideCols = 8;

template <int D>
__global__ __launch_bounds__(64 * kFoldWideCols) void split_fold_wide_kernel(AttnArgs a)
{
    constexpr int NSL = D / 64;
    const int b = blockIdx.z;
    int q0, q_len, seq_len;
    if (!row_ok(a, b, q0, q_len, seq_len))
        return;
    const int ncols = q_len * a.group;
    const int col[1] = {(int)(blockIdx.x / NSL) * kFoldWideCols + (int)(threadIdx.x >> 6)};
    if (ncols > a.split_cols || col[0] >= ncols)      // wave-uniform
        return;
    const int slice[1] = {(int)(blockIdx.x % NSL)};
    const bool on[1] = {true};
    fold_units<D, 1>(a, b, (int)blockIdx.y, q0, q_len, seq_len, col, slice, on);
}

// ---------------------------------------------------------------- direct K/V tile transfers

// The large-grid prefill fetches K/V tiles straight from HBM into LDS
// (global_load_lds: lane L of a wave writes 16 bytes at the wave's LDS base +
// 16 L, so each lane loads the unit that belongs at its swizzled slot); no
// staging registers.  Wave w stages page w of every tile (its K page or V
// page, four 1 KB chunks each); the page's block id is read ahead, so it has
// landed before the tile is issued.  V of keys at or beyond seq_len is
// zeroed in LDS once the tail tile has landed.

// Per-lane source byte offsets (inside one page) of the 16-byte units that
// chunk 0 of page `page` holds at this lane's LDS slots; chunk i adds i KB
// (the K swizzle and the V slot order do not depend on the chunk).
struct DbOffsets {
    uint32_t k, v;
};

__device__ __forceinline__ DbOffsets db_offsets(int page)
{
    const int lane = threadIdx.x & 63;
    DbOffsets o;
    // K: slot (du, tok') holds unit (du, ksw(tok', page))
    o.k = (uint32_t)(((lane >> 4) * 16 + ksw(lane & 15, page)) * 16);
    // V: slot vslot(d, half) holds unit (d, half), at source byte 32 d + 16 half
    o.v = (uint32_t)((lane & 31) * 32 + (lane >> 5) * 16);
    return o;
}

// Block id of this wave's page of `tile`, as a vector load (it is consumed
// only after the next tile barrier, which waits for it).
__device__ __forceinline__ int db_load_id(const int32_t *bt_row, int tile)
{
    return bt_row[tile * 8 + (int)(threadIdx.x >> 6)];
}

// Four consecutive 1 KB chunks of one page: global_load_lds_dwordx4 with a
// 64-bit SGPR base, a per-lane 32-bit offset and the wave's LDS destination
// in M0.  The instruction's immediate offset moves the global source and the
// LDS destination alike, so the four chunks share one base and one M0 value
// and the chunk step rides in the offset (no address arithmetic per chunk).
// Written as inline assembly so that the compiler's wait-count bookkeeping
// does not treat every later LDS read as dependent on the transfer (it would
// wait for all LDS reads at each use); the transfers are waited for
// explicitly (vmcnt before the tile barrier).  The leading s_nop covers the
// M0-write hazard.
__device__ __forceinline__ void db_chunks4(const char *base, uint32_t off, uint32_t lds_addr)
{
    asm volatile("s_nop 0\n\t"
                 "global_load_lds_dwordx4 %0, %1\n\t"
                 "global_load_lds_dwordx4 %0, %1 offset:1024\n\t"
                 "global_load_lds_dwordx4 %0, %1 offset:2048\n\t"
                 "global_load_lds_dwordx4 %0, %1 offset:3072"
                 :
                 : "v"(off), "s"(base), "{m0}"(lds_addr)
                 : "memory");
}

// This wave's page of a K (or V) tile: block `id` of `cache`, kv head kvh,
// copied to dst + page * PAGE in four 1 KB chunks.
template <int D>
__device__ __forceinline__ void db_issue_half(char *dst, const AttnArgs &a, const uint16_t *cache, int64_t block_stride,
                                              int id, int kvh, int page, uint32_t off)
{
    using G = Geo<D>;
    static_assert(G::PAGE == 4096, "four 1 KB chunks per page");
    const uint32_t nb = a.num_blocks > 0x7fffffff ? 0x7fffffffu : (uint32_t)a.num_blocks;
    id = (uint32_t)id < nb ? id : 0;                          // ids outside the pool read block 0
    const char *src = reinterpret_cast<const char *>(cache + (int64_t)id * block_stride + (int64_t)kvh * BS * D);
    const uint32_t d0 = (uint32_t)(size_t)(__attribute__((address_space(3))) char *)(dst + page * G::PAGE);
    db_chunks4(src, off, d0);
}

// Zero V of keys >= seq_len in a staged tile (only the tile holding seq_len - 1
// and later ones can have such keys).
template <int D, int NWV>
__device__ __forceinline__ void db_mask_tail(char *vl, int seq_len, int tile)
{
    using G = Geo<D>;
    constexpr int DB_NT = NWV * 64;
    for (int u = threadIdx.x; u < G::NKB * G::UPP; u += DB_NT) {
        const int pg = u / G::UPP, slot = u % G::UPP;
        const int valid = seq_len - (tile * G::NKB + pg) * BS;
        if (valid >= BS)
            continue;
        const int hf = (slot >> 5) & 1;                 // the slot's token half (vslot)
        u32x4 *q = reinterpret_cast<u32x4 *>(vl + pg * G::PAGE + slot * 16);
        *q = mask_tokens(*q, hf * 8, valid);
    }
}

// ---------------------------------------------------------------- split-KV partials, many columns

// P.V of one 16-column block from zero, per 16-dim block (32-key steps
// ascending, the same MFMA chain as every other kernel), stored as the
// tile's acc partial; the next step's V fragments are read while the
// current step's MFMAs run.
template <int D, int DG>
__device__ __forceinline__ void tile_pv_store(const char *vl, const bf16x8 (&pf)[Geo<D>::NKS], float *accp, bool store)
{
    using G = Geo<D>;
    static_assert(G::NDB % DG == 0, "whole groups");
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, c = lane & 15;
    auto vaddr = [&](int db, int stp) -> const char * {
        const int d = 16 * db + c;
        return vl + (g >> 1) * G::PAGE + vslot(d, g & 1) * 16 + 2 * stp * G::PAGE;
    };
#pragma unroll
    for (int db0 = 0; db0 < G::NDB; db0 += DG) {
        f32x4 o[DG];
        bf16x8 vf[DG], vn[DG];
#pragma unroll
        for (int d = 0; d < DG; ++d) {
            o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
            vf[d] = *reinterpret_cast<const bf16x8 *>(vaddr(db0 + d, 0));
        }
#pragma unroll
        for (int stp = 0; stp < G::NKS; ++stp) {
            if (stp + 1 < G::NKS) {
#pragma unroll
                for (int d = 0; d < DG; ++d)
                    vn[d] = *reinterpret_cast<const bf16x8 *>(vaddr(db0 + d, stp + 1));
            }
#pragma unroll
            for (int d = 0; d < DG; ++d)
                o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[d], pf[stp], o[d], 0, 0, 0);
#pragma unroll
            for (int d = 0; d < DG; ++d)
                vf[d] = vn[d];
        }
        if (store) {
#pragma unroll
            for (int d = 0; d < DG; ++d) {
                if (D == 512)
                    __builtin_nontemporal_store(o[d], reinterpret_cast<f32x4 *>(accp + 16 * (db0 + d)));
                else
                    *reinterpret_cast<f32x4 *>(accp + 16 * (db0 + d)) = o[d];
            }
        }
    }
}

// Split-KV partials for rows with many columns (split_cols > 16).
// Workgroup = (tile, kv head x group of kTileWaves column blocks, sequence).
// The tile's K and V pages are staged in LDS once (the prefill kernels'
// transfers and layout); each wave then runs the prefill tile step (tile_qk,
// tile_stats, P.V) for one 16-column block and stores the tile's (m, l, acc)
// partials for the fold instead of folding them.  Per column these are the
// operations of the split-KV partial kernel, so the same bits; there is no
// exchange between waves and no barrier after the staging.

template <int D>
__global__ __launch_bounds__(64 * kTileWaves) void split_tile_kernel(AttnArgs a)
{
    using G = Geo<D>;
    constexpr int NWV = kTileWaves;
    constexpr int HALF = G::NKB * G::PAGE;        // K (or V) part of one tile
    constexpr int CPP = G::PAGE / 1024;           // 1 KB chunks per page
    constexpr int CPW = G::NKB * CPP / NWV;       // K (or V) chunks per wave
    static_assert(CPW % 4 == 0 && CPP % 4 == 0 && (G::NKB * CPP) % NWV == 0, "runs of four chunks per wave");
    extern __shared__ __attribute__((aligned(16))) char lds[];
    char *const kbuf = lds;
    char *const vbuf = lds + HALF;

    const int tile = blockIdx.x;
    const int kvh = blockIdx.y % a.num_kv_heads;
    const int grp = blockIdx.y / a.num_kv_heads;
    const int b = blockIdx.z;
    int q0, q_len, seq_len;
    if (!row_ok(a, b, q0, q_len, seq_len))
        return;
    const int ncols = q_len * a.group;
    if (ncols > a.split_cols || grp * NWV * 16 >= ncols)
        return;
    const int n_tiles = (seq_len + G::T - 1) / G::T;
    if (tile >= n_tiles)
        return;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, c = lane & 15;

    // ---- stage the tile's K and V pages: this wave's chunks of each
    const int32_t *bt_row = a.block_tables + (int64_t)b * a.bt_stride;
    const ids_t<G::NKB> blk = tile_blocks<G::NKB>(a, bt_row, tile);
    auto lds_addr = [](const void *p) { return (uint32_t)(size_t)(const __attribute__((address_space(3))) char *)p; };
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
        char *const buf = kv ? vbuf : kbuf;
        const uint16_t *const cache = kv ? a.v_cache : a.k_cache;
        const int64_t stride = kv ? a.v_block_stride : a.k_block_stride;
#pragma unroll
        for (int i = 0; i < CPW; i += 4) {
            const int ch = wave * CPW + i;
            const int page = ch / CPP, part = ch % CPP;
            const int id = __builtin_amdgcn_readfirstlane(blk[page]);     // inside the pool (tile_blocks)
            const char *src = reinterpret_cast<const char *>(cache + (int64_t)id * stride + (int64_t)kvh * BS * D);
            const DbOffsets o = db_offsets(page);
            db_chunks4(src + part * 1024, kv ? o.v : o.k, lds_addr(buf + page * G::PAGE + part * 1024));
        }
    }
    // Q of this wave's column block while the pages land
    const int cb = grp * NWV + wave;
    const int col = cb * 16 + c;
    Cols<D> cols[1];
    load_q<D>(cols[0], a, col_info(a, col, kvh, q0, q_len, seq_len));
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if ((tile + 1) * G::T > seq_len) {
        db_mask_tail<D, NWV>(vbuf, seq_len, tile);
        __syncthreads();
    }
    if (cb * 16 >= ncols)                           // wave-uniform; no barrier follows
        return;

    f32x4 sc[1][G::NKB];
    tile_qk<D, 1>(kbuf, cols, sc);
    int min_lim = cols[0].lim;
#pragma unroll
    for (int off = 1; off < 64; off *= 2)
        min_lim = min(min_lim, __shfl_xor(min_lim, off, 64));
    float mx[1], lsum[1];
    bf16x8 pf[1][G::NKS];
    if ((tile + 1) * G::T > min_lim)
        tile_stats<D, 1, true>(sc, cols, tile, a.scale_log2, mx, lsum, pf);
    else
        tile_stats<D, 1, false>(sc, cols, tile, a.scale_log2, mx, lsum, pf);
    const int64_t slot = ((int64_t)b * a.num_kv_heads + kvh) * a.max_tiles + tile;
    tile_pv_store<D, (D == 128 ? 8 : 4)>(vbuf, pf[0], a.ws_acc + (slot * a.split_cols + col) * D + 4 * g, col < ncols);
    if (g == 0 && col < ncols) {
        a.ws_m[slot * a.split_cols + col] = mx[0];
        a.ws_l[slot * a.split_cols + col] = lsum[0];
    }
}

// ---------------------------------------------------------------- streaming prefill, direct loads

// vmcnt(N) with the other counters left alone (gfx9 s_waitcnt encoding).
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Block ids of this wave's pages of `tile` into LDS (one dword per page,
// lanes >= npages idle), as an LDS DMA counted by vmcnt like the tile
// transfers, so that no compiler-inserted wait stalls on the transfers.
__device__ __forceinline__ void id_dma(const int32_t *src, int npages, uint32_t lds_addr)
{
    // lane index from mbcnt (computed here rather than kept live from the
    // work-item id, which the tile loops would otherwise hold or spill)
    const uint32_t ln = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    if ((int)ln < npages)
        asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1"
                     :
                     : "v"(ln * 4u), "s"(src), "{m0}"(lds_addr)
                     : "memory");
}

// P.V of one 16-column block with the V fragments read through a ring of
// RD register sets (the single-buffer kernel's form: its registers leave no
// room for two dim blocks in flight): per 16-dim block the same chain
// (32-key steps ascending from zero) and the same fold fma(tile, h, ACC) as
// prefill_pv.  Each ring slot is reloaded with the fragment RD positions
// ahead as soon as its MFMA is issued, and a block is folded while the next
// block's MFMAs run.
template <int D, int RD, class Hook = NoHook>
__device__ __forceinline__ void prefill_pv_ring(const char *vl, const bf16x8 (&pf)[Geo<D>::NKS], const FoldF &f,
                                                State<D> &st, Hook hook = Hook{})
{
    using G = Geo<D>;
    constexpr int N = G::NDB * G::NKS;           // fragment j: dim block j / NKS, key step j % NKS
    static_assert(RD >= 1 && RD <= N, "ring depth");
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, c = lane & 15;
    // the lane's operand of dim block db lies (db / 2) KB + (db % 2) * 256 B
    // past its operand of block 0 (vslot of dim 16 db + c)
    const char *const vb = vl + (g >> 1) * G::PAGE + vslot(c, g & 1) * 16;
    auto frag = [&](int j) {
        const int db = j / G::NKS, stp = j % G::NKS;
        return *reinterpret_cast<const bf16x8 *>(vb + (db >> 1) * 1024 + (db & 1) * 256 + 2 * stp * G::PAGE);
    };
    bf16x8 ring[RD];
#pragma unroll
    for (int j = 0; j < RD; ++j)
        ring[j] = frag(j);
    f32x4 o, prev;
#pragma unroll
    for (int j = 0; j < N; ++j) {
        const int db = j / G::NKS, stp = j % G::NKS;
        o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ring[j % RD], pf[stp], stp == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : o,
                                                    0, 0, 0);
        if (j + RD < N)
            ring[j % RD] = frag(j + RD);
        if (stp == G::NKS - 1) {
            if (db > 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    st.acc[db - 1][i] = __builtin_fmaf(prev[i], f.h, st.acc[db - 1][i]);
            }
            prev = o;
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (j + RD < N)
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_barrier(0);
        hook(j);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        st.acc[G::NDB - 1][i] = __builtin_fmaf(prev[i], f.h, st.acc[G::NDB - 1][i]);
}

// Workgroup = (column group, kv head, sequence): NWV waves x CB column
// blocks.  One LDS buffer for the K tile and one for the V tile, each
// refilled straight from HBM as soon as its last reader is done: each wave
// copies its share of V(t) during QK(t) and of K(t+1) during the first half
// of P.V(t), one 1 KB chunk at a time between MFMAs (a wave waits while the
// CU's memory pipeline takes its transfer instructions, so the copies are
// spread rather than issued together between the phases).  V(t) lands during
// the softmax, K(t+1) during the rest of P.V; wave 0 fetches the block ids of
// tile t+2 (to LDS) during P.V(t).  Two barriers per tile; between the QK and
// the softmax there is none, so a SIMD's first wave starts its softmax while
// the second still runs its QK MFMAs.  Per column the arithmetic is exactly
// the tile step of the other prefill kernels.
template <int D, int CB, int NWV, int WPE>
__global__ __launch_bounds__(NWV * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void prefill_sb_kernel(AttnArgs a)
{
    using G = Geo<D>;
    constexpr int NCOL = NWV * CB * 16;
    constexpr int HALF = G::NKB * G::PAGE;        // K (or V) part of one tile
    constexpr int CPP = G::PAGE / 1024;           // 1 KB chunks per page
    constexpr int CPW = G::NKB * CPP / NWV;       // K (or V) chunks per wave per tile
    static_assert(CPW >= 1 && (G::NKB * CPP) % NWV == 0, "whole chunks per wave");
    static_assert(CPW + 1 < 64, "vmcnt range");
    extern __shared__ __attribute__((aligned(16))) char lds[];
    char *const kbuf = lds;
    char *const vbuf = lds + HALF;
    int32_t *const ids = reinterpret_cast<int32_t *>(lds + 2 * HALF);     // [2][NKB]

    int b, kvh, cgi;
    if (!wg_slot(a, b, kvh, cgi))
        return;
    const int cg = a.col_groups - 1 - cgi;           // heaviest (latest) columns first

    int q0, q_len, seq_len;
    if (!row_ok(a, b, q0, q_len, seq_len))
        return;
    const int ncols = q_len * a.group;
    if (cg * NCOL >= ncols || ncols <= a.split_cols)
        return;
    const int col_last = min((cg + 1) * NCOL, ncols) - 1;
    const int pos_last = seq_len - q_len + col_last / a.group;
    const int last = (a.causal ? pos_last : seq_len - 1) / G::T;
    const int32_t *bt_row = a.block_tables + (int64_t)b * a.bt_stride;

    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int c = threadIdx.x & 15;
    Cols<D> cols[CB];
    State<D> st[CB];
    bool active = false;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const int col = cg * NCOL + (wave * CB + cb) * 16 + c;
        const ColInfo ci = col_info(a, col, kvh, q0, q_len, seq_len);
        load_q<D>(cols[cb], a, ci);
        state_init<D>(st[cb]);
        active |= (cg * NCOL + (wave * CB + cb) * 16) < ncols;
    }
    int min_lim = 0x7fffffff;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
        min_lim = min(min_lim, cols[cb].lim);
#pragma unroll
    for (int off = 1; off < 64; off *= 2)
        min_lim = min(min_lim, __shfl_xor(min_lim, off, 64));

    auto lds_addr = [](const void *p) { return (uint32_t)(size_t)(const __attribute__((address_space(3))) char *)p; };
    // this wave's chunks of `tile`: block ids (from LDS) -> K or V chunks
    auto issue = [&](bool is_k, int tile) {
        char *const buf = is_k ? kbuf : vbuf;
        const uint16_t *const cache = is_k ? a.k_cache : a.v_cache;
        const int64_t stride = is_k ? a.k_block_stride : a.v_block_stride;
        const uint32_t nb = a.num_blocks > 0x7fffffff ? 0x7fffffffu : (uint32_t)a.num_blocks;
        static_assert(CPW % 4 == 0 && CPP % 4 == 0, "runs of four chunks");
#pragma unroll
        for (int i = 0; i < CPW; i += 4) {
            const int ch = wave * CPW + i;
            const int page = ch / CPP, part = ch % CPP;
            int id = __builtin_amdgcn_readfirstlane(ids[(tile & 1) * G::NKB + page]);
            id = (uint32_t)id < nb ? id : 0;                  // ids outside the pool read block 0
            const char *src = reinterpret_cast<const char *>(cache + (int64_t)id * stride + (int64_t)kvh * BS * D);
            const DbOffsets o = db_offsets(page);
            db_chunks4(src + part * 1024, is_k ? o.k : o.v, lds_addr(buf + page * G::PAGE + part * 1024));
        }
    };
    // This wave's chunks of a K (or V) tile in runs of four (one source base
    // and one M0 value per run), issued one chunk at a time from the hooks of
    // the MFMA loops.
    constexpr int NR = CPW / 4;
    static_assert(CPW <= CPP && CPP % CPW == 0, "a wave's chunks lie in one page");
    struct Runs {
        const char *base[NR];
        uint32_t m0[NR], off;
    };
    auto runs = [&](bool is_k, int tile) {
        Runs r;
        char *const buf = is_k ? kbuf : vbuf;
        const uint16_t *const cache = is_k ? a.k_cache : a.v_cache;
        const int64_t stride = is_k ? a.k_block_stride : a.v_block_stride;
        const uint32_t nb = a.num_blocks > 0x7fffffff ? 0x7fffffffu : (uint32_t)a.num_blocks;
#pragma unroll
        for (int q = 0; q < NR; ++q) {
            const int ch = wave * CPW + 4 * q;
            const int page = ch / CPP, part = ch % CPP;
            int id = __builtin_amdgcn_readfirstlane(ids[(tile & 1) * G::NKB + page]);
            id = (uint32_t)id < nb ? id : 0;
            r.base[q] = reinterpret_cast<const char *>(cache + (int64_t)id * stride + (int64_t)kvh * BS * D) + part * 1024;
            r.m0[q] = lds_addr(buf + page * G::PAGE + part * 1024);
        }
        const DbOffsets o = db_offsets(wave * CPW / CPP);
        r.off = is_k ? o.k : o.v;
        return r;
    };
    auto chunk = [&](const Runs &r, int c) {
        const int q = c / 4, i = c % 4;
        asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:%2"
                     :
                     : "v"(r.off), "s"(r.base[q]), "i"(i * 1024), "{m0}"(r.m0[q]));
    };
    auto fetch_ids = [&](int tile) {
        if (wave == 0)
            id_dma(bt_row + tile * G::NKB, G::NKB, lds_addr(ids + (tile & 1) * G::NKB));
    };

    // ---- prologue: ids of tile 0, then K(0) and the ids of tile 1
    fetch_ids(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    issue(true, 0);
    if (last >= 1)
        fetch_ids(1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // Per tile: V(t) is copied during QK(t) (one chunk per NQ MFMAs) and
    // K(t+1) during the first half of P.V(t), so the copies land during the
    // softmax (resp. the rest of P.V) and no wave waits on the memory
    // pipeline between the phases.
    constexpr int NQ = G::NDS * G::NKB / CPW;                 // QK MFMAs per chunk
    static_assert(CB == 1, "one column block per wave (P.V through a fragment ring)");
    static_assert(NQ >= 1 && G::NDB * G::NKS >= 4 * CPW, "chunks fit the loops");
    // Two barriers per tile: after the softmax (every wave's V(t) chunks
    // have landed and every wave has read K(t)) and at the end (every wave
    // has read V(t); K(t+1) and the ids of tile t+2 have landed).
    for (int t = 0; t <= last; ++t) {
        f32x4 sc[CB][G::NKB];
        bf16x8 pf[CB][G::NKS];
        FoldF f[CB];
        {
            const Runs rv = runs(false, t);
            if (active) {
                prefill_qk_wide<D, CB, 4>(kbuf, cols, sc, [&](int j) {
                    if (j % NQ == NQ - 1)
                        chunk(rv, j / NQ);
                });
            } else {
#pragma unroll
                for (int c = 0; c < CPW; ++c)
                    chunk(rv, c);
            }
        }
        if (active) {
            if ((t + 1) * G::T > min_lim)
                prefill_softmax<D, CB, true>(sc, cols, t, a.scale_log2, st, pf, f);
            else
                prefill_softmax<D, CB, false>(sc, cols, t, a.scale_log2, st, pf, f);
        }
        __builtin_amdgcn_s_waitcnt(0);                     // this wave's V(t) chunks landed
        __syncthreads();                                   // V(t) whole; K(t) read by every wave
        if ((t + 1) * G::T > seq_len) {
            db_mask_tail<D, NWV>(vbuf, seq_len, t);
            __syncthreads();
        }
        if (t + 2 <= last)
            fetch_ids(t + 2);                              // its slot held the ids of tile t
        {
            // K(t+1); past the last tile a spare copy (the slot's ids are
            // stale but sanitised) into kbuf, which no wave reads after QK(t)
            const Runs rk = runs(true, t + 1);
            if (active) {
                prefill_pv_ring<D, 3>(vbuf, pf[0], f[0], st[0], [&](int j) {
                    if (j % 4 == 0 && j / 4 < CPW)
                        chunk(rk, j / 4);
                });
            } else {
#pragma unroll
                for (int c = 0; c < CPW; ++c)
                    chunk(rk, c);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);                     // K(t+1) and the ids of t+2 landed
        __syncthreads();                                   // and V(t) read by every wave
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const ColInfo cj = col_info(a, cg * NCOL + (wave * CB + cb) * 16 + c, kvh, q0, q_len, seq_len);
        if (cj.lim > 0)
            store_out<D>(a, cj, st[cb]);
    }
}

// Double-buffered variant for workgroups that own a CU: two K+V tile
// buffers; tile t+1 (and the block ids of t+2) are fetched while tile t is
// computed, one barrier per tile.  Same chunk split and per-column arithmetic
// as prefill_sb_kernel.
template <int D, int CB, int NWV, int WPE>
__global__ __launch_bounds__(NWV * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void prefill_db_kernel(AttnArgs a)
{
    using G = Geo<D>;
    constexpr int NCOL = NWV * CB * 16;
    constexpr int HALF = G::NKB * G::PAGE;        // K (or V) part of one tile
    constexpr int CPP = G::PAGE / 1024;           // 1 KB chunks per page
    constexpr int CPW = G::NKB * CPP / NWV;       // K (or V) chunks per wave per tile
    static_assert(CPW >= 1 && (G::NKB * CPP) % NWV == 0, "whole chunks per wave");
    extern __shared__ __attribute__((aligned(16))) char lds[];
    int32_t *const ids = reinterpret_cast<int32_t *>(lds + 4 * HALF);     // [2][NKB]

    int b, kvh, cgi;
    if (!wg_slot(a, b, kvh, cgi))
        return;
    const int cg = a.col_groups - 1 - cgi;           // heaviest (latest) columns first

    int q0, q_len, seq_len;
    if (!row_ok(a, b, q0, q_len, seq_len))
        return;
    const int ncols = q_len * a.group;
    if (cg * NCOL >= ncols || ncols <= a.split_cols)
        return;
    const int col_last = min((cg + 1) * NCOL, ncols) - 1;
    const int pos_last = seq_len - q_len + col_last / a.group;
    const int last = (a.causal ? pos_last : seq_len - 1) / G::T;
    const int32_t *bt_row = a.block_tables + (int64_t)b * a.bt_stride;

    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int c = threadIdx.x & 15;
    Cols<D> cols[CB];
    State<D> st[CB];
    bool active = false;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const int col = cg * NCOL + (wave * CB + cb) * 16 + c;
        const ColInfo ci = col_info(a, col, kvh, q0, q_len, seq_len);
        load_q<D>(cols[cb], a, ci);
        state_init<D>(st[cb]);
        active |= (cg * NCOL + (wave * CB + cb) * 16) < ncols;
    }
    int min_lim = 0x7fffffff;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
        min_lim = min(min_lim, cols[cb].lim);
#pragma unroll
    for (int off = 1; off < 64; off *= 2)
        min_lim = min(min_lim, __shfl_xor(min_lim, off, 64));

    auto lds_addr = [](const void *p) { return (uint32_t)(size_t)(const __attribute__((address_space(3))) char *)p; };
    auto kbuf = [&](int tile) { return lds + (tile & 1) * 2 * HALF; };
    // this wave's chunks of `tile` (K and V): block ids (from LDS) -> chunks
    auto issue = [&](int tile) {
        char *const buf = kbuf(tile);
        const uint32_t nb = a.num_blocks > 0x7fffffff ? 0x7fffffffu : (uint32_t)a.num_blocks;
        static_assert(CPW % 4 == 0 && CPP % 4 == 0, "runs of four chunks");
#pragma unroll
        for (int i = 0; i < CPW; i += 4) {
            const int ch = wave * CPW + i;
            const int page = ch / CPP, part = ch % CPP;
            int id = __builtin_amdgcn_readfirstlane(ids[(tile & 1) * G::NKB + page]);
            id = (uint32_t)id < nb ? id : 0;                  // ids outside the pool read block 0
            const int64_t hoff = (int64_t)kvh * BS * D;
            const char *ks = reinterpret_cast<const char *>(a.k_cache + (int64_t)id * a.k_block_stride + hoff);
            const char *vs = reinterpret_cast<const char *>(a.v_cache + (int64_t)id * a.v_block_stride + hoff);
            const DbOffsets o = db_offsets(page);
            db_chunks4(ks + part * 1024, o.k, lds_addr(buf + page * G::PAGE + part * 1024));
            db_chunks4(vs + part * 1024, o.v, lds_addr(buf + HALF + page * G::PAGE + part * 1024));
        }
    };
    auto fetch_ids = [&](int tile) {
        if (wave == 0)
            id_dma(bt_row + tile * G::NKB, G::NKB, lds_addr(ids + (tile & 1) * G::NKB));
    };

    // ---- prologue: ids of tile 0, tile 0, ids of tile 1
    fetch_ids(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    issue(0);
    if (last >= 1)
        fetch_ids(1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int t = 0; t <= last; ++t) {
        // tile t+1 and the ids of t+2 go out while tile t is computed; the
        // buffers they fill were last read in iteration t-1
        if (t < last) {
            issue(t + 1);
            if (t + 2 <= last)
                fetch_ids(t + 2);
        }
        char *const cur = kbuf(t);
        if ((t + 1) * G::T > seq_len) {
            db_mask_tail<D, NWV>(cur + HALF, seq_len, t);
            __syncthreads();
        }
        if (active) {
            f32x4 sc[CB][G::NKB];
            bf16x8 pf[CB][G::NKS];
            FoldF f[CB];
            tile_qk<D, CB>(cur, cols, sc);
            if ((t + 1) * G::T > min_lim)
                prefill_softmax<D, CB, true>(sc, cols, t, a.scale_log2, st, pf, f);
            else
                prefill_softmax<D, CB, false>(sc, cols, t, a.scale_log2, st, pf, f);
            tile_pv<D, CB>(cur + HALF, pf, f, st);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const ColInfo cj = col_info(a, cg * NCOL + (wave * CB + cb) * 16 + c, kvh, q0, q_len, seq_len);
        if (cj.lim > 0)
            store_out<D>(a, cj, st[cb]);
    }
}

// ---------------------------------------------------------------- wave-pair prefill

// Two waves share CB 16-column blocks: wave half h of the pair computes S
// for key blocks [h NKB/2, (h+1) NKB/2) of the tile and P.V for dim blocks
// [h NDB/2, (h+1) NDB/2) of the output; the tile max, the per-lane partial
// sums and P^T go through LDS.  Per column the arithmetic is the tile step of
// the other kernels: the max is exact in any order; the partial sums are the
// two halves of the same fixed tree (blocks of half 0, then of half 1, then
// lanes xor 16 and xor 32); P^T and the fold are unchanged.  Used for
// head_dim 512 grids too small for two 128-column workgroups per CU: half of
// ACC per wave holds the state in registers without spills, and with CB = 2
// every K and V fragment read from LDS feeds two MFMAs.

template <int D>
struct HalfState {
    float R, L;
    f32x4 acc[Geo<D>::NDB / 2];
};

// Exchange area of one pair.
template <int D, int CB>
struct PairX {
    float mx[2][CB][16];
    float sum[2][CB][64];
    bf16x8 p[CB][Geo<D>::NKS][64];
};

template <int D, int CB, int RD = 6>
__device__ __forceinline__ void ws_qk(const char *kl, const Cols<D> (&cols)[CB], f32x4 (&s)[CB][Geo<D>::NKB / 2],
                                      int h)
{
    using G = Geo<D>;
    constexpr int HK = G::NKB / 2;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, c = lane & 15;
    const char *base[HK];
#pragma unroll
    for (int k = 0; k < HK; ++k) {
        const int kb = h * HK + k;
        const int stp = kb >> 1, e = kb & 1;
        const int page = 2 * stp + (c >> 3);
        const int tok = ((c >> 2) & 1) * 8 + e * 4 + (c & 3);
        base[k] = kl + page * G::PAGE + ksw(tok, page) * 16 + g * 256;
    }
#pragma unroll
    for (int k = 0; k < HK; ++k)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
            s[cb][k] = f32x4{0.f, 0.f, 0.f, 0.f};
    // fragment j = (dim step j / HK, key block j % HK), RD of them in flight
    constexpr int N = G::NDS * HK;
    auto frag = [&](int j) { return *reinterpret_cast<const bf16x8 *>(base[j % HK] + (j / HK) * 1024); };
    bf16x8 ring[RD];
#pragma unroll
    for (int j = 0; j < RD; ++j)
        ring[j] = frag(j);
#pragma unroll
    for (int j = 0; j < N; ++j) {
        const int ds = j / HK, k = j % HK;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
            s[cb][k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ring[j % RD], cols[cb].qf[ds], s[cb][k], 0, 0, 0);
        if (j + RD < N)
            ring[j % RD] = frag(j + RD);
        __builtin_amdgcn_sched_group_barrier(0x008, CB, 0);
        if (j + RD < N)
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Stage 1: mask, this half's max of raw scores (exact), to the pair's area.
template <int D, int CB, bool MASK>
__device__ __forceinline__ void ws_max(f32x4 (&s)[CB][Geo<D>::NKB / 2], const Cols<D> (&cols)[CB], int tile, int h,
                                       PairX<D, CB> &x)
{
    using G = Geo<D>;
    constexpr int HK = G::NKB / 2;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, c = lane & 15;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        float vals[4 * HK];
#pragma unroll
        for (int k = 0; k < HK; ++k) {
            if (MASK) {
                const int kb = h * HK + k;
                const int stp = kb >> 1, e = kb & 1;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = tile * G::T + 32 * stp + 8 * g + 4 * e + i;
                    s[cb][k][i] = key < cols[cb].lim ? s[cb][k][i] : -INFINITY;
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                vals[4 * k + i] = s[cb][k][i];
        }
        const float m = max_xor32(max_xor16(max_reduce<4 * HK>(vals)));
        if (g == 0)
            x.mx[h][cb][c] = m;
    }
}

// Stage 2: the tile max, p, this half's level of the sum tree and its P^T
// steps to the pair's area; m[cb] gets the scaled tile max.
template <int D, int CB>
__device__ __forceinline__ void ws_exp(f32x4 (&s)[CB][Geo<D>::NKB / 2], float scale_log2, int h, PairX<D, CB> &x,
                                       float (&m)[CB])
{
    using G = Geo<D>;
    constexpr int HK = G::NKB / 2;
    const int lane = threadIdx.x & 63;
    const int c = lane & 15;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        m[cb] = __fmul_rn(fmax2(x.mx[0][cb][c], x.mx[1][cb][c]), scale_log2);
        const float nmu = m[cb] == -INFINITY ? 0.f : -m[cb];
        float part[HK];
#pragma unroll
        for (int k = 0; k < HK; ++k) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                s[cb][k][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[cb][k][i], scale_log2, nmu));
            part[k] = __fadd_rn(__fadd_rn(s[cb][k][0], s[cb][k][1]), __fadd_rn(s[cb][k][2], s[cb][k][3]));
        }
#pragma unroll
        for (int w = 1; w < HK; w *= 2)
#pragma unroll
            for (int k = 0; k < HK; k += 2 * w)
                part[k] = __fadd_rn(part[k], part[k + w]);
        x.sum[h][cb][lane] = part[0];
#pragma unroll
        for (int sl = 0; sl < HK / 2; ++sl) {
            bf16x8 pv;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pv[i] = (__bf16)s[cb][2 * sl][i];
                pv[4 + i] = (__bf16)s[cb][2 * sl + 1][i];
            }
            x.p[cb][h * (HK / 2) + sl][lane] = pv;
        }
    }
}

// Stage 3: l (the tree's last levels), the fold of (R, L), the rescale of
// this half's ACC if some reference moved, then P.V for this half's dims
// folded with fma(tile, h, ACC); each V fragment feeds all CB blocks.
template <int D, int CB, int DG>
__device__ __forceinline__ void ws_fold_pv(const char *vl, const float (&m)[CB], int h, const PairX<D, CB> &x,
                                           HalfState<D> (&st)[CB])
{
    using G = Geo<D>;
    constexpr int HD = G::NDB / 2;
    static_assert(HD % DG == 0, "whole groups");
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, c = lane & 15;
    bf16x8 pf[CB][G::NKS];
    FoldF f[CB];
    bool any_up = false;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        float l = __fadd_rn(x.sum[0][cb][lane], x.sum[1][cb][lane]);
        l = sum_xor32(sum_xor16(l));
#pragma unroll
        for (int stp = 0; stp < G::NKS; ++stp)
            pf[cb][stp] = x.p[cb][stp][lane];
        f[cb] = fold_factors(st[cb].R, m[cb]);
        any_up |= __ballot(f[cb].up) != 0;
        st[cb].L = fold1v(st[cb].L, l, f[cb].gs, f[cb].h);
        st[cb].R = f[cb].Rn;
    }
    if (any_up) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int db = 0; db < HD; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    st[cb].acc[db][i] = __fmul_rn(st[cb].acc[db][i], f[cb].gs);
    }
    auto vaddr = [&](int db, int stp) -> const char * {
        const int d = 16 * db + c;
        return vl + (g >> 1) * G::PAGE + vslot(d, g & 1) * 16 + 2 * stp * G::PAGE;
    };
#pragma unroll
    for (int d0 = 0; d0 < HD; d0 += DG) {
        f32x4 o[CB][DG];
        bf16x8 vf[DG], vn[DG];
#pragma unroll
        for (int d = 0; d < DG; ++d) {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
                o[cb][d] = f32x4{0.f, 0.f, 0.f, 0.f};
            vf[d] = *reinterpret_cast<const bf16x8 *>(vaddr(h * HD + d0 + d, 0));
        }
#pragma unroll
        for (int stp = 0; stp < G::NKS; ++stp) {
            if (stp + 1 < G::NKS) {
#pragma unroll
                for (int d = 0; d < DG; ++d)
                    vn[d] = *reinterpret_cast<const bf16x8 *>(vaddr(h * HD + d0 + d, stp + 1));
            }
#pragma unroll
            for (int d = 0; d < DG; ++d)
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
                    o[cb][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[d], pf[cb][stp], o[cb][d], 0, 0, 0);
#pragma unroll
            for (int d = 0; d < DG; ++d)
                vf[d] = vn[d];
            if (stp + 1 < G::NKS)
                __builtin_amdgcn_sched_group_barrier(0x100, DG, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, DG * CB, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int d = 0; d < DG; ++d)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    st[cb].acc[d0 + d][i] = __builtin_fmaf(o[cb][d][i], f[cb].h, st[cb].acc[d0 + d][i]);
    }
}

// This half's dims of the column's output (and its lse from half 0).
template <int D>
__device__ __forceinline__ void ws_store(const AttnArgs &a, const ColInfo &ci, const HalfState<D> &st, int h)
{
    constexpr int HD = Geo<D>::NDB / 2;
    const int g = (threadIdx.x & 63) >> 4;
    if (a.lse && h == 0 && g == 0)
        a.lse[ci.row * a.lse_token_stride + ci.head] = lse_of(st.R, st.L);
    const float inv = 1.0f / st.L;
    uint16_t *dst = a.out + ci.row * a.out_token_stride + (int64_t)ci.head * D + 4 * g + 16 * h * HD;
#pragma unroll
    for (int db = 0; db < HD; ++db)
        *reinterpret_cast<u32x2 *>(dst + 16 * db) = finish4(st.acc[db], inv);
}

// Shared set-up of the wave-pair kernels: workgroup -> (column group, kv
// head, sequence) as in the other prefill kernels; wave w -> pair w / 2,
// half w % 2.
struct WsSetup {
    int b, kvh, cg, q0, q_len, seq_len, ncols, last, wave, pair, half;
    bool run;
};

template <int D, int NCOL>
__device__ __forceinline__ WsSetup ws_setup(const AttnArgs &a)
{
    WsSetup w{};
    w.run = false;
    int cgi;
    if (!wg_slot(a, w.b, w.kvh, cgi))
        return w;
    w.cg = a.col_groups - 1 - cgi;                  // heaviest (latest) columns first
    if (!row_ok(a, w.b, w.q0, w.q_len, w.seq_len))
        return w;
    w.ncols = w.q_len * a.group;
    if (w.cg * NCOL >= w.ncols || w.ncols <= a.split_cols)
        return w;
    const int col_last = min((w.cg + 1) * NCOL, w.ncols) - 1;
    const int pos_last = w.seq_len - w.q_len + col_last / a.group;
    w.last = (a.causal ? pos_last : w.seq_len - 1) / Geo<D>::T;
    w.wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    w.pair = w.wave >> 1;
    w.half = w.wave & 1;
    w.run = true;
    return w;
}

// Single-buffered wave-pair kernel (head_dim 512, whose K+V tile takes 128
// KB of LDS): the staging order of prefill_sb_kernel; the pair exchanges
// share its barriers (the maxima with "K(t) read", P^T and the sums with
// "V(t) landed").  NWV / 2 pairs of CB column blocks each.
template <int D, int NWV, int WPE, int CB>
__global__ __launch_bounds__(NWV * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void prefill_ws_sb_kernel(AttnArgs a)
{
    using G = Geo<D>;
    constexpr int NCOL = NWV / 2 * CB * 16;
    constexpr int HALF = G::NKB * G::PAGE;
    constexpr int CPP = G::PAGE / 1024;
    constexpr int CPW = G::NKB * CPP / NWV;
    static_assert(CPW >= 1 && (G::NKB * CPP) % NWV == 0, "whole chunks per wave");
    static_assert(CPW + 1 < 64, "vmcnt range");
    extern __shared__ __attribute__((aligned(16))) char lds[];
    char *const kbuf = lds;
    char *const vbuf = lds + HALF;
    int32_t *const ids = reinterpret_cast<int32_t *>(lds + 2 * HALF);                     // [2][NKB]
    PairX<D, CB> *const xs = reinterpret_cast<PairX<D, CB> *>(lds + 2 * HALF + 2 * G::NKB * 4);   // [NWV / 2]

    const WsSetup w = ws_setup<D, NCOL>(a);
    if (!w.run)
        return;
    const int c = threadIdx.x & 15;
    const int32_t *bt_row = a.block_tables + (int64_t)w.b * a.bt_stride;
    Cols<D> cols[CB];
    HalfState<D> st[CB];
    ColInfo ci[CB];
    bool active = false;
    int min_lim = 0x7fffffff;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const int col = w.cg * NCOL + (w.pair * CB + cb) * 16 + c;
        ci[cb] = col_info(a, col, w.kvh, w.q0, w.q_len, w.seq_len);
        load_q<D>(cols[cb], a, ci[cb]);
        st[cb].R = -INFINITY;
        st[cb].L = 0.f;
#pragma unroll
        for (int db = 0; db < G::NDB / 2; ++db)
            st[cb].acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
        active |= w.cg * NCOL + (w.pair * CB + cb) * 16 < w.ncols;
        min_lim = min(min_lim, cols[cb].lim);
    }
#pragma unroll
    for (int off = 1; off < 64; off *= 2)
        min_lim = min(min_lim, __shfl_xor(min_lim, off, 64));
    PairX<D, CB> &x = xs[w.pair];

    auto lds_addr = [](const void *p) { return (uint32_t)(size_t)(const __attribute__((address_space(3))) char *)p; };
    auto issue = [&](bool is_k, int tile) {
        char *const buf = is_k ? kbuf : vbuf;
        const uint16_t *const cache = is_k ? a.k_cache : a.v_cache;
        const int64_t stride = is_k ? a.k_block_stride : a.v_block_stride;
        const uint32_t nb = a.num_blocks > 0x7fffffff ? 0x7fffffffu : (uint32_t)a.num_blocks;
        static_assert(CPW % 4 == 0 && CPP % 4 == 0, "runs of four chunks");
#pragma unroll
        for (int i = 0; i < CPW; i += 4) {
            const int ch = w.wave * CPW + i;
            const int page = ch / CPP, part = ch % CPP;
            int id = __builtin_amdgcn_readfirstlane(ids[(tile & 1) * G::NKB + page]);
            id = (uint32_t)id < nb ? id : 0;                  // ids outside the pool read block 0
            const char *src = reinterpret_cast<const char *>(cache + (int64_t)id * stride + (int64_t)w.kvh * BS * D);
            const DbOffsets o = db_offsets(page);
            db_chunks4(src + part * 1024, is_k ? o.k : o.v, lds_addr(buf + page * G::PAGE + part * 1024));
        }
    };
    auto fetch_ids = [&](int tile) {
        if (w.wave == 0)
            id_dma(bt_row + tile * G::NKB, G::NKB, lds_addr(ids + (tile & 1) * G::NKB));
    };

    fetch_ids(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    issue(true, 0);
    issue(false, 0);
    if (w.last >= 1)
        fetch_ids(1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int t = 0; t <= w.last; ++t) {
        f32x4 s[CB][G::NKB / 2];
        float m[CB];
        if (active) {
            ws_qk<D, CB>(kbuf, cols, s, w.half);
            if ((t + 1) * G::T > min_lim)
                ws_max<D, CB, true>(s, cols, t, w.half, x);
            else
                ws_max<D, CB, false>(s, cols, t, w.half, x);
        }
        __syncthreads();                                   // K(t) read by every wave; maxima visible
        if (t < w.last)
            issue(true, t + 1);
        if (active)
            ws_exp<D, CB>(s, a.scale_log2, w.half, x, m);
        // V(t) (issued before K(t+1)) has landed
        if (t < w.last)
            wait_vm<CPW>();
        else
            wait_vm<0>();
        __syncthreads();                                   // sums and P^T visible
        if ((t + 1) * G::T > w.seq_len) {
            db_mask_tail<D, NWV>(vbuf, w.seq_len, t);
            __syncthreads();
        }
        if (active)
            ws_fold_pv<D, CB, 4>(vbuf, m, w.half, x, st);
        __syncthreads();                                   // V(t) read by every wave
        if (t < w.last) {
            if (t + 2 <= w.last)
                fetch_ids(t + 2);
            issue(false, t + 1);
            // K(t+1) and the ids of t+2 (issued before V(t+1)) have landed
            wait_vm<CPW>();
            __syncthreads();
        }
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
        if (ci[cb].lim > 0)
            ws_store<D>(a, ci[cb], st[cb], w.half);
}

// ---------------------------------------------------------------- producer / consumer prefill

// Two waves per 16-column block split the tile step by stage instead of by
// keys: the producer (waves 0-3) runs QK and the softmax statistics of tile
// t, folds (R, L) and hands the fold factors and P^T to its consumer (waves
// 4-7) through LDS; the consumer runs P.V of tile t-1 and folds it into ACC
// at the same time.  Both roles use the tile-step functions of the other
// kernels, so the bits are the same (the consumer takes ACC * gs inside its
// fold on every tile: gs is 1 unless the reference moved, and ACC * 1 is
// exact); the two waves of a SIMD are a stage apart, so one's MFMAs fill the
// other's softmax.  K and V tiles have two LDS buffers each (K(t+1) and V(t)
// load while K(t) and V(t-1) are read; the consumers copy V(t), the
// producers K(t+1)), two barriers per tile.  64 columns
// per workgroup, for grids that leave CUs idle with more columns per
// workgroup.
template <int D>
struct StageX {
    bf16x8 p[Geo<D>::NKS][64];
    float gs[64], h[64], R[64], L[64];
};

template <int D, int WPE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void prefill_ss_kernel(AttnArgs a)
{
    using G = Geo<D>;
    constexpr int NWV = 8;
    constexpr int NCOL = 64;
    constexpr int HALF = G::NKB * G::PAGE;
    constexpr int CPP = G::PAGE / 1024;
    constexpr int CPW = G::NKB * CPP / NWV;          // K (or V) chunks per wave per tile
    static_assert(CPW >= 1 && (G::NKB * CPP) % NWV == 0, "whole chunks per wave");
    extern __shared__ __attribute__((aligned(16))) char lds[];
    int32_t *const ids = reinterpret_cast<int32_t *>(lds + 4 * HALF);                   // [2][NKB]
    StageX<D> *const xs = reinterpret_cast<StageX<D> *>(lds + 4 * HALF + 2 * G::NKB * 4);   // [4]

    int b, kvh, cgi;
    if (!wg_slot(a, b, kvh, cgi))
        return;
    const int cg = a.col_groups - 1 - cgi;           // heaviest (latest) columns first
    int q0, q_len, seq_len;
    if (!row_ok(a, b, q0, q_len, seq_len))
        return;
    const int ncols = q_len * a.group;
    if (cg * NCOL >= ncols || ncols <= a.split_cols)
        return;
    const int col_last = min((cg + 1) * NCOL, ncols) - 1;
    const int pos_last = seq_len - q_len + col_last / a.group;
    const int last = (a.causal ? pos_last : seq_len - 1) / G::T;
    const int32_t *bt_row = a.block_tables + (int64_t)b * a.bt_stride;

    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int blk = wave & 3;                  // column block
    const bool producer = wave < 4;
    const int lane = threadIdx.x & 63;
    const int c = lane & 15;
    StageX<D> &x = xs[blk];
    const int col = cg * NCOL + blk * 16 + c;
    const ColInfo ci = col_info(a, col, kvh, q0, q_len, seq_len);
    const bool active = cg * NCOL + blk * 16 < ncols;
    Cols<D> cols[1];
    State<D> st[1];
    int min_lim = 0;
    if (producer) {
        load_q<D>(cols[0], a, ci);
        min_lim = cols[0].lim;
#pragma unroll
        for (int off = 1; off < 64; off *= 2)
            min_lim = min(min_lim, __shfl_xor(min_lim, off, 64));
    }
    state_init<D>(st[0]);

    auto lds_addr = [](const void *p) { return (uint32_t)(size_t)(const __attribute__((address_space(3))) char *)p; };
    auto stage = [&](int tile) { return lds + (tile & 1) * 2 * HALF; };
    // Chunks of the K (or V) part of `tile` copied by issuing wave iw of NI
    // (all eight waves for the first K tile, one role's four waves later).
    auto issue = [&](bool is_k, int tile, int iw, auto ni) {
        constexpr int NI = decltype(ni)::value;
        constexpr int CPI = G::NKB * CPP / NI;       // chunks per issuing wave
        char *const buf = stage(tile) + (is_k ? 0 : HALF);
        const uint16_t *const cache = is_k ? a.k_cache : a.v_cache;
        const int64_t stride = is_k ? a.k_block_stride : a.v_block_stride;
        const uint32_t nb = a.num_blocks > 0x7fffffff ? 0x7fffffffu : (uint32_t)a.num_blocks;
        static_assert(CPI % 4 == 0 && CPP % 4 == 0 && CPI * NI == G::NKB * CPP, "runs of four chunks");
#pragma unroll
        for (int i = 0; i < CPI; i += 4) {
            const int ch = iw * CPI + i;
            const int page = ch / CPP, part = ch % CPP;
            int id = __builtin_amdgcn_readfirstlane(ids[(tile & 1) * G::NKB + page]);
            id = (uint32_t)id < nb ? id : 0;                  // ids outside the pool read block 0
            const char *src = reinterpret_cast<const char *>(cache + (int64_t)id * stride + (int64_t)kvh * BS * D);
            const DbOffsets o = db_offsets(page);
            db_chunks4(src + part * 1024, is_k ? o.k : o.v, lds_addr(buf + page * G::PAGE + part * 1024));
        }
    };
    auto fetch_ids = [&](int tile) {
        if (wave == 0)
            id_dma(bt_row + tile * G::NKB, G::NKB, lds_addr(ids + (tile & 1) * G::NKB));
    };

    // ---- prologue: ids of tiles 0 and 1, then K(0)
    fetch_ids(0);
    if (last >= 1)
        fetch_ids(1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    issue(true, 0, wave, std::integral_constant<int, NWV>{});
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // step t: the producer computes tile t, the consumer tile t - 1.  Each
    // role runs its own copy of the step loop, with the same barriers in the
    // same order, so the two roles' values never meet at a join.
    // K(t+1) and V(t) go into buffers last read in step t - 1.  A wave
    // waits while the CU's memory pipeline takes its transfer instructions
    // (about 16 cycles per 1 KB chunk for the whole CU), so the consumers copy
    // V(t) at the start of the step and the producers copy K(t+1) after their
    // QK, rather than all eight waves copying both at the start.
    auto step_head = [&](int t) {
        if (!producer && t <= last)
            issue(false, t, wave - 4, std::integral_constant<int, 4>{});
        // V(t-1) of a tile that reaches seq_len: zero its keys >= seq_len
        if (t >= 1 && t * G::T > seq_len) {
            db_mask_tail<D, NWV>(stage(t - 1) + HALF, seq_len, t - 1);
            __syncthreads();
        }
    };
    if (producer) {
        for (int t = 0; t <= last + 1; ++t) {
            step_head(t);
            const bool work = active && t <= last;
            bf16x8 pf[1][G::NKS];
            FoldF f[1];
            f32x4 sc[1][G::NKB];
            if (work)
                tile_qk<D, 1>(stage(t), cols, sc);
            if (t + 1 <= last)
                issue(true, t + 1, wave, std::integral_constant<int, 4>{});
            if (work) {
                if ((t + 1) * G::T > min_lim)
                    prefill_softmax_stats<D, 1, true>(sc, cols, t, a.scale_log2, st, pf, f);
                else
                    prefill_softmax_stats<D, 1, false>(sc, cols, t, a.scale_log2, st, pf, f);
            }
            __syncthreads();                               // the consumer is done with the hand-off of t - 1
            if (t + 2 <= last)
                fetch_ids(t + 2);                          // its slot held the ids of V(t), issued above
            if (work) {
#pragma unroll
                for (int stp = 0; stp < G::NKS; ++stp)
                    x.p[stp][lane] = pf[0][stp];
                x.gs[lane] = f[0].gs;
                x.h[lane] = f[0].h;
                if (t == last) {
                    x.R[lane] = st[0].R;
                    x.L[lane] = st[0].L;
                }
            }
            if (t <= last) {
                __builtin_amdgcn_s_waitcnt(0);             // K(t+1), V(t), ids(t+2) landed
                __syncthreads();                           // and the hand-off of t is visible
            }
        }
    } else {
        for (int t = 0; t <= last + 1; ++t) {
            step_head(t);
            if (active && t >= 1) {
                bf16x8 pf[1][G::NKS];
                FoldF f[1];
#pragma unroll
                for (int stp = 0; stp < G::NKS; ++stp)
                    pf[0][stp] = x.p[stp][lane];
                f[0].gs = x.gs[lane];
                f[0].h = x.h[lane];
                // ACC * gs inside the fold, for every tile (ACC * 1 is exact)
                prefill_pv_grp<D, 1, (D == 128 ? 8 : 4), true>(stage(t - 1) + HALF, pf, f, st);
            }
            __syncthreads();                               // done with the hand-off of t - 1
            if (t <= last) {
                __builtin_amdgcn_s_waitcnt(0);             // K(t+1), V(t) landed
                __syncthreads();                           // and the hand-off of t is visible
            }
        }
        if (ci.lim > 0) {
            st[0].R = x.R[lane];
            st[0].L = x.L[lane];
            store_out<D>(a, ci, st[0]);
        }
    }
}

// ---------------------------------------------------------------- ping-pong prefill

// Same column/tile work and per-column arithmetic as prefill_db_kernel, for
// large grids (one workgroup of 8 waves and 256 columns per CU), with
// the two waves of each SIMD (waves w and w+4) kept half a tile apart:
// waves 0-3 (group A) run the softmax of tile t while waves 4-7 (group B)
// run the MFMAs of P.V(t-1) and QK(t), then the roles swap.  The wave in its
// MFMA half runs at raised issue priority.  Two barriers per tile separate
// the halves.
//   slot 1: A softmax(t)                 | B P.V(t-1), QK(t)
//   slot 2: A P.V(t), QK(t+1)            | B softmax(t)
// K and V tiles have two LDS buffers each.  During slot 2 of iteration t the
// waves of group A copy K(t+2) and V(t+1) into the buffers that slot 1
// released (K(t), V(t-1)), one 1 KB chunk after every eight of their MFMAs:
// a wave waits while the CU's memory pipeline takes its transfer
// instructions (about 16 cycles per chunk for the whole CU), and spread over
// the slot no wave queues behind the others.  The copies are waited for
// before the barrier that ends slot 1 of iteration t+1, one slot before
// their first use.  P of a wave is
// kept in the register space of its scores (the two are never live together
// in one wave).
template <int D, int CB>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_pp_kernel(AttnArgs a)
{
    using G = Geo<D>;
    constexpr int NWV = 8;
    constexpr int NCOL = NWV * CB * 16;
    constexpr int HALF = G::NKB * G::PAGE;        // K (or V) part of one tile
    static_assert(G::NKB == NWV, "one page of each tile per wave");
    static_assert(G::NKS <= G::NKB, "P fits in the score registers");
    extern __shared__ __attribute__((aligned(16))) char lds[];
    char *const kbuf0 = lds, *const kbuf1 = lds + HALF;
    char *const vbuf0 = lds + 2 * HALF, *const vbuf1 = lds + 3 * HALF;

    int b, kvh, cgi;
    if (!wg_slot(a, b, kvh, cgi))
        return;
    const int cg = a.col_groups - 1 - cgi;

    int q0, q_len, seq_len;
    if (!row_ok(a, b, q0, q_len, seq_len))
        return;
    const int ncols = q_len * a.group;
    if (cg * NCOL >= ncols || ncols <= a.split_cols)
        return;
    const int col_last = min((cg + 1) * NCOL, ncols) - 1;
    const int pos_last = seq_len - q_len + col_last / a.group;
    const int last = (a.causal ? pos_last : seq_len - 1) / G::T;
    const int32_t *bt_row = a.block_tables + (int64_t)b * a.bt_stride;

    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const bool grp_b = wave >= 4;
    const int c = threadIdx.x & 15;
    Cols<D> cols[CB];
    State<D> st[CB];
    bool active = false;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const int col = cg * NCOL + (wave * CB + cb) * 16 + c;
        const ColInfo ci = col_info(a, col, kvh, q0, q_len, seq_len);
        load_q<D>(cols[cb], a, ci);
        state_init<D>(st[cb]);
        active |= (cg * NCOL + (wave * CB + cb) * 16) < ncols;
    }
    int min_lim = 0x7fffffff;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
        min_lim = min(min_lim, cols[cb].lim);
#pragma unroll
    for (int off = 1; off < 64; off *= 2)
        min_lim = min(min_lim, __shfl_xor(min_lim, off, 64));

    const DbOffsets offs = db_offsets(wave);
    auto issue_k = [&](char *dst, int id) { db_issue_half<D>(dst, a, a.k_cache, a.k_block_stride, id, kvh, wave, offs.k); };
    auto issue_v = [&](char *dst, int id) { db_issue_half<D>(dst, a, a.v_cache, a.v_block_stride, id, kvh, wave, offs.v); };
    auto kbuf = [&](int t) { return (t & 1) ? kbuf1 : kbuf0; };
    auto vbuf = [&](int t) { return (t & 1) ? vbuf1 : vbuf0; };
    auto softmax = [&](int tile, f32x4 (&sc)[CB][G::NKB], bf16x8 (&pf)[CB][G::NKS], FoldF (&f)[CB]) {
        if ((tile + 1) * G::T > min_lim)
            prefill_softmax<D, CB, true>(sc, cols, tile, a.scale_log2, st, pf, f);
        else
            prefill_softmax<D, CB, false>(sc, cols, tile, a.scale_log2, st, pf, f);
    };

    // ---- prologue: K(0), V(0), K(1) staged
    {
        const int id0 = __builtin_amdgcn_readfirstlane(db_load_id(bt_row, 0));
        issue_k(kbuf0, id0);
        issue_v(vbuf0, id0);
    }
    if (last >= 1)
        issue_k(kbuf1, __builtin_amdgcn_readfirstlane(db_load_id(bt_row, 1)));
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // Between the two slots of iteration t (every wave): the transfers of
    // slot 2 of t-1 have landed; the tail tile's V is masked.
    auto mid = [&](int t) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if ((t + 1) * G::T > seq_len) {
            db_mask_tail<D, NWV>(vbuf(t), seq_len, t);
            __syncthreads();
        }
    };
    // Group A wave wa copies pages 2 wa and 2 wa + 1 of K(t+2) and V(t+1)
    // during its MFMA slot of iteration t.  Their block ids are read at the
    // top of the iteration with scalar loads (the table is read through the
    // constant address space, so the compiler emits s_load and its wait).
    // K(t+2) is copied even past the last tile, from the last tile's pages
    // into kbuf(t), which no wave reads after that slot (no branch in the
    // MFMA loop).
    static_assert(G::NKB == 8 && G::PAGE == 4096, "two pages of four chunks per group-A wave");
    const int wa = wave & 3;
    struct CpIds {
        int k0, k1, v0, v1;
    };
    using cint = const __attribute__((address_space(4))) int32_t;
    auto cp_ids = [&](int t) {
        CpIds r;
        const int tk = min(t + 2, last), tv = min(t + 1, last);
        cint *const tb = (cint *)bt_row;
        r.k0 = tb[tk * 8 + 2 * wa];
        r.k1 = tb[tk * 8 + 2 * wa + 1];
        r.v0 = tb[tv * 8 + 2 * wa];
        r.v1 = tb[tv * 8 + 2 * wa + 1];
        return r;
    };
    const uint32_t nbk = a.num_blocks > 0x7fffffff ? 0x7fffffffu : (uint32_t)a.num_blocks;
    auto cp_chunk = [&](const CpIds &r, int t, bool is_k, int c) {   // c = 0..7: page 2 wa + c / 4, chunk c % 4
        const int p = 2 * wa + c / 4, i = c % 4;
        int id = is_k ? (c < 4 ? r.k0 : r.k1) : (c < 4 ? r.v0 : r.v1);
        id = (uint32_t)id < nbk ? id : 0;
        const uint16_t *const cache = is_k ? a.k_cache : a.v_cache;
        const int64_t stride = is_k ? a.k_block_stride : a.v_block_stride;
        const char *base = reinterpret_cast<const char *>(cache + (int64_t)id * stride + (int64_t)kvh * BS * D);
        const DbOffsets o = db_offsets(p);
        char *const dst = (is_k ? kbuf(t) : vbuf(t + 1)) + p * G::PAGE;
        const uint32_t m0 = (uint32_t)(size_t)(__attribute__((address_space(3))) char *)dst;
        asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:%2"
                     :
                     : "v"(is_k ? o.k : o.v), "s"(base), "i"(i * 1024), "{m0}"(m0));
    };

    // The two groups run separate loops with the same barrier sequence
    // (the branch is wave-uniform; s_barrier counts waves, not call sites).
    // The last iteration is peeled so that no score array is carried through
    // a path that skips its producer (it would stay live across P.V).
    if (!grp_b) {
        f32x4 sc[CB][G::NKB];
        if (active)
            prefill_qk<D, CB>(kbuf0, cols, sc);
        __syncthreads();
        for (int t = 0; t < last; ++t) {
            bf16x8 pf[CB][G::NKS];
            FoldF f[CB];
            const CpIds ci = cp_ids(t);
            if (active)
                softmax(t, sc, pf, f);                         // slot 1
            mid(t);
            __builtin_amdgcn_s_setprio(1);
            if (active) {                                      // slot 2
                prefill_pv<D, CB>(vbuf(t), pf, f, st, [&](int db) { cp_chunk(ci, t, false, db); });
                prefill_qk<D, CB>(kbuf(t + 1), cols, sc, [&](int kb) { cp_chunk(ci, t, true, kb); });
            } else {
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    cp_chunk(ci, t, false, c);
                    cp_chunk(ci, t, true, c);
                }
            }
            __builtin_amdgcn_s_setprio(0);
            __syncthreads();
        }
        bf16x8 pf[CB][G::NKS];
        FoldF f[CB];
        if (active)
            softmax(last, sc, pf, f);
        mid(last);
        if (active)
            prefill_pv<D, CB>(vbuf(last), pf, f, st);
        __syncthreads();
    } else {
        bf16x8 pf[CB][G::NKS];
        FoldF f[CB];
        __syncthreads();
        {
            f32x4 sc[CB][G::NKB];
            if (active)
                prefill_qk<D, CB>(kbuf0, cols, sc);            // slot 1
            mid(0);
            if (active)
                softmax(0, sc, pf, f);                         // slot 2
            __syncthreads();
        }
        for (int t = 1; t <= last; ++t) {
            f32x4 sc[CB][G::NKB];
            __builtin_amdgcn_s_setprio(1);
            if (active) {                                      // slot 1
                prefill_pv<D, CB>(vbuf(t - 1), pf, f, st);
                prefill_qk<D, CB>(kbuf(t), cols, sc);
            }
            __builtin_amdgcn_s_setprio(0);
            mid(t);
            if (active)
                softmax(t, sc, pf, f);                         // slot 2
            __syncthreads();
        }
        if (active)
            prefill_pv<D, CB>(vbuf(last), pf, f, st);
    }

#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const ColInfo cj = col_info(a, cg * NCOL + (wave * CB + cb) * 16 + c, kvh, q0, q_len, seq_len);
        if (cj.lim > 0)
            store_out<D>(a, cj, st[cb]);
    }
}

}  // namespace

template <int D, int CB, int NWV, int WPE>
static hipError_t prefill_sb_launch(AttnArgs a, hipStream_t s, uint64_t *blocks, int max_query_len)
{
    constexpr int NCOL = NWV * CB * 16;
    constexpr int LDS_BYTES = Geo<D>::LDS + 2 * Geo<D>::NKB * 4;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    a.col_groups = (max_query_len * a.group + NCOL - 1) / NCOL;
    const int64_t n = (int64_t)a.num_seqs * a.num_kv_heads * a.col_groups;
    const int64_t grid = (n + 7) / 8 * 8;
    if (grid <= 0)
        return hipSuccess;
    if (grid > 0x7fffffff)
        return hipErrorInvalidValue;
    static const hipError_t attr = hipFuncSetAttribute((const void *)prefill_sb_kernel<D, CB, NWV, WPE>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    (void)attr;
    hipLaunchKernelGGL((prefill_sb_kernel<D, CB, NWV, WPE>), dim3((unsigned)grid), dim3(NWV * 64), LDS_BYTES, s, a);
    *blocks = (uint64_t)grid;
    return hipGetLastError();
}

template <int D, int CB, int NWV, int WPE>
static hipError_t prefill_db_launch(AttnArgs a, hipStream_t s, uint64_t *blocks, int max_query_len)
{
    constexpr int NCOL = NWV * CB * 16;
    constexpr int LDS_BYTES = 2 * Geo<D>::LDS + 2 * Geo<D>::NKB * 4;
    a.col_groups = (max_query_len * a.group + NCOL - 1) / NCOL;
    const int64_t n = (int64_t)a.num_seqs * a.num_kv_heads * a.col_groups;
    const int64_t grid = (n + 7) / 8 * 8;
    if (grid <= 0)
        return hipSuccess;
    if (grid > 0x7fffffff)
        return hipErrorInvalidValue;
    static const hipError_t attr = hipFuncSetAttribute((const void *)prefill_db_kernel<D, CB, NWV, WPE>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    (void)attr;
    hipLaunchKernelGGL((prefill_db_kernel<D, CB, NWV, WPE>), dim3((unsigned)grid), dim3(NWV * 64), LDS_BYTES, s, a);
    *blocks = (uint64_t)grid;
    return hipGetLastError();
}

template <int D, int NWV, int WPE, int CB>
static hipError_t prefill_ws_launch(AttnArgs a, hipStream_t s, uint64_t *blocks, int max_query_len)
{
    constexpr int NCOL = NWV / 2 * CB * 16;
    constexpr int LDS_BYTES = Geo<D>::LDS + 2 * Geo<D>::NKB * 4 + NWV / 2 * (int)sizeof(PairX<D, CB>);
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    a.col_groups = (max_query_len * a.group + NCOL - 1) / NCOL;
    const int64_t n = (int64_t)a.num_seqs * a.num_kv_heads * a.col_groups;
    const int64_t grid = (n + 7) / 8 * 8;
    if (grid <= 0)
        return hipSuccess;
    if (grid > 0x7fffffff)
        return hipErrorInvalidValue;
    static const hipError_t attr = hipFuncSetAttribute((const void *)prefill_ws_sb_kernel<D, NWV, WPE, CB>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    (void)attr;
    hipLaunchKernelGGL((prefill_ws_sb_kernel<D, NWV, WPE, CB>), dim3((unsigned)grid), dim3(NWV * 64), LDS_BYTES, s, a);
    *blocks = (uint64_t)grid;
    return hipGetLastError();
}

template <int D, int WPE>
static hipError_t prefill_ss_launch(AttnArgs a, hipStream_t s, uint64_t *blocks, int max_query_len)
{
    constexpr int NCOL = 64;
    constexpr int LDS_BYTES = 2 * Geo<D>::LDS + 2 * Geo<D>::NKB * 4 + 4 * (int)sizeof(StageX<D>);
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    a.col_groups = (max_query_len * a.group + NCOL - 1) / NCOL;
    const int64_t n = (int64_t)a.num_seqs * a.num_kv_heads * a.col_groups;
    const int64_t grid = (n + 7) / 8 * 8;
    if (grid <= 0)
        return hipSuccess;
    if (grid > 0x7fffffff)
        return hipErrorInvalidValue;
    static const hipError_t attr = hipFuncSetAttribute((const void *)prefill_ss_kernel<D, WPE>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    (void)attr;
    hipLaunchKernelGGL((prefill_ss_kernel<D, WPE>), dim3((unsigned)grid), dim3(512), LDS_BYTES, s, a);
    *blocks = (uint64_t)grid;
    return hipGetLastError();
}

template <int D, int CB>
static hipError_t prefill_pp_launch(AttnArgs a, hipStream_t s, uint64_t *blocks, int max_query_len)
{
    constexpr int NCOL = 8 * CB * 16;
    a.col_groups = (max_query_len * a.group + NCOL - 1) / NCOL;
    const int64_t n = (int64_t)a.num_seqs * a.num_kv_heads * a.col_groups;
    const int64_t grid = (n + 7) / 8 * 8;
    if (grid <= 0)
        return hipSuccess;
    if (grid > 0x7fffffff)
        return hipErrorInvalidValue;
    static const hipError_t attr = hipFuncSetAttribute((const void *)prefill_pp_kernel<D, CB>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, 2 * Geo<D>::LDS);
    (void)attr;
    hipLaunchKernelGGL((prefill_pp_kernel<D, CB>), dim3((unsigned)grid), dim3(512), 2 * Geo<D>::LDS, s, a);
    *blocks = (uint64_t)grid;
    return hipGetLastError();
}

hipError_t launch_prefill(const AttnArgs &a, int head_dim, int max_query_len, hipStream_t s, uint64_t *blocks)
{
    const int mq = max_query_len;
    // Dh 128: the ping-pong kernel (256 columns per workgroup) when it still
    // yields a workgroup per CU (256 CUs), else the double-buffered kernel
    // with 128 columns if that does, else the producer / consumer kernel (64
    // columns, twice the workgroups).  Dh 256: double-buffered or producer /
    // consumer by the same rule.  Dh 512 (one K and one V buffer; a
    // double-buffered tile would not fit in LDS): the single-buffer kernel
    // with 128 columns per workgroup when that yields a workgroup per CU,
    // else the wave-pair kernel (64 columns).
    const int64_t rows = (int64_t)a.num_seqs * a.num_kv_heads;
    const int64_t groups256 = rows * ((mq * a.group + 255) / 256);
    const int64_t groups128 = rows * ((mq * a.group + 127) / 128);
    switch (head_dim) {
    case 128:
        if (groups256 >= 256)
            return prefill_pp_launch<128, 2>(a, s, blocks, mq);
        if (groups128 >= 256)
            return prefill_db_launch<128, 1, 8, 2>(a, s, blocks, mq);
        return prefill_ss_launch<128, 2>(a, s, blocks, mq);
    case 256:
        if (groups128 >= 256)
            return prefill_db_launch<256, 1, 8, 2>(a, s, blocks, mq);
        return prefill_ss_launch<256, 2>(a, s, blocks, mq);
    case 512:
        if (groups128 >= 256)
            return prefill_sb_launch<512, 1, 8, 2>(a, s, blocks, mq);
        return prefill_ws_launch<512, 8, 2, 1>(a, s, blocks, mq);
    default: return hipErrorInvalidValue;
    }
}

template <int D>
static hipError_t split_launch(const AttnArgs &a, int max_query_len, hipStream_t s, uint64_t *blocks, bool fuse)
{
    if (a.max_tiles <= 0 || a.num_seqs <= 0)
        return hipSuccess;
    // columns a row of this call can have on the split path
    const int max_cols = (int)min((int64_t)a.split_cols, (int64_t)max_query_len * a.group);
    dim3 grid((unsigned)a.max_tiles, (unsigned)a.num_kv_heads, (unsigned)a.num_seqs);
    if (fuse) {   // one more column of workgroups for the cache write (one column block)
        hipLaunchKernelGGL((split_partial_kernel<D, true>), dim3(grid.x + 1, grid.y, grid.z), dim3(NT), 0, s, a);
    } else if (a.split_cols > kSplitCols) {
        // rows with many columns: tiles staged in LDS, one wave per 16-column block
        constexpr int LDS_BYTES = 2 * Geo<D>::NKB * Geo<D>::PAGE;
        const int tgroups = ((max_cols + 15) / 16 + kTileWaves - 1) / kTileWaves;
        static const hipError_t attr = hipFuncSetAttribute((const void *)split_tile_kernel<D>,
                                                           hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
        if (attr != hipSuccess)
            return attr;
        grid.y = (unsigned)(a.num_kv_heads * tgroups);
        hipLaunchKernelGGL((split_tile_kernel<D>), grid, dim3(64 * kTileWaves), LDS_BYTES, s, a);
    } else {
        hipLaunchKernelGGL((split_partial_kernel<D, false>), grid, dim3(NT), 0, s, a);
    }
    if (a.split_cols > kSplitCols) {
        // one fold workgroup per (kFoldWideCols columns, 64-dim slice)
        const dim3 fgrid((unsigned)((max_cols + kFoldWideCols - 1) / kFoldWideCols * (D / 64)),
                         (unsigned)a.num_kv_heads, (unsigned)a.num_seqs);
        hipLaunchKernelGGL((split_fold_wide_kernel<D>), fgrid, dim3(64 * kFoldWideCols), 0, s, a);
    } else {
        // one fold workgroup per (column that can exist, 32-dim slice)
        const dim3 fgrid((unsigned)(max_cols * (D / kFoldSlice)), (unsigned)a.num_kv_heads, (unsigned)a.num_seqs);
        hipLaunchKernelGGL((split_fold_kernel<D>), fgrid, dim3(NT), 0, s, a);
    }
    *blocks = (uint64_t)grid.x * grid.y * grid.z;
    return hipGetLastError();
}

hipError_t launch_split_kv(const AttnArgs &a, int head_dim, int max_query_len, hipStream_t s, uint64_t *blocks)
{
    switch (head_dim) {
    case 128: return split_launch<128>(a, max_query_len, s, blocks, false);
    case 256: return split_launch<256>(a, max_query_len, s, blocks, false);
    case 512: return split_launch<512>(a, max_query_len, s, blocks, false);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_split_kv_fused(const AttnArgs &a, int head_dim, int max_query_len, hipStream_t s, uint64_t *blocks)
{
    if (a.num_new > kMaxFusedTokens || a.split_cols != kSplitCols)
        return hipErrorInvalidValue;
    switch (head_dim) {
    case 128: return split_launch<128>(a, max_query_len, s, blocks, true);
    case 256: return split_launch<256>(a, max_query_len, s, blocks, true);
    case 512: return split_launch<512>(a, max_query_len, s, blocks, true);
    default: return hipErrorInvalidValue;
    }
}

Workspace workspace_layout(int64_t num_seqs, int64_t num_kv_heads, int64_t max_tiles, int64_t head_dim,
                           int64_t split_cols)
{
    // Per-tile partials of the split-KV path, split_cols columns per (row,
    // kv head, tile).  Every call rewrites the slots it reads before reading
    // them, so the workspace needs no initialisation and one workspace sized
    // for the largest bounds serves smaller calls.
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    Workspace w;
    const size_t slots = (size_t)num_seqs * num_kv_heads * max_tiles * split_cols;
    w.acc_off = 0;
    w.m_off = up(w.acc_off + slots * head_dim * sizeof(float));
    w.l_off = up(w.m_off + slots * sizeof(float));
    w.total = up(w.l_off + slots * sizeof(float));
    return w;
}

}  // namespace kvp
