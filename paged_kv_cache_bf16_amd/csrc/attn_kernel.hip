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
//       t = S * (scale*log2 e), -inf for keys the column does not see;
//       m = max t;  p = exp2(t - m) (v_exp_f32);  l = sum p in a fixed tree;
//       acc = P . V with P = bf16(p), MFMA over the tile's keys in 32-key
//           steps in ascending order.
//   * Tiles are folded into the running (M, L, ACC) in ascending order:
//       if m > M:  f = exp2(M - m);  ACC = fma(ACC, f, acc); L = fma(L, f, l); M = m
//       else:      f = exp2(m - M);  ACC = fma(acc, f, ACC); L = fma(l, f, L)
//     starting from M = -inf, L = 0, ACC = 0 (a tile a column cannot see is a
//     no-op).  The output is bf16(ACC * (1 / L) + 0).
//   * No implicit FMA contraction (the library is built -ffp-contract=off);
//     every FMA above is written explicitly.
// Who computes a tile (a streaming prefill workgroup, or one split-KV
// workgroup per tile whose partial the last-arriving workgroup folds) never
// changes these operations, so decode and prefill rows agree bit for bit.
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
// LDS: the K and V pages of the current tile are staged (one kv head), with
// a 16-byte-unit XOR swizzle that keeps the MFMA operand reads free of bank
// conflicts.  Keys at or beyond seq_len read as zero (K and V) so padded or
// poisoned page tails never reach the arithmetic.
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

__device__ __forceinline__ int vsw(int half, int d)
{
    return half ^ (((d >> 2) ^ (d >> 3)) & 1);
}

__device__ __forceinline__ float fmax2(float a, float b) { return a > b ? a : b; }

__device__ __forceinline__ float wave_xor(float v, int mask)
{
    return __shfl_xor(v, mask, 64);
}

// ---------------------------------------------------------------- staging

// Copies the K and V pages of tile `tile` (kv head kvh) into LDS.  Keys at or
// beyond seq_len are zero in both; block ids outside the pool read as zero.
template <int D>
__device__ __forceinline__ void stage_tile(char *lds, const AttnArgs &a, const int32_t *bt_row,
                                           int seq_len, int kvh, int tile)
{
    using G = Geo<D>;
    char *kl = lds;
    char *vl = lds + G::NKB * G::PAGE;
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < G::NKB * G::UPP / NT; ++it) {
        const int u = tid + it * NT;
        const int p = u / G::UPP;
        const int w = u % G::UPP;
        const int page = tile * G::NKB + p;
        const int valid = seq_len - page * BS;          // tokens of this page in range
        u32x4 kval = {0u, 0u, 0u, 0u}, vval = {0u, 0u, 0u, 0u};
        if (valid > 0) {
            const int32_t blk = bt_row[page];
            if (blk >= 0 && (int64_t)blk < a.num_blocks) {
                const int64_t hoff = (int64_t)kvh * BS * D + (int64_t)w * 8;
                kval = *reinterpret_cast<const u32x4 *>(a.k_cache + (int64_t)blk * a.k_block_stride + hoff);
                vval = *reinterpret_cast<const u32x4 *>(a.v_cache + (int64_t)blk * a.v_block_stride + hoff);
                if (valid < BS) {
                    // V unit w = (d, half): tokens half*8 .. half*8+7
                    const int t0 = (w & 1) * 8;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t lo = (t0 + 2 * j < valid) ? 0x0000FFFFu : 0u;
                        const uint32_t hi = (t0 + 2 * j + 1 < valid) ? 0xFFFF0000u : 0u;
                        vval[j] &= (lo | hi);
                    }
                    // K unit w = (du, tok)
                    if ((w & 15) >= valid)
                        kval = u32x4{0u, 0u, 0u, 0u};
                }
            }
        }
        const int du = w >> 4, tok = w & 15;
        *reinterpret_cast<u32x4 *>(kl + p * G::PAGE + (du * 16 + ksw(tok, p)) * 16) = kval;
        const int d = w >> 1, half = w & 1;
        *reinterpret_cast<u32x4 *>(vl + p * G::PAGE + (d * 2 + vsw(half, d)) * 16) = vval;
    }
}

// ---------------------------------------------------------------- tile step

// Per-lane view of one 16-column block: lane (g = lane/16, c = lane%16) owns
// column c.  Holds the Q fragments and the column's key limit.
template <int D>
struct Cols {
    bf16x8 qf[Geo<D>::NDS];
    int lim;         // keys < lim are visible (0: column inactive)
};

// Softmax statistics and BF16 probabilities of one tile for one column block.
template <int D>
struct Scores {
    float m, l;                       // tile max (scaled, log2 domain) and sum of p
    bf16x8 pf[Geo<D>::NKS];           // P^T operands, one per 32-key PV step
};

// Scores and softmax statistics of one tile for one column block.
template <int D>
__device__ __forceinline__ void tile_scores(const char *lds, const Cols<D> &col, int tile,
                                            float scale_log2, Scores<D> &o)
{
    using G = Geo<D>;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, c = lane & 15;
    const char *kl = lds;

    // S^T = K . Q^T, one 16-key block at a time, head dim ascending
    f32x4 s[G::NKB];
#pragma unroll
    for (int kb = 0; kb < G::NKB; ++kb) {
        const int st = kb >> 1, e = kb & 1;
        const int page = 2 * st + (c >> 3);
        const int tok = ((c >> 2) & 1) * 8 + e * 4 + (c & 3);
        const char *rowp = kl + page * G::PAGE + ksw(tok, page) * 16;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < G::NDS; ++ds) {
            const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(rowp + (4 * ds + g) * 256);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, col.qf[ds], acc, 0, 0, 0);
        }
        s[kb] = acc;
    }

    // scale, mask, max
    const int key0 = tile * G::T;
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < G::NKB; ++kb) {
        const int st = kb >> 1, e = kb & 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = key0 + 32 * st + 8 * g + 4 * e + i;
            const float t = __fmul_rn(s[kb][i], scale_log2);
            s[kb][i] = key < col.lim ? t : -INFINITY;
            mx = fmax2(mx, s[kb][i]);
        }
    }
    mx = fmax2(mx, wave_xor(mx, 16));
    mx = fmax2(mx, wave_xor(mx, 32));
    const float mu = mx == -INFINITY ? 0.f : mx;

    // p = exp2(t - m); l in a fixed tree: pairs inside a block, blocks pairwise
    float part[G::NKB];
#pragma unroll
    for (int kb = 0; kb < G::NKB; ++kb) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            s[kb][i] = __builtin_amdgcn_exp2f(__fsub_rn(s[kb][i], mu));
        part[kb] = __fadd_rn(__fadd_rn(s[kb][0], s[kb][1]), __fadd_rn(s[kb][2], s[kb][3]));
    }
#pragma unroll
    for (int w = 1; w < G::NKB; w *= 2)
#pragma unroll
        for (int kb = 0; kb < G::NKB; kb += 2 * w)
            part[kb] = __fadd_rn(part[kb], part[kb + w]);
    float l = part[0];
    l = __fadd_rn(l, wave_xor(l, 16));
    l = __fadd_rn(l, wave_xor(l, 32));
    o.m = mx;
    o.l = l;

    // P^T operands: step st = keys 32st + 8g + 0..7 = block 2st (i) then 2st+1 (i)
#pragma unroll
    for (int st = 0; st < G::NKS; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o.pf[st][i] = (__bf16)s[2 * st][i];
            o.pf[st][4 + i] = (__bf16)s[2 * st + 1][i];
        }
}

// O^T = V^T . P^T for each 16-dim block, keys ascending in 32-key steps;
// sink(db, acc) receives dims 16*db + 4*g + 0..3 of the lane's column.
template <int D, typename Sink>
__device__ __forceinline__ void tile_pv(const char *lds, const Scores<D> &sc, Sink &&sink)
{
    using G = Geo<D>;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, c = lane & 15;
    const char *vl = lds + G::NKB * G::PAGE;
#pragma unroll
    for (int db = 0; db < G::NDB; ++db) {
        const int d = 16 * db + c;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < G::NKS; ++st) {
            const int page = 2 * st + (g >> 1);
            const bf16x8 vf = *reinterpret_cast<const bf16x8 *>(vl + page * G::PAGE + (d * 2 + vsw(g & 1, d)) * 16);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, sc.pf[st], acc, 0, 0, 0);
        }
        sink(db, acc);
    }
}

// Running softmax state of one column (lane-replicated over g).
template <int D>
struct State {
    float M, L;
    f32x4 acc[Geo<D>::NDB];
};

template <int D>
__device__ __forceinline__ void state_init(State<D> &st)
{
    st.M = -INFINITY;
    st.L = 0.f;
#pragma unroll
    for (int db = 0; db < Geo<D>::NDB; ++db)
        st.acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Fold factor for folding a tile with max m into a state with max M:
// up = (m > M); f = exp2(M - m) if up else exp2(m - M); 0 for an empty tile.
__device__ __forceinline__ float fold_factor(float M, float m, bool &up)
{
    up = m > M;
    const float f = up ? __builtin_amdgcn_exp2f(__fsub_rn(M, m)) : __builtin_amdgcn_exp2f(__fsub_rn(m, M));
    return m == -INFINITY ? 0.f : f;
}

// acc' = up ? fma(acc, f, tile) : fma(tile, f, acc).  any_up (wave-uniform)
// only selects a cheaper instruction sequence with identical results.
__device__ __forceinline__ void fold_acc(f32x4 &acc, const f32x4 &tile, float f, bool up, bool any_up)
{
    if (!any_up) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc[i] = __builtin_fmaf(tile[i], f, acc[i]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float x = up ? acc[i] : tile[i];
            const float y = up ? tile[i] : acc[i];
            acc[i] = __builtin_fmaf(x, f, y);
        }
    }
}

__device__ __forceinline__ void fold_stats(float &M, float &L, float m, float l, float f, bool up)
{
    L = up ? __builtin_fmaf(L, f, l) : __builtin_fmaf(l, f, L);
    M = up ? m : M;
}

// bf16 output of 4 consecutive dims
__device__ __forceinline__ u32x2 finish4(const f32x4 &acc, float inv)
{
    u32x2 r;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const float a0 = __fadd_rn(__fmul_rn(acc[2 * j], inv), 0.f);
        const float a1 = __fadd_rn(__fmul_rn(acc[2 * j + 1], inv), 0.f);
        const __bf16 b0 = (__bf16)a0, b1 = (__bf16)a1;
        r[j] = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
    }
    return r;
}

// Column bookkeeping: column index -> (query row, head, key limit).
struct ColInfo {
    int64_t row;
    int head;
    int lim;
};

__device__ __forceinline__ ColInfo col_info(const AttnArgs &a, int col, int kvh, int q0, int q_len, int seq_len)
{
    ColInfo ci;
    const int pr = col / a.group;
    ci.head = kvh * a.group + col % a.group;
    ci.row = (int64_t)q0 + pr;
    const int pos = seq_len - q_len + pr;
    ci.lim = col < q_len * a.group ? (a.causal ? pos + 1 : seq_len) : 0;
    return ci;
}

template <int D>
__device__ __forceinline__ void load_q(Cols<D> &cf, const AttnArgs &a, const ColInfo &ci)
{
    const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int ds = 0; ds < Geo<D>::NDS; ++ds) {
        if (ci.lim > 0) {
            const uint16_t *src = a.q + ci.row * a.q_token_stride + (int64_t)ci.head * D + 32 * ds + 8 * g;
            cf.qf[ds] = *reinterpret_cast<const bf16x8 *>(src);
        } else {
            cf.qf[ds] = bf16x8{};
        }
    }
    cf.lim = ci.lim;
}

template <int D>
__device__ __forceinline__ void store_out(const AttnArgs &a, const ColInfo &ci, const State<D> &st)
{
    const int g = (threadIdx.x & 63) >> 4;
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

// ---------------------------------------------------------------- streaming prefill

// Workgroup = (column group, kv head, sequence); 4 waves x CB column blocks.
// Walks the tiles in ascending order, folding each into registers.
template <int D, int CB>
__global__ __launch_bounds__(NT) void prefill_kernel(AttnArgs a)
{
    using G = Geo<D>;
    extern __shared__ __attribute__((aligned(16))) char lds[];
    constexpr int NCOL = NW * CB * 16;

    // XCD-aware order: workgroup i runs on XCD i % 8; give each XCD a
    // contiguous run of work items so one kv head's pages stay in its L2.
    const int n = a.num_seqs * a.num_kv_heads * a.col_groups;
    const int per = (n + 7) / 8;
    const int j = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
    if (j >= n)
        return;
    const int cgi = j % a.col_groups;
    const int kvh = (j / a.col_groups) % a.num_kv_heads;
    const int b = j / (a.col_groups * a.num_kv_heads);
    const int cg = a.col_groups - 1 - cgi;           // heaviest (latest) columns first

    int q0, q_len, seq_len;
    if (!row_ok(a, b, q0, q_len, seq_len))
        return;
    const int ncols = q_len * a.group;
    if (cg * NCOL >= ncols)
        return;
    const int col_last = min((cg + 1) * NCOL, ncols) - 1;
    const int pos_last = seq_len - q_len + col_last / a.group;
    const int last_tile = (a.causal ? pos_last : seq_len - 1) / G::T;
    const int32_t *bt_row = a.block_tables + (int64_t)b * a.bt_stride;

    const int wave = threadIdx.x >> 6;
    const int c = threadIdx.x & 15;
    Cols<D> cols[CB];
    ColInfo ci[CB];
    State<D> st[CB];
    bool active = false;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const int col = cg * NCOL + (wave * CB + cb) * 16 + c;
        ci[cb] = col_info(a, col, kvh, q0, q_len, seq_len);
        load_q<D>(cols[cb], a, ci[cb]);
        state_init<D>(st[cb]);
        active |= (cg * NCOL + (wave * CB + cb) * 16) < ncols;
    }

    for (int tile = 0; tile <= last_tile; ++tile) {
        __syncthreads();
        stage_tile<D>(lds, a, bt_row, seq_len, kvh, tile);
        __syncthreads();
        if (active) {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                Scores<D> sc;
                tile_scores<D>(lds, cols[cb], tile, a.scale_log2, sc);
                bool up;
                const float f = fold_factor(st[cb].M, sc.m, up);
                const bool any_up = __ballot(up) != 0;
                State<D> &S = st[cb];
                tile_pv<D>(lds, sc, [&](int db, const f32x4 &acc) { fold_acc(S.acc[db], acc, f, up, any_up); });
                fold_stats(S.M, S.L, sc.m, sc.l, f, up);
            }
        }
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
        if (ci[cb].lim > 0)
            store_out<D>(a, ci[cb], st[cb]);
}

// ---------------------------------------------------------------- split-KV (decode)

// Workgroup = (tile, kv head, sequence) for rows whose q_len * G <= 16.
// All waves stage the tile; wave 0 computes the single column block and
// stores the tile's partial state.  The last workgroup of a (sequence, kv
// head) to finish folds the partials in tile order and writes the output.
template <int D>
__global__ __launch_bounds__(NT) void split_kv_kernel(AttnArgs a)
{
    using G = Geo<D>;
    extern __shared__ __attribute__((aligned(16))) char lds[];
    __shared__ int last_flag;

    const int tile = blockIdx.x;
    const int kvh = blockIdx.y;
    const int b = blockIdx.z;
    int q0, q_len, seq_len;
    if (!row_ok(a, b, q0, q_len, seq_len))
        return;
    const int ncols = q_len * a.group;
    if (ncols > kSplitCols)
        return;
    const int n_tiles = (seq_len + G::T - 1) / G::T;
    if (tile >= n_tiles)
        return;
    const int32_t *bt_row = a.block_tables + (int64_t)b * a.bt_stride;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, c = lane & 15;
    const int64_t slot = ((int64_t)b * a.num_kv_heads + kvh) * a.max_tiles;

    stage_tile<D>(lds, a, bt_row, seq_len, kvh, tile);
    __syncthreads();
    if (threadIdx.x < 64) {
        Cols<D> cols;
        const ColInfo ci = col_info(a, c, kvh, q0, q_len, seq_len);
        load_q<D>(cols, a, ci);
        Scores<D> sc;
        tile_scores<D>(lds, cols, tile, a.scale_log2, sc);
        float *accp = a.ws_acc + ((slot + tile) * kSplitCols + c) * D + 4 * g;
        tile_pv<D>(lds, sc, [&](int db, const f32x4 &acc) { *reinterpret_cast<f32x4 *>(accp + 16 * db) = acc; });
        if (g == 0) {
            a.ws_m[(slot + tile) * kSplitCols + c] = sc.m;
            a.ws_l[(slot + tile) * kSplitCols + c] = sc.l;
        }
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        int32_t *ticket = a.ws_ticket + (int64_t)b * a.num_kv_heads + kvh;
        const int prev = __hip_atomic_fetch_add(ticket, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        const int last = prev == n_tiles - 1;
        if (last)
            __hip_atomic_store(ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last_flag = last;
    }
    __syncthreads();
    if (!last_flag)
        return;
    __threadfence();

    // Fold: thread -> (column, 4 dims); tiles in ascending order.
    for (int e = threadIdx.x; e < ncols * (D / 4); e += NT) {
        const int col = e / (D / 4);
        const int d4 = (e % (D / 4)) * 4;
        float M = -INFINITY, L = 0.f;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int t = 0; t < n_tiles; ++t) {
            const int64_t si = (slot + t) * kSplitCols + col;
            const float m = a.ws_m[si];
            const float l = a.ws_l[si];
            const f32x4 pa = *reinterpret_cast<const f32x4 *>(a.ws_acc + si * D + d4);
            bool up;
            const float f = fold_factor(M, m, up);
            fold_acc(acc, pa, f, up, true);
            fold_stats(M, L, m, l, f, up);
        }
        const ColInfo ci = col_info(a, col, kvh, q0, q_len, seq_len);
        const float inv = 1.0f / L;
        *reinterpret_cast<u32x2 *>(a.out + ci.row * a.out_token_stride + (int64_t)ci.head * D + d4) = finish4(acc, inv);
    }
}

}  // namespace

template <int D, int CB>
static hipError_t prefill_launch(AttnArgs a, hipStream_t s, uint64_t *blocks, int max_query_len)
{
    constexpr int NCOL = NW * CB * 16;
    a.col_groups = (max_query_len * a.group + NCOL - 1) / NCOL;
    const int64_t n = (int64_t)a.num_seqs * a.num_kv_heads * a.col_groups;
    const int64_t grid = (n + 7) / 8 * 8;
    if (grid <= 0)
        return hipSuccess;
    if (grid > 0x7fffffff)
        return hipErrorInvalidValue;
    static const hipError_t attr = hipFuncSetAttribute((const void *)prefill_kernel<D, CB>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, Geo<D>::LDS);
    (void)attr;
    hipLaunchKernelGGL((prefill_kernel<D, CB>), dim3((unsigned)grid), dim3(NT), Geo<D>::LDS, s, a);
    *blocks = (uint64_t)grid;
    return hipGetLastError();
}

hipError_t launch_prefill(const AttnArgs &a, int head_dim, int max_query_len, hipStream_t s, uint64_t *blocks)
{
    const int mq = max_query_len;
    switch (head_dim) {
    case 128: return prefill_launch<128, 2>(a, s, blocks, mq);
    case 256: return prefill_launch<256, 1>(a, s, blocks, mq);
    case 512: return prefill_launch<512, 1>(a, s, blocks, mq);
    default: return hipErrorInvalidValue;
    }
}

template <int D>
static hipError_t split_launch(const AttnArgs &a, hipStream_t s, uint64_t *blocks)
{
    const dim3 grid((unsigned)a.max_tiles, (unsigned)a.num_kv_heads, (unsigned)a.num_seqs);
    if (a.max_tiles <= 0 || a.num_seqs <= 0)
        return hipSuccess;
    static const hipError_t attr = hipFuncSetAttribute((const void *)split_kv_kernel<D>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, Geo<D>::LDS);
    (void)attr;
    hipLaunchKernelGGL((split_kv_kernel<D>), grid, dim3(NT), Geo<D>::LDS, s, a);
    *blocks = (uint64_t)a.max_tiles * a.num_kv_heads * a.num_seqs;
    return hipGetLastError();
}

hipError_t launch_split_kv(const AttnArgs &a, int head_dim, hipStream_t s, uint64_t *blocks)
{
    switch (head_dim) {
    case 128: return split_launch<128>(a, s, blocks);
    case 256: return split_launch<256>(a, s, blocks);
    case 512: return split_launch<512>(a, s, blocks);
    default: return hipErrorInvalidValue;
    }
}

Workspace workspace_layout(int64_t num_seqs, int64_t num_kv_heads, int64_t max_tiles, int64_t head_dim)
{
    // The ticket counters sit at a fixed place (the start) whatever the call's
    // bounds, so calls with different batch sizes or lengths sharing one
    // workspace always find them zero; the partials after them are fully
    // rewritten by every call before they are read.
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    Workspace w;
    const size_t slots = (size_t)num_seqs * num_kv_heads * max_tiles * kSplitCols;
    w.ticket_off = 0;
    w.acc_off = (size_t)kMaxTickets * sizeof(int32_t);
    w.m_off = up(w.acc_off + slots * head_dim * sizeof(float));
    w.l_off = up(w.m_off + slots * sizeof(float));
    w.total = up(w.l_off + slots * sizeof(float));
    return w;
}

}  // namespace kvp
