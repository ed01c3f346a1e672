"""GPU parity of paged_attention against the oracle, and the bitwise
properties of the fixed arithmetic schedule.

Tolerance (BF16 output vs the FP32 oracle): max-abs 2e-2 and mean-abs 2e-3
per case.  Bitwise checks report mismatch_count / max_abs_diff like the
strict-agreement runs on "fix(rocm): stabilize direct paged CK attention for
bitwise R/R" (Validation)."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_bf16_amd as kvp
from paged_kv_cache_bf16_amd import workloads as wl
from harness import (GpuCase, bitwise, bf16_to_f32, compare, dev_bits, group_rows, host_bits,
                     oracle_attention, oracle_pool, sample_rows)

pytestmark = pytest.mark.gpu


def _run_and_compare(w, rows=None, what=""):
    print("case", what or w.name, flush=True)
    g = GpuCase(w)
    out = g.run()
    ref = oracle_attention(w, oracle_pool(w), rows=rows)
    got = out if rows is None else out[rows]
    return g, out, compare(got, ref, what or w.name)


# ------------------------------------------------------------ the pages' composition case

def test_tiny_prefill_and_decode_match_oracle_and_each_other():
    w = wl.tiny()
    g, out, _ = _run_and_compare(w)
    # decode of token 19: one query (the last position) over the same cache
    d = w.decode_view()
    g.set_queries(d.q, d.query_lens)
    dec = g.run()
    ref = oracle_attention(d, oracle_pool(w))
    compare(dec, ref, "tiny-decode")
    bitwise(dec[0], out[19], "tiny decode vs prefill row 19")
    c = kvp.kvp_get_counters()
    assert c["split_kv_launches"] >= 1 and c["prefill_launches"] >= 1


def test_tiny_swapped_blocks_change_output():
    """Anti-vacuity: swapping the two in-range logical blocks must change the
    causal rows (reads really go through the table).  The pool is zero-filled:
    after the swap some reads land on slots no token wrote."""
    w = wl.tiny()
    g = GpuCase(w, fill_bits=0)
    base = g.run()
    bt = w.block_tables.copy()
    bt[0, [0, 1]] = bt[0, [1, 0]]
    g.set_queries(w.q, w.query_lens, block_tables=bt)
    swapped = g.run()
    assert np.abs(bf16_to_f32(swapped) - bf16_to_f32(base)).max() > 0.1


# ------------------------------------------------------------ named workloads

def test_decode_b4_kv7168():
    w = wl.decode()
    g, out, stats = _run_and_compare(w)
    print(stats)
    assert kvp.kvp_get_counters()["split_kv_launches"] >= 1


def _rows(*parts):
    return np.array(sorted(set(np.concatenate(parts).tolist())), np.int64)


def test_prefill_b1_q4096_sampled():
    """Every row of the first, a middle and the last 256-column workgroup
    (64 query rows each at G = 4), plus a seeded sample."""
    w = wl.prefill()
    _run_and_compare(w, rows=_rows(group_rows(w, 64), sample_rows(w, 64)))


def test_suffix_b4_q128_kv7168_sampled():
    """Every row of the first, a middle and the last 64-column workgroup of
    each sequence (16 query rows each), plus a seeded sample."""
    w = wl.suffix()
    _run_and_compare(w, rows=_rows(group_rows(w, 16), sample_rows(w, 64)))


def test_ragged_mixed_batch_over_2gb_pool():
    w = wl.ragged()
    _run_and_compare(w)


@pytest.mark.parametrize("L", wl.WIDE_LENGTHS)
def test_wide_head_prefill_sampled_and_decode(L):
    w = wl.wide(L)
    # every row of the first, a middle and the last 128-column workgroup (16 rows at G = 8)
    g, out, _ = _run_and_compare(w, rows=_rows(group_rows(w, 16), sample_rows(w, 24)), what="wide%d" % L)
    d = w.decode_view()
    g.set_queries(d.q, d.query_lens)
    dec = g.run()
    compare(dec, oracle_attention(d, oracle_pool(w)), "wide%d-decode" % L)
    bitwise(dec[0], out[L - 1], "wide%d decode vs prefill last row" % L)


# ------------------------------------------------------------ sweeps: several tiles, ragged tails

CASES = [
    # seq_lens, q_lens, Hq, Hkv, D, causal
    ([1, 2, 15, 16, 17], [1, 2, 15, 16, 17], 4, 1, 128, True),
    ([127, 128, 129, 300], [127, 1, 129, 33], 8, 2, 128, True),
    ([513, 200], [513, 17], 8, 2, 128, True),
    ([64, 65, 250], [64, 65, 250], 16, 2, 512, True),
    ([100, 37], [100, 5], 8, 2, 256, True),
    ([300, 129], [300, 3], 8, 8, 128, False),
    ([90], [90], 16, 1, 128, True),
    ([200, 0, 70], [7, 0, 70], 8, 2, 128, True),
]


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_parity_sweep(case):
    seq, ql, Hq, Hkv, D, causal = case
    w = wl.random_case(100 + len(seq) + D, seq, ql, Hq, Hkv, D, causal=causal)
    _run_and_compare(w, what="sweep%s" % (case,))


def test_decode_many_sequences():
    """2048 decode rows of 1..400 keys in one call (a grid of 2048 rows of
    partial and fold workgroups): every output row matches the oracle."""
    rng = np.random.default_rng(5)
    lens = [int(x) for x in rng.integers(1, 401, size=2048)]
    w = wl.random_case(61, lens, [1] * len(lens), 8, 2, 128)
    _run_and_compare(w, what="decode-2048-rows")


def test_decode_only_sweep_many_lengths():
    lens = [1, 5, 16, 127, 128, 129, 255, 256, 257, 1000, 4100]
    w = wl.random_case(7, lens, [1] * len(lens), 8, 2, 128)
    _run_and_compare(w, what="decode-sweep")


# ------------------------------------------------------------ large grids (one workgroup per CU, Dh 128)

def _large_grid_blocks(w):
    """Workgroups the Dh-128 large-grid prefill launches (256 columns each,
    padded to a multiple of the 8 XCDs)."""
    G = w.num_q_heads // w.num_kv_heads
    n = w.batch * w.num_kv_heads * (-(-int(w.max_query_len) * G // 256))
    return -(-n // 8) * 8


@pytest.mark.parametrize("causal", [True, False])
def test_large_grid_prefill_ragged(causal):
    """Ragged full prefills big enough for the large-grid kernel: sampled rows
    against the oracle, every row's decode against its prefill row."""
    lens = [2049, 1000, 300, 1537]
    w = wl.random_case(31 + int(causal), lens, lens, 32, 8, 128, causal=causal)
    assert _large_grid_blocks(w) >= 256
    g, full, _ = _run_and_compare(w, rows=sample_rows(w, 96), what="large-grid causal=%d" % causal)
    assert kvp.kvp_get_counters()["last_grid_blocks"] == _large_grid_blocks(w)
    d = w.decode_view()
    g.set_queries(d.q, d.query_lens)
    bitwise(g.run(), full[w.query_start_loc[1:] - 1], "large-grid decode vs prefill last rows")


def test_large_grid_suffix_equals_full_rows():
    """Suffix chunks (bottom-right causal) through the large-grid kernel give
    the full prefill's rows bitwise."""
    lens = [3000, 2100, 3001, 2800]
    w = wl.random_case(41, lens, lens, 32, 8, 128)
    g = GpuCase(w)
    full = g.run()
    qsl = w.query_start_loc
    for tail in (512, 777):
        q = np.concatenate([w.q[qsl[b + 1] - tail:qsl[b + 1]] for b in range(w.batch)])
        g.set_queries(q, [tail] * w.batch)
        part = g.run()
        assert kvp.kvp_get_counters()["last_grid_blocks"] == -(-(4 * 8 * (-(-tail * 4 // 256))) // 8) * 8
        exp = np.concatenate([full[qsl[b + 1] - tail:qsl[b + 1]] for b in range(w.batch)])
        bitwise(part, exp, "large-grid suffix %d vs full" % tail)


def test_mixed_batch_split_and_prefill_paths_agree():
    """With a workspace, rows of a mixed batch whose q_len * G <= 16 take the
    split-KV path and the others a prefill kernel; without one, every row
    streams through the prefill kernel.  Both give the same bits."""
    w = wl.random_case(29, [300, 2000, 129, 700, 4100], [300, 1, 4, 33, 2], 8, 2, 128)
    g = GpuCase(w)
    before = kvp.kvp_get_counters()["split_kv_launches"]
    both = g.run()
    assert kvp.kvp_get_counters()["split_kv_launches"] == before + 1
    alone = g.run(use_workspace=False)
    assert kvp.kvp_get_counters()["split_kv_launches"] == before + 1
    bitwise(both, alone, "mixed batch: split + prefill vs prefill only")
    compare(both, oracle_attention(w, oracle_pool(w)), "mixed batch")


def test_mixed_batch_on_a_side_stream_is_complete_for_later_work():
    """A mixed batch given a workspace, called on a stream other than the
    default one: work enqueued on that stream after the call (a copy of the
    output, with no device-wide synchronisation) must see every row, the
    split-KV rows included, with the bits of the prefill-only run.  Short
    rows with long KV (a slow split path) beside one small prefill row;
    three calls in a row."""
    w = wl.random_case(41, [9000, 12000, 33, 7000], [1, 2, 33, 1], 8, 2, 128)
    g = GpuCase(w)
    ref = g.run(use_workspace=False)
    s = torch.cuda.Stream()
    before = kvp.kvp_get_counters()["split_kv_launches"]
    ms, mq = int(w.seq_lens.max()), int(w.max_query_len)
    copies = []
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        for _ in range(3):
            g.out.fill_(-1)
            kvp.paged_attention(g.pool, g.q, g.out, w.num_q_heads, g.bt, g.seq_lens, g.qsl, mq, ms, w.scale, True,
                                workspace=g.ws)
            copies.append(g.out.clone())
    s.synchronize()
    assert kvp.kvp_get_counters()["split_kv_launches"] == before + 3
    for i, c in enumerate(copies):
        bitwise(host_bits(c), ref, "mixed batch on a helper stream, copy %d" % i)


def _decode_step_case(seed, lens, Hq, Hkv, D, new_pos, extra_slots=()):
    """A decode batch plus new K/V rows for the given positions (one per row),
    optionally followed by extra (slot, k, v) rows."""
    w = wl.random_case(seed, lens, [1] * len(lens), Hq, Hkv, D)
    rng = np.random.default_rng(seed + 7)
    slots = [int(w.block_tables[b, p // 16]) * 16 + p % 16 for b, p in enumerate(new_pos)]
    slots += list(extra_slots)
    T = len(slots)
    kn = wl.to_bf16_bits(rng.standard_normal((T, Hkv, D)).astype(np.float32))
    vn = wl.to_bf16_bits(rng.standard_normal((T, Hkv, D)).astype(np.float32))
    return w, np.array(slots, np.int64), kn, vn


def _run_step(w, slots, kn, vn, fused):
    from harness import dev_bits
    g = GpuCase(w)
    k, v = dev_bits(kn), dev_bits(vn)
    sd = torch.from_numpy(slots).cuda()
    ms = int(w.seq_lens.max())
    mq = int(w.max_query_len)
    g.out.fill_(-1)
    torch.cuda.synchronize()
    before = kvp.kvp_get_counters()
    if fused:
        kvp.kvp_decode_step(g.pool, k, v, sd, g.q, g.out, w.num_q_heads, g.bt, g.seq_lens, g.qsl, mq, ms, w.scale,
                            True, workspace=g.ws)
    else:
        kvp.reshape_and_cache(g.pool, k, v, sd)
        kvp.paged_attention(g.pool, g.q, g.out, w.num_q_heads, g.bt, g.seq_lens, g.qsl, mq, ms, w.scale, True,
                            workspace=g.ws)
    torch.cuda.synchronize()
    after = kvp.kvp_get_counters()
    delta = {k: after[k] - before[k] for k in ("fused_decode_steps", "reshape_and_cache_launches")}
    return (g.out.cpu().numpy().view(np.uint16).copy(), g.pool.storage.cpu().numpy().view(np.uint16).copy(),
            delta)


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 8, 2), (256, 8, 2), (512, 16, 2)])
def test_decode_step_fused_equals_cache_then_attention(D, Hq, Hkv):
    """kvp_decode_step in one launch: the same pool bits and output bits as
    reshape_and_cache followed by paged_attention, with the new tokens at the
    last position, inside a middle tile, at the first key, skipped (-1) and
    beyond the pool."""
    lens = [700, 129, 2000, 1]
    w, slots, kn, vn = _decode_step_case(D + Hq, lens, Hq, Hkv, D, [699, 64, 1000, 0], extra_slots=(-1, 1 << 40))
    out_f, pool_f, delta = _run_step(w, slots, kn, vn, fused=True)
    assert delta == {"fused_decode_steps": 1, "reshape_and_cache_launches": 0}
    out_s, pool_s, _ = _run_step(w, slots, kn, vn, fused=False)
    bitwise(pool_f, pool_s, "pool after the fused step")
    bitwise(out_f, out_s, "output of the fused step")
    assert np.isfinite(bf16_to_f32(out_f)).all()


@pytest.mark.parametrize("D,Hq,Hkv,split_cols", [(128, 8, 2, 512), (128, 32, 8, 128), (256, 8, 2, 256),
                                                  (512, 16, 2, 384), (128, 8, 2, 1024)])
def test_wide_split_mixed_batch_equals_prefill(D, Hq, Hkv, split_cols):
    """A workspace of kvp_workspace_bytes_split(..., split_cols) sends the
    rows with q_len * G <= split_cols to the split-KV path (up to eight
    16-column blocks per partial workgroup against one KV tile staged in
    LDS, then the register fold); the others stream through a prefill
    kernel (split_cols 1024 is the widest the library takes).  Every row's output and lse equal the
    prefill-only call (no workspace) bitwise, and match the oracle."""
    G = Hq // Hkv
    lens = [2100, 900, 1500, 3000, 640, 2000]
    qls = [1, 5, max(1, 68 // G), max(1, split_cols // G), 300, max(1, split_cols // G + 1)]
    w = wl.random_case(800 + D + split_cols, lens, qls, Hq, Hkv, D)
    print("wide split D=%d G=%d split_cols=%d cols=%s" % (D, G, split_cols, [q * G for q in qls]), flush=True)
    g = GpuCase(w, split_cols=split_cols)
    c0 = kvp.kvp_get_counters()
    out, lse = g.run_lse()
    c1 = kvp.kvp_get_counters()
    assert c1["split_kv_launches"] == c0["split_kv_launches"] + 1
    assert c1["prefill_launches"] == c0["prefill_launches"] + 1
    ref_out, ref_lse = g.run_lse(use_workspace=False)
    bitwise(out, ref_out, "wide split vs prefill only")
    assert np.array_equal(lse.view(np.uint32), ref_lse.view(np.uint32)), "lse differs"
    rows = _rows(sample_rows(w, 48), group_rows(w, 4, groups=("last",)))
    compare(out[rows], oracle_attention(w, oracle_pool(w), rows=rows), "wide split vs oracle")


def test_wide_split_ragged_over_2gb():
    """The ragged batch on its 2.29 GB pool with a workspace wide enough for
    its 128- and 17-query rows (512 columns): same bits as with the minimal
    workspace (only the one-query row on the split path) and within tolerance
    of the oracle."""
    w = wl.ragged()
    g = GpuCase(w)
    base = g.run()
    ws_small = g.ws
    g.ws = kvp.alloc_workspace(g.pool, w.num_q_heads, w.batch, int(w.seq_lens.max()), split_cols=512)
    assert g.ws.numel() > ws_small.numel()
    wide = g.run()
    bitwise(wide, base, "ragged: wide split vs minimal workspace")
    compare(wide, oracle_attention(w, oracle_pool(w)), "ragged wide split vs oracle")


def _multi_token_step_case(seed, lens, n_new, Hq, Hkv, D):
    """A decode step that writes the last n_new positions of every row and
    queries exactly those positions (q_len = n_new, bottom-right causal)."""
    w = wl.random_case(seed, lens, [n_new] * len(lens), Hq, Hkv, D)
    rng = np.random.default_rng(seed + 11)
    slots = [int(w.block_tables[b, p // 16]) * 16 + p % 16 for b, L in enumerate(lens) for p in range(L - n_new, L)]
    T = len(slots)
    kn = wl.to_bf16_bits(rng.standard_normal((T, Hkv, D)).astype(np.float32))
    vn = wl.to_bf16_bits(rng.standard_normal((T, Hkv, D)).astype(np.float32))
    return w, np.array(slots, np.int64), kn, vn


# rows whose last positions cross a half-page (7/8), a page (15/16), a
# 128-key tile (127/128), a 64-key tile (63/64), or stay inside one
# half-page (696..699: several new values in one lane's 8-token V unit)
MULTI_LENS = [9, 17, 130, 66, 700]


@pytest.mark.parametrize("D,Hq,Hkv,n_new,lens", [
    (128, 8, 2, 2, MULTI_LENS), (128, 8, 2, 3, MULTI_LENS), (128, 8, 2, 4, MULTI_LENS),
    (256, 8, 2, 2, MULTI_LENS), (256, 8, 2, 3, MULTI_LENS), (256, 8, 2, 4, MULTI_LENS),
    (512, 8, 2, 2, MULTI_LENS), (512, 8, 2, 3, MULTI_LENS), (512, 8, 2, 4, MULTI_LENS),
    (512, 16, 2, 2, MULTI_LENS),
    (128, 2, 2, 16, [16, 40, 130, 700]), (256, 2, 2, 16, [16, 40, 130, 700]),
    (512, 2, 2, 16, [16, 40, 130, 700]),
], ids=lambda x: str(x) if not isinstance(x, list) else "L%d" % len(x))
def test_decode_step_several_new_tokens_per_row(D, Hq, Hkv, n_new, lens):
    """kvp_decode_step writing n_new consecutive tokens per row (all in one
    launch): pool and output bits equal reshape_and_cache followed by
    paged_attention, and the output matches the oracle run on the pool after
    the scatter ("test(rocm): ReshapeAndCache->PagedAttention composition at
    real dims", What changed: the cache write and the read that must see it)."""
    print("multi-token step D=%d Hq=%d Hkv=%d n=%d lens=%s" % (D, Hq, Hkv, n_new, lens), flush=True)
    w, slots, kn, vn = _multi_token_step_case(7 * D + 3 * n_new + Hq, lens, n_new, Hq, Hkv, D)
    out_f, pool_f, delta = _run_step(w, slots, kn, vn, fused=True)
    assert delta == {"fused_decode_steps": 1, "reshape_and_cache_launches": 0}
    out_s, pool_s, delta_s = _run_step(w, slots, kn, vn, fused=False)
    assert delta_s["reshape_and_cache_launches"] == 1
    bitwise(pool_f, pool_s, "pool after the fused step")
    bitwise(out_f, out_s, "output of the fused step")
    opool = oracle_pool(w)
    oracle.reshape_and_cache(opool, kn, vn, slots)
    np.testing.assert_array_equal(pool_f, opool.storage)
    compare(out_f, oracle_attention(w, opool), "multi-token step vs oracle")


def test_decode_step_many_tokens_falls_back_to_two_launches():
    lens = [300, 520]
    w, slots, kn, vn = _decode_step_case(11, lens, 8, 2, 128, [299, 519])
    extra = [s for s in range(16 * int(w.num_blocks - 5), 16 * int(w.num_blocks)) if s not in set(slots.tolist())]
    slots = np.concatenate([slots, np.array(extra[:70], np.int64)])     # 72 distinct slots
    rng = np.random.default_rng(3)
    kn = wl.to_bf16_bits(rng.standard_normal((len(slots), 2, 128)).astype(np.float32))
    vn = wl.to_bf16_bits(rng.standard_normal((len(slots), 2, 128)).astype(np.float32))
    out_f, pool_f, delta = _run_step(w, slots, kn, vn, fused=True)
    assert delta == {"fused_decode_steps": 0, "reshape_and_cache_launches": 1}
    out_s, pool_s, _ = _run_step(w, slots, kn, vn, fused=False)
    bitwise(pool_f, pool_s, "pool")
    bitwise(out_f, out_s, "output")


def test_decode_long_rows():
    """Decode rows of 2..235 tiles (the longest folds its partials in two
    staged rounds) match the oracle and their prefill rows bitwise."""
    lens = [8193, 16384, 20000, 129, 30000]
    w = wl.random_case(23, lens, lens, 8, 2, 128)
    d = w.decode_view()
    g = GpuCase(d)
    dec = g.run()
    compare(dec, oracle_attention(d, oracle_pool(d)), "long decode")
    g.set_queries(w.q, w.query_lens)
    full = g.run()
    bitwise(dec, full[w.query_start_loc[1:] - 1], "long decode vs prefill last rows")


@pytest.mark.parametrize("D,Hq,Hkv,L,peak,vs", [
    (128, 8, 2, 26000, 24999, 1.0),      # 128-key tiles: the peak in tile 195, past the first round of 192
    (512, 16, 2, 18432, 15007, 0.5),     # 64-key tiles: tile 234 of 288 (the wide-head geometry)
    (512, 16, 2, 13000, 12300, 0.5),     # tile 192: the first tile of the second fold round
])
def test_planted_peak_long_rows(D, Hq, Hkv, L, peak, vs):
    """A long row whose running maximum jumps late: the key at position
    `peak` is planted as alpha * q (q = the last query row's first head of
    each kv-head group), so that head's softmax is nearly one-hot on it and
    its output is ~V[peak] (magnitude ~1) while every other key's weight is
    ~1e-5.  Decode (split-KV, partials folded in rounds of 192 tiles) and
    the full prefill's last row must both find the peak: a fold that drops
    or misweights the second round, or a reference that does not move,
    returns ~mean(V) ~ 0 instead."""
    print("planted peak D=%d L=%d peak=%d" % (D, L, peak), flush=True)
    w = wl.random_case(500 + D + L, [L], [L], Hq, Hkv, D, value_scale=vs)
    G = Hq // Hkv
    alpha = 2.0 / vs                           # score ~ 22.6 natural-log units at either scale
    qlast = bf16_to_f32(w.q[L - 1])            # [Hq, D]
    k = w.k.copy()
    for g in range(Hkv):
        k[peak, g] = wl.to_bf16_bits(np.float32(alpha) * qlast[g * G])
    w.k = k
    g, full, dec = _prefill_then_decode(w)
    d = w.decode_view()
    ref = oracle_attention(d, oracle_pool(w))
    # the pin is live: the oracle's planted heads return V[peak]
    vpk = bf16_to_f32(w.v[peak])
    for gg in range(Hkv):
        assert np.abs(ref[0, gg * G] - vpk[gg]).max() < 1e-2
    compare(dec, ref, "planted peak decode L=%d" % L)
    bitwise(dec[0], full[L - 1], "planted peak decode vs prefill last row")
    rows = _rows(group_rows(w, 16, groups=("last",)), sample_rows(w, 8))
    compare(full[rows], oracle_attention(w, oracle_pool(w), rows=rows), "planted peak prefill L=%d" % L)


# ------------------------------------------------------------ bitwise properties

def _prefill_then_decode(w):
    g = GpuCase(w)
    full = g.run()
    d = w.decode_view()
    g.set_queries(d.q, d.query_lens)
    dec = g.run()
    return g, full, dec


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 8, 2), (128, 32, 8), (256, 8, 2), (512, 16, 2)])
def test_decode_equals_prefill_last_row(D, Hq, Hkv):
    lens = [1, 16, 129, 777, 2050]
    w = wl.random_case(D + Hq, lens, lens, Hq, Hkv, D)
    g, full, dec = _prefill_then_decode(w)
    last = w.query_start_loc[1:] - 1
    bitwise(dec, full[last], "decode vs prefill D=%d" % D)


def test_row_zero_is_v0_and_suffix_equals_full():
    w = wl.random_case(5, [300, 520], [300, 520], 8, 2, 128)
    g = GpuCase(w)
    full = g.run()
    # row 0 of each causal prefill sees only token 0: output == V[0] bitwise
    for b, start in enumerate(w.query_start_loc[:-1]):
        v0 = w.v[int(np.sum(w.seq_lens[:b]))]                     # [Hkv, D]
        G = w.num_q_heads // w.num_kv_heads
        exp = np.repeat(v0, G, axis=0)
        bitwise(full[start], exp, "row0 == V0 (seq %d)" % b)
    # suffix chunks of 130 and 1 queries give the same rows as the full prefill
    for tail in (130, 17, 1):
        qsl = w.query_start_loc
        q = np.concatenate([w.q[qsl[b + 1] - tail:qsl[b + 1]] for b in range(w.batch)])
        g.set_queries(q, [tail] * w.batch)
        part = g.run()
        exp = np.concatenate([full[qsl[b + 1] - tail:qsl[b + 1]] for b in range(w.batch)])
        bitwise(part, exp, "suffix %d vs full" % tail)


def test_page_permutation_and_batch_shape_are_bitwise_neutral():
    lens = [700, 129, 2000, 64]
    w = wl.random_case(9, lens, [1] * 4, 8, 2, 128, spare_blocks=11)
    g = GpuCase(w)
    base = g.run()
    # same values at new physical pages
    perm = np.random.default_rng(1).permutation(w.num_blocks).astype(np.int32)
    w2 = wl.build("perm", w.seq_lens, w.query_lens, 8, 2, 128, perm[w.block_tables], w.num_blocks, seed=3)
    w2.k, w2.v, w2.q = w.k, w.v, w.q
    bitwise(GpuCase(w2).run(), base, "page permutation")
    # shrinking batches 4 -> 3 -> 2 -> 1 and single rows give the same rows
    for n in (3, 2, 1):
        g.set_queries(w.q[:n], [1] * n, block_tables=w.block_tables[:n], seq_lens=w.seq_lens[:n])
        bitwise(g.run(), base[:n], "batch %d" % n)
    g.set_queries(w.q[2:3], [1], block_tables=w.block_tables[2:3], seq_lens=w.seq_lens[2:3])
    bitwise(g.run(), base[2:3], "row 2 alone")


def test_decode_with_larger_host_bound_is_bitwise_equal():
    """A looser max_seq_len bound (wider grid, more empty tiles) changes who
    computes, never what: the same rows give the same bits."""
    lens = [4000, 129, 1, 7000]
    w = wl.random_case(17, lens, [1] * 4, 8, 2, 128)
    g = GpuCase(w, ws_max_seq_len=8400)
    base = g.run()
    wide_bt = np.pad(w.block_tables, ((0, 0), (0, 100)))
    g.set_queries(w.q, w.query_lens, block_tables=wide_bt)
    bitwise(base, g.run(max_seq_len=8400), "looser max_seq_len")
    compare(base, oracle_attention(w, oracle_pool(w)), "decode")


def test_repeated_calls_are_deterministic():
    w = wl.random_case(12, [3000, 40], [1, 1], 8, 2, 128)
    g = GpuCase(w)
    a = g.run()
    for _ in range(20):
        b = g.run()
    bitwise(a, b, "repeat")


def test_empty_batch_and_zero_queries_are_noops():
    w = wl.random_case(13, [50], [1], 8, 2, 128)
    g = GpuCase(w)
    out = torch.full_like(g.q, 7)
    kvp.paged_attention(g.pool, g.q, out, 8, g.bt[:0], g.seq_lens[:0], g.qsl[:1], 0, 0, workspace=g.ws)
    kvp.paged_attention(g.pool, g.q, out, 8, g.bt, g.seq_lens, g.qsl, 0, 50, workspace=g.ws)
    torch.cuda.synchronize()
    assert bool((out == 7).all())


def test_invalid_arguments_rejected_before_launch():
    w = wl.random_case(14, [50], [1], 8, 2, 128)
    g = GpuCase(w)
    before = kvp.kvp_get_counters()
    with pytest.raises(kvp.KvpError) as e:          # too-small workspace
        kvp.paged_attention(g.pool, g.q, g.out, 8, g.bt, g.seq_lens, g.qsl, 1, 50, workspace=g.ws[:16])
    assert e.value.code == kvp.KVP_ERR_WORKSPACE_TOO_SMALL
    with pytest.raises(kvp.KvpError) as e:          # Hq not a multiple of Hkv
        kvp.paged_attention(g.pool, g.q, g.out, 7, g.bt, g.seq_lens, g.qsl, 1, 50, workspace=g.ws)
    assert e.value.code == kvp.KVP_ERR_UNSUPPORTED
    after = kvp.kvp_get_counters()
    assert after["split_kv_launches"] == before["split_kv_launches"]


def test_fused_qkv_view_strides():
    """q, k and v as column slices of one fused projection output [T, (Hq + 2 Hkv) * D]
    ("test(rocm): ReshapeAndCache->PagedAttention composition at real dims", review
    thread on fused-view strides): the cache write and attention read them through
    their token strides, and the output lands in a wider buffer; bits equal the
    contiguous run."""
    lens = [300, 129]
    w = wl.random_case(91, lens, lens, 8, 2, 128)
    print("fused qkv view", flush=True)
    Hq, Hkv, D = 8, 2, 128
    T = int(w.q.shape[0])
    assert T == int(w.k.shape[0])           # full prefill: one new token per query
    Wd = (Hq + 2 * Hkv) * D
    fused = torch.empty((T, Wd), dtype=torch.int16, device="cuda")
    fused[:, :Hq * D] = dev_bits(w.q).reshape(T, -1)
    fused[:, Hq * D:(Hq + Hkv) * D] = dev_bits(w.k).reshape(T, -1)
    fused[:, (Hq + Hkv) * D:] = dev_bits(w.v).reshape(T, -1)
    qv = fused[:, :Hq * D].unflatten(1, (Hq, D))
    kv = fused[:, Hq * D:(Hq + Hkv) * D].unflatten(1, (Hkv, D))
    vv = fused[:, (Hq + Hkv) * D:].unflatten(1, (Hkv, D))
    assert qv.stride(0) == Wd and kv.stride(0) == Wd
    pool = kvp.alloc_pool(w.num_blocks, Hkv, D, fill_bits=0x7FC1)
    kvp.reshape_and_cache(pool, kv, vv, torch.from_numpy(w.slot_mapping).cuda())
    bt = torch.from_numpy(kvp.kv_prepare_block_tables(pool, w.block_tables, w.seq_lens)).cuda()
    sl = torch.from_numpy(w.seq_lens).cuda()
    qsl = torch.from_numpy(w.query_start_loc).cuda()
    wide = torch.full((T, Hq * D + 64), -1, dtype=torch.int16, device="cuda")
    outv = wide[:, :Hq * D].unflatten(1, (Hq, D))
    kvp.paged_attention(pool, qv, outv, Hq, bt, sl, qsl, int(max(lens)), int(max(lens)), w.scale, True)
    torch.cuda.synchronize()
    g = GpuCase(w)
    ref = g.run()
    got = host_bits(outv.contiguous())
    bitwise(got, ref, "fused-view prefill")
    assert (host_bits(wide[:, Hq * D:]) == 0xFFFF).all(), "wrote past the output rows"
    np.testing.assert_array_equal(host_bits(pool.storage), g.pool_bits())
    # and against the oracle: the pool bit for bit, the output within tolerance
    opool = oracle_pool(w)
    np.testing.assert_array_equal(host_bits(pool.storage), opool.storage)
    compare(got, oracle_attention(w, opool), "fused-view prefill vs oracle")


def test_fused_qkv_view_decode_step():
    """kvp_decode_step (one launch) reading q, k and v as slices of a fused
    [B, (Hq + 2 Hkv) * D] projection: same output and pool bits as contiguous
    inputs."""
    lens = [700, 129, 2000]
    Hq, Hkv, D = 8, 2, 128
    w, slots, kn, vn = _decode_step_case(93, lens, Hq, Hkv, D, [699, 128, 1999])
    print("fused qkv view decode step", flush=True)
    out_c, pool_c, delta = _run_step(w, slots, kn, vn, fused=True)
    assert delta["fused_decode_steps"] == 1
    B = len(lens)
    Wd = (Hq + 2 * Hkv) * D
    fused = torch.empty((B, Wd), dtype=torch.int16, device="cuda")
    fused[:, :Hq * D] = dev_bits(w.q).reshape(B, -1)
    fused[:, Hq * D:(Hq + Hkv) * D] = dev_bits(kn).reshape(B, -1)
    fused[:, (Hq + Hkv) * D:] = dev_bits(vn).reshape(B, -1)
    g = GpuCase(w)
    out = torch.full((B, Hq, D), -1, dtype=torch.int16, device="cuda")
    kvp.kvp_decode_step(g.pool, fused[:, Hq * D:(Hq + Hkv) * D].unflatten(1, (Hkv, D)),
                        fused[:, (Hq + Hkv) * D:].unflatten(1, (Hkv, D)), torch.from_numpy(slots).cuda(),
                        fused[:, :Hq * D].unflatten(1, (Hq, D)), out, Hq, g.bt, g.seq_lens, g.qsl, 1,
                        int(max(lens)), w.scale, True, workspace=g.ws)
    torch.cuda.synchronize()
    bitwise(host_bits(out), out_c, "fused-view decode step output")
    np.testing.assert_array_equal(g.pool_bits(), pool_c)
    # and against the oracle run on the pool after the step's scatter
    opool = oracle_pool(w)
    oracle.reshape_and_cache(opool, kn, vn, slots)
    np.testing.assert_array_equal(g.pool_bits(), opool.storage)
    compare(host_bits(out), oracle_attention(w, opool), "fused-view decode step vs oracle")


@pytest.mark.parametrize("lens,Hq,Hkv,D,ncol", [
    ([1500], 32, 8, 128, 128),           # 376 workgroups of 128 columns: prefill_db_kernel<128>
    ([4100, 4100], 8, 2, 256, 128),      # 516 workgroups of 128 columns: prefill_db_kernel<256>
    ([300, 133], 32, 8, 128, 64),        # few columns: producer / consumer kernel, 64 columns per workgroup
    ([20, 45], 8, 2, 256, 64),           # the same at head_dim 256
    ([900], 16, 2, 512, 64),             # head_dim 512, small grid: wave-pair kernel
    ([2100], 16, 2, 512, 128),           # 264 workgroups of 128 columns: prefill_sb_kernel<512>
], ids=["db128", "db256", "ss128", "ss256", "ws512", "sb512"])
def test_prefill_kernel_per_grid_size(lens, Hq, Hkv, D, ncol):
    """Each prefill kernel the launcher picks by grid size (identified by its
    workgroup count) against the oracle on sampled rows, and every row's
    decode against its prefill row bitwise."""
    w = wl.random_case(97 + D + len(lens), lens, lens, Hq, Hkv, D)
    G = Hq // Hkv
    expect = -(-(w.batch * Hkv * (-(-int(w.max_query_len) * G // ncol))) // 8) * 8
    g, full, _ = _run_and_compare(w, rows=sample_rows(w, 48), what="kernel for %s D=%d" % (lens, D))
    assert kvp.kvp_get_counters()["last_grid_blocks"] == expect
    d = w.decode_view()
    g.set_queries(d.q, d.query_lens)
    bitwise(g.run(), full[w.query_start_loc[1:] - 1], "decode vs prefill last rows (%s, D=%d)" % (lens, D))


@pytest.mark.parametrize("lens,Hq,Hkv,D,ncol", [
    ([600, 550, 500], 8, 1, 128, 64),               # 3 rows, producer / consumer kernel
    ([1500], 24, 3, 128, 128),                      # 3 rows, double-buffered kernel
    ([1700], 40, 5, 128, 256),                      # 5 rows, ping-pong kernel
    ([300, 280, 260, 240, 220], 4, 1, 256, 64),     # 5 rows, producer / consumer kernel, head_dim 256
    ([1400, 1400, 1400], 8, 1, 512, 128),           # 3 rows, single-buffer kernel
    ([700, 600, 500], 8, 1, 512, 64),               # 3 rows, wave-pair kernel
    ([500, 470, 440, 410, 380, 350], 8, 1, 128, 64),   # 6 rows, producer / consumer kernel
], ids=["ss128_3", "db128_3", "pp_5", "ss256_5", "sb512_3", "ws512_3", "ss128_6"])
def test_prefill_workgroup_mapping_covers_every_row(lens, Hq, Hkv, D, ncol):
    """Grids whose rows (sequence x kv head) have more column groups than one
    XCD's share of the grid deal the (row, column group) pairs out over the
    XCDs one by one; with row counts that do not divide 8 an XCD cycles
    through the rows.  Every output row must be written exactly as the
    oracle says: no row left at the NaN fill, sampled rows against the
    oracle, decode against the prefill's last rows, and a reordered batch
    (every workgroup computes a different pair) bitwise equal per sequence."""
    w = wl.random_case(311 + D + len(lens) + Hkv, lens, lens, Hq, Hkv, D)
    G = Hq // Hkv
    cgs = -(-int(w.max_query_len) * G // ncol)
    rows_n = w.batch * Hkv
    assert rows_n % 8 != 0 and cgs > -(-rows_n * cgs // 8), "the case must take the dealt-out mapping"
    g, full, _ = _run_and_compare(w, rows=_rows(group_rows(w, 8, groups=("first", "last")), sample_rows(w, 40)),
                                  what="mapping %s Hkv=%d D=%d" % (lens, Hkv, D))
    assert kvp.kvp_get_counters()["last_grid_blocks"] == -(-(rows_n * cgs) // 8) * 8
    assert not np.isnan(bf16_to_f32(full)).any(), "some output row was never written"
    d = w.decode_view()
    g.set_queries(d.q, d.query_lens)
    bitwise(g.run(), full[w.query_start_loc[1:] - 1], "mapping: decode vs prefill last rows")
    if w.batch > 1:
        order = list(range(w.batch))[::-1]
        qsl = w.query_start_loc
        q = np.concatenate([w.q[qsl[b]:qsl[b + 1]] for b in order])
        g.set_queries(q, [int(w.query_lens[b]) for b in order], block_tables=w.block_tables[order],
                      seq_lens=w.seq_lens[order])
        rev = g.run()
        exp = np.concatenate([full[qsl[b]:qsl[b + 1]] for b in order])
        bitwise(rev, exp, "mapping: reversed batch")


def _random_shape(rng):
    D = int(rng.choice([128, 256, 512]))
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    B = int(rng.integers(1, 5))
    max_len = 700 if D == 512 else 1500
    seq = [int(x) for x in rng.integers(1, max_len, size=B)]
    ql = []
    for L in seq:
        kind = int(rng.integers(0, 4))
        ql.append({0: 1, 1: L, 2: min(L, max(1, 16 // G)), 3: int(rng.integers(1, L + 1))}[kind])
    return seq, ql, Hkv * G, Hkv, D, bool(rng.integers(0, 4) > 0)


@pytest.mark.parametrize("seed", range(12))
def test_random_shape_sweep(seed):
    """Seeded random shapes (head dims, group sizes 1..16, ragged lengths, q_len * G around
    the split-KV threshold, causal and not): sampled rows against the oracle, with and
    without a workspace (split-KV for short rows, or every row through a prefill kernel),
    which must give the same bits."""
    rng = np.random.default_rng(1000 + seed)
    seq, ql, Hq, Hkv, D, causal = _random_shape(rng)
    w = wl.random_case(2000 + seed, seq, ql, Hq, Hkv, D, causal=causal)
    print("random shape", seq, ql, Hq, Hkv, D, causal, flush=True)
    rows = sample_rows(w, 24, seed)
    g, out, _ = _run_and_compare(w, rows=rows, what="random %d" % seed)
    if w.batch > 1 and int(w.max_query_len) * (Hq // Hkv) > 16:
        bitwise(g.run(use_workspace=False), out, "random %d: with vs without workspace" % seed)


# ------------------------------------------------------------ score shapes that stress the fold

def _shaped(seed, lens, Hq, Hkv, D, slope, qk_scale=0.5):
    """Full causal prefills whose scores follow a trend along the key
    position: dim 0 of every key is slope * position and dim 0 of every query
    is 4, the other dims N(0, qk_scale^2); V ~ N(0, 1).  With the scale
    1/sqrt(D), slope = 0.37 raises the running maximum by ~24 log2 units per
    128-key tile (the state's reference moves on every tile and ACC is
    rescaled each time); a negative slope leaves the maximum in the first
    tile (later tiles fold with tiny factors)."""
    w = wl.random_case(seed, lens, lens, Hq, Hkv, D)
    pos = np.concatenate([np.arange(L, dtype=np.float32) for L in lens])
    rng = np.random.default_rng(seed + 100)
    k = rng.standard_normal((pos.size, Hkv, D), dtype=np.float32) * np.float32(qk_scale)
    k[:, :, 0] = (slope * pos)[:, None]
    q = rng.standard_normal(w.q.shape, dtype=np.float32) * np.float32(qk_scale)
    q[:, :, 0] = 4.0
    w.k = wl.to_bf16_bits(k)
    w.q = wl.to_bf16_bits(q)
    return w


@pytest.mark.parametrize("slope,D,Hq,Hkv", [(0.37, 128, 8, 2), (-0.37, 128, 8, 2), (0.37, 512, 16, 2),
                                            (-0.37, 256, 8, 2)])
def test_trending_scores(slope, D, Hq, Hkv):
    """Rising scores (the reference moves and ACC is rescaled on every tile)
    and falling scores (every later tile folds with a vanishing factor):
    sampled rows match the oracle, and decode rows equal the prefill's last
    rows bitwise."""
    w = _shaped(61, [1500, 700, 129], Hq, Hkv, D, slope)
    g, full, dec = _prefill_then_decode(w)
    rows = sample_rows(w, 48)
    compare(full[rows], oracle_attention(w, oracle_pool(w), rows=rows), "trend %g D%d" % (slope, D))
    bitwise(dec, full[w.query_start_loc[1:] - 1], "trend %g D%d decode vs prefill" % (slope, D))


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 8, 2), (512, 16, 2)])
def test_peaked_scores(D, Hq, Hkv):
    """Q and K ~ N(0, 9) (score spread ~9 natural-log units: nearly one-hot
    softmax rows), V ~ N(0, 1): sampled rows match the oracle and decode rows
    equal the prefill's last rows bitwise."""
    w = wl.random_case(67, [1100, 333], [1100, 333], Hq, Hkv, D)
    rng = np.random.default_rng(168)
    w.k = wl.to_bf16_bits(rng.standard_normal((w.k.shape), dtype=np.float32) * np.float32(3.0))
    w.q = wl.to_bf16_bits(rng.standard_normal((w.q.shape), dtype=np.float32) * np.float32(3.0))
    g, full, dec = _prefill_then_decode(w)
    rows = sample_rows(w, 48)
    compare(full[rows], oracle_attention(w, oracle_pool(w), rows=rows), "peaked D%d" % D)
    bitwise(dec, full[w.query_start_loc[1:] - 1], "peaked D%d decode vs prefill" % D)
