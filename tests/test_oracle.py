"""Pins for the CPU oracle (runs without a GPU).

The oracle is checked against things other than itself: the worked example
printed on the composition page, a library routine (torch's float64
scaled_dot_product_attention on the dense, un-paged sequence), closed forms
(length-1 KV, identical keys, constant V, two keys with one-hot V, a peaked
key), invariants (physical page permutation, batch independence, suffix rows
equal full-prefill rows) and negative controls (the rejected slot formula, a
swap of two in-range logical blocks).  The pool layout is checked against an
independent numpy reshape/transpose of the same layout definition.
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from paged_kv_cache_bf16_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_worked_example():
    vals = {}
    with open(os.path.join(GOLDEN, "composition_worked_example.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *rest = line.split()
            vals[key] = rest
    return vals


def make_pool(w: wl.Workload, fill_bits=0):
    return oracle.Pool(w.num_blocks, w.num_kv_heads, w.head_dim, interleaved=w.interleaved,
                       fill_bits=fill_bits)


def oracle_run(w: wl.Workload, rows=None, fill_bits=0, slots=None):
    pool = make_pool(w, fill_bits)
    oracle.reshape_and_cache(pool, w.k, w.v, w.slot_mapping if slots is None else slots)
    out = oracle.paged_attention(w.q, pool, w.block_tables, w.seq_lens, w.query_start_loc,
                                 w.num_q_heads, w.scale, w.causal, rows=rows)
    return out, pool


def sdpa_reference(w: wl.Workload):
    """float64 torch SDPA per sequence on the dense logical K/V (no paging)."""
    outs = []
    kf = torch.from_numpy(oracle.bf16_bits_to_f32(w.k)).double()
    vf = torch.from_numpy(oracle.bf16_bits_to_f32(w.v)).double()
    qf = torch.from_numpy(oracle.bf16_bits_to_f32(w.q)).double()
    qsl = w.query_start_loc
    koff = 0
    for b in range(w.batch):
        L, n = int(w.seq_lens[b]), int(w.query_lens[b])
        kb = kf[koff:koff + L].permute(1, 0, 2)[None]          # [1, Hkv, L, D]
        vb = vf[koff:koff + L].permute(1, 0, 2)[None]
        koff += L
        qb = qf[qsl[b]:qsl[b + 1]].permute(1, 0, 2)            # [Hq, n, D]
        if n == 0:
            continue
        if w.causal:
            # bottom-right alignment == top-left causal over the full sequence,
            # with the suffix queries placed at positions L-n .. L-1
            full = torch.zeros(w.num_q_heads, L, w.head_dim, dtype=torch.float64)
            full[:, L - n:] = qb
            o = F.scaled_dot_product_attention(full[None], kb, vb, is_causal=True, scale=w.scale,
                                               enable_gqa=True)[0, :, L - n:]
        else:
            o = F.scaled_dot_product_attention(qb[None], kb, vb, scale=w.scale, enable_gqa=True)[0]
        outs.append(o.permute(1, 0, 2))
    return torch.cat(outs).numpy()


# ---------------------------------------------------------------- worked example

def test_worked_example_slots_and_pool():
    ex = load_worked_example()
    bs = int(ex["block_size"][0])
    table = [int(x) for x in ex["block_table"]]
    expect = np.array([int(x) for x in ex["slots"]], np.int64)
    w = wl.tiny()
    assert bs == wl.BLOCK_SIZE and w.block_tables[0].tolist() == table
    assert int(ex["num_tokens"][0]) == w.seq_lens[0] == expect.shape[0]
    np.testing.assert_array_equal(w.slot_mapping, expect)
    _, pool = oracle_run(w)
    # the oracle must have placed token i at the printed physical slot
    kp, vp = layout_views(pool)
    for i, s in enumerate(expect):
        np.testing.assert_array_equal(kp[s // 16, s % 16], w.k[i])
        np.testing.assert_array_equal(vp[s // 16, s % 16], w.v[i])


def test_worked_example_matches_dense_and_bad_mapping_fails():
    w = wl.tiny()
    ref = sdpa_reference(w)
    out, _ = oracle_run(w)
    np.testing.assert_allclose(out, ref, atol=2e-5, rtol=0)
    # negative control: the rejected mapping (i*7+3)%64 writes slots the table
    # does not read, so the composition must disagree with the dense result
    bad = (np.arange(20, dtype=np.int64) * 7 + 3) % 64
    out_bad, _ = oracle_run(w, slots=bad)
    assert np.abs(out_bad - ref).max() > 0.1


def test_swap_of_in_range_blocks_changes_prefill():
    """Anti-vacuity: swapping logical blocks 0 and 1 (both hold real tokens) must change
    causal prefill rows, while the dense reference stays put."""
    w = wl.tiny()
    out, pool = oracle_run(w)
    bt = w.block_tables.copy()
    bt[0, [0, 1]] = bt[0, [1, 0]]
    out2 = oracle.paged_attention(w.q, pool, bt, w.seq_lens, w.query_start_loc, w.num_q_heads,
                                  w.scale, True)
    assert np.abs(out2 - out).max() > 0.1
    # a swap of columns past the logical range is vacuous: the output is bitwise unchanged
    bt3 = w.block_tables.copy()
    bt3[0, [2, 3]] = bt3[0, [3, 2]]
    out3 = oracle.paged_attention(w.q, pool, bt3, w.seq_lens, w.query_start_loc, w.num_q_heads,
                                  w.scale, True)
    np.testing.assert_array_equal(out3, out)


# ---------------------------------------------------------------- pool layout

def layout_views(pool: oracle.Pool):
    """Independent numpy view of the documented page layout: returns K and V as
    [num_blocks, 16, Hkv, D] arrays of BF16 bits."""
    nb, H, D = pool.num_blocks, pool.num_kv_heads, pool.head_dim
    st = pool.storage
    if pool.interleaved:
        blocks = st.reshape(nb, 2, H * 16 * D)
        kraw, vraw = blocks[:, 0], blocks[:, 1]
    else:
        kraw = st[:nb * H * 16 * D].reshape(nb, H * 16 * D)
        vraw = st[nb * H * 16 * D:].reshape(nb, H * 16 * D)
    k = kraw.reshape(nb, H, D // 8, 16, 8).transpose(0, 3, 1, 2, 4).reshape(nb, 16, H, D)
    v = vraw.reshape(nb, H, D, 16).transpose(0, 3, 1, 2)
    return k, v


@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("D", [128, 256, 512])
def test_layout_and_untouched_slots(interleaved, D):
    rng = np.random.default_rng(7)
    nb, H = 6, 2
    pool = oracle.Pool(nb, H, D, interleaved=interleaved, fill_bits=0x7FC1)  # NaN poison
    T = 37
    slots = rng.choice(nb * 16, size=T, replace=False).astype(np.int64)
    slots[5] = -1                                   # negative slots are skipped
    k = rng.integers(0, 2 ** 16, size=(T, H, D), dtype=np.uint16)
    v = rng.integers(0, 2 ** 16, size=(T, H, D), dtype=np.uint16)
    oracle.reshape_and_cache(pool, k, v, slots)
    kp, vp = layout_views(pool)
    written = np.zeros((nb, 16), bool)
    for i, s in enumerate(slots):
        if s < 0:
            continue
        written[s // 16, s % 16] = True
        np.testing.assert_array_equal(kp[s // 16, s % 16], k[i])
        np.testing.assert_array_equal(vp[s // 16, s % 16], v[i])
    assert (kp[~written] == 0x7FC1).all() and (vp[~written] == 0x7FC1).all()


def test_duplicate_or_out_of_range_slot_rejected_without_writes():
    pool = oracle.Pool(2, 1, 128, fill_bits=0x1234)
    k = np.zeros((3, 1, 128), np.uint16)
    for slots in ([0, 1, 1], [0, 1, 32]):
        with pytest.raises(oracle.OracleError):
            oracle.reshape_and_cache(pool, k, k, np.array(slots, np.int64))
        assert (pool.storage == 0x1234).all()


# ---------------------------------------------------------------- library routine

@pytest.mark.parametrize("case", [
    dict(seq=[1, 17, 40], q=[1, 17, 3], Hq=4, Hkv=1, D=128, causal=True),
    dict(seq=[33, 130], q=[33, 5], Hq=8, Hkv=2, D=128, causal=True),
    dict(seq=[20, 64], q=[2, 64], Hq=8, Hkv=2, D=256, causal=False),
    dict(seq=[45], q=[45], Hq=16, Hkv=2, D=512, causal=True),
    dict(seq=[300, 1, 129], q=[1, 1, 1], Hq=6, Hkv=3, D=128, causal=True),
])
def test_oracle_matches_float64_sdpa(case):
    w = wl.random_case(11, case["seq"], case["q"], case["Hq"], case["Hkv"], case["D"],
                       causal=case["causal"])
    out, _ = oracle_run(w)
    ref = sdpa_reference(w)
    err = np.abs(out - ref)
    assert err.max() < 3e-5, err.max()


def test_named_workloads_match_sdpa_on_sampled_rows():
    for w in (wl.tiny(), wl.random_case(3, [513, 200], [513, 17], 8, 2, 128)):
        ref = sdpa_reference(w)
        rows = np.unique(np.r_[0, w.q.shape[0] - 1, np.arange(0, w.q.shape[0], 37)])
        out, _ = oracle_run(w, rows=rows)
        assert np.abs(out - ref[rows]).max() < 3e-5


# ---------------------------------------------------------------- closed forms

def _single(q, k, v, scale, causal=False):
    """Run the oracle on one sequence given float arrays q [n,Hq,D], k/v [L,Hkv,D]."""
    L, Hkv, D = k.shape
    n, Hq, _ = q.shape
    npg = (L + 15) // 16
    bt = np.arange(npg, dtype=np.int32)[::-1].copy()[None]    # reversed pages
    pool = oracle.Pool(npg, Hkv, D)
    slots = (bt[0, np.arange(L) // 16].astype(np.int64) * 16 + np.arange(L) % 16)
    oracle.reshape_and_cache(pool, wl.to_bf16_bits(k), wl.to_bf16_bits(v), slots)
    return oracle.paged_attention(wl.to_bf16_bits(q), pool, bt, [L], [0, n], Hq, scale, causal)


def _bf(x):
    return oracle.bf16_bits_to_f32(wl.to_bf16_bits(np.asarray(x, np.float32)))


def test_length_one_kv_returns_v_exactly():
    rng = np.random.default_rng(1)
    q, k, v = (_bf(rng.standard_normal(s)) for s in ((1, 4, 128), (1, 2, 128), (1, 2, 128)))
    out = _single(q, k, v, 1 / math.sqrt(128))
    np.testing.assert_array_equal(out[0, :2], np.broadcast_to(v[0, 0], (2, 128)))
    np.testing.assert_array_equal(out[0, 2:], np.broadcast_to(v[0, 1], (2, 128)))


def test_causal_row_zero_is_v0():
    rng = np.random.default_rng(2)
    L = 40
    q, k, v = (_bf(rng.standard_normal(s)) for s in ((L, 2, 128), (L, 1, 128), (L, 1, 128)))
    out = _single(q, k, v, 0.1, causal=True)
    np.testing.assert_array_equal(out[0, 0], v[0, 0])


def test_identical_keys_give_mean_of_v():
    rng = np.random.default_rng(3)
    L = 300
    k = np.broadcast_to(_bf(rng.standard_normal((1, 1, 128))), (L, 1, 128)).copy()
    v = _bf(rng.standard_normal((L, 1, 128)))
    q = _bf(rng.standard_normal((1, 2, 128)))
    out = _single(q, k, v, 1 / math.sqrt(128))
    mean = v[:, 0].astype(np.float64).mean(0)
    np.testing.assert_allclose(out[0, 0], mean, atol=L * 2 ** -22)
    np.testing.assert_allclose(out[0, 1], mean, atol=L * 2 ** -22)


def test_constant_v_returns_constant():
    rng = np.random.default_rng(4)
    L = 77
    k = _bf(rng.standard_normal((L, 1, 128)))
    v = np.full((L, 1, 128), 1.75, np.float32)
    q = _bf(rng.standard_normal((3, 1, 128)))
    out = _single(q, k, v, 1 / math.sqrt(128))
    np.testing.assert_allclose(out, 1.75, rtol=L * 2 ** -23)


def test_two_keys_one_hot_v_is_sigmoid():
    rng = np.random.default_rng(5)
    q = _bf(rng.standard_normal((1, 1, 128)))
    k = _bf(rng.standard_normal((2, 1, 128)))
    v = np.zeros((2, 1, 128), np.float32)
    v[0, 0, 0] = 1.0
    v[1, 0, 1] = 1.0
    scale = 1 / math.sqrt(128)
    out = _single(q, k, v, scale)
    s = (k[:, 0].astype(np.float64) @ q[0, 0].astype(np.float64)) * scale
    sig = 1 / (1 + math.exp(-(s[0] - s[1])))
    np.testing.assert_allclose(out[0, 0, 0], sig, atol=1e-6)
    np.testing.assert_allclose(out[0, 0, 1], 1 - sig, atol=1e-6)
    assert (out[0, 0, 2:] == 0).all()


def test_softmax_rows_sum_to_one():
    rng = np.random.default_rng(6)
    L = 513
    k = _bf(rng.standard_normal((L, 2, 128)) * 3)
    q = _bf(rng.standard_normal((5, 4, 128)) * 3)
    v = np.ones((L, 2, 128), np.float32)
    out = _single(q, k, v, 1 / math.sqrt(128), causal=True)
    assert np.abs(out - 1).max() <= L * 2 ** -23


def test_peaked_key_returns_its_value():
    rng = np.random.default_rng(8)
    L = 200
    k = _bf(rng.standard_normal((L, 1, 128)))
    q = _bf(rng.standard_normal((1, 1, 128)))
    k[123, 0] = q[0, 0] * 4
    v = _bf(rng.standard_normal((L, 1, 128)))
    out = _single(q, k, v, 1 / math.sqrt(128))
    np.testing.assert_allclose(out[0, 0], v[123, 0], atol=2e-2)
    assert np.abs(out[0, 0] - v[123, 0]).max() < np.abs(v[123, 0]).max()


# ---------------------------------------------------------------- invariants

def test_page_permutation_is_bitwise_neutral():
    w = wl.random_case(21, [200, 77], [200, 3], 8, 2, 128, spare_blocks=5)
    out, _ = oracle_run(w)
    rng = np.random.default_rng(22)
    perm = rng.permutation(w.num_blocks).astype(np.int32)      # old block -> new block
    bt2 = perm[w.block_tables]
    w2 = wl.build("perm", w.seq_lens, w.query_lens, 8, 2, 128, bt2, w.num_blocks, seed=22)
    # same values, new physical placement
    w2.k, w2.v, w2.q = w.k, w.v, w.q
    out2, _ = oracle_run(w2)
    np.testing.assert_array_equal(out, out2)


def test_batch_independence_and_suffix_rows():
    w = wl.random_case(31, [150, 90], [150, 90], 4, 1, 128)
    out, pool = oracle_run(w)
    # sequence 1 alone, through the same pool
    bt1 = w.block_tables[1:2]
    o1 = oracle.paged_attention(w.q[150:], pool, bt1, w.seq_lens[1:], [0, 90], 4, w.scale, True)
    np.testing.assert_array_equal(o1, out[150:])
    # its last 7 queries as a suffix chunk give the same rows
    o2 = oracle.paged_attention(w.q[240 - 7:], pool, bt1, w.seq_lens[1:], [0, 7], 4, w.scale, True)
    np.testing.assert_array_equal(o2, out[240 - 7:])
    # and its last query alone (decode) gives the last row
    o3 = oracle.paged_attention(w.q[239:], pool, bt1, w.seq_lens[1:], [0, 1], 4, w.scale, True)
    np.testing.assert_array_equal(o3, out[239:])


def test_inconsistent_metadata_rejected():
    w = wl.tiny()
    pool = make_pool(w)
    with pytest.raises(oracle.OracleError):       # q_len > seq_len
        oracle.paged_attention(w.q, pool, w.block_tables, [10], [0, 20], 8, w.scale)
    with pytest.raises(oracle.OracleError):       # table entry out of range
        oracle.paged_attention(w.q, pool, np.array([[3, 9, 2, 0]], np.int32), [20], [0, 20], 8,
                               w.scale)


# ---------------------------------------------------------------- page-table prep

def test_prepare_tables_worked_cases():
    imax = np.iinfo(np.int32).max
    bt = np.array([[5, 7, -1, imax, -1, imax, -1, imax, -1],
                   [-1, -1, -1, -1, -1, -1, -1, -1, -1],
                   [1, 2, 3, 4, 5, 6, 7, 8, 9]], np.int32)
    out = oracle.prepare_block_tables(bt, [20, 0, 144], num_blocks=10)
    assert out.shape == (3, 16)
    assert out[0].tolist() == [5, 7] + [7] * 14
    assert out[1].tolist() == [0] * 16
    assert out[2].tolist() == list(range(1, 10)) + [9] * 7
    with pytest.raises(oracle.OracleError):        # active entry out of range
        oracle.prepare_block_tables(bt, [20, 0, 144], num_blocks=9)
    with pytest.raises(oracle.OracleError):        # table too narrow for seq_len
        oracle.prepare_block_tables(bt, [20, 0, 145], num_blocks=10)


# ---------------------------------------------------------------- LSE output and the merge of two results

def _dense_lse_out(q, k, v, scale, visible):
    """float64 torch reference over dense K/V: q [n,H,D], k/v [L,H,D] (heads already
    matched), visible [n,L] bool.  Returns (out [n,H,D], lse [n,H]) via torch.logsumexp."""
    qt, kt, vt = (torch.from_numpy(np.asarray(x, np.float64)).permute(1, 0, 2) for x in (q, k, v))
    s = torch.matmul(qt, kt.transpose(1, 2)) * scale                  # [H, n, L]
    s = s.masked_fill(~torch.from_numpy(visible)[None], float("-inf"))
    lse = torch.logsumexp(s, -1)                                      # [H, n]
    out = torch.matmul(torch.softmax(s, -1), vt)
    return out.permute(1, 0, 2).numpy(), lse.T.numpy()


def test_oracle_lse_matches_torch_logsumexp():
    w = wl.random_case(21, [1, 40, 300], [1, 40, 7], 8, 2, 128, causal=True)
    pool = make_pool(w)
    oracle.reshape_and_cache(pool, w.k, w.v, w.slot_mapping)
    out, lse = oracle.paged_attention(w.q, pool, w.block_tables, w.seq_lens, w.query_start_loc,
                                      w.num_q_heads, w.scale, True, return_lse=True)
    G = w.num_q_heads // w.num_kv_heads
    koff = 0
    for b in range(w.batch):
        L, n, q0 = int(w.seq_lens[b]), int(w.query_lens[b]), int(w.query_start_loc[b])
        k = np.repeat(oracle.bf16_bits_to_f32(w.k[koff:koff + L]), G, axis=1)
        v = np.repeat(oracle.bf16_bits_to_f32(w.v[koff:koff + L]), G, axis=1)
        koff += L
        pos = L - n + np.arange(n)
        vis = np.arange(L)[None] <= pos[:, None]
        ro, rl = _dense_lse_out(oracle.bf16_bits_to_f32(w.q[q0:q0 + n]), k, v, w.scale, vis)
        assert np.abs(lse[q0:q0 + n] - rl).max() < 1e-5
        assert np.abs(out[q0:q0 + n] - ro).max() < 3e-5


def test_lse_closed_forms():
    rng = np.random.default_rng(22)
    scale = 1 / math.sqrt(128)
    q, k, v = (_bf(rng.standard_normal(s)) for s in ((1, 1, 128), (1, 1, 128), (1, 1, 128)))
    L = 1
    npg = 1
    pool = oracle.Pool(npg, 1, 128)
    oracle.reshape_and_cache(pool, wl.to_bf16_bits(k), wl.to_bf16_bits(v), np.array([0]))
    _, lse = oracle.paged_attention(wl.to_bf16_bits(q), pool, np.zeros((1, 1), np.int32), [L], [0, 1], 1,
                                    scale, False, return_lse=True)
    # one key: the LSE is that key's scaled score
    assert abs(lse[0, 0] - scale * float(q[0, 0].astype(np.float64) @ k[0, 0].astype(np.float64))) < 1e-6
    # n identical keys: score + log(n)
    n = 300
    kk = np.broadcast_to(k, (n, 1, 128)).copy()
    vv = _bf(rng.standard_normal((n, 1, 128)))
    npg = (n + 15) // 16
    pool = oracle.Pool(npg, 1, 128)
    oracle.reshape_and_cache(pool, wl.to_bf16_bits(kk), wl.to_bf16_bits(vv), np.arange(n))
    _, lse_n = oracle.paged_attention(wl.to_bf16_bits(q), pool, np.arange(npg, dtype=np.int32)[None], [n],
                                      [0, 1], 1, scale, False, return_lse=True)
    assert abs(lse_n[0, 0] - (lse[0, 0] + math.log(n))) < 1e-5


def test_merge_of_disjoint_key_sets_is_attention_over_their_union():
    rng = np.random.default_rng(23)
    n, H, D, L = 5, 3, 64, 90
    q, k, v = (rng.standard_normal(s) for s in ((n, H, D), (L, H, D), (L, H, D)))
    for split in (1, 37, 89):
        vis = np.ones((n, L), bool)
        full_o, full_l = _dense_lse_out(q, k, v, 0.2, vis)
        oa, la = _dense_lse_out(q, k[:split], v[:split], 0.2, vis[:, :split])
        ob, lb = _dense_lse_out(q, k[split:], v[split:], 0.2, vis[:, split:])
        mo, ml = oracle.merge_states(oa, la, ob, lb)
        assert np.abs(mo - full_o).max() < 1e-12 and np.abs(ml - full_l).max() < 1e-12
        # the order of the two sides does not matter
        mo2, ml2 = oracle.merge_states(ob, lb, oa, la)
        assert np.abs(mo2 - mo).max() < 1e-14 and np.abs(ml2 - ml).max() < 1e-14


def test_merge_special_cases():
    rng = np.random.default_rng(24)
    a = rng.standard_normal((4, 2, 16))
    la = rng.standard_normal((4, 2)) * 5
    nan = np.full_like(a, np.nan)
    ninf = np.full_like(la, -np.inf)
    # an empty side contributes nothing, whatever its output holds
    mo, ml = oracle.merge_states(a, la, nan, ninf)
    np.testing.assert_array_equal(mo, a)
    np.testing.assert_array_equal(ml, la)
    mo, ml = oracle.merge_states(nan, ninf, a, la)
    np.testing.assert_array_equal(mo, a)
    # both empty: zero output, -inf LSE
    mo, ml = oracle.merge_states(nan, ninf, nan, ninf)
    assert (mo == 0).all() and (ml == -np.inf).all()
    # equal LSE: the mean of the outputs, LSE + log 2
    b = rng.standard_normal(a.shape)
    mo, ml = oracle.merge_states(a, la, b, la)
    np.testing.assert_allclose(mo, (a + b) / 2, rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(ml, la + math.log(2), rtol=1e-15)
    # a far smaller LSE leaves the other side (up to its weight exp(-diff))
    mo, ml = oracle.merge_states(a, la, b, la - 60)
    np.testing.assert_allclose(mo, a, atol=1e-25 + 1e-20 * np.abs(b).max())


def test_chunked_prefill_by_merging_prefix_and_chunk():
    """Prefix keys (all visible, non-causal) merged with the chunk's own keys
    (causal) equal a causal prefill over the whole row."""
    w = wl.random_case(25, [96 + 40], [40], 8, 2, 128, causal=True)
    pool = make_pool(w)
    oracle.reshape_and_cache(pool, w.k, w.v, w.slot_mapping)
    full = oracle.paged_attention(w.q, pool, w.block_tables, w.seq_lens, w.query_start_loc,
                                  w.num_q_heads, w.scale, True)
    oa, la = oracle.paged_attention(w.q, pool, w.block_tables, [96], [0, 40], w.num_q_heads, w.scale,
                                    False, return_lse=True)
    ob, lb = oracle.paged_attention(w.q, pool, w.block_tables[:, 96 // 16:], [40], [0, 40], w.num_q_heads,
                                    w.scale, True, return_lse=True)
    mo, _ = oracle.merge_states(oa, la, ob, lb)
    assert np.abs(mo - full).max() < 3e-6
