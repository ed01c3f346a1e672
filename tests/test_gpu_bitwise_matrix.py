"""The bit-pattern matrix of "fix(rocm): stabilize direct paged CK attention
for bitwise R/R" (Additional checks): full prefill against suffix chunks and
against decode, outputs and LSE, at KV lengths 513 / 4096 / 4171 / 7168,
batches of 4 and of 1, query tails full / 128 / 17 / 1, on separate,
interleaved and >2 GB interleaved pools, with reversed or shuffled pages.
Every comparison is bitwise (mismatch_count = 0); one full prefill per pool
is also checked against the oracle on sampled rows.

A pool that crosses 2**32 bytes (the stress size of the ragged workload)
gives the same bits as the same pages in a compact pool.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_bf16_amd as kvp
from paged_kv_cache_bf16_amd import workloads as wl
from harness import GpuCase, bitwise, compare, oracle_attention, oracle_pool, sample_rows

pytestmark = pytest.mark.gpu

LENS = [513, 4096, 4171, 7168]
Hq, Hkv, D = 8, 2, 128


def _pool_layout(kind, rng):
    """(block_tables [4, W], num_blocks, interleaved) for one pool kind."""
    npages = [-(-L // 16) for L in LENS]
    total, W = sum(npages), max(npages)
    if kind == "separate-reversed":
        nb = total + 5
        phys = (nb - 1 - np.arange(total)).astype(np.int32)
        interleaved = False
    elif kind == "interleaved-shuffled":
        nb = total + 5
        phys = rng.permutation(nb)[:total].astype(np.int32)
        interleaved = True
    elif kind == "interleaved-over-2gb":
        nb = wl.RAGGED_POOL_BLOCKS                     # 2.29 GB; pages above byte 2**31, one below
        block_bytes = 2 * 2 * 16 * D * 2
        first_high = 2 ** 31 // block_bytes + 1
        high = rng.choice(np.arange(first_high, nb), size=total - 1, replace=False)
        phys = rng.permutation(np.concatenate([high, [int(rng.integers(0, first_high))]])).astype(np.int32)
        interleaved = True
    else:
        raise ValueError(kind)
    bt = np.zeros((4, W), np.int32)
    off = 0
    for b, n in enumerate(npages):
        bt[b, :n] = phys[off:off + n]
        bt[b, n:] = phys[off + n - 1]
        off += n
    return bt, nb, interleaved


def _tail_queries(w, tails):
    qsl = w.query_start_loc
    q = np.concatenate([w.q[qsl[b + 1] - t:qsl[b + 1]] for b, t in enumerate(tails)])
    rows = np.concatenate([np.arange(qsl[b + 1] - t, qsl[b + 1]) for b, t in enumerate(tails)])
    return q, rows


@pytest.mark.parametrize("kind", ["separate-reversed", "interleaved-shuffled", "interleaved-over-2gb"])
def test_bit_pattern_matrix(kind):
    print("bit-pattern matrix", kind, flush=True)
    rng = np.random.default_rng(4242 + len(kind))
    bt, nb, interleaved = _pool_layout(kind, rng)
    w = wl.build("matrix-" + kind, LENS, LENS, Hq, Hkv, D, bt, nb, interleaved=interleaved, seed=4300 + len(kind))
    g = GpuCase(w)
    if kind == "interleaved-over-2gb":
        assert kvp.kv_pool_span_bytes(g.pool) > 2 ** 31
    full, full_lse = g.run_lse()
    rows = sample_rows(w, 48, seed=7)
    compare(full[rows], oracle_attention(w, oracle_pool(w), rows=rows), "matrix %s full prefill" % kind)
    n_checked = 0
    for tails in ([LENS[0], 128, 17, 1], [128] * 4, [17] * 4, [1] * 4):
        q, rows = _tail_queries(w, tails)
        # B = 4: the suffix chunks (tail 1: decode) give the full prefill's rows and lse
        g.set_queries(q, tails)
        out, lse = g.run_lse()
        bitwise(out, full[rows], "%s B4 tails %s vs full" % (kind, tails))
        assert np.array_equal(lse.view(np.uint32), full_lse[rows].view(np.uint32)), \
            "%s B4 tails %s: lse differs from the full prefill" % (kind, tails)
        n_checked += 2
        # B = 1: each row alone gives the same bits
        off = 0
        for b, t in enumerate(tails):
            g.set_queries(q[off:off + t], [t], block_tables=bt[b:b + 1], seq_lens=[LENS[b]])
            o1, l1 = g.run_lse()
            bitwise(o1, out[off:off + t], "%s B1 row %d tail %d vs B4" % (kind, b, t))
            assert np.array_equal(l1.view(np.uint32), lse[off:off + t].view(np.uint32))
            off += t
            n_checked += 2
        g.set_queries(w.q, w.query_lens)
    print("%s: %d bitwise comparisons, mismatch_count=0" % (kind, n_checked), flush=True)


def test_pool_over_4gb_matches_compact_pool():
    """Pages placed above byte 2**32 of a 4.9 GB interleaved pool (one page
    below 2**31): the same bits as the same pages in a compact pool, and the
    compact run within tolerance of the oracle ("fix(rocm): stabilize direct
    paged CK attention for bitwise R/R", Changes: 64-bit addressing when a
    K/V view spans more than 2 GB)."""
    lens, q_lens = [513, 4171, 7168], [513, 17, 1]
    npages = [-(-L // 16) for L in lens]
    total = sum(npages)
    nb_big = 300_000                                     # x 16 KB per block = 4.9 GB
    block_bytes = 2 * 2 * 16 * D * 2
    rng = np.random.default_rng(77)
    first_4g = 2 ** 32 // block_bytes + 1
    high = rng.choice(np.arange(first_4g, nb_big), size=total - 1, replace=False)
    phys_big = rng.permutation(np.concatenate([high, [3]])).astype(np.int32)
    W = max(npages)
    bt_big = np.zeros((3, W), np.int32)
    bt_small = np.zeros((3, W), np.int32)
    off = 0
    for b, n in enumerate(npages):
        bt_big[b, :n] = phys_big[off:off + n]
        bt_small[b, :n] = np.arange(off, off + n)
        off += n
    w_big = wl.build("over4g", lens, q_lens, Hq, Hkv, D, bt_big, nb_big, interleaved=True, seed=91)
    w_small = wl.build("over4g-compact", lens, q_lens, Hq, Hkv, D, bt_small, total, interleaved=True, seed=91)
    assert np.array_equal(w_big.k, w_small.k) and np.array_equal(w_big.q, w_small.q)
    print("pool over 4 GB", flush=True)
    g_small = GpuCase(w_small)
    small = g_small.run()
    compare(small, oracle_attention(w_small, oracle_pool(w_small)), "compact pool")
    del g_small
    g_big = GpuCase(w_big)
    assert kvp.kv_pool_span_bytes(g_big.pool) > 2 ** 32
    assert int(bt_big.max()) * block_bytes > 2 ** 32
    bitwise(g_big.run(), small, "pool over 4 GB vs compact pool")
    d = w_big.decode_view()
    g_big.set_queries(d.q, d.query_lens)
    dec = g_big.run()
    bitwise(dec, small[w_small.query_start_loc[1:] - 1], "decode over 4 GB vs compact prefill last rows")
    del g_big
    torch.cuda.empty_cache()
