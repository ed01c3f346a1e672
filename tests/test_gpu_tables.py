"""kv_prepare_block_tables_device: the page-table preparation ("fix(rocm):
stabilize direct paged CK attention for bitwise R/R", Changes: pad page
tables to complete KV tiles, sanitise unused columns of active and inactive
rows) run on the GPU from a device table.  Its output must equal the host
version's and the oracle's entry for entry on every table they accept; rows
they reject are flagged in the status word and written sanitised; attention
over a device-prepared table gives the host-prepared call's bits, also from
a captured graph replayed with new tables."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_bf16_amd as kvp
from paged_kv_cache_bf16_amd import workloads as wl

from harness import GpuCase, bitwise, host_bits

pytestmark = pytest.mark.gpu


def _random_table(rng, B, W, nb):
    sl = rng.integers(0, W * 16 + 1, size=B).astype(np.int32)
    sl[rng.random(B) < 0.2] = 0                                   # inactive rows
    bt = rng.integers(-7, nb + 7, size=(B, W)).astype(np.int32)   # garbage past each row's pages
    for b in range(B):
        n = (int(sl[b]) + 15) // 16
        bt[b, :n] = rng.integers(0, nb, size=n)
    return bt, sl


def _device_prep(pool, bt, sl):
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = kvp.kv_prepare_block_tables_device(pool, torch.from_numpy(bt).cuda(), torch.from_numpy(sl).cuda(),
                                             status=status)
    torch.cuda.synchronize()
    return out.cpu().numpy(), int(status.item())


@pytest.mark.parametrize("B,W", [(1, 1), (5, 9), (64, 37), (300, 8), (7, 130), (3, 0)])
def test_device_prep_equals_host_and_oracle(B, W):
    nb = 500
    rng = np.random.default_rng(B * 1000 + W)
    pool = kvp.alloc_pool(nb, 2, 128)
    bt, sl = _random_table(rng, B, W, nb)
    if W == 0:
        sl[:] = 0
    dev, status = _device_prep(pool, bt, sl)
    host = kvp.kv_prepare_block_tables(pool, bt, sl)
    assert status == 0
    assert dev.shape == host.shape == (B, kvp.kvp_padded_width(W))
    assert np.array_equal(dev, host), "device vs host preparation"
    if W > 0:                                  # (the library pads a zero-width table to one tile of zeros)
        assert np.array_equal(dev, oracle.prepare_block_tables(bt, sl, nb)), "device preparation vs oracle"


def test_device_prep_flags_and_sanitises_rows_the_host_rejects():
    nb, W = 50, 5
    pool = kvp.alloc_pool(nb, 2, 128)
    bt = np.arange(4 * W, dtype=np.int32).reshape(4, W) + 3
    bt[2, 1] = nb + 7                          # a kept entry outside the pool
    sl = np.array([-3, W * 16 + 1, 20, 0], np.int32)
    for b in range(3):                         # the host version rejects each of rows 0-2
        with pytest.raises(kvp.KvpError):
            kvp.kv_prepare_block_tables(pool, bt[b:b + 1], sl[b:b + 1])
    dev, status = _device_prep(pool, bt, sl)
    assert status == 1 | 2 | 4
    wp = kvp.kvp_padded_width(W)
    exp = np.zeros((4, wp), np.int32)
    exp[1, :W] = bt[1]                         # pages beyond the width dropped
    exp[1, W:] = bt[1, W - 1]
    exp[2, 0] = bt[2, 0]                       # the bad entry (and the fill repeating it) become block 0
    assert np.array_equal(dev, exp), dev


def test_attention_over_device_prepared_tables_and_graph_replays():
    """A ragged batch with its raw device table prepared on the GPU: the same
    output bits as with the host-prepared table.  Then the preparation and
    the attention call captured in one graph and replayed with new sequence
    lengths (a shortened row, inactive rows, the original again): every
    replay equals an eager call over a host-prepared table for the same
    lengths."""
    w = wl.random_case(77, [700, 129, 2000, 1, 300], [1, 1, 33, 1, 300], 8, 2, 128)
    g = GpuCase(w)
    ref = g.run()
    raw = torch.from_numpy(np.ascontiguousarray(w.block_tables)).cuda()
    bt_dev = kvp.kv_prepare_block_tables_device(g.pool, raw, g.seq_lens)
    ms, mq = int(w.seq_lens.max()), int(w.max_query_len)

    def call(bt, sl):
        g.out.fill_(-1)
        kvp.paged_attention(g.pool, g.q, g.out, w.num_q_heads, bt, sl, g.qsl, mq, ms, w.scale, True,
                            workspace=g.ws)
    call(bt_dev, g.seq_lens)
    torch.cuda.synchronize()
    bitwise(host_bits(g.out), ref, "device-prepared tables")

    sl_dev = g.seq_lens.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            kvp.kv_prepare_block_tables_device(g.pool, raw, sl_dev, out=bt_dev)
            call(bt_dev, sl_dev)
    torch.cuda.synchronize()
    base = np.asarray(w.seq_lens, np.int32)
    variants = [base.copy(), base.copy(), base.copy(), base.copy()]
    variants[1][2] = 1500                       # a shorter row: its later raw entries become padding
    variants[2][[0, 3]] = 0                     # inactive rows
    for i, sl in enumerate(variants):
        sl_dev.copy_(torch.from_numpy(sl))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = host_bits(g.out).copy()
        bt_h = torch.from_numpy(kvp.kv_prepare_block_tables(g.pool, w.block_tables, sl)).cuda()
        call(bt_h, torch.from_numpy(sl).cuda())
        torch.cuda.synchronize()
        bitwise(got, host_bits(g.out), "graph replay %d (seq_lens %s)" % (i, sl.tolist()))
