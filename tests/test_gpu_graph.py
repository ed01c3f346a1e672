"""HIP graph capture of the attention calls.  A graph is captured once with
a fixed grid (set by the host bounds num_seqs, max_query_len and
max_seq_len); between replays only device metadata changes, and the batch
shrinks 4 -> 3 -> 2 -> 1 by giving leaving rows seq_len 0 and no queries
(their table rows sanitised).  Every replay must equal the eager call
bitwise ("fix(rocm): stabilize direct paged CK attention for bitwise R/R",
Additional checks: HIP Graph vs eager and shrinking graph batches; Changes:
inactive graph rows).  Each replay is preceded by eager work on the same
stream (metadata copies, a sentinel fill) and followed by an eager check, so
replays after the first are exercised too."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_bf16_amd as kvp
from paged_kv_cache_bf16_amd import workloads as wl
from harness import GpuCase, bitwise, compare, dev_bits, host_bits, oracle_attention, oracle_pool

pytestmark = pytest.mark.gpu


class Meta:
    """Device metadata buffers the graph reads; refilled in place between replays."""

    def __init__(self, g: GpuCase, lens, qlens):
        self.g = g
        self.lens = np.asarray(lens, np.int32)
        self.W = g.w.block_tables.shape[1]
        self.bt = torch.from_numpy(kvp.kv_prepare_block_tables(g.pool, g.w.block_tables, self.lens)).cuda()
        self.seq = torch.from_numpy(self.lens.copy()).cuda()
        self.qsl = torch.from_numpy(np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)).cuda()

    def set_active(self, n, qlens):
        """Rows >= n leave the batch: seq_len 0, no queries, sanitised table row."""
        lens = self.lens.copy()
        lens[n:] = 0
        ql = np.asarray(qlens, np.int32).copy()
        ql[n:] = 0
        self.bt.copy_(torch.from_numpy(kvp.kv_prepare_block_tables(self.g.pool, self.g.w.block_tables, lens)))
        self.seq.copy_(torch.from_numpy(lens))
        self.qsl.copy_(torch.from_numpy(np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)))
        return lens, ql


def _attention(g, m, out, max_q, max_s):
    w = g.w
    kvp.paged_attention(g.pool, g.q, out, w.num_q_heads, m.bt, m.seq, m.qsl, max_q, max_s, w.scale, True,
                        workspace=g.ws)


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                       # eager warm-up: kernels loaded before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 8, 2), (512, 16, 2)])
def test_decode_graph_replays_equal_eager_while_batch_shrinks(D, Hq, Hkv):
    lens = [700, 2000, 129, 4100]
    w = wl.random_case(51 + D, lens, [1] * 4, Hq, Hkv, D)
    print("graph decode D=%d" % D, flush=True)
    g = GpuCase(w)
    m = Meta(g, lens, [1] * 4)
    max_s = int(max(lens))
    out_g = torch.zeros_like(g.q)
    graph = _capture(lambda: _attention(g, m, out_g, 1, max_s))
    first = None
    for n in (4, 3, 2, 1, 4):
        sl, ql = m.set_active(n, [1] * 4)
        out_g.fill_(-1)
        graph.replay()
        got = host_bits(out_g)
        # eager: the same padded batch, and the active rows alone as a batch of n
        out_e = torch.full_like(g.q, -1)        # the same sentinel as the graph's output
        _attention(g, m, out_e, 1, max_s)
        bitwise(got, host_bits(out_e), "graph vs eager, %d active" % n)
        alone = torch.zeros_like(g.q[:n])
        kvp.paged_attention(g.pool, g.q[:n], alone, Hq, m.bt[:n], m.seq[:n], m.qsl[:n + 1], 1, max_s, w.scale,
                            True, workspace=g.ws)
        bitwise(got[:n], host_bits(alone), "graph vs eager batch of %d" % n)
        assert (got[n:] == 0xFFFF).all(), "rows that left the batch were written"
        if first is None:
            first = got.copy()
            compare(got, oracle_attention(w, oracle_pool(w)), "graph decode")
        elif n == 4:
            bitwise(got, first, "replay after shrinking vs first replay")


def test_decode_step_graph_replays_equal_eager():
    """kvp_decode_step (cache write fused into the partial launch) captured
    once; each replay writes the same new rows (idempotent) and reads them."""
    lens = [700, 2000, 129, 4100]
    w = wl.random_case(61, lens, [1] * 4, 8, 2, 128)
    print("graph decode step", flush=True)
    g = GpuCase(w)
    m = Meta(g, lens, [1] * 4)
    rng = np.random.default_rng(5)
    kn_h = wl.to_bf16_bits(rng.standard_normal((4, 2, 128)).astype(np.float32))
    vn_h = wl.to_bf16_bits(rng.standard_normal((4, 2, 128)).astype(np.float32))
    kn, vn = dev_bits(kn_h), dev_bits(vn_h)
    slots_all = np.array([int(w.block_tables[b, (L - 1) // 16]) * 16 + (L - 1) % 16 for b, L in enumerate(lens)],
                         np.int64)
    slots = torch.from_numpy(slots_all.copy()).cuda()
    max_s = int(max(lens))
    out_g = torch.zeros_like(g.q)

    def step(out):
        kvp.kvp_decode_step(g.pool, kn, vn, slots, g.q, out, 8, m.bt, m.seq, m.qsl, 1, max_s, w.scale, True,
                            workspace=g.ws)

    before = kvp.kvp_get_counters()["fused_decode_steps"]
    graph = _capture(lambda: step(out_g))
    assert kvp.kvp_get_counters()["fused_decode_steps"] == before + 2     # warm-up + capture
    for n in (4, 3, 2, 1):
        m.set_active(n, [1] * 4)
        s = slots_all.copy()
        s[n:] = -1                                    # leaving rows write nothing
        slots.copy_(torch.from_numpy(s))
        out_g.fill_(-1)
        graph.replay()
        pool_g = host_bits(g.pool.storage)
        got = host_bits(out_g)
        out_e = torch.full_like(g.q, -1)        # the same sentinel as the graph's output
        step(out_e)
        torch.cuda.synchronize()
        bitwise(got, host_bits(out_e), "graph step vs eager, %d active" % n)
        bitwise(pool_g, host_bits(g.pool.storage), "pool after graph step vs eager, %d active" % n)
        assert (got[n:] == 0xFFFF).all()
    # the pool holds the new rows in their slots and nothing else changed
    exp = oracle_pool(w)
    oracle.reshape_and_cache(exp, kn_h, vn_h, slots_all)
    np.testing.assert_array_equal(host_bits(g.pool.storage), exp.storage)


def test_mixed_batch_graph_replays_equal_eager():
    """A mixed batch (split-KV rows and prefill rows: two kernels and the fold)
    captured once and replayed while rows leave."""
    lens = [300, 2000, 129, 700]
    ql = [300, 1, 4, 33]
    w = wl.random_case(71, lens, ql, 8, 2, 128)
    print("graph mixed batch", flush=True)
    g = GpuCase(w)
    m = Meta(g, lens, ql)
    max_q, max_s = int(max(ql)), int(max(lens))
    out_g = torch.zeros_like(g.q)
    graph = _capture(lambda: _attention(g, m, out_g, max_q, max_s))
    ref = None
    for n in (4, 3, 2, 1, 4):
        m.set_active(n, ql)
        out_g.fill_(-1)
        graph.replay()
        got = host_bits(out_g)
        out_e = torch.full_like(g.q, -1)        # the same sentinel as the graph's output
        _attention(g, m, out_e, max_q, max_s)
        bitwise(got, host_bits(out_e), "mixed graph vs eager, %d active" % n)
        rows = int(np.sum(ql[:n]))
        assert (got[rows:] == 0xFFFF).all()
        if ref is None:
            ref = got.copy()
            compare(got, oracle_attention(w, oracle_pool(w)), "mixed graph")
        elif n == 4:
            bitwise(got, ref, "mixed replay after shrinking")
