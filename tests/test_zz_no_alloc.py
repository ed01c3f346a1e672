"""paged_attention_noalloc: the split-KV partials in the library's static
scratch array instead of a caller workspace.  Its output must equal
paged_attention's (with a workspace) bit for bit, on two calls in a row (the
second with a smaller input, so the scratch holds the first call's partials
when it starts), and a decode call whose partials exceed the scratch is
rejected before anything is queued."""
import numpy as np
import pytest
import torch

import paged_kv_cache_bf16_amd as kvp
from paged_kv_cache_bf16_amd import workloads as wl
from harness import GpuCase, bitwise, compare, host_bits, oracle_attention, oracle_pool

pytestmark = pytest.mark.gpu


def _noalloc(g, w):
    g.out.fill_(-1)
    kvp.paged_attention_noalloc(g.pool, g.q, g.out, w.num_q_heads, g.bt, g.seq_lens, g.qsl,
                                int(w.max_query_len), int(w.seq_lens.max()), w.scale, w.causal)
    torch.cuda.synchronize()
    return host_bits(g.out).copy()


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 8, 2), (512, 16, 2)])
def test_noalloc_equals_workspace_call_twice_shrinking(D, Hq, Hkv):
    print("noalloc D=%d" % D, flush=True)
    big = wl.random_case(31 + D, [7168, 5000, 3000, 129], [1, 1, 1, 1], Hq, Hkv, D)
    small = wl.random_case(37 + D, [1000, 70], [1, 1], Hq, Hkv, D)
    need = kvp.kvp_workspace_bytes(GpuCase(small).pool, Hq, 4, 7168)
    assert need <= kvp.KVP_SCRATCH_BYTES
    outs = []
    for w in (big, small):
        g = GpuCase(w)
        ref = g.run()                                   # paged_attention with a workspace
        before = kvp.kvp_get_counters()["split_kv_launches"]
        got = _noalloc(g, w)
        assert kvp.kvp_get_counters()["split_kv_launches"] == before + 1
        bitwise(got, ref, "noalloc vs workspace call (B=%d)" % w.batch)
        compare(got, oracle_attention(w, oracle_pool(w)), "noalloc vs oracle (B=%d)" % w.batch)
        outs.append(got)
    assert outs[0].shape != outs[1].shape


def test_noalloc_mixed_batch_and_prefill():
    """A mixed batch (short rows through the split-KV path, long ones through
    a prefill kernel) gives the workspace call's bits."""
    w = wl.random_case(43, [300, 2000, 129, 700], [300, 1, 4, 33], 8, 2, 128)
    g = GpuCase(w)
    ref = g.run()
    bitwise(_noalloc(g, w), ref, "noalloc mixed batch")


def test_noalloc_rejects_partials_beyond_scratch():
    """A decode batch whose partials exceed KVP_SCRATCH_BYTES: rejected with
    KVP_ERR_WORKSPACE_TOO_SMALL before any launch (counters unchanged)."""
    w = wl.random_case(47, [64], [1], 8, 2, 128)
    g = GpuCase(w)
    B, L = 64, 16384
    assert kvp.kvp_workspace_bytes(g.pool, 8, B, L) > kvp.KVP_SCRATCH_BYTES
    q = torch.zeros((B, 8, 128), dtype=torch.int16, device="cuda")
    bt = torch.zeros((B, L // 16), dtype=torch.int32, device="cuda")
    sl = torch.full((B,), L, dtype=torch.int32, device="cuda")
    qsl = torch.arange(B + 1, dtype=torch.int32, device="cuda")
    before = kvp.kvp_get_counters()
    with pytest.raises(kvp.KvpError) as e:
        kvp.paged_attention_noalloc(g.pool, q, q, 8, bt, sl, qsl, 1, L)
    assert e.value.code == kvp.KVP_ERR_WORKSPACE_TOO_SMALL
    assert "scratch" in str(e.value)
    after = kvp.kvp_get_counters()
    assert after["split_kv_launches"] == before["split_kv_launches"]
    assert after["prefill_launches"] == before["prefill_launches"]
