"""GPU parity of the log-sum-exp output (paged_attention_lse) and of
kvp_merge_attention against the oracle, and the bitwise properties the
"fix(rocm): stabilize direct paged CK attention for bitwise R/R" page lists
under Additional checks (causal/LSE results compared with decode).

Tolerances:
  * lse vs the FP32 oracle: |diff| <= 2e-4 * max(1, |lse|).  Both sides sum
    the same FP32 exponentials; the GPU's scores come from an MFMA chain in
    another order and its exp2/log2 are the hardware approximations (about
    1 ulp each), which move lse by ~1e-6 relative; 2e-4 leaves a wide margin
    yet fails a base-2 logarithm (x0.69), a dropped max term or a wrong row.
  * merge output vs the FP64 oracle merge on the same inputs: within one
    BF16 ulp (2^-8 relative) -- the GPU rounds an FP32 value, the oracle's
    is exact to ~1e-16, so only a rounding tie can differ; merge lse within
    1e-6 * max(1, |lse|).
  * chunked prefill (prefix and chunk merged) vs the oracle's full causal
    prefill: the attention tolerance (max-abs 2e-2, mean-abs 2e-3), since
    the merged output rounds twice to BF16.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_bf16_amd as kvp
from paged_kv_cache_bf16_amd import workloads as wl
from harness import GpuCase, bitwise, bf16_to_f32, compare, dev_bits, host_bits, oracle_pool

pytestmark = pytest.mark.gpu

LSE_REL = 2e-4


def _oracle_lse(w, q_bits=None, query_lens=None, block_tables=None, seq_lens=None, causal=None):
    pool = oracle_pool(w)
    q = w.q if q_bits is None else q_bits
    ql = w.query_lens if query_lens is None else np.asarray(query_lens, np.int32)
    qsl = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    return oracle.paged_attention(q, pool, w.block_tables if block_tables is None else block_tables,
                                  w.seq_lens if seq_lens is None else seq_lens, qsl, w.num_q_heads, w.scale,
                                  w.causal if causal is None else causal, return_lse=True)


def _check_lse(got, ref, what):
    assert np.isfinite(got).all(), what
    err = np.abs(got.astype(np.float64) - ref) / np.maximum(1.0, np.abs(ref))
    assert err.max() <= LSE_REL, (what, float(err.max()))


@pytest.mark.parametrize("case", [
    dict(lens=[300, 1, 129], q=[300, 1, 17], Hq=8, Hkv=2, D=128),        # prefill + decode rows, mixed
    dict(lens=[2000, 777], q=[1, 1], Hq=8, Hkv=2, D=128),                # decode only (split-KV + fold)
    dict(lens=[333], q=[333], Hq=32, Hkv=8, D=128),
    dict(lens=[200, 65], q=[200, 1], Hq=8, Hkv=2, D=256),
    dict(lens=[150, 90], q=[150, 1], Hq=16, Hkv=2, D=512),
], ids=["mixed128", "decode128", "g4x8", "d256", "d512"])
def test_lse_matches_oracle_and_output_is_unchanged(case):
    w = wl.random_case(31 + case["D"], case["lens"], case["q"], case["Hq"], case["Hkv"], case["D"])
    print("case", case, flush=True)
    g = GpuCase(w)
    plain = g.run()
    out, lse = g.run_lse()
    bitwise(out, plain, "paged_attention_lse output vs paged_attention")
    ref_out, ref_lse = _oracle_lse(w)
    compare(out, ref_out, "lse case output")
    _check_lse(lse, ref_lse, "lse")


def test_lse_decode_equals_prefill_bitwise():
    lens = [1, 16, 129, 777, 2050]
    for D, Hq, Hkv in ((128, 8, 2), (256, 8, 2), (512, 16, 2)):
        w = wl.random_case(40 + D, lens, lens, Hq, Hkv, D)
        print("case D=%d" % D, flush=True)
        g = GpuCase(w)
        full, full_lse = g.run_lse()
        d = w.decode_view()
        g.set_queries(d.q, d.query_lens)
        dec, dec_lse = g.run_lse()
        last = w.query_start_loc[1:] - 1
        bitwise(dec, full[last], "decode vs prefill D=%d" % D)
        assert (dec_lse.view(np.uint32) == full_lse[last].view(np.uint32)).all(), "lse decode vs prefill D=%d" % D


def _merge_inputs(rng, T, H, D, empty_frac=0.1):
    a = wl.to_bf16_bits(rng.standard_normal((T, H, D)).astype(np.float32))
    b = wl.to_bf16_bits(rng.standard_normal((T, H, D)).astype(np.float32))
    la = (rng.standard_normal((T, H)) * 6).astype(np.float32)
    lb = (rng.standard_normal((T, H)) * 6).astype(np.float32)
    # some pairs with an empty side (NaN rows there must not leak), and both empty
    ea = rng.random((T, H)) < empty_frac
    eb = rng.random((T, H)) < empty_frac
    la[ea] = -np.inf
    lb[eb] = -np.inf
    a[ea] = 0x7FC1
    b[eb] = 0x7FC1
    return a, la, b, lb


@pytest.mark.parametrize("T,H,D", [(1, 1, 128), (37, 8, 128), (300, 4, 256), (19, 16, 512), (5, 3, 72)])
def test_merge_matches_oracle(T, H, D):
    rng = np.random.default_rng(T * 1000 + D)
    a, la, b, lb = _merge_inputs(rng, T, H, D)
    print("merge T=%d H=%d D=%d" % (T, H, D), flush=True)
    ta, tb = dev_bits(a), dev_bits(b)
    tla, tlb = torch.from_numpy(la).cuda(), torch.from_numpy(lb).cuda()
    out = torch.empty_like(ta)
    lse = torch.empty_like(tla)
    kvp.kvp_merge_attention(ta, tla, tb, tlb, out, lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.merge_states(a, la, b, lb)
    got = bf16_to_f32(host_bits(out)).astype(np.float64)
    assert np.isfinite(got).all()
    assert (np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30).all(), float(np.abs(got - ref).max())
    gl = lse.cpu().numpy().astype(np.float64)
    both = np.isneginf(ref_lse)
    assert (np.isneginf(gl) == both).all()
    assert (np.abs(gl[~both] - ref_lse[~both]) <= 1e-6 * np.maximum(1.0, np.abs(ref_lse[~both]))).all()
    # in place: out = out_a, lse = lse_a gives the same bits
    kvp.kvp_merge_attention(ta, tla, tb, tlb, ta, tla)
    torch.cuda.synchronize()
    bitwise(host_bits(ta), host_bits(out), "in-place merge")
    assert (tla.cpu().numpy().view(np.uint32) == lse.cpu().numpy().view(np.uint32)).all()
    assert kvp.kvp_get_counters()["merge_launches"] >= 2


@pytest.mark.parametrize("prefix,chunk,D,Hq,Hkv", [(96, 40, 128, 8, 2), (1024, 300, 128, 32, 8),
                                                   (512, 77, 256, 8, 2), (256, 100, 512, 16, 2)])
def test_chunked_prefill_by_merge_matches_full_prefill(prefix, chunk, D, Hq, Hkv):
    """Prefix keys (non-causal, all visible) merged with the chunk's own keys
    (causal, bottom-right) give the causal prefill of the chunk's queries over
    the whole row.  The prefix is a whole number of 16-token pages, so the
    chunk's keys are the table's columns from prefix / 16 on."""
    L = prefix + chunk
    w = wl.random_case(7 + D + prefix, [L], [chunk], Hq, Hkv, D)
    print("chunked prefix=%d chunk=%d D=%d" % (prefix, chunk, D), flush=True)
    g = GpuCase(w)
    # part A: prefix keys
    g.set_queries(w.q, [chunk], seq_lens=[prefix])
    oa, la = g.run_lse(causal=False)
    # part B: the chunk's keys through the table's later columns
    g.set_queries(w.q, [chunk], block_tables=np.ascontiguousarray(w.block_tables[:, prefix // 16:]),
                  seq_lens=[chunk])
    ob, lb = g.run_lse(causal=True)
    ta, tb = dev_bits(oa), dev_bits(ob)
    out = torch.empty_like(ta)
    lse = torch.empty((chunk, Hq), dtype=torch.float32, device="cuda")
    kvp.kvp_merge_attention(ta, torch.from_numpy(la).cuda(), tb, torch.from_numpy(lb).cuda(), out, lse)
    torch.cuda.synchronize()
    ref_out, ref_lse = _oracle_lse(w)
    compare(host_bits(out), ref_out, "chunked prefill by merge")
    # anti-vacuity: either part alone is far from the full result
    for part in (oa, ob):
        assert np.abs(bf16_to_f32(part).astype(np.float64) - ref_out).max() > 0.1
    _check_lse(lse.cpu().numpy(), ref_lse, "merged lse")
