"""Shared set-up for the GPU parity tests: upload a workload, run the HIP
path through the C ABI, and run the oracle on the same inputs."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import paged_kv_cache_bf16_amd as kvp
from paged_kv_cache_bf16_amd import workloads as wl

POISON = 0x7FC1          # a quiet-NaN BF16 pattern for never-written slots

MAX_ABS = 2e-2
MEAN_ABS = 2e-3
# Relative RMS error, per (query row, head) output vector and over the case.
# The absolute bars alone are weak on long rows: there the output's spread is
# ~0.5 / sqrt(L) (0.004 at L = 18432 with values x0.5), so an output off by a
# factor of two still passes max-abs 2e-2 / mean-abs 2e-3.  BF16 rounding of
# P and of the output bounds the expected relative error near 2e-3.
REL_RMS = 1e-2


def dev_bits(a: np.ndarray) -> torch.Tensor:
    """Host uint16 BF16 bits -> device int16 tensor holding the same bits."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    return oracle.bf16_bits_to_f32(a)


class GpuCase:
    """A workload resident on the GPU: pool filled through reshape_and_cache,
    prepared tables and metadata, and a workspace."""

    def __init__(self, w: wl.Workload, fill_bits=POISON, ws_max_seq_len=None, split_cols=16):
        self.w = w
        self.pool = kvp.alloc_pool(w.num_blocks, w.num_kv_heads, w.head_dim, interleaved=w.interleaved,
                                   fill_bits=fill_bits)
        self.k = dev_bits(w.k)
        self.v = dev_bits(w.v)
        self.slots = torch.from_numpy(w.slot_mapping).cuda()
        kvp.reshape_and_cache(self.pool, self.k, self.v, self.slots)
        self.set_queries(w.q, w.query_lens)
        self.ws = kvp.alloc_workspace(self.pool, w.num_q_heads, w.batch,
                                      int(ws_max_seq_len or w.seq_lens.max(initial=1)), split_cols=split_cols)

    def set_queries(self, q_bits, query_lens, block_tables=None, seq_lens=None):
        w = self.w
        bt = w.block_tables if block_tables is None else block_tables
        sl = w.seq_lens if seq_lens is None else np.asarray(seq_lens, np.int32)
        self.host_bt = kvp.kv_prepare_block_tables(self.pool, bt, sl)
        self.bt = torch.from_numpy(self.host_bt).cuda()
        self.seq_lens_h = sl
        self.seq_lens = torch.from_numpy(sl).cuda()
        self.qlens_h = np.asarray(query_lens, np.int32)
        qsl = np.concatenate([[0], np.cumsum(self.qlens_h)]).astype(np.int32)
        self.qsl_h = qsl
        self.qsl = torch.from_numpy(qsl).cuda()
        self.q_h = q_bits
        self.q = dev_bits(q_bits)
        self.out = torch.zeros_like(self.q)

    def run(self, causal=None, max_seq_len=None, use_workspace=True):
        """Run paged_attention; max_seq_len overrides the host bound (it must
        cover every row; a larger bound can select a different kernel path)."""
        w = self.w
        self.out.fill_(-1)                         # 0xFFFF: NaN bits, so unwritten rows show
        ms = int(self.seq_lens_h.max(initial=0)) if max_seq_len is None else int(max_seq_len)
        kvp.paged_attention(self.pool, self.q, self.out, w.num_q_heads, self.bt, self.seq_lens, self.qsl,
                            int(self.qlens_h.max(initial=0)), ms, w.scale,
                            w.causal if causal is None else causal,
                            workspace=self.ws if use_workspace else None)
        torch.cuda.synchronize()
        return host_bits(self.out)

    def run_lse(self, causal=None, max_seq_len=None, use_workspace=True):
        """paged_attention_lse: (output bits, lse float32); rows not computed keep NaN lse."""
        w = self.w
        self.out.fill_(-1)
        lse = torch.full((self.q.shape[0], w.num_q_heads), float("nan"), dtype=torch.float32, device="cuda")
        ms = int(self.seq_lens_h.max(initial=0)) if max_seq_len is None else int(max_seq_len)
        kvp.paged_attention_lse(self.pool, self.q, self.out, lse, w.num_q_heads, self.bt, self.seq_lens, self.qsl,
                                int(self.qlens_h.max(initial=0)), ms, w.scale,
                                w.causal if causal is None else causal,
                                workspace=self.ws if use_workspace else None)
        torch.cuda.synchronize()
        return host_bits(self.out), lse.cpu().numpy()

    def pool_bits(self) -> np.ndarray:
        return host_bits(self.pool.storage)


def oracle_pool(w: wl.Workload, fill_bits=POISON) -> oracle.Pool:
    p = oracle.Pool(w.num_blocks, w.num_kv_heads, w.head_dim, interleaved=w.interleaved, fill_bits=fill_bits)
    oracle.reshape_and_cache(p, w.k, w.v, w.slot_mapping)
    return p


def oracle_attention(w: wl.Workload, pool: oracle.Pool, q_bits=None, query_lens=None, rows=None,
                     block_tables=None):
    q = w.q if q_bits is None else q_bits
    ql = w.query_lens if query_lens is None else np.asarray(query_lens, np.int32)
    qsl = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    bt = w.block_tables if block_tables is None else block_tables
    return oracle.paged_attention(q, pool, bt, w.seq_lens, qsl, w.num_q_heads, w.scale, w.causal, rows=rows)


def compare(gpu_bits: np.ndarray, ref: np.ndarray, what: str = ""):
    """Tolerance parity of BF16 outputs against the FP32 oracle; returns stats."""
    g = bf16_to_f32(gpu_bits).astype(np.float64)
    r = ref.astype(np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.isfinite(g).all(), "%s: non-finite GPU output (%d values)" % (what, (~np.isfinite(g)).sum())
    err = np.abs(g - r)
    # per output vector (last axis = head_dim): ||gpu - ref|| / ||ref||
    vec_err = np.sqrt((err ** 2).sum(axis=-1))
    vec_ref = np.sqrt((r ** 2).sum(axis=-1))
    vec_rel = vec_err / np.maximum(vec_ref, 1e-6)
    stats = dict(max_abs=float(err.max()), mean_abs=float(err.mean()),
                 rel_rms=float(np.sqrt((err ** 2).sum() / max((r ** 2).sum(), 1e-30))),
                 max_vec_rel_rms=float(vec_rel.max()) if vec_rel.size else 0.0)
    assert stats["max_abs"] <= MAX_ABS, (what, stats)
    assert stats["mean_abs"] <= MEAN_ABS, (what, stats)
    assert stats["rel_rms"] <= REL_RMS, (what, stats)
    if vec_rel.size:
        worst = np.unravel_index(int(vec_rel.argmax()), vec_rel.shape)
        assert stats["max_vec_rel_rms"] <= REL_RMS, (what, "worst (row, head)", worst, stats)
    return stats


def bitwise(a: np.ndarray, b: np.ndarray, what: str = ""):
    """Strict agreement, reported as mismatch_count / max_abs_diff / equal."""
    mism = int((a.view(np.uint16) != b.view(np.uint16)).sum())
    diff = float(np.abs(bf16_to_f32(a).astype(np.float64) - bf16_to_f32(b).astype(np.float64)).max()) if a.size else 0.0
    assert mism == 0, "%s: mismatch_count=%d max_abs_diff=%g" % (what, mism, diff)


def group_rows(w: wl.Workload, rows_per_group: int, groups=("first", "middle", "last")) -> np.ndarray:
    """Every query row of the first, a middle and the last column-group
    workgroup of each sequence, for a prefill kernel whose workgroups own
    rows_per_group consecutive query rows of one (sequence, kv head)."""
    qsl = w.query_start_loc
    rows = []
    for b in range(w.batch):
        q0, q_len = int(qsl[b]), int(qsl[b + 1] - qsl[b])
        if q_len == 0:
            continue
        n_groups = -(-q_len // rows_per_group)
        pick = {"first": 0, "middle": n_groups // 2, "last": n_groups - 1}
        for name in groups:
            gi = pick[name]
            rows.extend(range(q0 + gi * rows_per_group, q0 + min((gi + 1) * rows_per_group, q_len)))
    return np.array(sorted(set(rows)), np.int64)


def sample_rows(w: wl.Workload, n: int, seed: int = 0) -> np.ndarray:
    """Query rows to check with the oracle: first and last of every sequence,
    plus a seeded random sample."""
    qsl = w.query_start_loc
    rng = np.random.default_rng(seed)
    rows = set()
    for b in range(w.batch):
        if qsl[b + 1] > qsl[b]:
            rows.update([int(qsl[b]), int(qsl[b + 1] - 1)])
    total = int(qsl[-1])
    rows.update(rng.choice(total, size=min(n, total), replace=False).tolist())
    return np.array(sorted(rows), np.int64)
