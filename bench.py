#!/usr/bin/env python3
"""Benchmark of the paged BF16 KV-cache hot path on one MI355X.

One step = one pass of the whole path over one batch: write the batch's new
K/V rows into the pool (reshape_and_cache), then paged attention over the
pool.  Inputs are seeded synthetic BF16 N(0,1) data resident in HBM.

Headline (the JSON line's `value`): decode B=4 sequences, one query each, KV
length 7168, Hq 8 / Hkv 2 / Dh 128, 16-token pages permuted at random.  The
pool holds 40 disjoint page sets (1.17 GB, well above the 256 MB Infinity
Cache) and step i uses set i % 40, so every step reads K/V from HBM.  The
timed steps are replayed from HIP graphs that each hold 40 consecutive steps
(the library's calls are capture-safe), so host launch work does not sit
between steps; the eagerly issued rate is reported beside it.
value = decode KV-read bytes per step / step time (GB/s).

`roofline`: the dominant kernels of that step -- one paged_attention decode
call (split-KV partial kernel + fold kernel) -- timed live with HIP events
around graph replays of 40 calls on the launch stream; algorithmic bytes per
call / that time, against the MI355X HBM peak (8 TB/s).

`configs`: every workload, each timed the same way (a HIP graph of n calls
on the launch stream, median of 5 replays), with its algorithmic work and
roofline fraction: the composition case (Dh 256), B4 KV7168 decode, the
causal prefill B1 Q=KV=4096, the B4 Q128 suffix on KV 7168, the ragged mixed
batch on a 2.29 GB interleaved pool, and the wide-head (Dh 512) prefill and
decode at L = 3072 / 11264 / 18432, plus reshape_and_cache and the merge.
Prefill FLOPs = 4 * Dh * Hq * (visible causal query/key pairs); decode
bytes = K/V pages read + q + out + block-table entries.  Decode rows are
timed cold (rotating page sets larger than the Infinity Cache) and warm (one
set).  Peaks: HBM 8 TB/s, dense BF16 MFMA 2.5 PFLOP/s.

cpu_baseline: the CPU oracle timed on this host on a bounded sample of the
headline workload (full decode calls, ~10 s).

    python bench.py [--steps K --warmup W]        the driver's run
    python bench.py --only NAME                    one config (for profilers)
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
METRIC = "decode KV-read GB/s (% HBM peak) + prefill TFLOP/s (% MFMA peak), µs/call"
CONFIG_NAMES = ("tiny", "decode", "prefill", "suffix", "ragged", "wide3072", "wide11264", "wide18432", "cache",
                "merge")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def omp_threads():
    env = os.environ.get("OMP_NUM_THREADS")
    return min(host_cores(), int(env)) if env and env.isdigit() else host_cores()


# ----------------------------------------------------------------------------- timing

def time_launches(fn, n, stream):
    """Average GPU time per call of fn() over n back-to-back calls (HIP events on `stream`)."""
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(n):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / n * 1e3          # us


def capture(fn, n):
    """One HIP graph holding fn(i) for i = 0 .. n-1 in order (no host work between the calls)."""
    import torch
    fn(0)                                             # eager first: kernels loaded before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    torch.cuda.synchronize()
    return g


def graph_us(fn, n, stream, groups=5, replays=3):
    """us per call: a graph of n calls fn(0..n-1), median over `groups` groups of `replays` replays."""
    g = capture(fn, n)
    g.replay()
    ts = [time_launches(g.replay, replays, stream) / n for _ in range(groups)]
    del g
    return float(np.median(ts)), ts


# ----------------------------------------------------------------------------- work formulas

def causal_pairs(seq_lens, q_lens, causal=True):
    """Visible (query, key) pairs, bottom-right aligned queries."""
    n = 0
    for L, q in zip(seq_lens, q_lens):
        L, q = int(L), int(q)
        n += q * (L - q) + q * (q + 1) // 2 if causal else q * L
    return n


def prefill_flops(D, Hq, seq_lens, q_lens, causal=True):
    return 4.0 * D * Hq * causal_pairs(seq_lens, q_lens, causal)


def attention_bytes(D, Hq, Hkv, seq_lens, q_lens):
    """K/V bytes read once + q read + out written + active table entries."""
    kv = sum(int(L) for L in seq_lens) * Hkv * D * 2 * 2
    qo = 2 * sum(int(q) for q in q_lens) * Hq * D * 2
    tab = sum(-(-int(L) // 16) for L in seq_lens) * 4
    return kv + qo + tab


def rates(us, flops=None, nbytes=None):
    r = {"us_per_call": round(us, 3)}
    if flops is not None:
        tf = flops / (us * 1e-6) / 1e12
        r.update(TFLOPs=round(tf, 2), mfma_frac=round(tf / BF16_PEAK_TFLOPS, 4), flops_per_call=flops)
    if nbytes is not None:
        gbs = nbytes / (us * 1e-6) / 1e9
        r.update(GBps=round(gbs, 1), hbm_frac=round(gbs / HBM_PEAK_GBS, 4), bytes_per_call=nbytes)
    return r


# ----------------------------------------------------------------------------- workloads on the GPU

def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


class Uploaded:
    """A workloads.Workload resident on the GPU: pool written through
    reshape_and_cache, prepared tables, queries, output and workspace."""

    def __init__(self, w, split_cols=16):
        import torch
        import paged_kv_cache_bf16_amd as kvp
        self.kvp, self.w = kvp, w
        self.pool = kvp.alloc_pool(w.num_blocks, w.num_kv_heads, w.head_dim, interleaved=w.interleaved)
        self.k, self.v = to_dev(w.k), to_dev(w.v)
        self.slots = torch.from_numpy(w.slot_mapping).cuda()
        kvp.reshape_and_cache(self.pool, self.k, self.v, self.slots)
        self.bt = torch.from_numpy(kvp.kv_prepare_block_tables(self.pool, w.block_tables, w.seq_lens)).cuda()
        self.sl = torch.from_numpy(w.seq_lens).cuda()
        self.qsl = torch.from_numpy(w.query_start_loc).cuda()
        self.q = to_dev(w.q)
        self.out = torch.zeros_like(self.q)
        self.max_q, self.max_s = int(w.max_query_len), int(w.seq_lens.max())
        # a workspace only when some row is short (q_len * G <= 16), as a caller would pass it
        G = w.num_q_heads // w.num_kv_heads
        short = bool((w.query_lens * G <= 16).any())
        self.ws = (kvp.alloc_workspace(self.pool, w.num_q_heads, w.batch, self.max_s, split_cols=split_cols)
                   if short or split_cols > 16 else None)
        torch.cuda.synchronize()

    def attention(self, _i=0):
        w = self.w
        self.kvp.paged_attention(self.pool, self.q, self.out, w.num_q_heads, self.bt, self.sl, self.qsl, self.max_q,
                                 self.max_s, w.scale, w.causal, workspace=self.ws)

    def cache_write(self, _i=0):
        self.kvp.reshape_and_cache(self.pool, self.k, self.v, self.slots)

    def free(self):
        import torch
        del self.pool, self.k, self.v, self.q, self.out, self.ws
        torch.cuda.empty_cache()


class DecodeBench:
    """B sequences of KV length L, one query each, over S rotating disjoint page sets
    (filled on the GPU with torch's seeded normal generator)."""

    def __init__(self, B=4, L=7168, Hq=8, Hkv=2, D=128, sets=40, seed=1235, value_scale=1.0):
        import torch
        import paged_kv_cache_bf16_amd as kvp
        self.kvp = kvp
        self.B, self.L, self.Hq, self.Hkv, self.D = B, L, Hq, Hkv, D
        self.S = sets
        W = -(-L // 16)
        rng = np.random.default_rng(seed)
        nb = sets * B * W
        bt = rng.permutation(nb).astype(np.int32).reshape(sets * B, W)
        self.pool = kvp.alloc_pool(nb, Hkv, D, interleaved=False)
        gen = torch.Generator(device="cuda").manual_seed(seed)
        self.sl = torch.full((B,), L, dtype=torch.int32, device="cuda")
        self.qsl = torch.arange(B + 1, dtype=torch.int32, device="cuda")
        self.bt, self.q, self.knew, self.vnew, self.slot_new = [], [], [], [], []
        pos = np.arange(L, dtype=np.int64)
        for s in range(sets):
            rows = bt[s * B:(s + 1) * B]
            slots = np.concatenate([rows[b, pos // 16].astype(np.int64) * 16 + pos % 16 for b in range(B)])
            T = slots.shape[0]
            k = (torch.randn(T, Hkv, D, generator=gen, device="cuda") * value_scale).to(torch.bfloat16).view(torch.int16)
            v = (torch.randn(T, Hkv, D, generator=gen, device="cuda") * value_scale).to(torch.bfloat16).view(torch.int16)
            sd = torch.from_numpy(slots).cuda()
            kvp.reshape_and_cache(self.pool, k, v, sd)
            last = torch.arange(B, device="cuda") * L + L - 1
            self.knew.append(k[last].contiguous())
            self.vnew.append(v[last].contiguous())
            self.slot_new.append(sd[last].contiguous())
            self.bt.append(torch.from_numpy(kvp.kv_prepare_block_tables(self.pool, rows, [L] * B)).cuda())
            self.q.append((torch.randn(B, Hq, D, generator=gen, device="cuda") * value_scale)
                          .to(torch.bfloat16).view(torch.int16))
            if s == 0:
                self.host0 = dict(k=k.cpu().numpy().view(np.uint16), v=v.cpu().numpy().view(np.uint16),
                                  slots=slots, bt=rows.copy(), q=self.q[0].cpu().numpy().view(np.uint16))
            del k, v
        self.out = torch.zeros(B, Hq, D, dtype=torch.int16, device="cuda")
        self.lse = torch.zeros(B, Hq, dtype=torch.float32, device="cuda")
        self.ws = kvp.alloc_workspace(self.pool, Hq, B, L)
        self.scale = 1.0 / math.sqrt(D)
        self.i = 0
        torch.cuda.synchronize()

    @property
    def kv_bytes(self):
        return self.B * self.L * self.Hkv * self.D * 2 * 2

    @property
    def algo_bytes(self):
        return attention_bytes(self.D, self.Hq, self.Hkv, [self.L] * self.B, [1] * self.B)

    def attention(self, s):
        self.kvp.paged_attention(self.pool, self.q[s % self.S], self.out, self.Hq, self.bt[s % self.S], self.sl,
                                 self.qsl, 1, self.L, self.scale, True, workspace=self.ws)

    def attention_lse(self, s):
        self.kvp.paged_attention_lse(self.pool, self.q[s % self.S], self.out, self.lse, self.Hq, self.bt[s % self.S],
                                     self.sl, self.qsl, 1, self.L, self.scale, True, workspace=self.ws)

    def step_set(self, s):
        """One step on page set s: reshape_and_cache of the B new tokens + decode attention, through
        kvp_decode_step (the cache write runs inside the split-KV partial launch)."""
        s %= self.S
        self.kvp.kvp_decode_step(self.pool, self.knew[s], self.vnew[s], self.slot_new[s], self.q[s], self.out,
                                 self.Hq, self.bt[s], self.sl, self.qsl, 1, self.L, self.scale, True,
                                 workspace=self.ws)

    def step(self):
        s = self.i % self.S
        self.i += 1
        self.step_set(s)

    def attention_only(self):
        s = self.i % self.S
        self.i += 1
        self.attention(s)

    def check_against_oracle(self):
        """Set 0 output vs the oracle (tolerance), so the timed path is a correct one."""
        import torch
        import oracle
        h = self.host0
        self.attention(0)
        torch.cuda.synchronize()
        got = oracle.bf16_bits_to_f32(self.out.cpu().numpy().view(np.uint16))
        pool = oracle.Pool(self.S * self.B * -(-self.L // 16), self.Hkv, self.D)
        oracle.reshape_and_cache(pool, h["k"], h["v"], h["slots"])
        ref = oracle.paged_attention(h["q"], pool, h["bt"], [self.L] * self.B, np.arange(self.B + 1),
                                     self.Hq, self.scale, True)
        err = np.abs(got.astype(np.float64) - ref)
        return float(err.max()), float(err.mean()), pool

    def cpu_baseline(self, pool, budget_s=10.0):
        import oracle
        h = self.host0
        n, t0 = 0, time.perf_counter()
        while True:
            oracle.paged_attention(h["q"], pool, h["bt"], [self.L] * self.B, np.arange(self.B + 1), self.Hq,
                                   self.scale, True)
            n += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = (time.perf_counter() - t0) / n
        threads = min(omp_threads(), self.B * self.Hq)
        return {"value": round(self.algo_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
                "host_cores": host_cores(), "kind": "oracle",
                "sample": "%d full decode calls (B4 KV7168, all 8 heads: 32 independent (row, head) outputs) in "
                          "%.1f s, %.2f ms/call; the oracle parallelises over (query row, head) with OpenMP, so "
                          "%d of the %d host cores were busy" % (n, n * dt, dt * 1e3, threads, host_cores())}


class MergeBench:
    """kvp_merge_attention over [T=4096, H=32, D=128]: read two BF16 results and their
    FP32 lse, write the merged result and lse (HBM-bound).  Calls rotate over 4
    buffer sets (400 MB, above the 256 MB Infinity Cache), so inputs come from HBM."""
    T, H, D = 4096, 32, 128
    bytes = 3 * T * H * D * 2 + 3 * T * H * 4
    SETS = 4

    def __init__(self, seed=1237):
        import torch
        import paged_kv_cache_bf16_amd as kvp
        self.kvp = kvp
        gen = torch.Generator(device="cuda").manual_seed(seed)
        shp = (self.T, self.H, self.D)
        self.sets = []
        for _ in range(self.SETS):
            a = torch.randn(shp, generator=gen, device="cuda").to(torch.bfloat16).view(torch.int16)
            b = torch.randn(shp, generator=gen, device="cuda").to(torch.bfloat16).view(torch.int16)
            la = torch.randn(self.T, self.H, generator=gen, device="cuda") * 4
            lb = torch.randn(self.T, self.H, generator=gen, device="cuda") * 4
            self.sets.append((a, la, b, lb, torch.empty_like(a), torch.empty_like(la)))
        torch.cuda.synchronize()

    def merge(self, i):
        a, la, b, lb, out, lse = self.sets[i % self.SETS]
        self.kvp.kvp_merge_attention(a, la, b, lb, out, lse)


class CacheBench:
    """reshape_and_cache of T tokens x Hkv x Dh (K and V) into reversed pages, rotating
    over several input sets and page regions (together above the 256 MB Infinity Cache),
    so rows are read from and pages written to HBM."""

    def __init__(self, T, H, D, sets, seed=1238):
        import torch
        import paged_kv_cache_bf16_amd as kvp
        self.kvp, self.T, self.H, self.D, self.S = kvp, T, H, D, sets
        self.bytes = 2 * 2 * T * H * D * 2 + 8 * T
        pages = -(-T // 16)
        self.pool = kvp.alloc_pool(sets * pages, H, D)
        gen = torch.Generator(device="cuda").manual_seed(seed)
        pos = np.arange(T, dtype=np.int64)
        self.sets = []
        for s in range(sets):
            k = torch.randn(T, H, D, generator=gen, device="cuda").to(torch.bfloat16).view(torch.int16)
            v = torch.randn(T, H, D, generator=gen, device="cuda").to(torch.bfloat16).view(torch.int16)
            blocks = s * pages + (pages - 1 - pos // 16)
            self.sets.append((k, v, torch.from_numpy(blocks * 16 + pos % 16).cuda()))
        torch.cuda.synchronize()

    def write(self, i):
        k, v, slots = self.sets[i % self.S]
        self.kvp.reshape_and_cache(self.pool, k, v, slots)


# ----------------------------------------------------------------------------- per-config timing

def decode_sets(set_bytes, target=640 << 20, lo=8, hi=40):
    """Rotating page sets: enough that one pass over them exceeds the 256 MB Infinity Cache twice over."""
    return int(min(hi, max(lo, -(-target // set_bytes))))


def bench_prefill_config(name, w, stream, n_calls, with_cache=False, split_cols=16):
    """A prefill-shaped workload from workloads.py: one paged_attention call per graph entry."""
    up = Uploaded(w, split_cols)
    G = w.num_q_heads // w.num_kv_heads
    flops = prefill_flops(w.head_dim, w.num_q_heads, w.seq_lens, w.query_lens, w.causal)
    nbytes = attention_bytes(w.head_dim, w.num_q_heads, w.num_kv_heads, w.seq_lens, w.query_lens)
    us, ts = graph_us(up.attention, n_calls, stream)
    r = rates(us, flops=flops, nbytes=nbytes)
    c0 = up.kvp.kvp_get_counters()
    r["kernel_grid_blocks"] = c0["last_grid_blocks"]
    r["groups_us"] = [round(t, 3) for t in ts]
    r["workspace"] = None if up.ws is None else "kvp_workspace_bytes_split(..., %d)" % split_cols
    if with_cache:
        cus, _ = graph_us(up.cache_write, max(1, n_calls), stream)
        cb = 2 * 2 * int(w.slot_mapping.shape[0]) * w.num_kv_heads * w.head_dim * 2 + 8 * int(w.slot_mapping.shape[0])
        r["reshape_and_cache"] = rates(cus, nbytes=cb)
        r["reshape_and_cache"]["note"] = "all of the workload's tokens, warm (pages written again in place)"
    up.free()
    log("%s: %.2f us/call%s" % (name, us, "" if "TFLOPs" not in r else ", %.1f TFLOP/s" % r["TFLOPs"]))
    return r


def bench_decode_config(name, B, L, Hq, Hkv, D, stream, value_scale=1.0, calls=None):
    """Decode of one query per sequence: cold (rotating page sets) and warm (one set)."""
    set_bytes = B * L * Hkv * D * 4
    S = decode_sets(set_bytes)
    db = DecodeBench(B, L, Hq, Hkv, D, sets=S, value_scale=value_scale)
    cold, ts = graph_us(db.attention, S, stream)
    warm, _ = graph_us(lambda i: db.attention(0), 50, stream)
    step, _ = graph_us(db.step_set, S, stream)
    r = rates(cold, nbytes=db.algo_bytes)
    r["groups_us"] = [round(t, 3) for t in ts]
    r["warm"] = rates(warm, nbytes=db.algo_bytes)
    # kvp_decode_step (the new token's cache write in the partial launch), cold; rate over the
    # same KV-read bytes as the call
    r["step"] = rates(step, nbytes=db.algo_bytes)
    r["page_sets"] = S
    r["pool_GB"] = round(S * set_bytes / 1e9, 3)
    del db
    import torch
    torch.cuda.empty_cache()
    log("%s decode: cold %.2f us/call, warm %.2f us/call, step %.2f us" % (name, cold, warm, step))
    return r


def run_config(name, stream):
    from paged_kv_cache_bf16_amd import workloads as wl
    if name == "tiny":
        w = wl.tiny()
        return {"workload": "composition case: 1 sequence, 20 tokens, Hq 8, Hkv 2, Dh 256, table {3,1,2,0}",
                "prefill": bench_prefill_config("tiny prefill", w, stream, 50),
                "decode": bench_prefill_config("tiny decode", w.decode_view(), stream, 50)}
    if name == "decode":
        return {"workload": "decode B4 Q1 KV7168 Hq8 Hkv2 Dh128, random page permutation",
                "decode": bench_decode_config("B4 KV7168", 4, 7168, 8, 2, 128, stream)}
    if name == "prefill":
        return {"workload": "causal prefill B1 Q4096 KV4096 Hq32 Hkv8 Dh128, reversed pages",
                "prefill": bench_prefill_config("prefill B1 Q4096", wl.prefill(), stream, 20, with_cache=True)}
    if name == "suffix":
        return {"workload": "suffix prefill B4 Q128 on KV7168 Hq32 Hkv8 Dh128, reversed pages",
                "prefill": bench_prefill_config("suffix B4 Q128", wl.suffix(), stream, 20)}
    if name == "ragged":
        w = wl.ragged()
        return {"workload": "ragged B4 KV {513,4096,4171,7168}, query tails {full,128,17,1}, Hq8 Hkv2 Dh128, "
                            "2.29 GB interleaved pool (pages above 2^31 B), padded poisoned tables",
                "prefill": bench_prefill_config("ragged", w, stream, 20),
                "prefill_wide_split": bench_prefill_config("ragged, split_cols 512", w, stream, 20, split_cols=512)}
    if name.startswith("wide"):
        L = int(name[4:])
        w = wl.wide(L)
        pre = bench_prefill_config("wide L=%d prefill" % L, w, stream, 3 if L > 8000 else 10, with_cache=True)
        del w
        return {"workload": "wide-head GQA Hq16 Hkv2 Dh512, L=%d, values N(0,1)*0.5, sparse shuffled pages" % L,
                "prefill": pre,
                "decode": bench_decode_config("wide L=%d" % L, 1, L, 16, 2, 512, stream, value_scale=0.5)}
    if name == "cache":
        cb = CacheBench(4096, 8, 128, 6)
        us, _ = graph_us(cb.write, 24, stream)
        r = {"workload": "reshape_and_cache 4096 tokens x Hkv 8 x Dh 128 (K and V) into reversed pages, rotating "
                         "over 6 input sets and page regions (400 MB)", "cold": rates(us, nbytes=cb.bytes)}
        del cb
        cb = CacheBench(18432, 2, 512, 4)
        us, _ = graph_us(cb.write, 8, stream)
        r["wide18432"] = rates(us, nbytes=cb.bytes)
        r["wide18432"]["workload"] = "18432 tokens x Hkv 2 x Dh 512 (151 MB moved), rotating over 4 sets"
        del cb
        log("reshape_and_cache: %.2f us (4096 x 8 x 128), %.2f us (18432 x 2 x 512)"
            % (r["cold"]["us_per_call"], r["wide18432"]["us_per_call"]))
        return r
    if name == "merge":
        mg = MergeBench()
        us, _ = graph_us(mg.merge, 40, stream)
        log("merge: %.2f us/call" % us)
        return {"workload": "kvp_merge_attention of two [4096, 32, 128] BF16 results with FP32 lse, rotating over "
                            "4 buffer sets (400 MB)", "merge": rates(us, nbytes=MergeBench.bytes)}
    raise ValueError(name)


# ----------------------------------------------------------------------------- recorded HBM traffic

COUNTERS = os.path.join(ROOT, "profiles", "decode_b4_kv7168_hbm_counters.md")
KERNEL_SRC = os.path.join(ROOT, "paged_kv_cache_bf16_amd", "csrc", "attn_kernel.hip")


def recorded_traffic(kernel):
    """HBM bytes per launch (read + write) of `kernel` from the committed rocprofv3
    counter summary, or None when that summary was taken on other kernel source."""
    import hashlib
    try:
        text = open(COUNTERS).read()
    except OSError:
        return None
    sha = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()
    if ("kernel_source_sha256: " + sha) not in text:
        return None
    for line in text.splitlines():
        if line.startswith("traffic " + kernel + " "):
            f = dict(x.split("=") for x in line.split()[2:])
            return int(f["read_bytes"]) + int(f["write_bytes"])
    return None


def _sum_or_none(*xs):
    return None if any(x is None for x in xs) else sum(xs)


# ----------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1400)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--sets", type=int, default=40, help="rotating decode page sets of the headline")
    ap.add_argument("--only", choices=CONFIG_NAMES, help="time only this config (no headline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="headline only")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run 3 device copies of this many MiB (a known-size kernel for HBM counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the pool lives on one device); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_bf16_amd as kvp
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()

    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration: 3 copies of %d MiB (read %d B + write %d B each)" % (args.calibrate_copy_mib, 4 * n, 4 * n))
        del src, dst

    if args.only:
        print(json.dumps({"only": args.only, args.only: run_config(args.only, stream)}), flush=True)
        return

    log("setting up decode workload (%d page sets)" % args.sets)
    dec = DecodeBench(sets=args.sets)
    log("decode set-up done; checking against the oracle")
    mx, mean, opool = dec.check_against_oracle()
    log("decode parity: max_abs=%.3g mean_abs=%.3g" % (mx, mean))
    assert mx <= 2e-2 and mean <= 2e-3, "decode output out of tolerance"

    # eager issue first (kernels loaded, and the eager rate for reference)
    for _ in range(args.warmup):
        dec.step()
    torch.cuda.synchronize()
    eager_us = time_launches(dec.step, args.steps, stream)
    log("decode, eager issue: %.2f us/step" % eager_us)

    # timed steps: replayed from HIP graphs that hold the S page sets' steps in
    # order, so no host launch work sits between steps (issued eagerly from
    # Python, two kernel launches alone take ~10 us)
    full, rem = divmod(args.steps, dec.S)
    g_full = capture(dec.step_set, dec.S)
    g_rem = capture(dec.step_set, rem) if rem else None
    for _ in range(max(1, -(-args.warmup // dec.S))):
        g_full.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(full):
        g_full.replay()
    if g_rem is not None:
        g_rem.replay()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(end) / args.steps
    log("decode: %.2f us/step (wall %.2f us/step)" % (ms_step * 1e3, wall / args.steps * 1e6))
    del g_full, g_rem

    # dominant kernels alone (one paged_attention call: partial + fold): a graph
    # of S calls over the rotating page sets, 7 groups of 5 replays, median
    attn_us, groups = graph_us(dec.attention, dec.S, stream, groups=7, replays=5)
    log("decode attention: %.2f us/call (groups %s)" % (attn_us, ["%.2f" % g for g in groups]))
    lse_us, _ = graph_us(dec.attention_lse, dec.S, stream)
    log("decode attention with lse: %.2f us/call" % lse_us)
    warm_us, _ = graph_us(lambda i: dec.attention(0), 50, stream)
    eager_attn_us = float(np.median([time_launches(dec.attention_only, 200, stream) for _ in range(5)]))
    c0 = kvp.kvp_get_counters()
    assert c0["split_kv_launches"] > 0 and c0["fused_decode_steps"] > 0

    result = {
        "metric": METRIC,
        "value": round(dec.algo_bytes / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode B4 Q1 KV7168 Hq8 Hkv2 Dh128 page16 (random page permutation), "
                               "%d rotating page sets over a %.2f GB pool; step = kvp_decode_step: reshape_and_cache of "
                               "the 4 new tokens + split-KV decode (cache write fused into the partial kernel); steps "
                               "replayed from HIP graphs of %d consecutive steps" % (dec.S, dec.S * dec.kv_bytes / 1e9,
                                                                                 dec.S),
                   "global_batch": dec.B, "seq_len": dec.L, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(dec.algo_bytes / (attn_us * 1e-6) / 1e9, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dec.algo_bytes / (attn_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": _sum_or_none(recorded_traffic("split_partial_kernel<128,false>"),
                                             recorded_traffic("split_fold_kernel<128>")),
                     "kernel": "split_partial_kernel<128,false> + split_fold_kernel<128> (one paged_attention "
                               "decode call, timed with HIP events around graph replays of %d calls)" % dec.S,
                     "us_per_call": round(attn_us, 3),
                     "algo_bytes_per_call": dec.algo_bytes},
        "decode_eager": {"us_per_step": round(eager_us, 3), "GBps": round(dec.algo_bytes / (eager_us * 1e-6) / 1e9, 2),
                         "attention_us_per_call": round(eager_attn_us, 3),
                         "note": "the same steps issued one by one from Python (host launch cost included)"},
        "decode_lse": {"us_per_call": round(lse_us, 3), "note": "paged_attention_lse on the decode workload"},
        "decode_warm_cache": rates(warm_us, nbytes=dec.algo_bytes),
        "parity": {"decode_max_abs": mx, "decode_mean_abs": mean},
        "host_cores": host_cores(),
        "context": "the pages report 0.272859 ms for B4 Q1 KV7168 paged attention on MI300X (head counts not "
                   "given); not comparable as a target",
    }

    if not args.no_configs:
        cfgs = {}
        for name in CONFIG_NAMES:
            if name == "decode":
                continue                                 # the headline's call is the cold decode of this config
            cfgs[name] = run_config(name, stream)
        cfgs["decode"] = {"workload": "decode B4 Q1 KV7168 Hq8 Hkv2 Dh128 (the headline's call)",
                          "decode": dict(rates(attn_us, nbytes=dec.algo_bytes), warm=rates(warm_us,
                                                                                             nbytes=dec.algo_bytes),
                                         page_sets=dec.S)}
        result["configs"] = cfgs

    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        result["cpu_baseline"] = dec.cpu_baseline(opool, budget_s=args.cpu_seconds)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
