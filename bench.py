#!/usr/bin/env python3
"""Benchmark of the paged BF16 KV-cache hot path on one MI355X.

One step = one pass of the whole path over one batch: write the batch's new
K/V rows into the pool (reshape_and_cache), then paged attention over the
pool.  Inputs are seeded synthetic BF16 N(0,1) data resident in HBM.

Headline (default --workload decode): B=4 sequences, one query each, KV
length 7168, Hq 8 / Hkv 2 / Dh 128, 16-token pages permuted at random.  The
pool holds 40 disjoint page sets (1.17 GB, well above the 256 MB Infinity
Cache) and step i uses set i % 40, so every step reads K/V from HBM.
The timed steps are replayed from HIP graphs that each hold 40 consecutive
steps (the library's calls are capture-safe), so host launch work does not
sit between steps; the eagerly issued rate is reported beside it.
value = decode KV-read bytes per step / step time (GB/s).  The causal
prefill B=1 Q=KV=4096 Hq 32 / Hkv 8 is measured in the same run and
reported under "prefill" (TFLOP/s vs the BF16 MFMA peak).

Roofline: the dominant kernels' average duration (one paged_attention call:
partial + fold) is timed live with HIP events around graph replays of 40
calls on the launch stream; algorithmic bytes
(or FLOPs) per launch / that duration, against MI355X peaks (HBM 8 TB/s,
dense BF16 MFMA 2.5 PFLOP/s).  cpu_baseline: the CPU oracle timed on this
host on a bounded sample of the same workload.
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- set-up helpers

def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


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


class DecodeBench:
    """B=4 x KV7168 decode over S rotating page sets."""

    def __init__(self, sets=40, seed=1235):
        import torch
        import paged_kv_cache_bf16_amd as kvp
        from paged_kv_cache_bf16_amd import workloads as wl
        self.kvp = kvp
        self.B, self.L, self.Hq, self.Hkv, self.D = 4, 7168, 8, 2, 128
        self.S = sets
        W = self.L // 16
        rng = np.random.default_rng(seed)
        nb = sets * self.B * W
        bt = rng.permutation(nb).astype(np.int32).reshape(sets * self.B, W)
        self.pool = kvp.alloc_pool(nb, self.Hkv, self.D, interleaved=False)
        # fill every page with seeded N(0,1) BF16 through reshape_and_cache, one set at a time
        gen = torch.Generator(device="cuda").manual_seed(seed)
        self.sl = torch.full((self.B,), self.L, dtype=torch.int32, device="cuda")
        self.qsl = torch.arange(self.B + 1, dtype=torch.int32, device="cuda")
        self.bt, self.q, self.knew, self.vnew, self.slot_new = [], [], [], [], []
        pos = np.arange(self.L, dtype=np.int64)
        for s in range(sets):
            rows = bt[s * self.B:(s + 1) * self.B]
            slots = np.concatenate([rows[b, pos // 16].astype(np.int64) * 16 + pos % 16 for b in range(self.B)])
            T = slots.shape[0]
            k = torch.randn(T, self.Hkv, self.D, generator=gen, device="cuda").to(torch.bfloat16).view(torch.int16)
            v = torch.randn(T, self.Hkv, self.D, generator=gen, device="cuda").to(torch.bfloat16).view(torch.int16)
            sd = torch.from_numpy(slots).cuda()
            kvp.reshape_and_cache(self.pool, k, v, sd)
            last = torch.arange(self.B, device="cuda") * self.L + self.L - 1
            self.knew.append(k[last].contiguous())
            self.vnew.append(v[last].contiguous())
            self.slot_new.append(sd[last].contiguous())
            self.bt.append(torch.from_numpy(kvp.kv_prepare_block_tables(self.pool, rows, [self.L] * self.B)).cuda())
            self.q.append(torch.randn(self.B, self.Hq, self.D, generator=gen, device="cuda")
                          .to(torch.bfloat16).view(torch.int16))
            if s == 0:
                self.host0 = dict(k=k.cpu().numpy().view(np.uint16), v=v.cpu().numpy().view(np.uint16),
                                  slots=slots, bt=rows.copy(), q=self.q[0].cpu().numpy().view(np.uint16))
            del k, v
        self.out = torch.zeros(self.B, self.Hq, self.D, dtype=torch.int16, device="cuda")
        self.lse = torch.zeros(self.B, self.Hq, dtype=torch.float32, device="cuda")
        self.ws = kvp.alloc_workspace(self.pool, self.Hq, self.B, self.L)
        self.scale = 1.0 / math.sqrt(self.D)
        self.i = 0
        torch.cuda.synchronize()

    @property
    def kv_bytes(self):
        return self.B * self.L * self.Hkv * self.D * 2 * 2

    @property
    def algo_bytes(self):
        # K/V read + q read + out write + active block-table entries
        return self.kv_bytes + 2 * self.B * self.Hq * self.D * 2 + self.B * (self.L // 16) * 4

    def attention(self, s):
        self.kvp.paged_attention(self.pool, self.q[s], self.out, self.Hq, self.bt[s], self.sl, self.qsl, 1, self.L,
                                 self.scale, True, workspace=self.ws)

    def step_set(self, s):
        # one step on page set s: reshape_and_cache of the 4 new tokens + decode
        # attention, through kvp_decode_step (one partial launch + the fold)
        self.kvp.kvp_decode_step(self.pool, self.knew[s], self.vnew[s], self.slot_new[s], self.q[s], self.out,
                                 self.Hq, self.bt[s], self.sl, self.qsl, 1, self.L, self.scale, True,
                                 workspace=self.ws)

    def step(self):
        s = self.i % self.S
        self.i += 1
        self.step_set(s)

    def capture(self, fn, n):
        """One HIP graph holding fn(s) for page sets s = 0 .. n-1 in order (no host work between them)."""
        import torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for s in range(n):
                fn(s)
        torch.cuda.synchronize()
        return g

    def attention_lse(self, s):
        self.kvp.paged_attention_lse(self.pool, self.q[s], self.out, self.lse, self.Hq, self.bt[s], self.sl,
                                     self.qsl, 1, self.L, self.scale, True, workspace=self.ws)

    def attention_only(self):
        s = self.i % self.S
        self.i += 1
        self.attention(s)

    def check_against_oracle(self):
        """Set 0 output vs the oracle (tolerance), so the timed path is a correct one."""
        import oracle
        h = self.host0
        self.attention(0)
        import torch
        torch.cuda.synchronize()
        got = oracle.bf16_bits_to_f32(self.out.cpu().numpy().view(np.uint16))
        pool = oracle.Pool(self.S * self.B * (self.L // 16), self.Hkv, self.D)
        oracle.reshape_and_cache(pool, h["k"], h["v"], h["slots"])
        ref = oracle.paged_attention(h["q"], pool, h["bt"], [self.L] * self.B, np.arange(self.B + 1),
                                     self.Hq, self.scale, True)
        err = np.abs(got.astype(np.float64) - ref)
        return float(err.max()), float(err.mean()), pool, ref

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
        threads = min(_omp_threads(), self.B)
        return {"value": round(self.algo_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
                "kind": "oracle",
                "sample": "%d full decode calls (B4 KV7168, all 8 heads) in %.1f s, %.1f ms/call; the oracle "
                          "parallelises over query rows, so %d threads were busy" % (n, n * dt, dt * 1e3, threads)}


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
        self.i = 0
        torch.cuda.synchronize()

    def merge(self):
        a, la, b, lb, out, lse = self.sets[self.i % self.SETS]
        self.i += 1
        self.kvp.kvp_merge_attention(a, la, b, lb, out, lse)


class CacheBench:
    """reshape_and_cache of 4096 tokens x Hkv 8 x Dh 128 (K and V) into reversed pages,
    rotating over 6 input sets and 6 page regions (400 MB, above the 256 MB Infinity
    Cache), so rows are read from and pages written to HBM."""
    T, H, D, SETS = 4096, 8, 128, 6
    bytes = 2 * 2 * T * H * D * 2 + 8 * T

    def __init__(self, seed=1238):
        import torch
        import paged_kv_cache_bf16_amd as kvp
        self.kvp = kvp
        pages = self.T // 16
        self.pool = kvp.alloc_pool(self.SETS * pages, self.H, self.D)
        gen = torch.Generator(device="cuda").manual_seed(seed)
        pos = np.arange(self.T, dtype=np.int64)
        self.sets = []
        for s in range(self.SETS):
            k = torch.randn(self.T, self.H, self.D, generator=gen, device="cuda").to(torch.bfloat16).view(torch.int16)
            v = torch.randn(self.T, self.H, self.D, generator=gen, device="cuda").to(torch.bfloat16).view(torch.int16)
            blocks = s * pages + (pages - 1 - pos // 16)
            slots = torch.from_numpy(blocks * 16 + pos % 16).cuda()
            self.sets.append((k, v, slots))
        self.i = 0
        torch.cuda.synchronize()

    def write(self):
        k, v, slots = self.sets[self.i % self.SETS]
        self.i += 1
        self.kvp.reshape_and_cache(self.pool, k, v, slots)


class PrefillBench:
    """Causal prefill B=1, Q=KV=4096, Hq 32 / Hkv 8, Dh 128, reversed pages."""

    def __init__(self, seed=1236):
        import torch
        import paged_kv_cache_bf16_amd as kvp
        from paged_kv_cache_bf16_amd import workloads as wl
        self.kvp = kvp
        self.w = w = wl.prefill()
        self.pool = kvp.alloc_pool(w.num_blocks, w.num_kv_heads, w.head_dim)
        self.k, self.v = to_dev(w.k), to_dev(w.v)
        self.slots = torch.from_numpy(w.slot_mapping).cuda()
        kvp.reshape_and_cache(self.pool, self.k, self.v, self.slots)
        self.bt = torch.from_numpy(kvp.kv_prepare_block_tables(self.pool, w.block_tables, w.seq_lens)).cuda()
        self.sl = torch.from_numpy(w.seq_lens).cuda()
        self.qsl = torch.from_numpy(w.query_start_loc).cuda()
        self.q = to_dev(w.q)
        self.out = torch.zeros_like(self.q)
        self.L = int(w.seq_lens[0])
        torch.cuda.synchronize()

    @property
    def flops(self):
        w = self.w
        return 4.0 * w.head_dim * w.num_q_heads * (self.L * (self.L + 1) / 2)

    def attention(self):
        w = self.w
        self.kvp.paged_attention(self.pool, self.q, self.out, w.num_q_heads, self.bt, self.sl, self.qsl, self.L,
                                 self.L, w.scale, True)

    def cache_write(self):
        self.kvp.reshape_and_cache(self.pool, self.k, self.v, self.slots)

    def step(self):
        self.cache_write()
        self.attention()


COUNTERS = os.path.join(ROOT, "profiles", "bench_default_hbm_counters.md")
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


def _omp_threads():
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    return min(aff, int(env)) if env and env.isdigit() else aff


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1400)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--sets", type=int, default=40, help="rotating decode page sets")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
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

    log("setting up decode workload (%d page sets)" % args.sets)
    dec = DecodeBench(sets=args.sets)
    log("decode set-up done; checking against the oracle")
    mx, mean, opool, _ = dec.check_against_oracle()
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
    g_full = dec.capture(dec.step_set, dec.S)
    g_rem = dec.capture(dec.step_set, rem) if rem else None
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
    g_attn = dec.capture(dec.attention, dec.S)
    g_attn.replay()
    groups = [time_launches(g_attn.replay, 5, stream) / dec.S for _ in range(7)]
    attn_us = float(np.median(groups))
    log("decode attention: %.2f us/call (groups %s)" % (attn_us, ["%.2f" % g for g in groups]))
    del g_attn
    g_lse = dec.capture(dec.attention_lse, dec.S)
    g_lse.replay()
    lse_us = float(np.median([time_launches(g_lse.replay, 5, stream) / dec.S for _ in range(5)]))
    log("decode attention with lse: %.2f us/call" % lse_us)
    del g_lse
    # the same with the pool warm in the Infinity Cache (one page set), eager
    warm_us = time_launches(lambda: dec.attention(0), 400, stream)
    eager_attn_us = float(np.median([time_launches(dec.attention_only, 200, stream) for _ in range(5)]))

    c0 = kvp.kvp_get_counters()
    assert c0["split_kv_launches"] > 0 and c0["fused_decode_steps"] > 0

    # merge of two results over disjoint key sets at the prefill shape (4096 tokens x 32 heads x 128)
    mg = MergeBench()
    m_us = float(np.median([time_launches(mg.merge, 50, stream) for _ in range(5)]))
    log("merge: %.2f us/call, %.0f GB/s" % (m_us, mg.bytes / (m_us * 1e-6) / 1e9))
    del mg

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
                     "kernel": "split_partial_kernel<128> + split_fold_kernel<128> (one paged_attention call)",
                     "us_per_call": round(attn_us, 3),
                     "algo_bytes_per_call": dec.algo_bytes},
        "decode_eager": {"us_per_step": round(eager_us, 3), "GBps": round(dec.algo_bytes / (eager_us * 1e-6) / 1e9, 2),
                         "attention_us_per_call": round(eager_attn_us, 3),
                         "note": "the same steps issued one by one from Python (host launch cost included)"},
        "decode_lse": {"us_per_call": round(lse_us, 3), "note": "paged_attention_lse on the decode workload"},
        "merge": {"workload": "kvp_merge_attention of two [4096, 32, 128] BF16 results with FP32 lse",
                  "us_per_call": round(m_us, 3), "bytes_per_call": MergeBench.bytes,
                  "GBps": round(MergeBench.bytes / (m_us * 1e-6) / 1e9, 1),
                  "frac": round(MergeBench.bytes / (m_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
        "decode_warm_cache": {"us_per_call": round(warm_us, 3),
                              "GBps": round(dec.algo_bytes / (warm_us * 1e-6) / 1e9, 1)},
        "parity": {"decode_max_abs": mx, "decode_mean_abs": mean},
        "context": "the pages report 0.272859 ms for B4 Q1 KV7168 paged attention on MI300X (head counts not "
                   "given); not comparable as a target",
    }

    if not args.no_prefill:
        log("setting up prefill workload")
        pre = PrefillBench()
        for _ in range(3):
            pre.step()
        torch.cuda.synchronize()
        step_us = time_launches(pre.step, 20, stream)
        pgroups = [time_launches(pre.attention, 20, stream) for _ in range(5)]
        p_us = float(np.median(pgroups))
        tf = pre.flops / (p_us * 1e-6) / 1e12
        result["prefill"] = {"workload": "causal prefill B1 Q4096 KV4096 Hq32 Hkv8 Dh128 page16 reversed pages",
                             "us_per_call": round(p_us, 2), "us_per_step_with_cache_write": round(step_us, 2),
                             "TFLOPs": round(tf, 2), "peak_TFLOPs": BF16_PEAK_TFLOPS,
                             "frac": round(tf / BF16_PEAK_TFLOPS, 4), "flops_per_call": pre.flops,
                             "kernel": "prefill_pp_kernel<128, 2>",
                             "hbm_traffic_bytes": recorded_traffic("prefill_pp_kernel<128,2>")}
        log("prefill: %.2f us/call, %.1f TFLOP/s" % (p_us, tf))
        cb = CacheBench()
        cb.write()
        c_us = float(np.median([time_launches(cb.write, 24, stream) for _ in range(5)]))
        result["reshape_and_cache"] = {"workload": "4096 tokens x Hkv 8 x Dh 128 (K and V) into reversed pages, "
                                                   "rotating over 6 input sets and page regions (400 MB)",
                                       "us_per_call": round(c_us, 3), "bytes_per_call": CacheBench.bytes,
                                       "GBps": round(CacheBench.bytes / (c_us * 1e-6) / 1e9, 1),
                                       "frac": round(CacheBench.bytes / (c_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        del cb
        log("reshape_and_cache: %.2f us/call" % c_us)
        del pre

    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        result["cpu_baseline"] = dec.cpu_baseline(opool, budget_s=args.cpu_seconds)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
