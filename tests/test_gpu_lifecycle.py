"""Lifecycle gate of "ROCm: harden compact peer-local KV prefill for
Gemma-4" (Required hardening: repeated sequential requests must not grow
VRAM or host RAM): 1,000 calls of each entry point, with device free memory
and host resident memory read after a warm-up and at the end.  The library
allocates no device memory (the caller passes every buffer), so device free
memory must not move at all; host memory may move only by allocator noise.
"""
import os

import numpy as np
import pytest
import torch

import paged_kv_cache_bf16_amd as kvp
from paged_kv_cache_bf16_amd import workloads as wl
from harness import GpuCase, bitwise, dev_bits

pytestmark = pytest.mark.gpu


def _rss_bytes():
    with open("/proc/self/statm") as f:
        return int(f.read().split()[1]) * os.sysconf("SC_PAGE_SIZE")


def test_thousand_calls_no_memory_growth():
    w = wl.random_case(1717, [700, 2000, 129, 40], [1, 1, 1, 1], 8, 2, 128)
    g = GpuCase(w)
    wp = wl.random_case(1718, [600, 300], [600, 300], 8, 2, 128)
    gp = GpuCase(wp)
    rng = np.random.default_rng(5)
    kn = dev_bits(wl.to_bf16_bits(rng.standard_normal((4, 2, 128)).astype(np.float32)))
    vn = dev_bits(wl.to_bf16_bits(rng.standard_normal((4, 2, 128)).astype(np.float32)))
    slots = torch.from_numpy(np.array([int(w.block_tables[b, (L - 1) // 16]) * 16 + (L - 1) % 16
                                       for b, L in enumerate(w.seq_lens)], np.int64)).cuda()
    lse = torch.empty((4, 8), dtype=torch.float32, device="cuda")
    ms = int(w.seq_lens.max())

    def one_round():
        kvp.kvp_decode_step(g.pool, kn, vn, slots, g.q, g.out, 8, g.bt, g.seq_lens, g.qsl, 1, ms, w.scale, True,
                            workspace=g.ws)
        kvp.paged_attention_lse(g.pool, g.q, g.out, lse, 8, g.bt, g.seq_lens, g.qsl, 1, ms, w.scale, True,
                                workspace=g.ws)
        kvp.reshape_and_cache(gp.pool, gp.k, gp.v, gp.slots)
        kvp.paged_attention(gp.pool, gp.q, gp.out, 8, gp.bt, gp.seq_lens, gp.qsl, 600, 600, wp.scale, True)

    st = g.pool.storage
    page = 2 * 16 * 128
    for _ in range(50):
        one_round()
    torch.cuda.synchronize()
    first = g.out.clone()
    free0, _ = torch.cuda.mem_get_info()
    alloc0 = torch.cuda.memory_allocated()
    rss0 = _rss_bytes()
    for i in range(1000):
        one_round()
        # a pool descriptor created and destroyed per request (host-side only)
        h = kvp.kv_pool_create((st, 0), (st, page * w.num_blocks), w.num_blocks, 2, 128, page, page, storage=st)
        del h
        if i % 250 == 249:
            torch.cuda.synchronize()
            print("calls %d: device free %d B, host rss %d B" % (i + 1, torch.cuda.mem_get_info()[0], _rss_bytes()),
                  flush=True)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    rss1 = _rss_bytes()
    print("device free: %d -> %d B; torch allocated %d -> %d B; host rss %d -> %d B"
          % (free0, free1, alloc0, torch.cuda.memory_allocated(), rss0, rss1), flush=True)
    assert free1 == free0, "device free memory moved by %d B over 1000 calls" % (free0 - free1)
    assert torch.cuda.memory_allocated() == alloc0
    assert rss1 - rss0 < 8 << 20, "host resident memory grew by %d B over 1000 calls" % (rss1 - rss0)
    bitwise(g.out.cpu().numpy().view(np.uint16), first.cpu().numpy().view(np.uint16), "call 1050 vs call 50")
