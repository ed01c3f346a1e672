"""Seeded synthetic workloads for the paged KV-cache composition.

This module only draws inputs: BF16 tensors, block tables, slot mappings,
sequence lengths and query offsets.  It holds none of the attention or cache
arithmetic, and both the HIP path's tests and the CPU oracle read from it.

Shapes follow the workloads on the pages:
  * tiny      -- the composition case of "test(rocm): ReshapeAndCache->
                 PagedAttention composition at real dims" (Dh 256, Hq 8,
                 Hkv 2, 16-token pages, table {3,1,2,0}, 20 tokens).
  * decode, prefill, suffix, ragged -- the operator-benchmark and
                 additional-check shapes of "fix(rocm): stabilize direct paged
                 CK attention for bitwise R/R" (B4 Q1 KV7168; B1 Q4096 KV4096;
                 B4 Q128 KV7168; KV lengths 513/4096/4171/7168 with full /
                 128 / 17 / 1 query tails, >2 GB interleaved pool).
  * wide*     -- the geometry of "ROCm: harden compact peer-local KV prefill
                 for Gemma-4" (Hq 16, Hkv 2, d 512, ~3k / ~11k / ~18k).

Values are FP32 N(0, 1) drawn with numpy's PCG64, rounded to BF16 (nearest
even), seed 1234 + the workload's index.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

BLOCK_SIZE = 16
BASE_SEED = 1234


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> BF16 bit patterns, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@dataclasses.dataclass
class Workload:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    interleaved: bool
    block_tables: np.ndarray      # [B, W] int32, raw (unsanitised padding allowed)
    seq_lens: np.ndarray          # [B] int32
    query_lens: np.ndarray        # [B] int32
    kv_tokens: np.ndarray         # [T] int64: (sequence, position) order of the K/V rows below
    slot_mapping: np.ndarray      # [T] int64
    k: np.ndarray                 # [T, Hkv, D] uint16 (BF16 bits)
    v: np.ndarray                 # [T, Hkv, D] uint16
    q: np.ndarray                 # [Tq, Hq, D] uint16
    scale: float
    causal: bool = True

    @property
    def batch(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def query_start_loc(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.query_lens)]).astype(np.int32)

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max()) if self.batch else 0

    def decode_view(self) -> "Workload":
        """The same cache with one query per sequence: the last position of each row."""
        qsl = self.query_start_loc
        last = qsl[1:] - 1
        return dataclasses.replace(self, name=self.name + "-decode", q=self.q[last].copy(),
                                   query_lens=np.ones_like(self.query_lens))


def _slots_for(block_tables, seq_lens):
    """Slot of logical token i of row b: block_tables[b][i // 16] * 16 + i % 16."""
    slots = []
    for b, L in enumerate(seq_lens):
        i = np.arange(int(L), dtype=np.int64)
        slots.append(block_tables[b, i // BLOCK_SIZE].astype(np.int64) * BLOCK_SIZE + i % BLOCK_SIZE)
    return np.concatenate(slots) if slots else np.zeros(0, np.int64)


def _draw(rng, shape, mult=1.0):
    return to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(mult))


def build(name, seq_lens, query_lens, Hq, Hkv, D, block_tables, num_blocks, *, interleaved=False,
          seed=BASE_SEED, value_scale=1.0, causal=True, scale=None) -> Workload:
    rng = np.random.default_rng(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    query_lens = np.asarray(query_lens, dtype=np.int32)
    block_tables = np.asarray(block_tables, dtype=np.int32)
    slots = _slots_for(block_tables, seq_lens)
    T = slots.shape[0]
    k = _draw(rng, (T, Hkv, D), value_scale)
    v = _draw(rng, (T, Hkv, D), value_scale)
    q = _draw(rng, (int(query_lens.sum()), Hq, D), value_scale)
    kv_tokens = np.arange(T, dtype=np.int64)
    return Workload(name, Hq, Hkv, D, int(num_blocks), interleaved, block_tables, seq_lens,
                    query_lens, kv_tokens, slots, k, v, q,
                    float(scale if scale is not None else 1.0 / math.sqrt(D)), causal)


def _pages(L):
    return (int(L) + BLOCK_SIZE - 1) // BLOCK_SIZE


def tiny(seed=BASE_SEED + 0):
    bt = np.array([[3, 1, 2, 0]], np.int32)
    return build("tiny", [20], [20], 8, 2, 256, bt, 4, seed=seed)


def decode(seed=BASE_SEED + 1, batch=4, kv_len=7168, sets=1):
    """B sequences of kv_len tokens, pages permuted at random over a shared pool.

    With sets > 1 the pool holds `sets` disjoint copies of the active page
    set, and `block_tables` is [sets * B, W]: rows s*B .. s*B+B-1 are set s.
    """
    rng = np.random.default_rng(seed)
    W = _pages(kv_len)
    nb = sets * batch * W
    perm = rng.permutation(nb).astype(np.int32)
    bt = perm.reshape(sets * batch, W)
    wl = build("decode", [kv_len] * (sets * batch), [1] * (sets * batch), 8, 2, 128, bt, nb,
               seed=seed)
    return wl


def prefill(seed=BASE_SEED + 2, L=4096):
    W = _pages(L)
    bt = (W - 1 - np.arange(W, dtype=np.int32))[None, :]          # reversed physical order
    return build("prefill", [L], [L], 32, 8, 128, bt, W, seed=seed)


def suffix(seed=BASE_SEED + 3, batch=4, kv_len=7168, q_len=128):
    W = _pages(kv_len)
    nb = batch * W
    bt = (nb - 1 - np.arange(nb, dtype=np.int32)).reshape(batch, W)  # reversed over the pool
    return build("suffix", [kv_len] * batch, [q_len] * batch, 32, 8, 128, bt, nb, seed=seed)


RAGGED_POOL_BLOCKS = 140_000          # x 16 KB per block = 2.29 GB > 2**31 bytes


def ragged(seed=BASE_SEED + 4, num_blocks=RAGGED_POOL_BLOCKS, pad_cols=5):
    """KV lengths {513, 4096, 4171, 7168}, query tails {full, 128, 17, 1}.

    One interleaved pool (each block: K pages then V pages, 16 KB).  Active
    pages are shuffled; all but one sit above byte offset 2**31 and one sits
    below it.  Table rows are padded past their last page with poison values
    (-1 and INT32_MAX) that page-table preparation must sanitise.
    """
    rng = np.random.default_rng(seed)
    seq_lens = [513, 4096, 4171, 7168]
    q_lens = [513, 128, 17, 1]
    npages = [_pages(L) for L in seq_lens]
    total = sum(npages)
    block_bytes = 2 * 2 * BLOCK_SIZE * 128 * 2
    first_high = (2 ** 31) // block_bytes + 1
    high = rng.choice(np.arange(first_high, num_blocks, dtype=np.int64), size=total - 1, replace=False)
    low = rng.integers(0, first_high, size=1)
    phys = rng.permutation(np.concatenate([high, low])).astype(np.int32)
    W = max(npages) + pad_cols
    bt = np.empty((4, W), np.int32)
    off = 0
    for b, n in enumerate(npages):
        bt[b, :n] = phys[off:off + n]
        off += n
        bt[b, n:] = np.where(np.arange(W - n) % 2 == 0, -1, np.iinfo(np.int32).max)
    return build("ragged", seq_lens, q_lens, 8, 2, 128, bt, num_blocks, interleaved=True, seed=seed)


WIDE_LENGTHS = (3072, 11264, 18432)


def wide(L, seed=BASE_SEED + 5):
    """Hq 16 / Hkv 2 / Dh 512, values N(0,1)*0.5, pages drawn sparsely from a pool 4x larger."""
    rng = np.random.default_rng(seed + L)
    W = _pages(L)
    nb = 4 * W
    bt = rng.choice(nb, size=W, replace=False).astype(np.int32)[None, :]
    return build("wide%d" % L, [L], [L], 16, 2, 512, bt, nb, seed=seed + L, value_scale=0.5)


def random_case(seed, seq_lens, query_lens, Hq, Hkv, D, *, spare_blocks=3, interleaved=False,
                causal=True, value_scale=1.0):
    """A small ragged case with a shuffled pool (for parity sweeps)."""
    rng = np.random.default_rng(seed)
    npages = [_pages(L) for L in seq_lens]
    nb = sum(npages) + spare_blocks
    perm = rng.permutation(nb).astype(np.int32)
    W = max(npages + [1])
    bt = np.zeros((len(seq_lens), W), np.int32)
    off = 0
    for b, n in enumerate(npages):
        bt[b, :n] = perm[off:off + n]
        off += n
    return build("random", seq_lens, query_lens, Hq, Hkv, D, bt, nb, seed=seed + 1,
                 interleaved=interleaved, causal=causal, value_scale=value_scale)


CONFIGS = {
    "tiny": tiny,
    "decode": decode,
    "prefill": prefill,
    "suffix": suffix,
    "ragged": ragged,
    "wide3072": lambda: wide(3072),
    "wide11264": lambda: wide(11264),
    "wide18432": lambda: wide(18432),
}
