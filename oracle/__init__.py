"""CPU oracle for the paged BF16 KV-cache composition -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package.  The product path (the HIP
library and its Python binding) never imports, links or calls it, and it
shares no code with them.

The arithmetic lives in ``kvp_oracle.c`` (plain C, FP32 accumulation, OpenMP
only across independent output rows).  This module builds it with gcc and
marshals numpy arrays; it adds no arithmetic of its own apart from the
float32 -> bf16 bit conversion used for display.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvp_oracle.c")
_LIB = os.path.join(_HERE, "libkvp_oracle.so")
_lib = None

BLOCK_SIZE = 16


def build(force: bool = False) -> str:
    """Compile kvp_oracle.c into libkvp_oracle.so with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                               "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32, f32 = ctypes.c_int64, ctypes.c_int, ctypes.c_float
        lib.oracle_reshape_and_cache.argtypes = [P, P, i64, i32, i32, i64, i64, P, P, i64, i64, i64, P]
        lib.oracle_reshape_and_cache.restype = ctypes.c_int
        lib.oracle_paged_attention.argtypes = [P, P, P, P, i64, i64, i64, P, i32, i32, P, P, i32, i32,
                                               i32, f32, i32, P, i64, P]
        lib.oracle_paged_attention.restype = ctypes.c_int
        lib.oracle_prepare_block_tables.argtypes = [P, P, i32, i32, P, i64]
        lib.oracle_prepare_block_tables.restype = ctypes.c_int
        lib.oracle_merge_states.argtypes = [P, P, P, P, P, P, i64, i32]
        lib.oracle_merge_states.restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


class OracleError(ValueError):
    pass


class Pool:
    """A host KV pool in the shared page layout.

    ``storage`` is one flat uint16 array (BF16 bits).  K pages start at
    element ``k_offset`` and V pages at ``v_offset``; block b's pages are
    ``k_block_stride`` / ``v_block_stride`` elements after block b-1's.
    Separate pools use two disjoint ranges; an interleaved pool puts each
    block's V pages right after its K pages.
    """

    def __init__(self, num_blocks, num_kv_heads, head_dim, interleaved=False, fill_bits=0):
        self.num_blocks = int(num_blocks)
        self.num_kv_heads = int(num_kv_heads)
        self.head_dim = int(head_dim)
        page = num_kv_heads * BLOCK_SIZE * head_dim
        self.interleaved = interleaved
        if interleaved:
            self.k_block_stride = self.v_block_stride = 2 * page
            self.k_offset, self.v_offset = 0, page
        else:
            self.k_block_stride = self.v_block_stride = page
            self.k_offset, self.v_offset = 0, num_blocks * page
        n = 2 * num_blocks * page
        # np.zeros maps untouched pages lazily, so very large sparse pools are cheap
        self.storage = np.zeros(n, dtype=np.uint16) if fill_bits == 0 else np.full(n, fill_bits, np.uint16)

    def _kv_ptrs(self):
        base = self.storage.ctypes.data
        return ctypes.c_void_p(base + 2 * self.k_offset), ctypes.c_void_p(base + 2 * self.v_offset)


def reshape_and_cache(pool: Pool, k: np.ndarray, v: np.ndarray, slot_mapping: np.ndarray) -> None:
    """Scatter k, v ([T, Hkv, D] uint16 BF16 bits) into ``pool`` at ``slot_mapping`` ([T] int64)."""
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    slots = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    T = slots.shape[0]
    assert k.shape == (T, pool.num_kv_heads, pool.head_dim) == v.shape
    kp, vp = pool._kv_ptrs()
    rc = _load().oracle_reshape_and_cache(kp, vp, pool.num_blocks, pool.num_kv_heads, pool.head_dim,
                                          pool.k_block_stride, pool.v_block_stride, _ptr(k), _ptr(v),
                                          T, pool.num_kv_heads * pool.head_dim,
                                          pool.num_kv_heads * pool.head_dim, _ptr(slots))
    if rc != 0:
        raise OracleError("reshape_and_cache: invalid slot mapping")


def paged_attention(q: np.ndarray, pool: Pool, block_tables: np.ndarray, seq_lens, query_start_loc,
                    num_q_heads: int, scale: float, causal: bool = True, rows=None, return_lse: bool = False):
    """FP32 attention output for the requested query rows (all rows if ``rows`` is None).

    q: [Tq, Hq, D] uint16 BF16 bits.  Returns [n_rows, Hq, D] float32, and with
    ``return_lse`` also the [n_rows, Hq] float32 log-sum-exp of the scaled scores.
    """
    q = np.ascontiguousarray(q, dtype=np.uint16)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    qsl = np.ascontiguousarray(query_start_loc, dtype=np.int32)
    B, W = bt.shape
    Tq = int(qsl[-1])
    assert q.shape == (Tq, num_q_heads, pool.head_dim)
    if rows is None:
        rows_arr, n = None, Tq
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        n = rows_arr.shape[0]
    out = np.empty((n, num_q_heads, pool.head_dim), dtype=np.float32)
    lse = np.empty((n, num_q_heads), dtype=np.float32) if return_lse else None
    kp, vp = pool._kv_ptrs()
    rc = _load().oracle_paged_attention(_ptr(out), _ptr(q), kp, vp, pool.num_blocks,
                                        pool.k_block_stride, pool.v_block_stride, _ptr(bt), B, W,
                                        _ptr(sl), _ptr(qsl), num_q_heads, pool.num_kv_heads,
                                        pool.head_dim, float(scale), int(bool(causal)),
                                        None if rows_arr is None else _ptr(rows_arr), n,
                                        None if lse is None else _ptr(lse))
    if rc != 0:
        raise OracleError("paged_attention: inconsistent metadata")
    return (out, lse) if return_lse else out


def merge_states(out_a, lse_a, out_b, lse_b):
    """Merge two attention results over disjoint key sets (FP64).

    out_*: [..., D] values (float, or uint16 BF16 bits), lse_*: [...] natural-log
    LSE.  Returns (out [..., D] float64, lse [...] float64).
    """
    def as_f64(x):
        x = np.asarray(x)
        return bf16_bits_to_f32(x).astype(np.float64) if x.dtype == np.uint16 else x.astype(np.float64)
    a, b = np.ascontiguousarray(as_f64(out_a)), np.ascontiguousarray(as_f64(out_b))
    la = np.ascontiguousarray(np.asarray(lse_a, dtype=np.float64))
    lb = np.ascontiguousarray(np.asarray(lse_b, dtype=np.float64))
    assert a.shape == b.shape and la.shape == lb.shape == a.shape[:-1]
    D = a.shape[-1]
    n = int(np.prod(la.shape))
    out = np.empty(a.shape, dtype=np.float64)
    lse = np.empty(la.shape, dtype=np.float64)
    _load().oracle_merge_states(_ptr(out), _ptr(lse), _ptr(a), _ptr(la), _ptr(b), _ptr(lb), n, D)
    return out, lse


def prepare_block_tables(block_tables: np.ndarray, seq_lens, num_blocks: int) -> np.ndarray:
    """Padded, sanitised copy of ``block_tables`` ([B, W] int32 -> [B, ceil(W/8)*8])."""
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    B, W = bt.shape
    out = np.empty((B, (W + 7) // 8 * 8), dtype=np.int32)
    rc = _load().oracle_prepare_block_tables(_ptr(out), _ptr(bt), B, W, _ptr(sl), int(num_blocks))
    if rc != 0:
        raise OracleError("prepare_block_tables: invalid table")
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> BF16 bit patterns (NaN kept quiet)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
