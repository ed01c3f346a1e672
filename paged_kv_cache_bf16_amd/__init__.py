"""Python binding of libkvp.so: the MI355X paged BF16 KV-cache library.

Every function here has the name of the C entry point it calls (see
include/kvp.h) and only marshals arguments: torch tensors become device
pointers, torch's current stream becomes the HIP stream.  All arithmetic
runs in the library's HIP kernels; there is no fallback of any kind.  If
libkvp.so has not been built, the first call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvp.so")
BLOCK_SIZE = 16

KVP_OK = 0
KVP_ERR_INVALID_ARGUMENT = -1
KVP_ERR_UNSUPPORTED = -2
KVP_ERR_WORKSPACE_TOO_SMALL = -3
KVP_ERR_HIP = -4

_lib = None


class KvpError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("kvp error %d: %s" % (code, msg))
        self.code = code


class PoolDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int64), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("k_cache", ctypes.c_void_p),
                ("v_cache", ctypes.c_void_p), ("k_block_stride", ctypes.c_int64),
                ("v_block_stride", ctypes.c_int64)]


class Counters(ctypes.Structure):
    _fields_ = [("reshape_and_cache_launches", ctypes.c_uint64), ("split_kv_launches", ctypes.c_uint64),
                ("prefill_launches", ctypes.c_uint64), ("workspace_init_launches", ctypes.c_uint64),
                ("last_grid_blocks", ctypes.c_uint64), ("fused_decode_steps", ctypes.c_uint64),
                ("merge_launches", ctypes.c_uint64)]


def load_library(path: str = LIB_PATH):
    """Load libkvp.so (raises if it is missing: the library must be built first)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libkvp.so not found at %s; build it with "
                           "`python -m paged_kv_cache_bf16_amd.build`" % path)
    lib = ctypes.CDLL(path)
    P, I, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    sigs = {
        "kv_pool_create": ([ctypes.POINTER(PoolDesc), ctypes.POINTER(P)], I),
        "kv_pool_destroy": ([P], I),
        "kv_pool_span_bytes": ([P, ctypes.POINTER(I64)], I),
        "reshape_and_cache": ([P, P, P, I64, I64, I64, P, P], I),
        "kv_prepare_block_tables": ([P, P, ctypes.c_int32, ctypes.c_int32, P, P], I),
        "kv_prepare_block_tables_device": ([P, P, ctypes.c_int32, ctypes.c_int32, P, P, P, P], I),
        "kvp_padded_width": ([ctypes.c_int32], ctypes.c_int32),
        "kvp_check_slot_mapping": ([P, P, I64], I),
        "kvp_workspace_bytes": ([P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(SZ)], I),
        "kvp_workspace_bytes_split": ([P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.POINTER(SZ)], I),
        "kvp_workspace_init": ([P, SZ, P], I),
        "paged_attention": ([P, P, I64, P, I64, ctypes.c_int32, ctypes.c_int32, P, ctypes.c_int32, P, P,
                             ctypes.c_int32, ctypes.c_int32, ctypes.c_float, I, P, SZ, P], I),
        "paged_attention_lse": ([P, P, I64, P, I64, P, I64, ctypes.c_int32, ctypes.c_int32, P, ctypes.c_int32,
                                 P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, I, P, SZ, P], I),
        "paged_attention_noalloc": ([P, P, I64, P, I64, ctypes.c_int32, ctypes.c_int32, P, ctypes.c_int32, P, P,
                                     ctypes.c_int32, ctypes.c_int32, ctypes.c_float, I, P], I),
        "kvp_merge_attention": ([P, P, P, P, P, P, I64, ctypes.c_int32, ctypes.c_int32, P], I),
        "kvp_decode_step": ([P, P, P, I64, I64, I64, P, P, I64, P, I64, ctypes.c_int32, ctypes.c_int32, P,
                             ctypes.c_int32, P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, I, P, SZ, P], I),
        "kvp_get_counters": ([ctypes.POINTER(Counters)], I),
        "kvp_reset_counters": ([], I),
        "kvp_last_error": ([], ctypes.c_char_p),
        "kvp_version": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(rc: int):
    if rc != KVP_OK:
        raise KvpError(rc, load_library().kvp_last_error().decode())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _host_i32(a):
    return np.ascontiguousarray(np.asarray(a), dtype=np.int32)


# ------------------------------------------------------------------ pool


class KVPool:
    """A pool descriptor over caller-owned device memory (K and V page sets)."""

    def __init__(self, handle, desc: PoolDesc, storage):
        self.handle = handle
        self.desc = desc
        self.storage = storage            # keeps the device memory alive
        self.num_blocks = desc.num_blocks
        self.num_kv_heads = desc.num_kv_heads
        self.head_dim = desc.head_dim

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.kv_pool_destroy(self.handle)
            self.handle = None


def kv_pool_create(k_cache, v_cache, num_blocks: int, num_kv_heads: int, head_dim: int,
                   k_block_stride: int, v_block_stride: int, storage=None) -> KVPool:
    """Wrap device memory as a pool.  k_cache / v_cache are torch tensors (or
    (tensor, element offset) pairs into one allocation for interleaved pools)."""
    lib = load_library()

    def addr(x):
        if isinstance(x, tuple):
            t, off = x
            return t.data_ptr() + 2 * int(off)
        return x.data_ptr()

    d = PoolDesc(int(num_blocks), BLOCK_SIZE, int(num_kv_heads), int(head_dim), 0, addr(k_cache),
                 addr(v_cache), int(k_block_stride), int(v_block_stride))
    h = ctypes.c_void_p()
    _check(lib.kv_pool_create(ctypes.byref(d), ctypes.byref(h)))
    return KVPool(h, d, storage if storage is not None else (k_cache, v_cache))


def alloc_pool(num_blocks: int, num_kv_heads: int, head_dim: int, interleaved: bool = False,
               device="cuda", fill_bits: int | None = None) -> KVPool:
    """Allocate pool memory with torch (uint16 BF16 bits) and wrap it.

    Separate: one tensor holding all K pages then all V pages.  Interleaved:
    each block is its K pages followed by its V pages.
    """
    import torch
    page = num_kv_heads * BLOCK_SIZE * head_dim
    storage = torch.empty(2 * num_blocks * page, dtype=torch.int16, device=device)
    if fill_bits is not None:
        storage.fill_(int(np.int16(np.uint16(fill_bits))))
    if interleaved:
        return kv_pool_create((storage, 0), (storage, page), num_blocks, num_kv_heads, head_dim,
                              2 * page, 2 * page, storage=storage)
    return kv_pool_create((storage, 0), (storage, num_blocks * page), num_blocks, num_kv_heads, head_dim,
                          page, page, storage=storage)


def kv_pool_span_bytes(pool: KVPool) -> int:
    out = ctypes.c_int64()
    _check(load_library().kv_pool_span_bytes(pool.handle, ctypes.byref(out)))
    return out.value


# ------------------------------------------------------------------ cache scatter


def reshape_and_cache(pool: KVPool, k, v, slot_mapping, stream=None) -> None:
    """Scatter k, v ([T, Hkv, D] BF16 device tensors) into the pool at slot_mapping ([T] int64)."""
    T = int(slot_mapping.shape[0])
    _check(load_library().reshape_and_cache(pool.handle, _ptr(k), _ptr(v), T, int(k.stride(0)),
                                            int(v.stride(0)), _ptr(slot_mapping), _stream(stream)))


# ------------------------------------------------------------------ metadata


def kvp_check_slot_mapping(pool: KVPool, slot_mapping) -> None:
    """Host-side check: slots inside the pool and no slot used twice (raises KvpError)."""
    s = np.ascontiguousarray(np.asarray(slot_mapping), dtype=np.int64)
    _check(load_library().kvp_check_slot_mapping(pool.handle, s.ctypes.data_as(ctypes.c_void_p), int(s.shape[0])))


def kvp_padded_width(width: int) -> int:
    return int(load_library().kvp_padded_width(int(width)))


def kv_prepare_block_tables(pool: KVPool, block_tables, seq_lens) -> np.ndarray:
    """Pad and sanitise a host block table ([B, W] int32) -> [B, padded W] int32 (host)."""
    bt = _host_i32(block_tables)
    sl = _host_i32(seq_lens)
    B, W = bt.shape
    out = np.empty((B, kvp_padded_width(W)), np.int32)
    _check(load_library().kv_prepare_block_tables(pool.handle, bt.ctypes.data_as(ctypes.c_void_p), B, W,
                                                  sl.ctypes.data_as(ctypes.c_void_p),
                                                  out.ctypes.data_as(ctypes.c_void_p)))
    return out


def kv_prepare_block_tables_device(pool: KVPool, block_tables, seq_lens, out=None, status=None, stream=None):
    """The same on the device: block_tables [B, W] and seq_lens [B] int32 device tensors ->
    out [B, padded W] int32 device tensor (allocated here when not given), on the stream.
    status: an optional device int32 tensor of one element into which the kernel ORs the
    problem bits of rows the host version would reject (see include/kvp.h)."""
    import torch
    B, W = int(block_tables.shape[0]), int(block_tables.shape[1])
    if out is None:
        out = torch.empty((B, kvp_padded_width(W)), dtype=torch.int32, device=block_tables.device)
    _check(load_library().kv_prepare_block_tables_device(pool.handle, _ptr(block_tables), B, W, _ptr(seq_lens),
                                                         _ptr(out), _ptr(status), _stream(stream)))
    return out


def kvp_workspace_bytes(pool: KVPool, num_q_heads: int, num_seqs: int, max_seq_len: int) -> int:
    out = ctypes.c_size_t()
    _check(load_library().kvp_workspace_bytes(pool.handle, int(num_q_heads), int(num_seqs), int(max_seq_len),
                                              ctypes.byref(out)))
    return out.value


def kvp_workspace_bytes_split(pool: KVPool, num_q_heads: int, num_seqs: int, max_seq_len: int,
                              split_cols: int) -> int:
    out = ctypes.c_size_t()
    _check(load_library().kvp_workspace_bytes_split(pool.handle, int(num_q_heads), int(num_seqs), int(max_seq_len),
                                                    int(split_cols), ctypes.byref(out)))
    return out.value


def kvp_workspace_init(workspace, stream=None) -> None:
    _check(load_library().kvp_workspace_init(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                             _stream(stream)))


def alloc_workspace(pool: KVPool, num_q_heads: int, num_seqs: int, max_seq_len: int, device="cuda",
                    split_cols: int = 16):
    import torch
    n = (kvp_workspace_bytes(pool, num_q_heads, num_seqs, max_seq_len) if split_cols == 16 else
         kvp_workspace_bytes_split(pool, num_q_heads, num_seqs, max_seq_len, split_cols))
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=device)
    kvp_workspace_init(ws)
    return ws


# ------------------------------------------------------------------ attention


def paged_attention(pool: KVPool, q, out, num_q_heads: int, block_tables, seq_lens, query_start_loc,
                    max_query_len: int, max_seq_len: int, scale: float | None = None, causal: bool = True,
                    workspace=None, stream=None) -> None:
    """out[...] = paged GQA attention of q over the pool (device tensors; see include/kvp.h)."""
    if scale is None:
        scale = 1.0 / math.sqrt(pool.head_dim)
    B = int(seq_lens.shape[0])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().paged_attention(
        pool.handle, _ptr(q), int(q.stride(0)), _ptr(out), int(out.stride(0)), int(num_q_heads), B,
        _ptr(block_tables), int(block_tables.stride(0)), _ptr(seq_lens), _ptr(query_start_loc),
        int(max_query_len), int(max_seq_len), float(scale), int(bool(causal)), _ptr(workspace), ws_bytes,
        _stream(stream)))


KVP_SCRATCH_BYTES = 32 << 20


def paged_attention_noalloc(pool: KVPool, q, out, num_q_heads: int, block_tables, seq_lens, query_start_loc,
                            max_query_len: int, max_seq_len: int, scale: float | None = None, causal: bool = True,
                            stream=None) -> None:
    """paged_attention with the split-KV partials in the library's own scratch
    array (KVP_SCRATCH_BYTES per device; no workspace, nothing allocated)."""
    if scale is None:
        scale = 1.0 / math.sqrt(pool.head_dim)
    B = int(seq_lens.shape[0])
    _check(load_library().paged_attention_noalloc(
        pool.handle, _ptr(q), int(q.stride(0)), _ptr(out), int(out.stride(0)), int(num_q_heads), B,
        _ptr(block_tables), int(block_tables.stride(0)), _ptr(seq_lens), _ptr(query_start_loc),
        int(max_query_len), int(max_seq_len), float(scale), int(bool(causal)), _stream(stream)))


def paged_attention_lse(pool: KVPool, q, out, lse, num_q_heads: int, block_tables, seq_lens, query_start_loc,
                        max_query_len: int, max_seq_len: int, scale: float | None = None, causal: bool = True,
                        workspace=None, stream=None) -> None:
    """paged_attention that also writes lse[token, head] (float32 device tensor; see include/kvp.h)."""
    if scale is None:
        scale = 1.0 / math.sqrt(pool.head_dim)
    B = int(seq_lens.shape[0])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().paged_attention_lse(
        pool.handle, _ptr(q), int(q.stride(0)), _ptr(out), int(out.stride(0)), _ptr(lse), int(lse.stride(0)),
        int(num_q_heads), B, _ptr(block_tables), int(block_tables.stride(0)), _ptr(seq_lens),
        _ptr(query_start_loc), int(max_query_len), int(max_seq_len), float(scale), int(bool(causal)),
        _ptr(workspace), ws_bytes, _stream(stream)))


def kvp_merge_attention(out_a, lse_a, out_b, lse_b, out, lse=None, stream=None) -> None:
    """Merge two results over disjoint key sets: out/lse from (out_a, lse_a) and (out_b, lse_b).

    out_*: [T, H, D] bf16 contiguous device tensors; lse_*: [T, H] float32 (see include/kvp.h)."""
    T, H, D = (int(x) for x in out_a.shape)
    for t in (out_a, out_b, out, lse_a, lse_b) + ((lse,) if lse is not None else ()):
        if not t.is_contiguous():
            raise ValueError("kvp_merge_attention takes contiguous tensors")
    if tuple(out_b.shape) != (T, H, D) or tuple(out.shape) != (T, H, D):
        raise ValueError("kvp_merge_attention: output shapes differ")
    if tuple(lse_a.shape) != (T, H) or tuple(lse_b.shape) != (T, H) or (lse is not None and tuple(lse.shape) != (T, H)):
        raise ValueError("kvp_merge_attention: lse shapes must be [T, H]")
    _check(load_library().kvp_merge_attention(_ptr(out_a), _ptr(lse_a), _ptr(out_b), _ptr(lse_b), _ptr(out),
                                              _ptr(lse), T, H, D, _stream(stream)))


def kvp_decode_step(pool: KVPool, k, v, slot_mapping, q, out, num_q_heads: int, block_tables, seq_lens,
                    query_start_loc, max_query_len: int, max_seq_len: int, scale: float | None = None,
                    causal: bool = True, workspace=None, stream=None) -> None:
    """reshape_and_cache(pool, k, v, slot_mapping) then paged_attention(...), one launch when possible
    (see include/kvp.h)."""
    if scale is None:
        scale = 1.0 / math.sqrt(pool.head_dim)
    T = int(slot_mapping.shape[0])
    B = int(seq_lens.shape[0])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().kvp_decode_step(
        pool.handle, _ptr(k), _ptr(v), T, int(k.stride(0)), int(v.stride(0)), _ptr(slot_mapping),
        _ptr(q), int(q.stride(0)), _ptr(out), int(out.stride(0)), int(num_q_heads), B,
        _ptr(block_tables), int(block_tables.stride(0)), _ptr(seq_lens), _ptr(query_start_loc),
        int(max_query_len), int(max_seq_len), float(scale), int(bool(causal)), _ptr(workspace), ws_bytes,
        _stream(stream)))


def kvp_get_counters() -> dict:
    c = Counters()
    _check(load_library().kvp_get_counters(ctypes.byref(c)))
    return {name: getattr(c, name) for name, _ in Counters._fields_}


def kvp_reset_counters() -> None:
    _check(load_library().kvp_reset_counters())


def kvp_version() -> str:
    return load_library().kvp_version().decode()
