"""CPU tests of the C ABI: the library loads and exports every declared entry
point; argument validation rejects bad calls before anything is launched;
page-table preparation (host logic) matches the oracle bit for bit.  No test
here makes a GPU call."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import paged_kv_cache_bf16_amd as kvp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvp.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kvp.LIB_PATH):
        from paged_kv_cache_bf16_amd import build
        build.build()
    return kvp.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"kv_pool_create", "reshape_and_cache", "paged_attention", "kv_prepare_block_tables",
            "kvp_workspace_bytes"} <= set(names), names
    for n in names:
        assert hasattr(lib, n), "missing export %s" % n
    assert kvp.kvp_version().startswith("kvp")


FAKE_K, FAKE_V = 0x10000000, 0x20000000   # never dereferenced: validation only


def make_desc(**kw):
    d = dict(num_blocks=8, block_size=16, num_kv_heads=2, head_dim=128, reserved=0, k_cache=FAKE_K,
             v_cache=FAKE_V, k_block_stride=2 * 16 * 128, v_block_stride=2 * 16 * 128)
    d.update(kw)
    return kvp.PoolDesc(**d)


def create(lib, **kw):
    h = ctypes.c_void_p()
    rc = lib.kv_pool_create(ctypes.byref(make_desc(**kw)), ctypes.byref(h))
    return rc, h


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=64), kvp.KVP_ERR_UNSUPPORTED),
    (dict(block_size=32), kvp.KVP_ERR_UNSUPPORTED),
    (dict(num_blocks=0), kvp.KVP_ERR_INVALID_ARGUMENT),
    (dict(k_cache=FAKE_K + 2), kvp.KVP_ERR_INVALID_ARGUMENT),
    (dict(k_block_stride=100), kvp.KVP_ERR_INVALID_ARGUMENT),
    (dict(v_cache=FAKE_K + 64), kvp.KVP_ERR_INVALID_ARGUMENT),        # K and V pages overlap
    (dict(v_cache=None), kvp.KVP_ERR_INVALID_ARGUMENT),
])
def test_pool_create_rejects(lib, kw, code):
    rc, h = create(lib, **kw)
    assert rc == code
    assert lib.kvp_last_error().decode()


def test_pool_create_overlap_matches_brute_force(lib):
    # K page i covers elements [i*sk, i*sk + pg) from k_cache, V page j
    # [x0 + j*sv, x0 + j*sv + pg); creation must fail exactly when some pair
    # shares an element (equal and unequal strides, V before or after K)
    pg = 16 * 128                                  # one kv head, Dh 128
    rng = np.random.default_rng(7)
    seen = {True: 0, False: 0}
    for trial in range(400):
        n = int(rng.integers(1, 7))
        sk = pg + 8 * int(rng.integers(0, 3 * pg // 8))
        sv = sk if trial % 3 == 0 else pg + 8 * int(rng.integers(0, 3 * pg // 8))
        x0 = 8 * int(rng.integers(-(n * max(sk, sv)) // 8 - pg // 8, (n * max(sk, sv)) // 8 + pg // 8))
        overlap = any(x0 + j * sv < i * sk + pg and i * sk < x0 + j * sv + pg for i in range(n) for j in range(n))
        rc, h = create(lib, num_blocks=n, num_kv_heads=1, k_block_stride=sk, v_block_stride=sv,
                       v_cache=FAKE_K + 2 * x0)
        assert rc == (kvp.KVP_ERR_INVALID_ARGUMENT if overlap else 0), (n, sk, sv, x0, lib.kvp_last_error())
        if rc == 0:
            lib.kv_pool_destroy(h)
        seen[overlap] += 1
    assert seen[True] > 50 and seen[False] > 50
    # unequal strides interleaved without touching: K pages at 2i*pg, V pages at (4j+1)*pg
    rc, h = create(lib, num_blocks=1000, num_kv_heads=1, k_block_stride=2 * pg, v_block_stride=4 * pg,
                   v_cache=FAKE_K + 2 * pg)
    assert rc == 0, lib.kvp_last_error()
    lib.kv_pool_destroy(h)
    # and with V page 0 on K page 1
    rc, h = create(lib, num_blocks=1000, num_kv_heads=1, k_block_stride=2 * pg, v_block_stride=3 * pg,
                   v_cache=FAKE_K + 4 * pg)
    assert rc == kvp.KVP_ERR_INVALID_ARGUMENT


def test_pool_create_interleaved_and_span(lib):
    page = 2 * 16 * 128
    rc, h = create(lib, v_cache=FAKE_K + 2 * page, k_block_stride=2 * page, v_block_stride=2 * page,
                   num_blocks=140000)
    assert rc == 0, lib.kvp_last_error()
    span = ctypes.c_int64()
    assert lib.kv_pool_span_bytes(h, ctypes.byref(span)) == 0
    assert span.value == 140000 * 2 * page * 2 > 2 ** 31
    lib.kv_pool_destroy(h)


def test_prepare_tables_matches_oracle(lib):
    rc, h = create(lib, num_blocks=1000)
    assert rc == 0
    pool = kvp.KVPool(h, make_desc(num_blocks=1000), None)
    rng = np.random.default_rng(0)
    imax = np.iinfo(np.int32).max
    for trial in range(50):
        B = int(rng.integers(1, 6))
        W = int(rng.integers(1, 40))
        seq = rng.integers(0, 16 * W + 1, size=B).astype(np.int32)
        bt = rng.integers(0, 1000, size=(B, W)).astype(np.int32)
        for b in range(B):                        # poison past each row's pages
            n = -(-int(seq[b]) // 16)
            bt[b, n:] = rng.choice([-1, imax, 12345678], size=W - n)
        got = kvp.kv_prepare_block_tables(pool, bt, seq)
        exp = oracle.prepare_block_tables(bt, seq, 1000)
        np.testing.assert_array_equal(got, exp)
        assert got.shape[1] == kvp.kvp_padded_width(W) == -(-W // 8) * 8


def test_prepare_tables_rejects_without_writing(lib):
    rc, h = create(lib, num_blocks=10)
    pool = kvp.KVPool(h, make_desc(num_blocks=10), None)
    out = np.full((1, 8), 77, np.int32)
    bt = np.array([[1, 2, 10]], np.int32)
    seq = np.array([40], np.int32)
    rc = lib.kv_prepare_block_tables(h, bt.ctypes.data_as(ctypes.c_void_p), 1, 3,
                                     seq.ctypes.data_as(ctypes.c_void_p), out.ctypes.data_as(ctypes.c_void_p))
    assert rc == kvp.KVP_ERR_INVALID_ARGUMENT
    assert (out == 77).all()
    with pytest.raises(kvp.KvpError):
        kvp.kv_prepare_block_tables(pool, np.array([[1, 2]], np.int32), [33])   # needs 3 pages


def _attn(lib, h, **kw):
    a = dict(q=0x30000000, qs=8 * 128, out=0x40000000, os=8 * 128, Hq=8, B=1, bt=0x50000000, bts=8,
             sl=0x60000000, qsl=0x70000000, mq=1, ms=100, scale=0.1, causal=1, ws=0x80000000, wsb=1 << 30,
             stream=None)
    a.update(kw)
    return lib.paged_attention(h, a["q"], a["qs"], a["out"], a["os"], a["Hq"], a["B"], a["bt"], a["bts"], a["sl"],
                               a["qsl"], a["mq"], a["ms"], a["scale"], a["causal"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(Hq=7), kvp.KVP_ERR_UNSUPPORTED),
    (dict(Hq=2 * 17), kvp.KVP_ERR_UNSUPPORTED),           # group of 17 > 16
    (dict(q=0x30000002), kvp.KVP_ERR_INVALID_ARGUMENT),
    (dict(qs=8 * 128 - 8), kvp.KVP_ERR_INVALID_ARGUMENT),
    (dict(bts=6), kvp.KVP_ERR_INVALID_ARGUMENT),           # 100 tokens need 7 pages
    (dict(bts=12, ms=10), kvp.KVP_ERR_INVALID_ARGUMENT),   # stride not a multiple of 8
    (dict(bt=0x50000010), kvp.KVP_ERR_INVALID_ARGUMENT),   # table not 32-byte aligned
    (dict(mq=200), kvp.KVP_ERR_INVALID_ARGUMENT),          # max_query_len > max_seq_len
    (dict(causal=2), kvp.KVP_ERR_INVALID_ARGUMENT),
    (dict(scale=float("nan")), kvp.KVP_ERR_INVALID_ARGUMENT),
    (dict(scale=0.0), kvp.KVP_ERR_INVALID_ARGUMENT),
    (dict(scale=-0.1), kvp.KVP_ERR_INVALID_ARGUMENT),
    (dict(scale=3e38), kvp.KVP_ERR_INVALID_ARGUMENT),
    (dict(ws=None), kvp.KVP_ERR_INVALID_ARGUMENT),
    (dict(wsb=64), kvp.KVP_ERR_WORKSPACE_TOO_SMALL),
    (dict(sl=None), kvp.KVP_ERR_INVALID_ARGUMENT),
])
def test_attention_rejects_before_launch(lib, kw, code):
    rc, h = create(lib)
    assert rc == 0
    kvp.kvp_reset_counters()
    assert _attn(lib, h, **kw) == code
    c = kvp.kvp_get_counters()
    assert c["split_kv_launches"] == 0 and c["prefill_launches"] == 0
    lib.kv_pool_destroy(h)


def test_attention_empty_batch_is_ok_without_launch(lib):
    rc, h = create(lib)
    kvp.kvp_reset_counters()
    assert _attn(lib, h, B=0) == 0
    assert _attn(lib, h, mq=0) == 0
    assert kvp.kvp_get_counters()["split_kv_launches"] == 0
    lib.kv_pool_destroy(h)


@pytest.mark.parametrize("args,code", [
    (dict(T=-1), kvp.KVP_ERR_INVALID_ARGUMENT),
    (dict(k=0x30000004), kvp.KVP_ERR_INVALID_ARGUMENT),
    (dict(ks=100), kvp.KVP_ERR_INVALID_ARGUMENT),
    (dict(slots=None), kvp.KVP_ERR_INVALID_ARGUMENT),
])
def test_reshape_rejects_before_launch(lib, args, code):
    rc, h = create(lib)
    a = dict(k=0x30000000, v=0x40000000, T=5, ks=256, vs=256, slots=0x50000000)
    a.update(args)
    kvp.kvp_reset_counters()
    assert lib.reshape_and_cache(h, a["k"], a["v"], a["T"], a["ks"], a["vs"], a["slots"], None) == code
    assert kvp.kvp_get_counters()["reshape_and_cache_launches"] == 0
    assert lib.reshape_and_cache(h, a["k"], a["v"], 0, 256, 256, None, None) == 0   # empty is a no-op
    lib.kv_pool_destroy(h)


@pytest.mark.parametrize("args", [
    dict(pool=None), dict(B=-1), dict(W=-1), dict(bt=None), dict(sl=None), dict(out=None),
    dict(out=0x30000010),                     # overlaps the input table
    dict(bt=0x32000010),                      # the input table overlaps the output
])
def test_prepare_tables_device_rejects_before_launch(lib, args):
    """kv_prepare_block_tables_device: bad arguments fail before anything is
    queued (the pointers are never dereferenced); an empty batch is a no-op."""
    rc, h = create(lib)
    a = dict(pool=h, bt=0x30000000, B=3, W=10, sl=0x31000000, out=0x32000000)
    a.update(args)
    kvp.kvp_reset_counters()
    f = lib.kv_prepare_block_tables_device
    assert f(a["pool"], a["bt"], a["B"], a["W"], a["sl"], a["out"], None, None) == kvp.KVP_ERR_INVALID_ARGUMENT
    assert kvp.kvp_get_counters()["last_grid_blocks"] == 0
    assert f(h, None, 0, 10, None, None, None, None) == 0
    lib.kv_pool_destroy(h)


def test_workspace_bytes_scales_with_tiles(lib):
    rc, h = create(lib)
    pool = kvp.KVPool(h, make_desc(), None)
    a = kvp.kvp_workspace_bytes(pool, 8, 4, 7168)
    b = kvp.kvp_workspace_bytes(pool, 8, 4, 7168 * 2)
    assert a >= 4 * 2 * 56 * 16 * 128 * 4 and b > a


@pytest.mark.parametrize("lse,lss,code", [
    (None, 8, kvp.KVP_ERR_INVALID_ARGUMENT),
    (0x90000002, 8, kvp.KVP_ERR_INVALID_ARGUMENT),        # not 4-byte aligned
    (0x90000000, 7, kvp.KVP_ERR_INVALID_ARGUMENT),        # stride < num_q_heads
])
def test_attention_lse_rejects_before_launch(lib, lse, lss, code):
    rc, h = create(lib)
    kvp.kvp_reset_counters()
    rc = lib.paged_attention_lse(h, 0x30000000, 8 * 128, 0x40000000, 8 * 128, lse, lss, 8, 1, 0x50000000, 8,
                                 0x60000000, 0x70000000, 1, 100, 0.1, 1, 0x80000000, 1 << 30, None)
    assert rc == code
    c = kvp.kvp_get_counters()
    assert c["split_kv_launches"] == 0 and c["prefill_launches"] == 0
    # the checks paged_attention makes come first and are the same
    assert lib.paged_attention_lse(h, 0x30000000, 8 * 128, 0x40000000, 8 * 128, 0x90000000, 8, 7, 1, 0x50000000,
                                   8, 0x60000000, 0x70000000, 1, 100, 0.1, 1, 0x80000000, 1 << 30,
                                   None) == kvp.KVP_ERR_UNSUPPORTED
    lib.kv_pool_destroy(h)


@pytest.mark.parametrize("kw,code", [
    (dict(D=12), kvp.KVP_ERR_UNSUPPORTED),
    (dict(D=1024), kvp.KVP_ERR_UNSUPPORTED),
    (dict(T=-1), kvp.KVP_ERR_INVALID_ARGUMENT),
    (dict(H=0), kvp.KVP_ERR_INVALID_ARGUMENT),
    (dict(a=None), kvp.KVP_ERR_INVALID_ARGUMENT),
    (dict(lb=None), kvp.KVP_ERR_INVALID_ARGUMENT),
    (dict(a=0x10000008), kvp.KVP_ERR_INVALID_ARGUMENT),     # rows not 16-byte aligned
    (dict(lse=0x60000002), kvp.KVP_ERR_INVALID_ARGUMENT),   # lse not 4-byte aligned
    (dict(out=0x10000010), kvp.KVP_ERR_INVALID_ARGUMENT),   # partial overlap with out_a
    (dict(lse=0x40000004), kvp.KVP_ERR_INVALID_ARGUMENT),   # partial overlap with lse_a
])
def test_merge_rejects_before_launch(lib, kw, code):
    a = dict(a=0x10000000, la=0x40000000, b=0x20000000, lb=0x50000000, out=0x30000000, lse=0x60000000,
             T=4, H=8, D=128)
    a.update(kw)
    kvp.kvp_reset_counters()
    rc = lib.kvp_merge_attention(a["a"], a["la"], a["b"], a["lb"], a["out"], a["lse"], a["T"], a["H"], a["D"], None)
    assert rc == code
    assert kvp.kvp_get_counters()["merge_launches"] == 0


def test_merge_empty_is_ok_without_launch(lib):
    kvp.kvp_reset_counters()
    assert lib.kvp_merge_attention(None, None, None, None, None, None, 0, 8, 128, None) == 0
    assert kvp.kvp_get_counters()["merge_launches"] == 0


def test_check_slot_mapping_agrees_with_the_oracle(lib):
    """The host-side slot check accepts exactly the mappings the oracle's
    scatter accepts (negative slots skipped; duplicates and slots beyond the
    pool rejected), on random mappings of a 6-block pool."""
    rc, h = create(lib, num_blocks=6)
    pool = kvp.KVPool(h, make_desc(num_blocks=6), None)
    rng = np.random.default_rng(12)
    seen = {True: 0, False: 0}
    for trial in range(300):
        n = int(rng.integers(1, 12))
        slots = rng.integers(-3, 6 * 16 + 4, size=n).astype(np.int64)
        if trial % 3 == 0:
            slots = rng.permutation(6 * 16)[:n].astype(np.int64)        # always valid
        opool = oracle.Pool(6, 2, 128)
        kv = np.zeros((n, 2, 128), np.uint16)
        try:
            oracle.reshape_and_cache(opool, kv, kv, slots)
            ok_oracle = True
        except oracle.OracleError:
            ok_oracle = False
        try:
            kvp.kvp_check_slot_mapping(pool, slots)
            ok_lib = True
        except kvp.KvpError as e:
            ok_lib = False
            assert e.code == kvp.KVP_ERR_INVALID_ARGUMENT
            assert "share slot" in str(e) or "beyond the pool" in str(e)
        assert ok_lib == ok_oracle, slots
        seen[ok_lib] += 1
    assert seen[True] > 50 and seen[False] > 50
    kvp.kvp_check_slot_mapping(pool, np.array([], np.int64))
    del pool                                  # the wrapper destroys the descriptor


def test_workspace_bytes_split_sizes_and_errors(lib):
    h = create(lib)[1]
    pool = kvp.KVPool(h, make_desc(), None)
    base = kvp.kvp_workspace_bytes(pool, 8, 4, 7168)
    assert kvp.kvp_workspace_bytes_split(pool, 8, 4, 7168, 16) == base
    w512 = kvp.kvp_workspace_bytes_split(pool, 8, 4, 7168, 512)
    # 4 rows x 2 kv heads x 56 tiles x 512 columns x (128 + 2) floats, in 256-byte aligned parts
    assert w512 >= 4 * 2 * 56 * 512 * (128 + 2) * 4 and w512 < 4 * 2 * 56 * 512 * (128 + 2) * 4 + 3 * 256
    for bad in (0, 8, 24, 1040):
        with pytest.raises(kvp.KvpError):
            kvp.kvp_workspace_bytes_split(pool, 8, 4, 7168, bad)
