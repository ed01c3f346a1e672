"""The library's C ABI from C callers.

CPU: the header compiles as strict C99 and C++17, and a C program drives the
host-side entry points (descriptor checks, block tables, slot checks,
workspace sizes, calls rejected before submission) -- tests/c_abi/host_check.c.
GPU: a C library (tests/c_abi/e2e.c, built by __graft_entry__.build()) runs
the cache write, a causal prefill and the decode of each row's last token
through the ABI with hipMalloc'd buffers and a HIP stream, and checks them
against the CPU oracle (pool bit for bit, prefill within tolerance, decode
bitwise the prefill's last row); it is called in this process through ctypes.
"""
import ctypes
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CABI = os.path.join(ROOT, "tests", "c_abi")
LIBDIR = os.path.join(ROOT, "paged_kv_cache_bf16_amd")

# The CPU tests start compilers and a C program as child processes; on a
# machine with a GPU the test process may already hold it, so they run only
# where there is none.
cpu_only = pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="starts child processes: CPU hosts only")


@cpu_only
def test_header_compiles_as_strict_c99_and_cxx17(tmp_path):
    if not shutil.which("gcc") or not shutil.which("g++"):
        pytest.skip("no host compiler")
    src = tmp_path / "inc.c"
    src.write_text('#include "kvp.h"\nint main(void) { kvp_counters c; return kvp_get_counters(&c) != KVP_OK; }\n')
    for cc, std in (("gcc", "-std=c99"), ("g++", "-std=c++17")):
        lang = ["-x", "c++"] if cc == "g++" else []
        subprocess.run([cc, std, "-Wall", "-Wextra", "-Werror", "-pedantic", "-fsyntax-only", "-I",
                        os.path.join(ROOT, "include")] + lang + [str(src)], check=True)


@cpu_only
def test_c_program_host_entry_points(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("no host compiler")
    lib = os.path.join(LIBDIR, "libkvp.so")
    assert os.path.exists(lib), "build libkvp.so first"
    exe = tmp_path / "host_check"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    os.path.join(CABI, "host_check.c"), "-o", str(exe), "-L", LIBDIR, "-lkvp",
                    "-Wl,-rpath," + LIBDIR, "-Wl,-rpath-link,/opt/rocm/lib"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout, r.stderr)


@pytest.mark.gpu
@pytest.mark.parametrize("head_dim", [128, 256, 512])
def test_c_caller_end_to_end(head_dim):
    import paged_kv_cache_bf16_amd as kvp
    kvp.load_library()                       # the in-tree libkvp.so, the one the C library links
    path = os.path.join(CABI, "libkvp_c_e2e.so")
    assert os.path.exists(path), "build tests/c_abi/libkvp_c_e2e.so first (__graft_entry__.build())"
    print("C caller, head_dim", head_dim, flush=True)
    lib = ctypes.CDLL(path)
    lib.kvp_c_e2e.argtypes = [ctypes.c_int, ctypes.c_char_p, ctypes.c_int]
    lib.kvp_c_e2e.restype = ctypes.c_int
    msg = ctypes.create_string_buffer(512)
    rc = lib.kvp_c_e2e(head_dim, msg, len(msg))
    assert rc == 0 and msg.value == b"ok", msg.value.decode()
