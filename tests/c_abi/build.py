"""Build the C-caller test library (tests/c_abi/libkvp_c_e2e.so): e2e.c in
strict C99 with gcc, linked against the in-tree libkvp.so, the CPU oracle
and the HIP runtime (run paths relative to this directory, so the tree can
move).  Test infrastructure, built by __graft_entry__.build() after the
library and the oracle."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
OUT = os.path.join(HERE, "libkvp_c_e2e.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    for need in (os.path.join(ROOT, "paged_kv_cache_bf16_amd", "libkvp.so"), os.path.join(ROOT, "oracle", "libkvp_oracle.so")):
        if not os.path.exists(need):
            raise RuntimeError("build %s first" % need)
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-pedantic", "-fPIC", "-shared",
           "-D__HIP_PLATFORM_AMD__", "-isystem", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "e2e.c"), "-o", OUT,
           "-L", os.path.join(ROOT, "paged_kv_cache_bf16_amd"), "-lkvp",
           "-L", os.path.join(ROOT, "oracle"), "-lkvp_oracle",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../paged_kv_cache_bf16_amd:$ORIGIN/../../oracle",
           "-Wl,-rpath-link," + os.path.join(ROCM, "lib")]
    subprocess.run(cmd, check=True)
    return OUT


if __name__ == "__main__":
    print("built", build())
