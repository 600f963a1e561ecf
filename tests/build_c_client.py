"""Build tests/c_abi_client (plain C against include/kvp.h, linked to the
in-tree libkvp.so and the HIP runtime) with gcc.  Test infrastructure: the
C-ABI client tests run the binary; they never build it."""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c_abi_client.c")
BIN = os.path.join(HERE, "c_abi_client")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    pkg = os.path.join(ROOT, "future_attention_scoring_kvp_amd")
    if not os.path.exists(os.path.join(pkg, "libkvp.so")):
        raise RuntimeError("libkvp.so is not built")
    cc = shutil.which("gcc") or "gcc"
    tmp = BIN + ".tmp"
    cmd = [cc, "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), SRC, "-o", tmp,
           "-L", pkg, "-lkvp", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../future_attention_scoring_kvp_amd",
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"c_abi_client build failed:\n{proc.stdout}")
    os.replace(tmp, BIN)
    return BIN


if __name__ == "__main__":
    print(build())
