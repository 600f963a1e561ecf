"""Build libkvp.so (HIP kernels + C ABI) and libkvp_probe.so (the matrix-core
throughput probe the benchmark reports beside the datasheet peak) for gfx950
with hipcc, in-tree."""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(HERE, "libkvp.so")
PROBE_LIB_PATH = os.path.join(HERE, "libkvp_probe.so")

SOURCES = ["kvp_api.cpp", "lse_kernel.hip", "mass_kernel.hip", "select_kernel.hip",
           "target_kernel.hip", "cutoff_kernel.hip", "softtopk_kernel.hip", "f32_kernel.hip"]
PROBE_SOURCES = ["probe_kernel.hip"]
ARCH = "gfx950"

# Packed fp32 VALU forms are disabled for every device compilation.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-result"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build libkvp)")
    return path


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the device-only feature; drop that note.
    noise = "packed-fp32-ops' is not a recognized feature"
    out = "\n".join(l for l in proc.stdout.splitlines() if noise not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source for gfx950 and link libkvp.so and libkvp_probe.so
    next to this file.  The translation units compile concurrently (``jobs``
    processes, default one per source up to the CPU count, at most 16)."""
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="kvp_build_") as tmp:
        srcs = SOURCES + PROBE_SOURCES
        objs = [os.path.join(tmp, os.path.splitext(src)[0] + ".o") for src in srcs]
        cmds = [[cc, "-x", "hip", *COMMON, *DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
                for src, obj in zip(srcs, objs)]
        n = jobs or max(1, min(len(cmds), os.cpu_count() or 1, 16))
        with concurrent.futures.ThreadPoolExecutor(max_workers=n) as pool:
            for out in pool.map(_run, cmds):
                if verbose and out.strip():
                    print(out)
        for lib_objs, dest in ((objs[:len(SOURCES)], LIB_PATH),
                               (objs[len(SOURCES):], PROBE_LIB_PATH)):
            tmp_lib = os.path.join(tmp, os.path.basename(dest))
            _run([cc, "-shared", f"--offload-arch={ARCH}", *lib_objs, "-o", tmp_lib])
            shutil.copyfile(tmp_lib, dest + ".tmp")
            os.replace(dest + ".tmp", dest)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
