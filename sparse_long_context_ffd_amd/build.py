"""Build libffd.so (HIP kernels + C ABI) for gfx950 with hipcc.

Usage: ``python -m sparse_long_context_ffd_amd.build`` (or ``build()`` from
Python).  The shared library is written next to this file so that it travels
with the source tree.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libffd.so")
ARCH = os.environ.get("FFD_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    # keep packed-FP32 (v_pk_*_f32) instructions out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; ROCm is required to build libffd")
    return exe


# per-source extra hipcc flags (none at present)
FILE_FLAGS = {}
OBJ_DIR = os.path.join(HERE, "_build")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed with exit code {r.returncode}: {' '.join(cmd[-3:])}")


def build(verbose: bool = False) -> str:
    """Compile every HIP source to an object (in parallel), then link libffd.so."""
    from concurrent.futures import ThreadPoolExecutor
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    os.makedirs(OBJ_DIR, exist_ok=True)
    inc = ["-I", os.path.join(HERE, "..", "include")]
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    jobs = []
    for src in srcs:
        obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
        jobs.append((obj, [hipcc(), *compile_flags, *FILE_FLAGS.get(os.path.basename(src), []), *inc, "-c", src,
                           "-o", obj]))
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1, 8)) as ex:
        for f in [ex.submit(_run, cmd, verbose) for _, cmd in jobs]:
            f.result()
    tmp = LIB + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *[o for o, _ in jobs], "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
