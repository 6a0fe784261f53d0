"""Build libpkv.so in-tree with hipcc for gfx950.

Usage: ``python -m pagedattention_pkv_store_amd.build`` (or
``__graft_entry__.build()``).  The library is written next to this file, so it
travels with the source tree; a JIT cache is never used.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libpkv.so")
ARCH = "gfx950"

# Packed-FP32 VALU ops are kept out of the generated code; hipcc's host pass
# warns that it does not know the feature, which is harmless.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in res.stdout.splitlines() if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False) -> str:
    """Compile csrc/ into libpkv.so; return its path.  Always recompiles."""
    hipcc = _hipcc()
    include = os.path.join(REPO_DIR, "include")
    with tempfile.TemporaryDirectory(prefix="pkv_build_") as tmp:
        dev_o = os.path.join(tmp, "device.o")
        host_o = os.path.join(tmp, "host.o")
        _run([hipcc, *HIP_FLAGS, "-I", include, "-c", os.path.join(CSRC, "device.hip"), "-o", dev_o],
             verbose)
        _run([hipcc, *HOST_FLAGS, "-I", include, "-c", os.path.join(CSRC, "host.cpp"), "-o", host_o],
             verbose)
        tmp_lib = os.path.join(tmp, "libpkv.so")
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_lib, dev_o, host_o],
             verbose)
        staged = LIB_PATH + ".tmp"
        shutil.copyfile(tmp_lib, staged)
        os.replace(staged, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
