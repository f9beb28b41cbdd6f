"""Build libgdn.so (all HIP kernels + the C ABI) in-tree for gfx950 with hipcc.

Usage: ``python -m gated_deltanet_03_amd._build`` (or ``__graft_entry__.build()``).
Always recompiles; objects go to ``gated_deltanet_03_amd/_build/``.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgdn.so")
SOURCES = ["gdn_api.cpp", "gdn_profile.cpp", "gdn_recurrent.hip", "gdn_prefill.hip"]
ARCH = os.environ.get("GDN_OFFLOAD_ARCH", "gfx950")

# Packed fp32 VALU forms are disabled for every HIP translation unit.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # keep MFMA accumulators in VGPRs (no AGPR round trips around VALU work)
          "-mllvm", "-amdgpu-mfma-vgpr-form",
          # the register-resident substitution and fragment loops rely on full unrolling
          "-mllvm", "-pragma-unroll-threshold=1000000",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the GDN HIP library cannot be built")


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
