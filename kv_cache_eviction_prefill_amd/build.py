"""Build ``libh2o.so`` (the C-ABI library) for gfx950 with hipcc, in-tree.

Every ``csrc/*.hip`` file is compiled to an object in ``_build/`` (in parallel),
then linked into ``kv_cache_eviction_prefill_amd/libh2o.so``.  Each call
recompiles.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libh2o.so")

ARCH = "gfx950"
# Packed fp32 instructions stay off: hipcc -O3 would otherwise form them from
# plain float code.
# MFMA results go straight to VGPRs (no AGPR round trips in the softmax epilogues).
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form",
          "-I", INCLUDE, "-I", CSRC]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libh2o.so)")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "not a recognized feature for this target" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {os.path.basename(src)}:\n{out}")
    if verbose and out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    # A kernel template whose host-side instantiation fails leaves its launch stub
    # undefined without a compile error; refuse such a library here.
    nm = shutil.which("nm")
    if nm:
        res = subprocess.run([nm, "-uC", tmp], capture_output=True, text=True)
        missing = [l.strip() for l in res.stdout.splitlines() if "__device_stub__" in l]
        if missing:
            os.remove(tmp)
            raise RuntimeError("undefined kernel launch stubs in libh2o.so:\n" + "\n".join(missing))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
