"""Build libmla.so (the C-ABI library with the gfx950 HIP kernels) in-tree.

    python -m mla_paged_kv_amd.build

compiles every source under ``csrc/`` with hipcc for gfx950 and links
``mla_paged_kv_amd/libmla.so``.  Object files go to ``_build/`` at the repo
root.  Always recompiles (a few tens of seconds).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmla.so")
ARCH = "gfx950"

SOURCES = ["mla_sched.cpp", "mla_sched_dev.hip", "mla_api.cpp", "mla_splitkv.hip",
           "mla_decode_576.hip", "mla_decode_512.hip", "mla_decode_576_f16.hip",
           "mla_decode_512_f16.hip", "mla_combine.hip"]

# Packed-FP32 VALU ops are turned off for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"--offload-arch={ARCH}", f"-I{INCLUDE}",
          f"-I{CSRC}"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libmla.so)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "argument unused" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    jobs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        jobs.append([cc, *COMMON, *DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        for out in ex.map(_run, jobs):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    out = _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs])
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
