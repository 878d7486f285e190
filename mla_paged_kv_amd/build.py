"""Build libmla.so (the C-ABI library with the gfx950 HIP kernels) in-tree.

    python -m mla_paged_kv_amd.build

compiles every source under ``csrc/`` with hipcc for gfx950 and links
``mla_paged_kv_amd/libmla.so``.  Object files go to ``_build/`` at the repo
root.  Always recompiles (a few tens of seconds).
"""
from __future__ import annotations

import os
import re
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
           "mla_splitkv_f16.hip", "mla_decode_576.hip", "mla_decode_512.hip", "mla_decode_576_f16.hip",
           "mla_decode_512_f16.hip", "mla_narrow.hip", "mla_combine.hip", "mla_noalloc.hip"]

# Packed-FP32 VALU ops are turned off for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"--offload-arch={ARCH}", f"-I{INCLUDE}",
          f"-I{CSRC}"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libmla.so)")


# The decode kernels order their direct-to-LDS and query loads with exact
# vector-memory counts; scratch accesses share that counter (and a spill could
# copy a register a load has not written yet), so every decode kernel except
# the 64-bit-address (WIDE) ones must be free of scratch.  The compiler's
# resource remarks say so per kernel.
DECODE_SOURCES = {"mla_decode_576.hip", "mla_decode_512.hip", "mla_decode_576_f16.hip",
                  "mla_decode_512_f16.hip", "mla_narrow.hip"}
_KERNEL = re.compile(r"Function Name: (_ZN3mla10mla_decodeILi(\d+)ELb([01])ELb([01])ELb([01])ELi(\d+)E\S*)")
# the narrow kernel (units of at most 16 rows) is scratch-free too: a spill
# inside its loop would be a memory round trip per tile
_NARROW = re.compile(r"Function Name: (_ZN3mla10mla_narrowI\S*)")
_SCRATCH = re.compile(r"ScratchSize \[bytes/lane\]: (\d+)")


def check_scratch(remarks: str, src: str) -> int:
    """Number of decode kernels in the remarks; raises if a non-WIDE one uses scratch."""
    name, wide, seen = None, False, 0
    for line in remarks.splitlines():
        m = _KERNEL.search(line)
        if m:
            name, wide, seen = m.group(1), m.group(4) == "1", seen + 1
            continue
        m = _NARROW.search(line)
        if m:
            name, wide, seen = m.group(1), False, seen + 1
            continue
        m = _SCRATCH.search(line)
        if m and name is not None:
            if int(m.group(1)) > 0 and not wide:
                raise RuntimeError(f"{src}: {name} uses {m.group(1)} bytes/lane of scratch; the "
                                   "decode and narrow kernels must be scratch-free")
            name = None
    return seen


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "argument unused" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    src = os.path.basename(cmd[cmd.index("-c") + 1]) if "-c" in cmd else ""
    if src in DECODE_SOURCES:
        if check_scratch(out, src) == 0:
            raise RuntimeError(f"{src}: no resource remarks for the decode kernels")
        out = "\n".join(l for l in out.splitlines()
                         if "kernel-resource-usage" not in l and "In file included from" not in l
                         and not re.match(r"^\s*\d*\s*\|", l))
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    jobs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        extra = ["-Rpass-analysis=kernel-resource-usage"] if src in DECODE_SOURCES else []
        jobs.append([cc, *COMMON, *DEVICE_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj])
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
