"""Build libsm.so (the HIP library behind the C ABI in include/sm.h) in-tree.

Each csrc/*.hip unit is compiled for gfx950 with hipcc in parallel, then
linked into matrix_aware_optimizer_momentum_amd/libsm.so.  Always rebuilds.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsm.so")

ARCH = os.environ.get("SM_OFFLOAD_ARCH", "gfx950")
# Packed float32 VALU ops are kept out of the generated code on purpose.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=off",  # roundings happen where the source writes them
    "-Wall", "-Wno-unused-function", "-Werror=return-type",
    "-Wno-inline-asm",  # the direct-to-LDS loads name M0 as clobbered on purpose
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    lines = [ln for ln in proc.stdout.splitlines() if "packed-fp32-ops" not in ln]
    return proc.returncode, "\n".join(lines)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    objs = []
    cmds = []
    for f in srcs:
        obj = os.path.join(BUILD, f[:-4] + ".o")
        objs.append(obj)
        cmds.append([hipcc, *HIP_FLAGS, "-c", os.path.join(CSRC, f), "-o", obj])
    jobs = jobs or min(len(cmds), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_run, cmds))
    failed = False
    for cmd, (rc, out) in zip(cmds, results):
        if verbose or rc != 0:
            print(" ".join(cmd[-3:]), file=sys.stderr)
            if out:
                print(out, file=sys.stderr)
        failed |= rc != 0
    if failed:
        raise RuntimeError("HIP compilation failed")
    tmp = LIB + ".tmp"
    rc, out = _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    if rc != 0:
        print(out, file=sys.stderr)
        raise RuntimeError("linking libsm.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
