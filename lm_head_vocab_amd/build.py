"""Build libheadloss.so (gfx950) in-tree with hipcc.

Usage: python -m lm_head_vocab_amd.build  [-j JOBS]

Every call recompiles every source (no stale objects), in parallel, then
links the shared library next to this file. Each kernel's resource report is
checked: a kernel that spills vector registers or uses private (scratch)
memory fails the build, since the kernels are designed to keep their row slices in
registers and a spill would silently move them to memory.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libheadloss.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # packed fp32 (v_pk_fma_f32 / v_pk_mul_f32 / v_pk_add_f32) stays off
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def sources():
    out = []
    for name in sorted(os.listdir(CSRC)):
        if name.endswith(".hip") or name.endswith(".cpp"):
            out.append(os.path.join(CSRC, name))
    return out


def resource_problems(remarks: str) -> list[str]:
    """Kernels whose resource report shows VGPR spills or scratch use. (SGPR
    spills go to VGPR lanes, not to memory, and are allowed.)"""
    bad = []
    name = None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"(ScratchSize \[bytes/lane\]|VGPRs Spill): (\d+)", line)
        if m and name and int(m.group(2)) > 0:
            bad.append(f"{name}: {m.group(1)} = {m.group(2)}")
    return bad


def _compile(src: str) -> tuple[str, float]:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    t0 = time.time()
    cmd = [HIPCC, *COMMON, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    bad = resource_problems(res.stderr)
    if bad:
        raise RuntimeError(f"{os.path.basename(src)}: kernels spill or use scratch memory:\n  " + "\n  ".join(bad))
    return obj, time.time() - t0


def build(jobs: int | None = None, verbose: bool = True) -> str:
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    t0 = time.time()
    objs = []
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for obj, dt in ex.map(_compile, srcs):
            objs.append(obj)
            if verbose:
                print(f"  compiled {os.path.basename(obj)} in {dt:.1f}s", flush=True)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f}s", flush=True)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", "--jobs", type=int, default=None)
    args = ap.parse_args(argv)
    build(args.jobs)


if __name__ == "__main__":
    sys.exit(main())
