"""Build the HIP library libmoe_mi355x.so in-tree for gfx950.

    python -m mixture_experts_ffn_top_amd.build [--jobs N]

Every .hip file under csrc/ is compiled with hipcc to an object in _build/,
then all objects are linked into mixture_experts_ffn_top_amd/libmoe_mi355x.so.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe_mi355x.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Wall", "-Wno-unused-function",
    # keep hand-written and compiler-made code off the packed fp32 VALU forms
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _compile(src: str, obj: str) -> None:
    cmd = [_hipcc(), *HIPCC_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    err = "\n".join(line for line in (r.stderr or "").splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {os.path.basename(src)}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")


def build(jobs: int | None = None, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    objs = [os.path.join(BUILD, f[:-4] + ".o") for f in srcs]
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_compile, os.path.join(CSRC, s), o) for s, o in zip(srcs, objs)]
        for f in futs:
            f.result()
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    build(ap.parse_args().jobs)
