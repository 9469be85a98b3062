"""Build libfarskip_moe.so for gfx950 (MI355X) with hipcc, in-tree.

    python -m mixture_experts_layer_sum_amd.build

Compiles every csrc/*.hip to an object in csrc/_build/ (in parallel) and links them into
mixture_experts_layer_sum_amd/libfarskip_moe.so.  Works without a GPU (hipcc cross-compiles).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libfarskip_moe.so")
ARCH = os.environ.get("FARSKIP_MOE_ARCH", "gfx950")

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    # packed fp32 ops are left to neither the compiler nor hand code on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libfarskip_moe")
    return path


def _compile(src: str, obj: str) -> tuple[str, int, str]:
    cmd = [hipcc(), *CFLAGS, "-c", src, "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; drop that noise
    err = "\n".join(l for l in (p.stdout + p.stderr).splitlines()
                    if "packed-fp32-ops" not in l or "error" in l.lower())
    return src, p.returncode, err


def build(verbose: bool = True) -> str:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    bdir = os.path.join(CSRC, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = []
    jobs = []
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        for s in srcs:
            o = os.path.join(bdir, os.path.basename(s)[:-4] + ".o")
            objs.append(o)
            jobs.append(ex.submit(_compile, s, o))
        failed = []
        for j in jobs:
            src, rc, err = j.result()
            if err.strip() and verbose:
                print(f"[build] {os.path.basename(src)}:\n{err}", file=sys.stderr)
            if rc != 0:
                failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for: {', '.join(map(os.path.basename, failed))}")
    tmp = OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{p.stdout}\n{p.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"[build] wrote {OUT}", file=sys.stderr)
    return OUT


if __name__ == "__main__":
    build()
