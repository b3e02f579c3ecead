"""Build the HIP library ``_kda.so`` (gfx950) in-tree with hipcc.

Every source under ``csrc/`` is compiled for gfx950 only.  Packed-fp32 instructions are
disabled (``-packed-fp32-ops``).  The library links the HIP runtime by soname, so when
loaded after ``import torch`` it shares torch's runtime (one HIP runtime per process).
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "_kda.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
    ]


def build_library(verbose: bool = False, jobs: int = 8) -> str:
    """Compile csrc/*.hip and csrc/*.cpp to objects (in parallel), link ``_kda.so``."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs, objs = [], []
    for s in srcs:
        o = os.path.join(objdir, os.path.basename(s) + ".o")
        objs.append(o)
        cmd = [hipcc()] + compile_flags() + ["-c", s, "-o", o]
        if s.endswith(".cpp"):
            cmd = [hipcc(), "-x", "hip"] + compile_flags() + ["-c", s, "-o", o]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((s, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _wait(procs.pop(0))
    for p in procs:
        _wait(p)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def _wait(item):
    src, p = item
    out, _ = p.communicate()
    text = out.decode(errors="replace")
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{text}")
    lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]
    if any(lines):
        print("\n".join(lines), flush=True)


if __name__ == "__main__":
    print(build_library(verbose=True))
