"""Build ``libmxq.so`` in-tree with hipcc for gfx950.

    python -m mx_microscaling_quantization_amd._build

Compiles every HIP source under ``csrc/`` into one shared library next to
this file. Always rebuilds (the caller asked for a build).
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libmxq.so")

ARCH = "gfx950"
# -packed-fp32-ops: keep the compiler from forming v_pk_{add,mul,fma}_f32.
HIPCC_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmxq.so)")


def build(verbose: bool = False) -> str:
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not sources:
        raise RuntimeError("no HIP sources under %s" % CSRC)
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + HIPCC_FLAGS + ["-I" + INCLUDE, "-I" + CSRC, "-o", tmp] + sources
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that noise
    noise = ("packed-fp32-ops", "not a recognized feature")
    err = "\n".join(l for l in proc.stderr.splitlines() if not any(n in l for n in noise)).strip()
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (proc.returncode, err))
    if err and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
