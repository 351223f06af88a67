"""Build libnupaged.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libnupaged.so")
ARCH = "gfx950"
# Packed fp32 vector instructions are kept out of the generated code.
NO_PACKED_FP32 = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hc = hipcc()
    inc = ["-I", os.path.join(os.path.dirname(HERE), "include")]
    kobj = os.path.join(BUILD, "kernels.o")
    hobj = os.path.join(BUILD, "host.o")
    _run([hc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", *NO_PACKED_FP32, *inc,
          "-c", os.path.join(CSRC, "kernels.hip"), "-o", kobj], verbose)
    _run([hc, "-O2", "-std=c++17", "-fPIC", "-Wall", *inc,
          "-c", os.path.join(CSRC, "host.cpp"), "-o", hobj], verbose)
    tmp = LIB + ".tmp"
    _run([hc, f"--offload-arch={ARCH}", "-shared", "-fPIC", kobj, hobj, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
