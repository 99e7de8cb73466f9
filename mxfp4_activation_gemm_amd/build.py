"""Builds librfq.so in-tree with hipcc for gfx950 (no GPU needed to build).

Usage: python -m mxfp4_activation_gemm_amd.build
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "librfq.so")
SOURCES = ["quantize.hip", "gemm.hip", "backward.hip", "noalloc.hip", "api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep the compiler from forming packed fp32 ops (v_pk_{add,mul,fma}_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def build(verbose=False):
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("packed-fp32-ops", "argument unused during compilation")
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if not any(n in l for n in noise)]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if msgs and verbose:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
