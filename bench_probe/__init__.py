"""Benchmark-only MFMA ceiling probe (librfqprobe.so), loaded by bench.py.

The probe is a measurement tool, not part of the RFQ layer: it lives in its
own shared library so that librfq.so exports only the layer's entry points.
build() compiles it in-tree with hipcc for gfx950 (no GPU needed); load()
returns the ctypes library, building it first if it is missing.
"""
import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librfqprobe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep the compiler from forming packed fp32 ops (v_pk_{add,mul,fma}_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-I", HERE,
]

_p, _sz, _i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
SIGNATURES = {
    "rfq_probe_mfma_ceiling": (_i, [_p, _sz, _p, _sz, _i, _i, _p, _p, _p]),
    "rfq_probe_mfma_ceiling_e4m3": (_i, [_p, _sz, _p, _sz, _i, _i, _p, _p, _p]),
}
_LIB = None


def build(verbose=False):
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, *FLAGS, os.path.join(HERE, "probe.hip"), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def load():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            build()
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def check(status):
    if status != 0:
        raise RuntimeError(f"probe call failed with status {status}")
