"""The C ABI used from C: tests/c_abi_example.c includes include/rfq.h,
links librfq.so and the HIP runtime, and runs the layer with no Python in
between. Without a GPU it is compiled and linked; on the GPU it runs, and its
Y must equal, bit for bit, what the Python binding returns for the same
inputs (the same entry point), and the oracle within the per-output bound."""
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "mxfp4_activation_gemm_amd")
SRC = os.path.join(ROOT, "tests", "c_abi_example.c")
ROCM = "/opt/rocm"
M, N, K = 300, 520, 1024


def build(out_dir):
    if not os.path.exists(os.path.join(PKG, "librfq.so")):
        pytest.skip("librfq.so is not built")
    exe = os.path.join(out_dir, "c_abi_example")
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC,
           "-L", PKG, "-lrfq", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath," + PKG, "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return exe


def inputs():
    """The program's input formulas (values bfloat16 holds exactly)."""
    m, n, k = np.arange(M)[:, None], np.arange(N)[:, None], np.arange(K)[None, :]
    x = ((131 * m + 71 * k) % 97 - 48) / 16.0
    w = ((37 * n + 53 * k) % 89 - 44) / 32.0
    return x, w


def test_c_program_compiles_and_links(tmp_path):
    build(str(tmp_path))


@pytest.mark.gpu
def test_c_program_matches_the_binding_and_the_oracle(tmp_path):
    import torch

    import mxfp4_activation_gemm_amd as rfq
    import oracle
    import workloads
    from gpu_helpers import check_y, dev_bf16, host, log

    exe = build(str(tmp_path))
    out = os.path.join(str(tmp_path), "y.bin")
    log("[c-abi] running the C program")
    res = subprocess.run([exe, out], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("K = 33: "), res.stdout   # the rejected call (the program checks its status)
    y_c = np.fromfile(out, dtype=np.float32).reshape(M, N)

    x, w = inputs()
    xb, wb = workloads.f32_to_bf16_bits(x.astype(np.float32)), workloads.f32_to_bf16_bits(w.astype(np.float32))
    assert (oracle.bf16_bits_to_f64(xb) == x).all() and (oracle.bf16_bits_to_f64(wb) == w).all()
    wq, sw = rfq.quantize_mxfp4(dev_bf16(wb))
    y_py = host(rfq.linear(dev_bf16(xb), wq, sw, out_dtype=torch.float32))
    assert np.array_equal(y_c.view(np.uint32), y_py.view(np.uint32)), "C and Python calls differ"

    owq, osw = oracle.quantize_mxfp4(w)
    qx, sx, qr, sr = oracle.residual_quantize(x)
    y_ref, s_ref = oracle.gemm_w4a4(qx, sx, qr, sr, owq, osw)
    check_y(y_c, y_ref, s_ref, torch.float32, "C program Y")
