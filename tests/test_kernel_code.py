"""Checks on the generated gfx950 code of the HIP sources (no GPU needed).

Every kernel must be one function: the GEMM kernel reads its parameter block
again from the kernel-argument segment once per tile, and in a called
function that segment's pointer is not available (the compiler substitutes
0, so the read faults). The kernel body's lambdas are therefore forced
inline; this test compiles each source to assembly and checks that no
kernel calls a function or touches scratch memory (which would also mean
spilled or stack-resident arrays)."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mxfp4_activation_gemm_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
PROBE = os.path.join(ROOT, "bench_probe")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="hipcc not available")
@pytest.mark.parametrize("source", [os.path.join(CSRC, "gemm.hip"), os.path.join(CSRC, "quantize.hip"),
                                    os.path.join(CSRC, "backward.hip"), os.path.join(PROBE, "probe.hip")])
def test_kernels_make_no_calls_and_use_no_scratch(source, tmp_path):
    out = tmp_path / (os.path.basename(source) + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", INCLUDE, "-I", CSRC, "-I", PROBE, "-S", "--cuda-device-only", source,
           "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    text = out.read_text()
    functions = re.findall(r"^(_Z\S+):", text, flags=re.M)
    assert functions
    assert not re.search(r"\bs_swappc_b64\b|\bs_setpc_b64\b", text), "a kernel calls a function"
    assert not re.search(r"\bscratch_(load|store)", text), "a kernel uses scratch memory"
    assert not re.search(r"private_segment_fixed_size:\s*[1-9]", text), "a kernel reserves scratch"
