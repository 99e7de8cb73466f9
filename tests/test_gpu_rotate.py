"""GPU parity of the fp32-input quantize paths and of the block-Hadamard
rotated paths (activation X H with the RFQ residual, weight W H / 32):
codes and scales bit-exact against the oracle, and the rotated layer's Y
within the per-output tolerance."""
import numpy as np
import pytest
import torch

import mxfp4_activation_gemm_amd as rfq
import oracle
import workloads
from gpu_helpers import assert_bytes_equal, check_y, dev_bf16, host, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rfq.library()


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def check_mx(got, want, what):
    (gc, gs), (wc, ws) = got, want
    assert_bytes_equal(host(gc), oracle.pack_codes(wc), what + " codes")
    assert_bytes_equal(host(gs), ws, what + " scales")


def check_rfq(got, want, what):
    check_mx(got[:2], want[:2], what + " Q(X)")
    check_mx(got[2:], want[2:], what + " Q(R)")


def near_midpoints(rng, rows, K):
    """fp32 blocks that pin every E2M1 rounding decision: one element at
    4 * 2^se fixes the scale, the rest sit at midpoints and a few float32
    ulps either side of them (and of 6, the saturation edge), with random
    signs, scale exponents and positions."""
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.5, 3.0], dtype=np.float32)
    base = rng.choice(mids, size=(rows, K)).astype(np.float32)
    k = rng.integers(-3, 4, size=(rows, K))
    v = base.copy()
    for step in range(3):
        up, dn = k > step, k < -step
        v = np.where(up, np.nextafter(v, np.float32(np.inf)), v)
        v = np.where(dn, np.nextafter(v, np.float32(0)), v)
    v[:, ::32] = 4.0
    v *= rng.choice([-1.0, 1.0], size=(rows, K)).astype(np.float32)
    se = rng.integers(-20, 20, size=(rows, K // 32))
    return (v * np.repeat(np.exp2(se), 32, axis=1)).astype(np.float32)


def heavy_f32(rng, rows, K):
    x = rng.standard_t(3, size=(rows, K)) * np.exp(rng.uniform(-6, 6, size=(rows, 1)))
    x[:, rng.choice(K, size=3, replace=False)] *= 80
    x = x.astype(np.float32)
    x[0, :32] = 0.0
    x[0, 32:64] = -0.0
    x[1, :16] = np.float32(1e-40)            # float32 subnormals
    return x


@pytest.mark.parametrize("kind", ["midpoints", "heavy"])
def test_fp32_input_quantize_and_residual(kind):
    rng = np.random.default_rng(31 if kind == "midpoints" else 32)
    rows, K = 96, 1024
    x = near_midpoints(rng, rows, K) if kind == "midpoints" else heavy_f32(rng, rows, K)
    log(f"[rotate] fp32 input {kind}")
    xd = dev_f32(x)
    got_q = rfq.quantize_mxfp4(xd)
    got_r = rfq.residual_quantize(xd)
    torch.cuda.synchronize()
    x64 = x.astype(np.float64)
    check_mx(got_q, oracle.quantize_mxfp4(x64), f"fp32 {kind}")
    check_rfq(got_r, oracle.residual_quantize(x64), f"fp32 {kind}")


def spiky_bf16(rng, rows, K):
    x = rng.laplace(0, 1, size=(rows, K)).astype(np.float32)
    x[:, rng.choice(K, size=8, replace=False)] *= 80.0
    x[2, 5] = 3e38
    bits = workloads.f32_to_bf16_bits(x)
    bits[3, 40] = 0x7FC0          # NaN
    bits[4, 70] = 0xFF80          # -Inf
    bits[5, :32] = 0x8000         # -0.0 block
    return bits


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_rotated_activation_and_weight_bit_exact(dtype):
    rng = np.random.default_rng(41)
    M, N, K = 200, 72, 640
    if dtype == "bf16":
        xb = spiky_bf16(rng, M, K)
        wb = workloads.f32_to_bf16_bits(rng.normal(0, 0.02, (N, K)).astype(np.float32))
        xd, wd = dev_bf16(xb), dev_bf16(wb)
        x64, w64 = oracle.bf16_bits_to_f64(xb), oracle.bf16_bits_to_f64(wb)
    else:
        x = heavy_f32(rng, M, K)
        x[7, 100] = np.nan
        w = (rng.normal(0, 0.02, (N, K)) * np.exp(rng.uniform(-30, 3, (N, 1)))).astype(np.float32)
        xd, wd = dev_f32(x), dev_f32(w)
        x64, w64 = x.astype(np.float64), w.astype(np.float64)
    log(f"[rotate] rotated quantize {dtype}")
    got_x = rfq.rotate_residual_quantize(xd)
    got_w = rfq.rotate_quantize_weight(wd)
    torch.cuda.synchronize()
    check_rfq(got_x, oracle.rotate_residual_quantize(x64), f"rotated X {dtype}")
    check_mx(got_w, oracle.rotate_quantize_weight(w64), f"rotated W {dtype}")


@pytest.mark.parametrize("M,N,K", [(130, 200, 512), (64, 96, 160)])
def test_rotated_layer_every_output(M, N, K):
    """Q(XH), Q(R) and Q(WH/32) from the GPU into the unchanged W4A4 GEMM;
    Y against the oracle's rotated layer, and the rotation's effect on the
    error against the float64 product X W^T logged beside plain RFQ's."""
    rng = np.random.default_rng(M + N + K)
    x = rng.standard_t(3, size=(M, K)).astype(np.float32)
    x[:, rng.choice(K, size=4, replace=False)] *= 60
    xb = workloads.f32_to_bf16_bits(x)
    wb = workloads.f32_to_bf16_bits(rng.normal(0, 0.02, (N, K)).astype(np.float32))
    log(f"[rotate] rotated layer {M}x{N}x{K}")
    xd, wd = dev_bf16(xb), dev_bf16(wb)
    qx, sx, qr, sr = rfq.rotate_residual_quantize(xd)
    wq, sw = rfq.rotate_quantize_weight(wd)
    y = host(rfq.gemm_w4a4(qx, sx, qr, sr, wq, sw, out_dtype=torch.float32)).astype(np.float64)
    x64, w64 = oracle.bf16_bits_to_f64(xb), oracle.bf16_bits_to_f64(wb)
    y_ref, s_ref, _, _ = oracle.linear_rotated(x64, w64)
    worst = check_y(y, y_ref, s_ref, torch.float32, "rotated layer")
    exact = x64 @ w64.T
    y_plain, _, _, _ = oracle.linear(x64, w64)
    err = lambda a: float(np.linalg.norm(a - exact) / np.linalg.norm(exact))
    log(f"   max |dY|/S = {worst:.2e}; relative error vs X W^T: rotated RFQ {err(y):.3e}, plain RFQ {err(y_plain):.3e}")


def test_rotated_full_size_sampled():
    """The Wan2.2-style layer's full X through the rotated activation pass
    (the launch the benchmark's rotated line times); sampled rows bit-exact."""
    cfg = workloads.CONFIGS["wan22_ffn"]
    log(f"[rotate] full size {cfg.name}")
    xb = workloads.x_bf16(cfg)
    qx, sx, qr, sr = rfq.rotate_residual_quantize(dev_bf16(xb))
    torch.cuda.synchronize()
    rows = workloads.sample_rows(cfg, n_random=62)
    want = oracle.rotate_residual_quantize(oracle.bf16_bits_to_f64(xb[rows]))
    got = tuple(t[torch.from_numpy(rows).cuda()] for t in (qx, sx, qr, sr))
    check_rfq(got, want, "rotated wan22 rows")
