"""GPU parity of the straight-through backward pass against the oracle:
dX = dY deq(Wq) and dW = dY^T (deq Q(X) + deq Q(R)), every output (or
sampled outputs at full size) within the bound of bf16 matrix instructions
with fp32 accumulation (gpu_helpers.check_grad)."""
import numpy as np
import pytest
import torch

import mxfp4_activation_gemm_amd as rfq
import oracle
import workloads
from gpu_helpers import check_grad, dev_bf16, host, host_bf16_as_f64, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rfq.library()


def g_host(t):
    return host_bf16_as_f64(t) if t.dtype == torch.bfloat16 else host(t).astype(np.float64)


def make(rng, M, N, K):
    x = rng.standard_t(3, size=(M, K)).astype(np.float32)
    x[:, rng.choice(K, size=min(3, K), replace=False)] *= 50
    w = rng.normal(0, 0.02, size=(N, K)).astype(np.float32)
    dy = (rng.normal(0, 1, size=(M, N)) * np.exp(rng.uniform(-3, 3, size=(M, 1)))).astype(np.float32)
    return workloads.f32_to_bf16_bits(x), workloads.f32_to_bf16_bits(w), workloads.f32_to_bf16_bits(dy)


@pytest.mark.parametrize("M,N,K", [(130, 264, 96), (256, 512, 256), (1, 8, 32), (300, 1000, 160), (64, 384, 640)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_dx_every_output(M, N, K, out_dtype):
    rng = np.random.default_rng(M + 3 * N + 7 * K)
    xb, wb, dyb = make(rng, M, N, K)
    log(f"[backward] dX M={M} N={N} K={K} {out_dtype}")
    wq, sw = rfq.quantize_mxfp4(dev_bf16(wb))
    dx = rfq.backward_dx(dev_bf16(dyb), wq, sw, out_dtype=out_dtype)
    owq, osw = oracle.quantize_mxfp4(oracle.bf16_bits_to_f64(wb))
    ref, s = oracle.backward_dx(oracle.bf16_bits_to_f64(dyb), owq, osw)
    check_grad(g_host(dx), ref, s, N, out_dtype, f"dX {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(130, 264, 96), (512, 384, 512), (1, 5, 32), (1000, 77, 64), (257, 256, 288)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_dw_every_output(M, N, K, out_dtype):
    rng = np.random.default_rng(5 * M + N + 11 * K)
    xb, _, dyb = make(rng, M, N, K)
    log(f"[backward] dW M={M} N={N} K={K} {out_dtype}")
    qx, sx, qr, sr = rfq.residual_quantize(dev_bf16(xb))
    dw = rfq.backward_dw(dev_bf16(dyb), qx, sx, qr, sr, out_dtype=out_dtype)
    oqx, osx, oqr, osr = oracle.residual_quantize(oracle.bf16_bits_to_f64(xb))
    ref, s = oracle.backward_dw(oracle.bf16_bits_to_f64(dyb), oqx, osx, oqr, osr)
    check_grad(g_host(dw), ref, s, 2 * ((M + 7) // 8 * 8), out_dtype, f"dW {M}x{N}x{K}")


def test_strided_gradients_and_workspace_contents():
    """dX and dW written into column slices of wider buffers (row strides
    lddx, lddw > K), the rest untouched; dY with a row stride for dW; the
    documented workspace contents."""
    rng = np.random.default_rng(77)
    M, N, K = 72, 136, 160
    xb, wb, dyb = make(rng, M, N, K)
    log("[backward] strided outputs and workspaces")
    wq, sw = rfq.quantize_mxfp4(dev_bf16(wb))
    qx, sx, qr, sr = rfq.residual_quantize(dev_bf16(xb))
    big_dx = torch.full((M, K + 40), 3.0, dtype=torch.float32, device="cuda")
    wsx = torch.empty(rfq.library().rfq_backward_dx_workspace_size(N, K), dtype=torch.uint8, device="cuda")
    rfq.backward_dx(dev_bf16(dyb), wq, sw, out=big_dx[:, 8:8 + K], workspace=wsx)
    wide_dy = torch.zeros((M, N + 24), dtype=torch.bfloat16, device="cuda")
    wide_dy[:, :N] = dev_bf16(dyb)
    big_dw = torch.full((N, K + 16), 3.0, dtype=torch.bfloat16, device="cuda")
    wsw = torch.empty(rfq.library().rfq_backward_dw_workspace_size(M, N, K), dtype=torch.uint8, device="cuda")
    rfq.backward_dw(wide_dy[:, :N], qx, sx, qr, sr, out=big_dw[:, 16:], workspace=wsw)
    torch.cuda.synchronize()
    hx, hw = host(big_dx), g_host(big_dw)
    assert (hx[:, :8] == 3.0).all() and (hx[:, 8 + K:] == 3.0).all() and (hw[:, :16] == 3.0).all()
    owq, osw = oracle.quantize_mxfp4(oracle.bf16_bits_to_f64(wb))
    dy64 = oracle.bf16_bits_to_f64(dyb)
    ref, s = oracle.backward_dx(dy64, owq, osw)
    check_grad(hx[:, 8:8 + K], ref, s, N, torch.float32, "strided dX")
    oqx, osx, oqr, osr = oracle.residual_quantize(oracle.bf16_bits_to_f64(xb))
    ref, s = oracle.backward_dw(dy64, oqx, osx, oqr, osr)
    check_grad(hw[:, 16:], ref, s, 2 * M, torch.bfloat16, "strided dW")
    # workspaces: deq(Wq)^T [K, N]; dY^T [N, Mp], deq Q(X)^T, deq Q(R)^T [K, Mp]
    bf = lambda a: a.view(np.uint16).astype(np.uint32).__lshift__(16).view(np.float32).astype(np.float64)
    wdt = bf(host(wsx)[:K * N * 2].copy()).reshape(K, N)
    assert np.array_equal(wdt, oracle.dequantize(owq, osw).T)
    mp = (M + 7) // 8 * 8
    r256 = lambda b: (b + 255) // 256 * 256
    h = host(wsw)
    dyt = bf(h[:N * mp * 2].copy()).reshape(N, mp)
    xqt = bf(h[r256(N * mp * 2):r256(N * mp * 2) + K * mp * 2].copy()).reshape(K, mp)
    assert np.array_equal(dyt[:, :M], dy64.T) and not dyt[:, M:].any()
    assert np.array_equal(xqt[:, :M], oracle.dequantize(oqx, osx).T) and not xqt[:, M:].any()


def test_full_size_sampled_and_adjoint():
    """The Wan2.2-style layer at full size (dY [4096, 13824], X [4096, 5120],
    W [13824, 5120]): sampled rows of dX and of dW against the oracle, and the
    adjoint identity <dY, Y> = <dX, Xh> on the GPU's own Y and dX."""
    cfg = workloads.CONFIGS["wan22_ffn"]
    M, N, K = cfg.M, cfg.N, cfg.K
    log("[backward] full size: generating")
    xb, wb = workloads.x_bf16(cfg), workloads.w_bf16(cfg)
    rng = np.random.default_rng(cfg.seed + 100)
    dyb = workloads.f32_to_bf16_bits(rng.normal(0, 1, size=(M, N)).astype(np.float32))
    x, dy = dev_bf16(xb), dev_bf16(dyb)
    wq, sw = rfq.quantize_mxfp4(dev_bf16(wb))
    qx, sx, qr, sr = rfq.residual_quantize(x)
    log("   running on the GPU")
    dx = rfq.backward_dx(dy, wq, sw)
    dw = rfq.backward_dw(dy, qx, sx, qr, sr)
    y = rfq.gemm_w4a4(qx, sx, qr, sr, wq, sw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = workloads.sample_rows(cfg, n_random=30)
    owq, osw = oracle.quantize_mxfp4(oracle.bf16_bits_to_f64(wb))
    dy64 = oracle.bf16_bits_to_f64(dyb)
    ref, s = oracle.backward_dx(dy64[rows], owq, osw)
    check_grad(host(dx)[rows], ref, s, N, torch.float32, "full dX rows")
    oqx, osx, oqr, osr = oracle.residual_quantize(oracle.bf16_bits_to_f64(xb))
    ncols = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 30, replace=False)]))
    ref, s = oracle.backward_dw(dy64[:, ncols], oqx, osx, oqr, osr)
    check_grad(host(dw)[ncols], ref, s, 2 * M, torch.float32, "full dW rows")
    xh = oracle.dequantize(oqx, osx) + oracle.dequantize(oqr, osr)
    a = float(np.sum(dy64 * host(y).astype(np.float64)))
    b = float(np.sum(host(dx).astype(np.float64) * xh))
    scale = float(np.sum(np.abs(dy64) @ np.abs(oracle.dequantize(owq, osw)) * np.abs(xh)))
    log(f"   <dY, Y> = {a:.6e}, <dX, Xh> = {b:.6e}, scale {scale:.3e}")
    assert abs(a - b) <= 1e-4 * scale


@pytest.mark.parametrize("M", [4096, 8192])
def test_wide_tiles_every_output(M):
    """dX outputs [M, 5120] that 256 x 320 tiles cover in whole rounds on 256
    CUs (256 tiles: one per CU; 512: two streamed per CU) while 256 x 256
    tiles would leave a partial round, the planner's case for the wide tiles
    (as in dX of the 4096 x 5120 x 13824 layer): every output against the
    oracle, with a short contraction N (a multiple of 128, which the wide
    tiles need: the contraction in whole 512-element groups of the GEMM's
    E2M1-sized K units)."""
    N, K = 128, 5120
    rng = np.random.default_rng(M + 13)
    _, wb, dyb = make(rng, M, N, K)
    log(f"[backward] wide-tile dX M={M} N={N} K={K}")
    wq, sw = rfq.quantize_mxfp4(dev_bf16(wb))
    dx = rfq.backward_dx(dev_bf16(dyb), wq, sw, out_dtype=torch.bfloat16)
    owq, osw = oracle.quantize_mxfp4(oracle.bf16_bits_to_f64(wb))
    ref, s = oracle.backward_dx(oracle.bf16_bits_to_f64(dyb), owq, osw)
    check_grad(g_host(dx), ref, s, N, torch.bfloat16, f"wide dX {M}x{N}x{K}")


@pytest.mark.parametrize("which,M,N,K", [("dx", 4096, 128, 8192), ("dw", 128, 8192, 4096)])
def test_streamed_tiles_every_output(which, M, N, K):
    """Output shapes of two whole rounds of 256 x 256 tiles on 256 CUs, so
    that each workgroup streams its tiles back to back (for dW with the
    transposed store): every output checked."""
    rng = np.random.default_rng(M + N + K + (1 if which == "dw" else 0))
    xb, wb, dyb = make(rng, M, N, K)
    log(f"[backward] streamed {which} M={M} N={N} K={K}")
    dy64 = oracle.bf16_bits_to_f64(dyb)
    if which == "dx":
        wq, sw = rfq.quantize_mxfp4(dev_bf16(wb))
        got = host(rfq.backward_dx(dev_bf16(dyb), wq, sw)).astype(np.float64)
        owq, osw = oracle.quantize_mxfp4(oracle.bf16_bits_to_f64(wb))
        ref, s = oracle.backward_dx(dy64, owq, osw)
        check_grad(got, ref, s, N, torch.float32, "streamed dX")
    else:
        qx, sx, qr, sr = rfq.residual_quantize(dev_bf16(xb))
        got = g_host(rfq.backward_dw(dev_bf16(dyb), qx, sx, qr, sr, out_dtype=torch.bfloat16))
        oqx, osx, oqr, osr = oracle.residual_quantize(oracle.bf16_bits_to_f64(xb))
        ref, s = oracle.backward_dw(dy64, oqx, osx, oqr, osr)
        check_grad(got, ref, s, 2 * M, torch.bfloat16, "streamed dW")
