"""GPU parity of the RFQ layer with the quantization inside the GEMM
(rfq_linear_fused): every output against the oracle within 1e-5 of its
condition scale (plus the bf16 half-ulp for bf16 Y), and Y bit-equal to the
two-kernel rfq_linear, whose codes the oracle pins byte for byte (the fused
GEMM encodes each tile with the same instructions and accumulates in the
same order)."""
import numpy as np
import pytest
import torch

import mxfp4_activation_gemm_amd as rfq
import oracle
import workloads
from gpu_helpers import check_exact_where_covered, check_y, dev_bf16, host, host_bf16_as_f64, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rfq.library()


def bits(y):
    return host(y.view(torch.int16)) if y.dtype == torch.bfloat16 else host(y.view(torch.int32))


def y_host(y):
    return host_bf16_as_f64(y) if y.dtype == torch.bfloat16 else host(y).astype(np.float64)


def operands(M, N, K, seed, outliers=3):
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3, size=(M, K)).astype(np.float32)
    if outliers:
        x[:, rng.choice(K, size=min(outliers, K), replace=False)] *= 60
    return (workloads.f32_to_bf16_bits(x),
            workloads.f32_to_bf16_bits(rng.normal(0, 0.02, (N, K)).astype(np.float32)))


def oracle_y(xb, wb, with_scales=False):
    """Oracle Y and S; with_scales adds the E8M0 codes of each product's
    operands, [(sx, sw), (sr, sw)]."""
    y, s, (_, sx, _, sr), (_, sw) = oracle.linear(oracle.bf16_bits_to_f64(xb), oracle.bf16_bits_to_f64(wb))
    return (y, s, [(sx, sw), (sr, sw)]) if with_scales else (y, s)


@pytest.mark.parametrize("M,N,K", [(1, 1, 512), (33, 65, 512), (128, 256, 512), (300, 520, 1024), (257, 255, 1536),
                                   (130, 600, 2048)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_fused_every_output(M, N, K, out_dtype):
    xb, wb = operands(M, N, K, M * 7 + N * 13 + K)
    log(f"[fused] M={M} N={N} K={K} {out_dtype}")
    x = dev_bf16(xb)
    wq, sw = rfq.quantize_mxfp4(dev_bf16(wb))
    y = rfq.linear_fused(x, wq, sw, out_dtype=out_dtype)
    y2 = rfq.linear(x, wq, sw, out_dtype=out_dtype)
    torch.cuda.synchronize()
    y_ref, s_ref, pairs = oracle_y(xb, wb, with_scales=True)
    worst = check_y(y_host(y), y_ref, s_ref, out_dtype, f"fused {M}x{N}x{K}")
    check_exact_where_covered(y_host(y), y_ref, s_ref, pairs, out_dtype, f"fused {M}x{N}x{K}")
    assert np.array_equal(bits(y), bits(y2)), "fused Y differs from rfq_linear's"
    log(f"   ok, max |dY|/S = {worst:.2e}, bit-equal to rfq_linear")


@pytest.mark.parametrize("M,N,K", [(4096, 8192, 1024), (4096, 8448, 512), (2048, 4096, 2048)])
def test_fused_streamed_tiles_every_output(M, N, K):
    """Tiles inside Y: one workgroup per CU streams several 128 x 256 tiles
    back to back (4096 x 8448 leaves a partial last round: some workgroups
    take one tile more). Every output checked (fp32 Y)."""
    xb, wb = operands(M, N, K, M + N + K)
    log(f"[fused] streamed M={M} N={N} K={K}")
    x = dev_bf16(xb)
    wq, sw = rfq.quantize_mxfp4(dev_bf16(wb))
    y = rfq.linear_fused(x, wq, sw, out_dtype=torch.float32)
    y2 = rfq.linear(x, wq, sw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y), bits(y2)), "fused Y differs from rfq_linear's"
    y_ref, s_ref, pairs = oracle_y(xb, wb, with_scales=True)
    worst = check_y(y_host(y), y_ref, s_ref, torch.float32, f"fused streamed {M}x{N}x{K}")
    check_exact_where_covered(y_host(y), y_ref, s_ref, pairs, torch.float32, f"fused streamed {M}x{N}x{K}")
    log(f"   ok, max |dY|/S = {worst:.2e}")


def test_fused_strided_x_and_y_nan_block():
    """X as a column slice of a wider tensor (ldx > K), Y written into a
    strided view; a NaN in one block of X poisons exactly its row, as in the
    two-kernel layer."""
    M, N, K = 200, 300, 1024
    xb, wb = operands(M, N, K, 5)
    wide = np.zeros((M, K + 512), np.uint16)
    wide[:, 256:256 + K] = xb
    wide[17, 256 + 40] = 0x7FC0                  # NaN in block 1 of row 17
    xw = dev_bf16(wide)
    x = xw[:, 256:256 + K]
    wq, sw = rfq.quantize_mxfp4(dev_bf16(wb))
    ybig = torch.full((M, N + 64), 7.0, dtype=torch.float32, device="cuda")
    y = ybig[:, 32:32 + N]
    rfq.linear_fused(x, wq, sw, out=y)
    y2 = rfq.linear(x, wq, sw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    yh = host(ybig)
    assert (yh[:, :32] == 7.0).all() and (yh[:, 32 + N:] == 7.0).all()
    assert np.array_equal(bits(y.contiguous()), bits(y2))
    assert np.isnan(yh[17, 32:32 + N]).all()
    rows = np.array([r for r in range(M) if r != 17])
    xs = wide[:, 256:256 + K]
    y_ref, s_ref = oracle_y(xs[rows], wb)
    check_y(yh[rows, 32:32 + N].astype(np.float64), y_ref, s_ref, torch.float32, "fused strided")


def test_fused_rejects_what_it_does_not_cover():
    x = torch.zeros((8, 256), dtype=torch.bfloat16, device="cuda")
    wq = torch.zeros((8, 128), dtype=torch.uint8, device="cuda")
    sw = torch.zeros((8, 8), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="multiple of 512"):
        rfq.linear_fused(x, wq, sw)
    x32 = torch.zeros((8, 512), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="bf16"):
        rfq.linear_fused(x32, torch.zeros((8, 256), dtype=torch.uint8, device="cuda"),
                         torch.zeros((8, 16), dtype=torch.uint8, device="cuda"))


@pytest.mark.parametrize("name", ["qwen3vl_attn_proj", "wan22_ffn", "dit_ffn_down"])
def test_fused_full_size_config(name):
    """The configuration at full size through rfq_linear_fused: Y bit-equal to
    rfq_linear's over the whole output (bf16 and fp32), and against the oracle
    at 128 sampled rows x 256 sampled columns."""
    cfg = workloads.CONFIGS[name]
    log(f"[fused] full size {name} M={cfg.M} N={cfg.N} K={cfg.K}")
    xb, wb = workloads.x_bf16(cfg), workloads.w_bf16(cfg)
    x = dev_bf16(xb)
    wq, sw = rfq.quantize_mxfp4(dev_bf16(wb))
    for od in (torch.bfloat16, torch.float32):
        y = rfq.linear_fused(x, wq, sw, out_dtype=od)
        y2 = rfq.linear(x, wq, sw, out_dtype=od)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16 if od == torch.bfloat16 else torch.int32),
                           y2.view(torch.int16 if od == torch.bfloat16 else torch.int32)), f"{od}: fused != linear"
        del y2
        if od == torch.float32:
            rows = workloads.sample_rows(cfg, n_random=126)
            cols = np.unique(np.concatenate([[0, cfg.N - 1],
                                             np.random.default_rng(cfg.seed).choice(cfg.N, 254, replace=False)]))
            yh = host(y)[np.ix_(rows, cols)].astype(np.float64)
            y_ref, s_ref = oracle_y(xb[rows], wb[cols])
            worst = check_y(yh, y_ref, s_ref, od, f"fused {name}")
            log(f"   ok, max |dY|/S = {worst:.2e}; bf16 and fp32 Y bit-equal to rfq_linear")
        del y
