"""GPU parity of the W4A4 GEMM and the whole RFQ linear layer against the
oracle: codes and scales bit-exact, Y within 1e-5 of the condition scale
per output (plus the bf16 rounding half-ulp for bf16 outputs), and, at every
output whose sum the arithmetic makes exact in fp32 (gpu_helpers.exact_cover),
Y bit-equal to the exact sum (fp32) or to its RNE to bf16."""
import numpy as np
import pytest
import torch

import mxfp4_activation_gemm_amd as rfq
import oracle
import workloads
from gpu_helpers import (REL_TOL, assert_bytes_equal, check_exact_where_covered, check_y, dev_bf16, dev_u8, host,
                         host_bf16_as_f64, log, oracle_mx, oracle_rfq)

pytestmark = pytest.mark.gpu

SPEC_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rfq.library()


def y_host(y):
    return host_bf16_as_f64(y) if y.dtype == torch.bfloat16 else host(y).astype(np.float64)


def oracle_y(x_bits, w_bits, resid=True, with_scales=False):
    """Oracle Y and S; with_scales adds the E8M0 codes of each product's
    operands, [(sx, sw), (sr, sw)] (the residual pair only with resid)."""
    x = oracle.bf16_bits_to_f64(x_bits)
    w = oracle.bf16_bits_to_f64(w_bits)
    wq, sw = oracle.quantize_mxfp4(w)
    qx, sx, qr, sr = oracle.residual_quantize(x)
    if not resid:
        qr = sr = None
    y, s = oracle.gemm_w4a4(qx, sx, qr, sr, wq, sw)
    if with_scales:
        return y, s, [(sx, sw)] + ([(sr, sw)] if resid else [])
    return y, s


def heavy(rng, rows, K, outliers=3):
    x = rng.standard_t(3, size=(rows, K)).astype(np.float32)
    if outliers:
        x[:, rng.choice(K, size=min(outliers, K), replace=False)] *= 60
    return workloads.f32_to_bf16_bits(x)


def test_tiny_config_every_output_fp32():
    cfg = workloads.CONFIGS["tiny"]
    xb, wb = workloads.x_bf16(cfg), workloads.w_bf16(cfg)
    log("[gemm] tiny config")
    wq, sw = rfq.quantize_mxfp4(dev_bf16(wb))
    y = rfq.linear(dev_bf16(xb), wq, sw, out_dtype=torch.float32)
    y_ref, s_ref = oracle_y(xb, wb)
    worst = check_y(y_host(y), y_ref, s_ref, torch.float32, "tiny")
    log(f"   max |dY|/S = {worst:.2e}")


@pytest.mark.parametrize("M,N,K", [(300, 520, 416), (1, 1, 32), (33, 65, 96), (257, 255, 128), (70, 300, 4128),
                                   (512, 512, 1024), (300, 520, 1024), (257, 1000, 512)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_ragged_shapes_every_output(M, N, K, out_dtype):
    rng = np.random.default_rng(M * 7 + N * 13 + K)
    xb, wb = heavy(rng, M, K), workloads.f32_to_bf16_bits(rng.normal(0, 0.02, (N, K)).astype(np.float32))
    log(f"[gemm] ragged M={M} N={N} K={K} {out_dtype}")
    x = dev_bf16(xb)
    wq, sw = rfq.quantize_mxfp4(dev_bf16(wb))
    y = rfq.linear(x, wq, sw, out_dtype=out_dtype)
    y_ref, s_ref, pairs = oracle_y(xb, wb, with_scales=True)
    check_y(y_host(y), y_ref, s_ref, out_dtype, f"rfq {M}x{N}x{K}")
    cov = check_exact_where_covered(y_host(y), y_ref, s_ref, pairs, out_dtype, f"rfq {M}x{N}x{K}")
    # plain W4A4 through the same kernel family
    qx, sx, _, _ = rfq.residual_quantize(x)
    y1 = rfq.gemm_w4a4(qx, sx, None, None, wq, sw, out_dtype=out_dtype)
    y1_ref, s1_ref, pairs1 = oracle_y(xb, wb, resid=False, with_scales=True)
    check_y(y_host(y1), y1_ref, s1_ref, out_dtype, f"w4a4 {M}x{N}x{K}")
    cov1 = check_exact_where_covered(y_host(y1), y1_ref, s1_ref, pairs1, out_dtype, f"w4a4 {M}x{N}x{K}")
    log(f"   exact sums (Y bit-equal to the exact result) at {100 * cov:.1f}% (RFQ), {100 * cov1:.1f}% (W4A4)")


def test_all_code_pairs_single_block():
    # row a of Q(X) holds code a at k = 7, row b of W holds code b there; unit
    # scales: Y[a, b] = value(a) * value(b) exactly
    qx = np.zeros((16, 32), np.uint8)
    wq = np.zeros((16, 32), np.uint8)
    qx[:, 7] = np.arange(16)
    wq[:, 7] = np.arange(16)
    ones = np.full((16, 1), 127, np.uint8)
    log("[gemm] code pairs")
    y = rfq.gemm_w4a4(dev_u8(oracle.pack_codes(qx)), dev_u8(ones), None, None, dev_u8(oracle.pack_codes(wq)),
                      dev_u8(ones), out_dtype=torch.float32)
    vals = np.array(SPEC_E2M1 + [-v for v in SPEC_E2M1])
    assert (host(y) == np.outer(vals, vals)).all()


def test_every_code_in_every_lane_position():
    # random codes at every (row, k) with scale codes spread over a wide range
    rng = np.random.default_rng(21)
    M, N, K = 96, 160, 640
    qx = rng.integers(0, 16, (M, K)).astype(np.uint8)
    qr = rng.integers(0, 16, (M, K)).astype(np.uint8)
    wq = rng.integers(0, 16, (N, K)).astype(np.uint8)
    sx = rng.integers(64, 170, (M, K // 32)).astype(np.uint8)
    sr = rng.integers(64, 170, (M, K // 32)).astype(np.uint8)
    sw = rng.integers(64, 170, (N, K // 32)).astype(np.uint8)
    log("[gemm] random codes and scales")
    y = rfq.gemm_w4a4(dev_u8(oracle.pack_codes(qx)), dev_u8(sx), dev_u8(oracle.pack_codes(qr)), dev_u8(sr),
                      dev_u8(oracle.pack_codes(wq)), dev_u8(sw), out_dtype=torch.float32)
    y_ref, s_ref = oracle.gemm_w4a4(qx, sx, qr, sr, wq, sw)
    check_y(host(y), y_ref, s_ref, torch.float32, "random codes")


def test_selector_weight_returns_dequantized_activations():
    cfg = workloads.CONFIGS["tiny"]
    xb = workloads.x_bf16(cfg)
    K = cfg.K
    w = np.eye(K, dtype=np.float32)[:128]
    wb = workloads.f32_to_bf16_bits(w)
    log("[gemm] selector")
    wq, sw = rfq.quantize_mxfp4(dev_bf16(wb))
    y = rfq.linear(dev_bf16(xb), wq, sw, out_dtype=torch.float32)
    qx, sx, qr, sr = oracle.residual_quantize(oracle.bf16_bits_to_f64(xb))
    want = (oracle.dequantize(qx, sx) + oracle.dequantize(qr, sr))[:, :128]
    assert (host(y).astype(np.float64) == want).all()


def test_nan_block_gives_nan_outputs_only_in_its_row():
    rng = np.random.default_rng(22)
    M, N, K = 64, 96, 256
    xb = heavy(rng, M, K)
    xb[5, 40] = 0x7FC0          # NaN
    xb[9, 200] = 0x7F80         # +Inf
    wb = workloads.f32_to_bf16_bits(rng.normal(0, 0.02, (N, K)).astype(np.float32))
    log("[gemm] NaN/Inf blocks")
    x = dev_bf16(xb)
    qx, sx, qr, sr = rfq.residual_quantize(x)
    oqx, osx, oqr, osr = oracle_rfq(xb)
    assert_bytes_equal(host(sx), osx, "SX")
    assert_bytes_equal(host(sr), osr, "SR")
    assert_bytes_equal(host(qx), oqx, "QX")
    assert_bytes_equal(host(qr), oqr, "QR")
    wq, sw = rfq.quantize_mxfp4(dev_bf16(wb))
    y = host(rfq.gemm_w4a4(qx, sx, qr, sr, wq, sw, out_dtype=torch.float32))
    assert np.isnan(y[5]).all() and np.isnan(y[9]).all()
    ok_rows = [r for r in range(M) if r not in (5, 9)]
    assert np.isfinite(y[ok_rows]).all()


def test_maximum_k_every_output():
    """K at the ABI's limit, 2^22 (32768 stages, 131072 scale blocks per row):
    every output of a 4 x 8 RFQ layer against the oracle. The fp32
    accumulator takes 2K/128 step sums here, so the bound is the worst case
    (2K/128 + 1) 2^-24 S of that many roundings rather than 1e-5 S."""
    M, N, K = 4, 8, 1 << 22
    rng = np.random.default_rng(99)
    xb = heavy(rng, M, K)
    wb = workloads.f32_to_bf16_bits(rng.normal(0, 0.02, (N, K)).astype(np.float32))
    log(f"[gemm] maximum K = {K}")
    x = dev_bf16(xb)
    y = rfq.linear(x, *rfq.quantize_mxfp4(dev_bf16(wb)), out_dtype=torch.float32)
    # the quantize pass at this K too: codes and scales byte-equal
    for got, want, what in zip(rfq.residual_quantize(x), oracle_rfq(xb), ("QX", "SX", "QR", "SR")):
        assert_bytes_equal(host(got), want, f"max-K {what}")
    y_ref, s_ref = oracle_y(xb, wb)
    err = np.abs(y_host(y) - y_ref)
    tol = (2 * K // 128 + 1) * 2.0 ** -24 * s_ref + 2.0 ** -126
    assert (err <= tol).all(), f"max err / S = {float(np.max(err / s_ref)):.3e}"
    log(f"   max |dY|/S = {float(np.max(err / s_ref)):.2e}")


def test_residual_term_is_the_difference_of_rfq_and_w4a4():
    """End to end: Y_rfq - Y_w4a4, from two GPU GEMM calls on the same codes
    (with and without the residual term), equals deq(Q(R)) deq(W)^T, the
    residual path's contribution, within the two calls' accumulation bounds."""
    rng = np.random.default_rng(321)
    M, N, K = 200, 300, 1024
    xb = heavy(rng, M, K)
    wb = workloads.f32_to_bf16_bits(rng.normal(0, 0.02, (N, K)).astype(np.float32))
    log("[gemm] residual term = RFQ - W4A4")
    x = dev_bf16(xb)
    wq, sw = rfq.quantize_mxfp4(dev_bf16(wb))
    qx, sx, qr, sr = rfq.residual_quantize(x)
    y = rfq.gemm_w4a4(qx, sx, qr, sr, wq, sw, out_dtype=torch.float32)
    y1 = rfq.gemm_w4a4(qx, sx, None, None, wq, sw, out_dtype=torch.float32)
    diff = y_host(y) - y_host(y1)
    oqx, osx, oqr, osr = oracle.residual_quantize(oracle.bf16_bits_to_f64(xb))
    owq, osw = oracle.quantize_mxfp4(oracle.bf16_bits_to_f64(wb))
    ref = oracle.dequantize(oqr, osr) @ oracle.dequantize(owq, osw).T
    _, s = oracle.gemm_w4a4(oqx, osx, oqr, osr, owq, osw)
    _, s1 = oracle.gemm_w4a4(oqx, osx, None, None, owq, osw)
    err = np.abs(diff - ref)
    assert (err <= REL_TOL * (s + s1) + 2.0 ** -125).all(), f"max err / S = {float(np.max(err / s)):.3e}"
    assert np.abs(ref).max() > 0


def test_linear_equals_quantize_then_gemm_bitwise_and_is_deterministic():
    rng = np.random.default_rng(23)
    M, N, K = 384, 640, 2048
    xb = heavy(rng, M, K)
    wb = workloads.f32_to_bf16_bits(rng.normal(0, 0.02, (N, K)).astype(np.float32))
    x = dev_bf16(xb)
    wq, sw = rfq.quantize_mxfp4(dev_bf16(wb))
    log("[gemm] linear vs two calls")
    ws = torch.empty(rfq.linear_workspace_size(M, K), dtype=torch.uint8, device="cuda")
    y1 = rfq.linear(x, wq, sw, out_dtype=torch.float32, workspace=ws)
    qx, sx, qr, sr = rfq.residual_quantize(x)
    y2 = rfq.gemm_w4a4(qx, sx, qr, sr, wq, sw, out_dtype=torch.float32)
    y3 = rfq.linear(x, wq, sw, out_dtype=torch.float32)
    assert torch.equal(y1, y2) and torch.equal(y1, y3)
    # the workspace holds Q(X) | SX | Q(R) | SR at 256-byte-rounded offsets
    r256 = lambda b: (b + 255) // 256 * 256
    c, s = r256(M * K // 2), r256(M * K // 32)
    wsh = host(ws)
    assert (wsh[:M * K // 2] == host(qx).ravel()).all()
    assert (wsh[c:c + M * K // 32] == host(sx).ravel()).all()
    assert (wsh[c + s:c + s + M * K // 2] == host(qr).ravel()).all()
    assert (wsh[2 * c + s:2 * c + s + M * K // 32] == host(sr).ravel()).all()


@pytest.mark.parametrize("out_dtype,ldy,offset", [(torch.float32, 96, 0), (torch.float32, 96, 1), (torch.float32, 98, 0),
                                                  (torch.bfloat16, 96, 0), (torch.bfloat16, 96, 2),
                                                  (torch.bfloat16, 97, 0)])
def test_output_row_stride(out_dtype, ldy, offset):
    """Y as a column slice of a wider buffer, at a row stride and base offset
    that do or do not allow four-element vector stores; the columns around
    the slice stay untouched."""
    rng = np.random.default_rng(24)
    M, N, K = 40, 73, 192
    xb, wb = heavy(rng, M, K), workloads.f32_to_bf16_bits(rng.normal(0, 0.02, (N, K)).astype(np.float32))
    wq, sw = rfq.quantize_mxfp4(dev_bf16(wb))
    big = torch.full((M, ldy), 7.0, dtype=out_dtype, device="cuda")
    log(f"[gemm] strided output {out_dtype} ldy={ldy} base offset {offset}")
    rfq.linear(dev_bf16(xb), wq, sw, out=big[:, offset:offset + N])
    yh = y_host(big)
    assert (yh[:, :offset] == 7.0).all() and (yh[:, offset + N:] == 7.0).all()
    y_ref, s_ref = oracle_y(xb, wb)
    check_y(yh[:, offset:offset + N], y_ref, s_ref, out_dtype, "strided out")


@pytest.mark.parametrize("M,N,K", [(4100, 4200, 1024), (4100, 4200, 640), (2304, 7000, 512)])
def test_two_launch_split_sampled(M, N, K):
    """Shapes whose 256 x 256 tile count leaves a partial last round: whole
    rounds run as big tiles and the rest as upper and lower halves, with
    partial edge tiles in both (the last tile row's lower halves lie wholly
    past M); sampled rows x columns against the oracle (fp32 out)."""
    rng = np.random.default_rng(M + N + K)
    xb = heavy(rng, M, K)
    wb = workloads.f32_to_bf16_bits(rng.normal(0, 0.02, (N, K)).astype(np.float32))
    log(f"[gemm] two-launch split M={M} N={N} K={K}")
    wq, sw = rfq.quantize_mxfp4(dev_bf16(wb))
    y = host(rfq.linear(dev_bf16(xb), wq, sw, out_dtype=torch.float32))
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1, M - 4], rng.choice(M, 59, replace=False)]))
    cols = np.unique(np.concatenate([[0, 127, 128, 255, 256, N - 1, N - 100], rng.choice(N, 57, replace=False)]))
    y_ref, s_ref = oracle_y(xb[rows], wb[cols])
    check_y(y[np.ix_(rows, cols)], y_ref, s_ref, torch.float32, f"split {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,out_dtype", [(4096, 12288, 512, torch.float32), (4096, 8192, 1024, torch.bfloat16),
                                               (4096, 8448, 512, torch.bfloat16)])
def test_streamed_tiles_every_output(M, N, K, out_dtype):
    """M and N multiples of 256 with two or three whole rounds of tiles on
    256 CUs: each workgroup computes its tiles back to back, fetching the
    next tile's first stages while it finishes the previous one (with K =
    512 every scale group starts a new tile). 4096 x 8448 has 528 tiles:
    two streamed rounds, then 16 tiles as 32 halves in a second launch.
    Every output checked."""
    rng = np.random.default_rng(M + N + K + 7)
    xb = heavy(rng, M, K)
    wb = workloads.f32_to_bf16_bits(rng.normal(0, 0.02, (N, K)).astype(np.float32))
    log(f"[gemm] streamed tiles M={M} N={N} K={K} {out_dtype}")
    wq, sw = rfq.quantize_mxfp4(dev_bf16(wb))
    y = y_host(rfq.linear(dev_bf16(xb), wq, sw, out_dtype=out_dtype))
    y_ref, s_ref, pairs = oracle_y(xb, wb, with_scales=True)
    check_y(y, y_ref, s_ref, out_dtype, f"streamed {M}x{N}x{K}")
    cov = check_exact_where_covered(y, y_ref, s_ref, pairs, out_dtype, f"streamed {M}x{N}x{K}")
    log(f"   exact sums at {100 * cov:.1f}% of the outputs, each bit-equal to the exact result")


def _sweep_shapes():
    """Seeded random shapes (mostly one partial round, ragged edges, K with
    and without whole scale groups), then shapes whose tile counts exercise
    each plan for the last partial round behind streamed rounds: halves
    (4096 x 10240), and rectangle pieces over a last group of 1, 2 and 3
    tile rows (1280 x 26368, 3584 x 9472, 1792 x 19712)."""
    rng = np.random.default_rng(2026)
    shapes = []
    for i in range(24):
        M = int([rng.integers(1, 600), rng.integers(600, 5000), 256 * rng.integers(1, 20)][i % 3])
        N = int([rng.integers(1, 900), 256 * rng.integers(1, 40), rng.integers(900, 9000)][(i // 3) % 3])
        K = int(32 * [rng.integers(1, 24), 16 * rng.integers(1, 5)][i % 2])
        shapes.append((M, N, K))
    return shapes + [(4096, 10240, 512), (1280, 26368, 512), (3584, 9472, 512), (1792, 19712, 512)]


@pytest.mark.parametrize("i,M,N,K", [(i,) + s for i, s in enumerate(_sweep_shapes())])
def test_shape_sweep_sampled(i, M, N, K):
    """Every launch plan on sampled outputs: the RFQ layer (fp32 Y on even
    cases, bf16 Y on odd ones) and plain W4A4, at rows and columns that
    include the edges and the last 512 rows and 2048 columns (where a last
    partial round lies)."""
    rng = np.random.default_rng(5000 + i)
    out_dtype = torch.float32 if i % 2 == 0 else torch.bfloat16
    xb = heavy(rng, M, K)
    wb = workloads.f32_to_bf16_bits(rng.normal(0, 0.02, (N, K)).astype(np.float32))
    log(f"[gemm] sweep {i}: M={M} N={N} K={K} {out_dtype}")
    x = dev_bf16(xb)
    wq, sw = rfq.quantize_mxfp4(dev_bf16(wb))
    y = y_host(rfq.linear(x, wq, sw, out_dtype=out_dtype))
    qx, sx, _, _ = rfq.residual_quantize(x)
    y4 = y_host(rfq.gemm_w4a4(qx, sx, None, None, wq, sw, out_dtype=out_dtype))
    pick = lambda n, lo, k: rng.integers(lo, n, size=k) if n > lo else np.zeros(0, np.int64)
    rows = np.unique(np.concatenate([[0, M - 1, M // 2], rng.integers(0, M, 24), pick(M, max(M - 512, 0), 8)]))
    cols = np.unique(np.concatenate([[0, N - 1, N // 2], rng.integers(0, N, 40), pick(N, max(N - 2048, 0), 16)]))
    y_ref, s_ref, pairs = oracle_y(xb[rows], wb[cols], with_scales=True)
    check_y(y[np.ix_(rows, cols)], y_ref, s_ref, out_dtype, f"sweep {i} rfq")
    check_exact_where_covered(y[np.ix_(rows, cols)], y_ref, s_ref, pairs, out_dtype, f"sweep {i} rfq")
    y_ref, s_ref, pairs = oracle_y(xb[rows], wb[cols], resid=False, with_scales=True)
    check_y(y4[np.ix_(rows, cols)], y_ref, s_ref, out_dtype, f"sweep {i} w4a4")
    check_exact_where_covered(y4[np.ix_(rows, cols)], y_ref, s_ref, pairs, out_dtype, f"sweep {i} w4a4")


@pytest.mark.parametrize("M,N,K,out_dtype", [(4096, 13824, 512, torch.float32), (1024, 34304, 512, torch.bfloat16)])
def test_streamed_rounds_then_rectangle_pieces(M, N, K, out_dtype):
    """Whole streamed rounds, then the last partial round's tiles, which form
    a rectangle of whole tile columns, as 128 x 192 pieces in the same
    launch: 4096 x 13824 (the 4096 x 5120 x 13824 layer's tile grid at
    K = 512) has 864 tiles, three rounds and a 1024 x 6144 rectangle of 256
    pieces; 1024 x 34304 has 536 tiles, two rounds and a 1024 x 1536
    rectangle of 64 pieces. Every output of the RFQ GEMM and of the plain
    W4A4 GEMM on the same operands checked."""
    rng = np.random.default_rng(M + N + K + 11)
    xb = heavy(rng, M, K)
    wb = workloads.f32_to_bf16_bits(rng.normal(0, 0.02, (N, K)).astype(np.float32))
    log(f"[gemm] streamed rounds + rectangle pieces M={M} N={N} K={K} {out_dtype}")
    wq, sw = rfq.quantize_mxfp4(dev_bf16(wb))
    qx, sx, qr, sr = rfq.residual_quantize(dev_bf16(xb))
    y = y_host(rfq.gemm_w4a4(qx, sx, qr, sr, wq, sw, out_dtype=out_dtype))
    y4 = y_host(rfq.gemm_w4a4(qx, sx, None, None, wq, sw, out_dtype=out_dtype))
    x = oracle.bf16_bits_to_f64(xb)
    owq, osw = oracle.quantize_mxfp4(oracle.bf16_bits_to_f64(wb))
    oqx, osx, oqr, osr = oracle.residual_quantize(x)
    y_ref, s_ref = oracle.gemm_w4a4(oqx, osx, oqr, osr, owq, osw)
    check_y(y, y_ref, s_ref, out_dtype, f"rectangle pieces RFQ {M}x{N}x{K}")
    check_exact_where_covered(y, y_ref, s_ref, [(osx, osw), (osr, osw)], out_dtype, f"rectangle pieces RFQ {M}x{N}x{K}")
    y_ref, s_ref = oracle.gemm_w4a4(oqx, osx, None, None, owq, osw)
    check_y(y4, y_ref, s_ref, out_dtype, f"rectangle pieces W4A4 {M}x{N}x{K}")
    check_exact_where_covered(y4, y_ref, s_ref, [(osx, osw)], out_dtype, f"rectangle pieces W4A4 {M}x{N}x{K}")


def _rne_bf16_bits(y32):
    """fp32 to bfloat16 bits by round to nearest even, in integer arithmetic
    (NaNs are checked separately)."""
    u = y32.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("M,N,K", [(300, 520, 1024), (4096, 8192, 512), (4096, 13824, 512)])
def test_bf16_output_is_rne_of_fp32_output(M, N, K):
    """The bf16 epilogue rounds each fp32 accumulator to nearest even: every
    bf16 output equals the RNE rounding of the fp32 output of the same GEMM
    on the same operands, bit for bit, and NaN stays NaN. Three store paths:
    one partial round of single tiles (300 x 520), streamed whole rounds
    (4096 x 8192) and streamed rounds followed by rectangle pieces (4096 x
    13824). Codes are random bytes; each row's E8M0 scales are a base drawn
    from 0..246 plus 0..7 per block, so that the product of a row pair's
    scales, which sets the output's magnitude, spans the fp32 denormal
    range, the normal range and values past the largest finite one (inf);
    a few blocks carry the NaN scale."""
    rng = np.random.default_rng(M * 7 + N + K)
    kb = K // 32

    def scales(rows):
        return (rng.integers(0, 247, size=(rows, 1)) + rng.integers(0, 8, size=(rows, kb))).astype(np.uint8)

    qx, qr, wq = (dev_u8(rng.integers(0, 256, size=(r, K // 2), dtype=np.uint8)) for r in (M, M, N))
    sx_h, sr_h, sw_h = scales(M), scales(M), scales(N)
    sx_h[rng.integers(0, M, 2), rng.integers(0, kb, 2)] = 255
    sx, sr, sw = dev_u8(sx_h), dev_u8(sr_h), dev_u8(sw_h)
    log(f"[gemm] bf16 epilogue against RNE of the fp32 output M={M} N={N} K={K}")
    y32 = host(rfq.gemm_w4a4(qx, sx, qr, sr, wq, sw, out_dtype=torch.float32))
    y16 = rfq.gemm_w4a4(qx, sx, qr, sr, wq, sw, out_dtype=torch.bfloat16).cpu().view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(y32)
    assert nan.any() and np.isinf(y32).any()
    tiny = (y32 != 0) & (np.abs(y32) < np.float32(2.0 ** -126))
    assert tiny.any(), "no fp32 denormal outputs drawn"
    h_nan = y16[nan]
    assert ((h_nan & 0x7F80) == 0x7F80).all() and ((h_nan & 0x7F) != 0).all(), "NaN outputs must stay NaN"
    want = _rne_bf16_bits(y32)
    bad = np.flatnonzero((y16 != want) & ~nan)
    assert bad.size == 0, (f"{bad.size} bf16 outputs differ from RNE of fp32, first at {bad[0]}: "
                           f"fp32 {y32.flat[bad[0]]!r} bf16 {y16.flat[bad[0]]:#06x} want {want.flat[bad[0]]:#06x}")
    log(f"   {y32.size} outputs: {int(tiny.sum())} denormal, {int(np.isinf(y32).sum())} inf, {int(nan.sum())} NaN")


@pytest.mark.parametrize("name", ["qwen3vl_attn_proj", "qwen3vl_ffn_up", "wan22_ffn", "dit_ffn_down"])
def test_full_size_config(name):
    """The configuration as the benchmark runs it (full X, full W, one
    rfq_linear call, on the streamed-tile path wherever the benchmark takes
    it):
      * Q(X), Q(R) and their scales, as left in the workspace, byte-equal to
        the oracle over the WHOLE tensor (the oracle runs in row chunks on a
        CPU process pool while the GPU works);
      * the weight's codes and scales at sampled rows;
      * Y at 128 sampled rows x 256 sampled columns, both as bf16 Y (the
        benchmark's output) and as fp32 Y from a second call, the latter at
        the plain 1e-5 S + 2^-126 gate (with K/128 fp32 accumulations per
        product: 80 at K = 5120, 216 at K = 13824) and, beyond it, equal to
        the oracle's exact sum rounded once to fp32 (see below)."""
    import oracle_pool
    cfg = workloads.CONFIGS[name]
    log(f"[gemm] full size {name} M={cfg.M} N={cfg.N} K={cfg.K}: oracle codes on {oracle_pool.workers()} "
        f"processes; generating inputs")
    codes_job = oracle_pool.RfqCodesFull(cfg)
    try:
        xb = workloads.x_bf16(cfg)
        wb = workloads.w_bf16(cfg)
        x, w = dev_bf16(xb), dev_bf16(wb)
        log("   running on the GPU")
        wq, sw = rfq.quantize_mxfp4(w)
        del w
        ws = torch.empty(rfq.linear_workspace_size(cfg.M, cfg.K), dtype=torch.uint8, device="cuda")
        y = rfq.linear(x, wq, sw, out_dtype=torch.bfloat16, workspace=ws)
        y32 = rfq.linear(x, wq, sw, out_dtype=torch.float32)
        torch.cuda.synchronize()
        rows = workloads.sample_rows(cfg, n_random=126)
        cols = np.unique(np.concatenate([[0, cfg.N - 1],
                                         np.random.default_rng(cfg.seed).choice(cfg.N, 254, replace=False)]))
        M, K = cfg.M, cfg.K
        r256 = lambda b: (b + 255) // 256 * 256
        c, s = r256(M * K // 2), r256(M * K // 32)
        wsh = host(ws)
        yh = host_bf16_as_f64(y)[np.ix_(rows, cols)]
        y32h = host(y32)[np.ix_(rows, cols)].astype(np.float64)
        del ws, y, y32, x
        log(f"   oracle Y on {len(rows)} rows x {len(cols)} columns")
        owq, osw = oracle_mx(wb[cols])
        assert_bytes_equal(host(wq)[cols], owq, "W codes sampled rows")
        assert_bytes_equal(host(sw)[cols], osw, "W scales sampled rows")
        y_ref, s_ref = oracle_y(xb[rows], wb[cols])
        worst = check_y(yh, y_ref, s_ref, torch.bfloat16, f"{name} bf16 Y")
        worst32 = check_y(y32h, y_ref, s_ref, torch.float32, f"{name} fp32 Y")
        # where every partial sum is exact in fp32 (exact_cover), Y must be
        # the exact sum itself (fp32) or its RNE to bf16, bit for bit
        _, osx_s, _, osr_s = oracle.residual_quantize(oracle.bf16_bits_to_f64(xb[rows]))
        pairs = [(osx_s, osw), (osr_s, osw)]
        cov = check_exact_where_covered(y32h, y_ref, s_ref, pairs, torch.float32, f"{name} fp32 Y")
        check_exact_where_covered(yh, y_ref, s_ref, pairs, torch.bfloat16, f"{name} bf16 Y")
        log(f"   Y ok: max |dY|/S = {worst:.2e} (bf16 Y), {worst32:.2e} (fp32 Y); sums exact in fp32 at "
            f"{100 * cov:.2f}% of the sampled outputs, where fp32 Y is the exact sum and bf16 Y its RNE, bit for bit")
        assert cov > 0.99, f"{name}: sums exact in fp32 at only {100 * cov:.2f}% of the sampled outputs"
        del xb, wb
        log("   waiting for the oracle's codes of all rows")
        oqx, osx, oqr, osr = codes_job.result(timeout=600)
    finally:
        codes_job.close()
    assert_bytes_equal(wsh[:M * K // 2].reshape(M, K // 2), oqx, "Q(X) codes, all rows")
    assert_bytes_equal(wsh[c:c + M * K // 32].reshape(M, K // 32), osx, "Q(X) scales, all rows")
    assert_bytes_equal(wsh[c + s:c + s + M * K // 2].reshape(M, K // 2), oqr, "Q(R) codes, all rows")
    assert_bytes_equal(wsh[2 * c + s:2 * c + s + M * K // 32].reshape(M, K // 32), osr, "Q(R) scales, all rows")
    log(f"   Q(X), Q(R) and scales byte-equal on all {M} rows")
