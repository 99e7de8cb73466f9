"""Pins of the condition scale S that every GPU tolerance is scaled by.

S[m, n] is the sum over both products of the K-doubled contraction of
|term| = |a_k w_k| (the componentwise bound that fp32 accumulation error is
measured against). Here it is rebuilt for every oracle GEMM and gradient as
an exact rational sum, term by term, from operand values decoded without the
oracle (E2M1 from its value listing, E4M3 through PyTorch's float8_e4m3fn,
E8M0 as an exact power of two), and compared with the oracle's S. A wrong S
would silently loosen (too large) or break (too small) the GPU gates, so each
planted mistake below -- the weight counted twice, the residual product
dropped, S taken as |Y|, S taken from unquantized X -- must fail the same
comparison."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads

SPEC_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def e2m1(c):
    v = Fraction(SPEC_E2M1[int(c) & 7])
    return -v if int(c) & 8 else v


def e4m3(c):
    f = torch.tensor([int(c)], dtype=torch.uint8).view(torch.float8_e4m3fn).float().item()
    return Fraction(f)


def scale(s):
    return Fraction(2) ** (int(s) - 127)


def decode(codes, scales, elem):
    rows, K = codes.shape
    return [[elem(codes[r, k]) * scale(scales[r, k // 32]) for k in range(K)] for r in range(rows)]


def exact_s(pairs):
    """sum over (A, W) operand pairs of sum_k |A[m][k] W[n][k]|, exactly."""
    A0, W0 = pairs[0]
    M, N = len(A0), len(W0)
    return [[sum(abs(a[m][k] * w[n][k]) for a, w in pairs for k in range(len(a[m]))) for n in range(N)]
            for m in range(M)]


def matches(s, exact):
    """The oracle's float64 S equals the exact sum to float64 summation
    accuracy (all terms positive: relative error below 1e-13 here)."""
    s = np.asarray(s, dtype=np.float64)
    return all(abs(Fraction(float(s[m, n])) - exact[m][n]) <= Fraction(1, 10 ** 13) * exact[m][n]
               for m in range(len(exact)) for n in range(len(exact[0])))


def heavy_operands(seed, M=3, N=4, K=96):
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3, size=(M, K)).astype(np.float32)
    x[:, rng.choice(K, 3, replace=False)] *= 50
    w = rng.normal(0, 0.02, (N, K)).astype(np.float32)
    dy = rng.normal(0, 1, (M, N)).astype(np.float32)
    bf = lambda a: oracle.bf16_bits_to_f64(workloads.f32_to_bf16_bits(a))
    return bf(x), bf(w), bf(dy)


def test_rfq_gemm_s_is_the_exact_sum_over_both_products_and_planted_mistakes_fail():
    x, w, _ = heavy_operands(11)
    wq, sw = oracle.quantize_mxfp4(w)
    qx, sx, qr, sr = oracle.residual_quantize(x)
    y, s = oracle.gemm_w4a4(qx, sx, qr, sr, wq, sw)
    A, R, W = decode(qx, sx, e2m1), decode(qr, sr, e2m1), decode(wq, sw, e2m1)
    exact = exact_s([(A, W), (R, W)])
    assert matches(s, exact)
    # residual products are not negligible here, so dropping them is visible
    assert not matches(s, exact_s([(A, W)]))
    # planted mistakes in S, each of which must fail the pin
    a, r, wd = oracle.dequantize(qx, sx), oracle.dequantize(qr, sr), oracle.dequantize(wq, sw)
    planted = {
        "weight counted twice": np.abs(a) @ np.abs(2 * wd).T + np.abs(r) @ np.abs(2 * wd).T,
        "residual product dropped": np.abs(a) @ np.abs(wd).T,
        "S taken as |Y|": np.abs(y),
        "S from unquantized X": np.abs(x) @ np.abs(wd).T,
        "|a + r| instead of |a| + |r|": np.abs(a + r) @ np.abs(wd).T,
    }
    for what, bad in planted.items():
        assert not matches(bad, exact), what


def test_plain_w4a4_s():
    x, w, _ = heavy_operands(12)
    wq, sw = oracle.quantize_mxfp4(w)
    qx, sx = oracle.quantize_mxfp4(x)
    _, s = oracle.gemm_w4a4(qx, sx, None, None, wq, sw)
    assert matches(s, exact_s([(decode(qx, sx, e2m1), decode(wq, sw, e2m1))]))


def test_random_codes_and_scales_s():
    # arbitrary codes (both signs, every magnitude) and scales 2^-20 .. 2^20
    rng = np.random.default_rng(13)
    M, N, K = 3, 5, 64
    qx, qr, wq = (rng.integers(0, 16, (r, K)).astype(np.uint8) for r in (M, M, N))
    sx, sr, sw = (rng.integers(107, 148, (r, K // 32)).astype(np.uint8) for r in (M, M, N))
    _, s = oracle.gemm_w4a4(qx, sx, qr, sr, wq, sw)
    W = decode(wq, sw, e2m1)
    assert matches(s, exact_s([(decode(qx, sx, e2m1), W), (decode(qr, sr, e2m1), W)]))


def test_mxfp8_gemm_s():
    x, w, _ = heavy_operands(14)
    wq, sw = oracle.quantize_mxfp4(w)
    W = decode(wq, sw, e2m1)
    qx8, sx8 = oracle.quantize_mxfp8(x)
    _, s = oracle.gemm_w4a8(qx8, sx8, wq, sw)
    exact = exact_s([(decode(qx8, sx8, e4m3), W)])
    assert matches(s, exact)
    assert not matches(2 * s, exact)
    qx, sx, qr8, sr = oracle.residual_quantize_fp8(x)
    _, s = oracle.gemm_w4a4_fp8_residual(qx, sx, qr8, sr, wq, sw)
    exact = exact_s([(decode(qx, sx, e2m1), W), (decode(qr8, sr, e4m3), W)])
    assert matches(s, exact)
    assert not matches(s, exact_s([(decode(qx, sx, e2m1), W)]))


def test_backward_s():
    x, w, dy = heavy_operands(15, M=4, N=5, K=64)
    wq, sw = oracle.quantize_mxfp4(w)
    qx, sx, qr, sr = oracle.residual_quantize(x)
    _, sdx = oracle.backward_dx(dy, wq, sw)
    _, sdw = oracle.backward_dw(dy, qx, sx, qr, sr)
    D = [[Fraction(v) for v in row] for row in dy]
    W = decode(wq, sw, e2m1)
    A, R = decode(qx, sx, e2m1), decode(qr, sr, e2m1)
    M, N, K = 4, 5, 64
    # dX[m, k] = sum_n dY[m, n] Wd[n, k]: S over n
    ex_dx = [[sum(abs(D[m][n] * W[n][k]) for n in range(N)) for k in range(K)] for m in range(M)]
    assert matches(sdx, ex_dx)
    # dW[n, k] = sum_m dY[m, n] (A[m, k] + R[m, k]) over both products: S over m of |dY A| + |dY R|
    ex_dw = [[sum(abs(D[m][n] * A[m][k]) + abs(D[m][n] * R[m][k]) for m in range(M)) for k in range(K)]
             for n in range(N)]
    assert matches(sdw, ex_dw)
    # the combined-operand form |dY| |A + R| is smaller where A and R differ in sign: it must fail
    wrong = np.abs(dy).T @ np.abs(oracle.dequantize(qx, sx) + oracle.dequantize(qr, sr))
    assert not matches(wrong, ex_dw)
