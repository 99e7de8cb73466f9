"""Pins of the oracle's straight-through backward pass.

* exact rational sums by the definition on tiny inputs;
* the adjoint identities of the forward product Y = Xh Wd^T, with Y from
  the forward oracle (a different code path): <dY, Y> = <dX, Xh> = <dW, Wd>;
* a one-hot dY returns a row of Wd (dX) and a scaled row of Xh (dW);
* the residual path: on MXFP4-representable X, Q(R) is zero and dW is
  dY^T X exactly.
"""
from fractions import Fraction

import numpy as np

import oracle
import workloads


def _inputs(seed, M, N, K):
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3, size=(M, K)).astype(np.float32)
    x[:, rng.choice(K, size=2, replace=False)] *= 40
    w = rng.normal(0, 0.02, size=(N, K)).astype(np.float32)
    dy = rng.normal(0, 1, size=(M, N)).astype(np.float32)
    bf = lambda a: oracle.bf16_bits_to_f64(workloads.f32_to_bf16_bits(a))
    return bf(x), bf(w), bf(dy)


def test_exact_rational_sums():
    x, w, dy = _inputs(1, 3, 4, 64)
    wq, sw = oracle.quantize_mxfp4(w)
    qx, sx, qr, sr = oracle.residual_quantize(x)
    dx, sdx = oracle.backward_dx(dy, wq, sw)
    dw, sdw = oracle.backward_dw(dy, qx, sx, qr, sr)
    wd = [[Fraction(v) for v in row] for row in oracle.dequantize(wq, sw)]
    xh = [[Fraction(a) + Fraction(b) for a, b in zip(r1, r2)]
          for r1, r2 in zip(oracle.dequantize(qx, sx), oracle.dequantize(qr, sr))]
    f = [[Fraction(v) for v in row] for row in dy]
    M, N, K = 3, 4, 64
    for m in range(M):
        for k in range(K):
            ref = sum(f[m][n] * wd[n][k] for n in range(N))
            assert abs(float(ref) - dx[m, k]) <= 1e-14 * (sdx[m, k] + 1e-300)
    for n in range(N):
        for k in range(K):
            ref = sum(f[m][n] * xh[m][k] for m in range(M))
            assert abs(float(ref) - dw[n, k]) <= 1e-14 * (sdw[n, k] + 1e-300)


def test_adjoint_identities_against_the_forward_oracle():
    x, w, dy = _inputs(2, 48, 40, 256)
    y, _, (qx, sx, qr, sr), (wq, sw) = oracle.linear(x, w)
    dx, _, dw, _ = oracle.linear_backward(dy, x, w)
    xh = oracle.dequantize(qx, sx) + oracle.dequantize(qr, sr)
    wd = oracle.dequantize(wq, sw)
    a = np.sum(dy * y)
    b = np.sum(dx * xh)
    c = np.sum(dw * wd)
    scale = np.sum(np.abs(dy) @ np.abs(wd) * np.abs(xh))
    assert abs(a - b) <= 1e-12 * scale and abs(a - c) <= 1e-12 * scale


def test_one_hot_gradient():
    x, w, _ = _inputs(3, 8, 12, 96)
    dy = np.zeros((8, 12))
    dy[5, 7] = 2.0
    dx, _, dw, _ = oracle.linear_backward(dy, x, w)
    wq, sw = oracle.quantize_mxfp4(w)
    qx, sx, qr, sr = oracle.residual_quantize(x)
    assert np.array_equal(dx[5], 2.0 * oracle.dequantize(wq, sw)[7])
    assert not dx[np.arange(8) != 5].any()
    xh = oracle.dequantize(qx, sx) + oracle.dequantize(qr, sr)
    assert np.array_equal(dw[7], 2.0 * xh[5])
    assert not dw[np.arange(12) != 7].any()


def test_residual_path_vanishes_on_representable_input():
    rng = np.random.default_rng(4)
    q = rng.integers(0, 16, size=(6, 64)).astype(np.uint8)
    q[:, ::32] = 7
    s = rng.integers(120, 134, size=(6, 2)).astype(np.uint8)
    x = oracle.dequantize(q, s)
    w = rng.normal(0, 0.02, size=(5, 64))
    dy = rng.normal(size=(6, 5))
    _, _, dw, _ = oracle.linear_backward(dy, x, w)
    assert np.array_equal(dw, dy.T @ x)
