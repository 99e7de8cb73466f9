"""Pins of the oracle's W4A4 GEMM (the K-doubled contraction of Q(X), Q(R) with Wq)."""
import json
import os
from fractions import Fraction

import numpy as np

import oracle
import workloads

SPEC_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "toy_block.json")


def _frac_code(c):
    v = Fraction(SPEC_E2M1[c & 7]).limit_denominator()
    return -v if c & 8 else v


def _frac_scale(s):
    return Fraction(2) ** (int(s) - 127)


def brute_force_y(qx, sx, qr, sr, wq, sw):
    """Exact rational Y by the definition: for every output, the sum over
    blocks of scale products times the 32-term code dot products, for the
    primary and (when given) the residual operand. Pure Python."""
    M, K = qx.shape
    N = wq.shape[0]
    out = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for b in range(K // 32):
                for (q, s) in ((qx, sx), (qr, sr)) if qr is not None else ((qx, sx),):
                    dot = sum(_frac_code(q[m, 32 * b + i]) * _frac_code(wq[n, 32 * b + i]) for i in range(32))
                    acc += _frac_scale(s[m, b]) * _frac_scale(sw[n, b]) * dot
            out[m][n] = acc
    return out


def test_gemm_equals_exact_rational_definition():
    rng = np.random.default_rng(7)
    M, N, K = 3, 4, 96
    qx = rng.integers(0, 16, (M, K)).astype(np.uint8)
    qr = rng.integers(0, 16, (M, K)).astype(np.uint8)
    wq = rng.integers(0, 16, (N, K)).astype(np.uint8)
    sx = rng.integers(110, 140, (M, K // 32)).astype(np.uint8)
    sr = rng.integers(100, 130, (M, K // 32)).astype(np.uint8)
    sw = rng.integers(110, 140, (N, K // 32)).astype(np.uint8)
    y, s = oracle.gemm_w4a4(qx, sx, qr, sr, wq, sw)
    exact = brute_force_y(qx, sx, qr, sr, wq, sw)
    for m in range(M):
        for n in range(N):
            assert Fraction(y[m, n]) == exact[m][n]     # every partial sum is exact here
    y1, _ = oracle.gemm_w4a4(qx, sx, None, None, wq, sw)
    exact1 = brute_force_y(qx, sx, None, None, wq, sw)
    assert all(Fraction(y1[m, n]) == exact1[m][n] for m in range(M) for n in range(N))


def test_all_code_pairs_single_block():
    # K = 32, one nonzero element per row: Y[a, b] is the product of the two
    # code values (unit scales), for all 16 x 16 code pairs.
    qx = np.zeros((16, 32), np.uint8)
    wq = np.zeros((16, 32), np.uint8)
    qx[:, 7] = np.arange(16)
    wq[:, 7] = np.arange(16)
    ones = np.full((16, 1), 127, np.uint8)
    y, _ = oracle.gemm_w4a4(qx, ones, None, None, wq, ones)
    vals = np.array(SPEC_E2M1 + [-v for v in SPEC_E2M1])
    assert (y == np.outer(vals, vals)).all()


def test_selector_weight_recovers_dequantized_activations():
    # Row n of W holds 1.0 at k = n: its block gets scale 2^-2 and code 6 there,
    # every other block is all zero; so Y[m, n] = deq Q(X)[m, n] + deq Q(R)[m, n].
    cfg = workloads.CONFIGS["tiny"]
    x = oracle.bf16_bits_to_f64(workloads.x_bf16(cfg))
    K = x.shape[1]
    w = np.eye(K)[:128]
    wq, sw = oracle.quantize_mxfp4(w)
    qx, sx, qr, sr = oracle.residual_quantize(x)
    y, _ = oracle.gemm_w4a4(qx, sx, qr, sr, wq, sw)
    want = (oracle.dequantize(qx, sx) + oracle.dequantize(qr, sr))[:, :128]
    assert (y == want).all()


def test_residual_term_is_linear_and_blocks_permute():
    rng = np.random.default_rng(8)
    x = rng.laplace(size=(8, 128))
    w = rng.normal(0, 0.02, size=(6, 128))
    y, s, (qx, sx, qr, sr), (wq, sw) = oracle.linear(x, w)
    y1, _ = oracle.gemm_w4a4(qx, sx, None, None, wq, sw)
    dr = oracle.dequantize(qr, sr) @ oracle.dequantize(wq, sw).T
    assert np.allclose(y - y1, dr, rtol=0, atol=1e-12 * s.max())
    perm = rng.permutation(4)
    cols = np.concatenate([np.arange(32 * p, 32 * p + 32) for p in perm])
    yp, _ = oracle.gemm_w4a4(qx[:, cols], sx[:, perm], qr[:, cols], sr[:, perm], wq[:, cols], sw[:, perm])
    assert np.allclose(yp, y, rtol=0, atol=1e-12 * s.max())
    assert (s >= np.abs(y)).all()


def test_toy_block_gemm():
    g = json.load(open(GOLDEN))
    bits = np.zeros((1, 32), np.uint16)
    bits[0, :4] = [int(h, 16) for h in g["x_bf16_bits_first4"]]
    w = np.zeros((1, 32))
    w[0, :4] = g["w_row_first4"]
    y, _, _, (wq, sw) = oracle.linear(oracle.bf16_bits_to_f64(bits), w)
    assert sw[0, 0] == int(g["w_scale"], 16) and list(wq[0, :4]) == g["w_codes_first4"]
    assert y[0, 0] == g["y_rfq"]
    qx, sx = oracle.quantize_mxfp4(oracle.bf16_bits_to_f64(bits))
    y1, _ = oracle.gemm_w4a4(qx, sx, None, None, wq, sw)
    assert y1[0, 0] == g["y_w4a4"]
    exact = float(oracle.bf16_bits_to_f64(bits)[0, :4].sum())
    assert exact == g["y_exact_bf16_inputs"]
    assert abs(y[0, 0] - exact) < abs(y1[0, 0] - exact)


def test_rfq_output_closer_to_unquantized_activation_product():
    cfg = workloads.CONFIGS["tiny"]
    x = oracle.bf16_bits_to_f64(workloads.x_bf16(cfg))
    w = oracle.bf16_bits_to_f64(workloads.w_bf16(cfg))
    y, _, (qx, sx, _, _), (wq, sw) = oracle.linear(x, w)
    y1, _ = oracle.gemm_w4a4(qx, sx, None, None, wq, sw)
    ref = x @ oracle.dequantize(wq, sw).T
    assert np.linalg.norm(y - ref) < 0.3 * np.linalg.norm(y1 - ref)
