"""The test helper that marks outputs whose fp32 accumulation is exact
(gpu_helpers.exact_cover), checked without a GPU: on small random E2M1
operands with spread-out E8M0 scales, every output it marks has an exact
rational sum that fp32 holds exactly and that any fp32 summation order
reproduces; the bit-equality check built on it rejects a one-ulp change."""
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import check_exact_where_covered, exact_cover, rne_bf16

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def decode(codes, scales):
    """Exact rationals of unpacked E2M1 codes [rows, K] with E8M0 scales [rows, K/32]."""
    rows, K = codes.shape
    out = []
    for r in range(rows):
        row = []
        for k in range(K):
            c = int(codes[r, k])
            v = Fraction(E2M1[c & 7]) * (-1 if c & 8 else 1)
            row.append(v * Fraction(2) ** (int(scales[r, k // 32]) - 127))
        out.append(row)
    return out


def operands(rng, rows, K, lo, hi):
    codes = rng.integers(0, 16, size=(rows, K)).astype(np.uint8)
    scales = rng.integers(lo, hi, size=(rows, K // 32)).astype(np.uint8)
    return codes, scales


@pytest.mark.parametrize("spread", [6, 40])
def test_marked_outputs_have_sums_exact_in_fp32(spread):
    rng = np.random.default_rng(spread)
    M, N, K = 6, 5, 128
    qx, sx = operands(rng, M, K, 120, 120 + spread)
    qr, sr = operands(rng, M, K, 120, 120 + spread)
    wq, sw = operands(rng, N, K, 120, 120 + spread)
    y, s = oracle.gemm_w4a4(qx, sx, qr, sr, wq, sw)
    cov = exact_cover(s, [(sx, sw), (sr, sw)])
    X, R, W = decode(qx, sx), decode(qr, sr), decode(wq, sw)
    order = list(range(2 * K))
    inexact_unmarked = 0
    for m in range(M):
        for n in range(N):
            terms = [X[m][k] * W[n][k] for k in range(K)] + [R[m][k] * W[n][k] for k in range(K)]
            exact = sum(terms)
            if not cov[m, n]:
                acc = np.float32(0)
                for t in terms:
                    acc = np.float32(acc + np.float32(float(t)))
                inexact_unmarked += Fraction(float(acc)) != exact
                continue
            assert float(np.float32(float(exact))) == exact, (m, n)      # fp32 holds it
            assert y[m, n] == exact
            for _ in range(3):                                          # any order, fp32 adds
                random.Random(m * 7 + n).shuffle(order)
                acc = np.float32(0)
                for i in order:
                    acc = np.float32(acc + np.float32(float(terms[i])))
                assert Fraction(float(acc)) == exact, (m, n)
    if spread == 6:
        assert cov.all()              # narrow scale ranges: every output marked
    else:
        # 40 binades of scale spread: outputs go unmarked, and there fp32
        # accumulation does round
        assert not cov.all() and inexact_unmarked > 0


def test_check_rejects_a_one_ulp_change():
    rng = np.random.default_rng(1)
    qx, sx = operands(rng, 8, 64, 120, 126)
    wq, sw = operands(rng, 9, 64, 120, 126)
    y, s = oracle.gemm_w4a4(qx, sx, None, None, wq, sw)
    pairs = [(sx, sw)]
    assert check_exact_where_covered(y.astype(np.float32), y, s, pairs, torch.float32, "exact") == 1.0
    assert check_exact_where_covered(rne_bf16(y), y, s, pairs, torch.bfloat16, "exact bf16") == 1.0
    bad = y.astype(np.float32)
    bad[3, 4] = np.nextafter(bad[3, 4], np.float32(np.inf))
    with pytest.raises(AssertionError):
        check_exact_where_covered(bad, y, s, pairs, torch.float32, "planted")
