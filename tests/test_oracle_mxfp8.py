"""Pins of the oracle's MXFP8 (E4M3) encoder and the layers built on it.

* the E4M3 value table against the OCP specification's listed landmarks and
  against PyTorch's float8_e4m3fn decoding of all 256 codes (a library);
* element rounding against PyTorch's float8_e4m3fn conversion (round to
  nearest even, a library routine) wherever that conversion does not
  overflow, and saturation at 448 above it by its closed form;
* element rounding against brute force over every E4M3 value;
* the scale rule against its bit-field form, and the block-maximum invariant;
* the per-element error bound, NaN/Inf/zero blocks;
* both GEMM variants against exact rational sums by the definition.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from test_oracle_gemm import _frac_code, _frac_scale

ALL_BF16 = np.arange(65536, dtype=np.uint16)
X_ALL = oracle.bf16_bits_to_f64(ALL_BF16)
FINITE = np.isfinite(X_ALL)


def test_e4m3_landmarks_from_the_spec():
    assert oracle.e4m3_value(0x7E) == 448.0                 # S.1111.110, largest normal
    assert oracle.e4m3_value(0x08) == 2.0 ** -6             # S.0001.000, smallest normal
    assert oracle.e4m3_value(0x07) == 0.875 * 2.0 ** -6     # S.0000.111, largest subnormal
    assert oracle.e4m3_value(0x01) == 2.0 ** -9             # S.0000.001, smallest subnormal
    assert oracle.e4m3_value(0x38) == 1.0                   # exponent field 7 = bias
    assert oracle.e4m3_value(0xFE) == -448.0
    assert np.isnan(oracle.e4m3_value(0x7F)) and np.isnan(oracle.e4m3_value(0xFF))
    assert oracle.e4m3_value(0x80) == 0.0 and np.signbit(oracle.e4m3_value(0x80))
    mags = oracle.E4M3_MAGNITUDES
    assert len(mags) == 127 and (np.diff(mags) > 0).all() and mags[-1] == oracle.E4M3_MAX


def test_e4m3_decode_matches_torch_for_every_code():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    assert ((got == ref) | (np.isnan(got) & np.isnan(ref))).all()
    assert (np.signbit(got) == np.signbit(ref))[~np.isnan(ref)].all()


def torch_e4m3(v):
    """PyTorch's float32 -> float8_e4m3fn conversion codes (RNE; NaN on overflow)."""
    t = torch.from_numpy(np.asarray(v, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


@pytest.mark.parametrize("se", [-127, -126, -120, -9, -3, 0, 4, 8, 100, 119])
def test_encoder_equals_torch_rounding_on_all_bf16_patterns(se):
    x = X_ALL[FINITE]
    v = np.ldexp(x, -se)
    v = np.where(np.abs(v) < 1e30, v, 0.0)
    exact32 = (v.astype(np.float32).astype(np.float64) == v) & (v != 0.0)
    x, v = x[exact32], v[exact32]
    got = oracle.encode_e4m3(x, se)
    in_range = np.abs(v) <= 464.0                            # torch saturates nothing; up to 464 it rounds to 448
    assert (got[in_range] == torch_e4m3(v[in_range])).all()
    over = ~in_range
    assert (got[over] == (0x7E | (np.signbit(x[over]).astype(np.uint8) << 7))).all()


def brute_force_e4m3(x, se):
    """Nearest E4M3 value of x's sign among all 127 magnitudes (|v| capped at
    1024, where 448 is nearest whatever v is); ties to the even code."""
    v = np.minimum(np.abs(np.ldexp(x, -se)), 1024.0)
    best = np.zeros(x.shape, np.int64)
    bestd = np.full(x.shape, np.inf)
    for code in range(127):
        d = np.abs(v - oracle.e4m3_value(code))
        better = (d < bestd) | ((d == bestd) & (code % 2 == 0))
        best = np.where(better, code, best)
        bestd = np.where(better, d, bestd)
    return (best | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)


def test_encoder_equals_brute_force_near_every_midpoint():
    rng = np.random.default_rng(5)
    mags = oracle.E4M3_MAGNITUDES
    mids = np.concatenate([(mags[:-1] + mags[1:]) / 2, [448.0, 464.0, 480.0, 500.0]])
    v = np.repeat(mids, 9).astype(np.float32)
    ulps = np.tile(np.arange(-4, 5), len(mids))
    for _ in range(4):
        step = ulps > 0
        v = np.where(step, np.nextafter(v, np.float32(np.inf)), v)
        v = np.where(ulps < 0, np.nextafter(v, np.float32(0)), v)
        ulps = ulps - np.sign(ulps)
    v = v.astype(np.float64) * rng.choice([-1.0, 1.0], size=v.shape)
    for se in (-127, -5, 0, 13):
        x = np.ldexp(v, se)
        assert (oracle.encode_e4m3(x, se) == brute_force_e4m3(x, se)).all(), se


def test_scale_rule_bit_field_form_and_block_maximum():
    x = np.abs(X_ALL[FINITE & (X_ALL != 0)])
    se, code = oracle.scale_exponent_e4m3(x)
    biased = (ALL_BF16[FINITE & (X_ALL != 0)].astype(np.int64) >> 7) & 0xFF
    assert (code == np.maximum(biased - 8, 0)).all()
    # the block maximum lands in [256, 512) and encodes with exponent field 15
    # unless the scale was clamped at 2^-127
    unclamped = code > 0
    c = oracle.encode_e4m3(x[unclamped], se[unclamped])
    assert ((c >> 3) == 15).all()
    assert oracle.scale_exponent_e4m3(0.0)[1] == 0
    assert oracle.scale_exponent_e4m3(np.inf)[1] == 255


def test_quantize_blocks_error_bound_and_special_blocks():
    rng = np.random.default_rng(9)
    x = rng.standard_t(3, size=(16, 256)) * np.exp(rng.uniform(-20, 20, size=(16, 1)))
    x = x.astype(np.float32).astype(np.float64)
    x[0, :32] = 0.0
    x[0, 32:64] = -0.0
    x[1, 5] = np.nan
    x[2, 40] = -np.inf
    codes, scales = oracle.quantize_mxfp8(x)
    assert scales[0, 0] == 0 and (codes[0, :32] == 0).all() and (codes[0, 32:64] == 0x80).all()
    assert scales[1, 0] == 255 and (codes[1, :32] == 0).all()
    assert scales[2, 1] == 255 and (codes[2, 32:64] == 0).all()
    ok = np.repeat(scales != 255, 32, axis=1)
    d = oracle.dequantize_mxfp8(codes, scales)
    se = np.repeat(scales.astype(np.int64) - 127, 32, axis=1)
    err = np.abs(x - d)
    # half a step: 2^-4 relative in the normal range, 2^(se - 10) absolute
    # below it; past 464 * 2^se (only a block maximum in [1.8125, 2) * 2^(se + 8)
    # gets there) the value saturates to 448 * 2^se
    bound = np.maximum(np.abs(x) * 2.0 ** -4, np.ldexp(1.0, se - 10))
    sat = np.abs(x) > np.ldexp(464.0, se)
    assert (err[ok & ~sat] <= bound[ok & ~sat]).all()
    assert (err[ok & sat] == (np.abs(x) - np.ldexp(448.0, se))[ok & sat]).all()
    assert sat[ok].any()


def _frac_e4m3(c):
    return Fraction(oracle.e4m3_value(c))


def test_gemm_w4a8_equals_exact_rational_sum():
    rng = np.random.default_rng(3)
    M, N, K = 3, 4, 64
    x = rng.normal(size=(M, K)) * np.exp(rng.uniform(-3, 3, size=(M, 1)))
    w = rng.normal(size=(N, K))
    qx8, sx = oracle.quantize_mxfp8(x)
    wq, sw = oracle.quantize_mxfp4(w)
    y, s = oracle.gemm_w4a8(qx8, sx, wq, sw)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for b in range(K // 32):
                dot = sum(_frac_e4m3(qx8[m, 32 * b + i]) * _frac_code(wq[n, 32 * b + i]) for i in range(32))
                acc += _frac_scale(sx[m, b]) * _frac_scale(sw[n, b]) * dot
            assert abs(float(acc) - y[m, n]) <= 1e-12 * s[m, n]


def test_fp8_residual_gemm_equals_exact_rational_sum_and_error_shrinks():
    rng = np.random.default_rng(4)
    M, N, K = 3, 3, 64
    x = rng.standard_t(3, size=(M, K))
    x[:, 7] *= 50
    w = rng.normal(size=(N, K))
    qx, sx, qr8, sr = oracle.residual_quantize_fp8(x)
    wq, sw = oracle.quantize_mxfp4(w)
    y, s = oracle.gemm_w4a4_fp8_residual(qx, sx, qr8, sr, wq, sw)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for b in range(K // 32):
                d4 = sum(_frac_code(qx[m, 32 * b + i]) * _frac_code(wq[n, 32 * b + i]) for i in range(32))
                d8 = sum(_frac_e4m3(qr8[m, 32 * b + i]) * _frac_code(wq[n, 32 * b + i]) for i in range(32))
                acc += _frac_scale(sw[n, b]) * (_frac_scale(sx[m, b]) * d4 + _frac_scale(sr[m, b]) * d8)
            assert abs(float(acc) - y[m, n]) <= 1e-12 * s[m, n]
    # the reconstruction deq Q4(X) + deq Q8(R) misses X by what Q8 misses R:
    # at most half an E4M3 step, or the saturation of R's block maximum when it
    # lies past 464 * 2^se
    r = x - oracle.dequantize(qx, sx)
    xhat = oracle.dequantize(qx, sx) + oracle.dequantize_mxfp8(qr8, sr)
    se_r = np.repeat(sr.astype(np.int64) - 127, 32, axis=1)
    bound = np.maximum(np.maximum(np.abs(r) * 2.0 ** -4, np.ldexp(1.0, se_r - 10)),
                       np.abs(r) - np.ldexp(448.0, se_r))
    assert (np.abs(x - xhat) <= bound).all()
    assert np.linalg.norm(x - xhat) < 0.1 * np.linalg.norm(r)


def test_fp8_residual_vanishes_on_representable_input():
    """X already exact in MXFP4: R = 0, so Q8(R) is all zero codes at the
    smallest scale and the layer equals plain W4A4."""
    rng = np.random.default_rng(6)
    q = rng.integers(0, 16, size=(5, 96)).astype(np.uint8)
    s = rng.integers(120, 135, size=(5, 3)).astype(np.uint8)
    q[:, ::32] = 7                                         # a 6 in every block fixes the scale
    x = oracle.dequantize(q, s)
    qx, sx, qr8, sr = oracle.residual_quantize_fp8(x)
    assert (qx == q).all() and (sx == s).all()
    assert (qr8 == 0).all() and (sr == 0).all()
    w = rng.normal(size=(4, 96))
    y8 = oracle.linear_fp8_residual(x, w)[0]
    y4, _, _, _ = oracle.linear(x, w)
    assert np.array_equal(y8, y4)
