"""Property tests of the oracle's MXFP4 block encoding and RFQ residual pass,
driven by hypothesis over arbitrary finite bf16 blocks (derandomized, so the
examples are the same on every run).

The properties come from the format and the method, not from the oracle's
code: OCP MX v1.0 (shared E8M0 scale with the block maximum in E2M1's top
binade, round to nearest E2M1 magnitude, saturation at 6), and "Activation
Outliers Matter: Robust Recovery for Quantized Multimodal LLMs", §1 (the
residual is the whole quantization error, quantized by a second pass of the
same format).
"""
import numpy as np
from hypothesis import given, settings, strategies as st

import oracle

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])   # E2M1 magnitudes (OCP MX v1.0)
FINITE_BF16 = st.integers(0, 0xFFFF).filter(lambda b: (b >> 7) & 0xFF != 0xFF)
BLOCK = st.lists(FINITE_BF16, min_size=32, max_size=32)
SETTINGS = settings(max_examples=400, deadline=None, derandomize=True)


def block(bits):
    return oracle.bf16_bits_to_f64(np.array(bits, dtype=np.uint16).reshape(1, 32))


def se_of(code):
    return int(code) - 127


@SETTINGS
@given(BLOCK)
def test_scale_and_rounding_on_any_block(bits):
    x = block(bits)
    q, s = oracle.quantize_mxfp4(x)
    d = oracle.dequantize(q, s)
    amax = float(np.abs(x).max())
    se = se_of(s[0, 0])
    unit = 2.0 ** se
    if amax > 0 and se > -127:
        assert 4 <= amax / unit < 8                       # block maximum in the top binade
    v = np.abs(x[0]) / unit
    err = np.abs(x[0] - d[0])
    # nearest grid magnitude (times 2^se) for unsaturated elements, 6 x 2^se above
    best = np.min(np.abs(v[:, None] - GRID[None, :]), axis=1) * unit
    inside = v <= 6
    assert (err[inside] == best[inside]).all()
    assert (np.abs(d[0][~inside]) == 6 * unit).all()
    assert (err <= 2 * unit).all()
    # sign kept on every element, zeros included
    assert (np.signbit(d[0]) == np.signbit(x[0])).all()


@SETTINGS
@given(BLOCK)
def test_idempotence_and_sign_symmetry_on_any_block(bits):
    x = block(bits)
    q, s = oracle.quantize_mxfp4(x)
    d = oracle.dequantize(q, s)
    q2, s2 = oracle.quantize_mxfp4(d)
    assert (q2 == q).all() and (s2 == s).all()
    qn, sn = oracle.quantize_mxfp4(-x)
    assert (qn == (q ^ 8)).all() and (sn == s).all()


@SETTINGS
@given(BLOCK, st.integers(-20, 20))
def test_power_of_two_covariance_on_any_block(bits, j):
    x = block(bits)
    q, s = oracle.quantize_mxfp4(x)
    qj, sj = oracle.quantize_mxfp4(np.ldexp(x, j))
    se, sej = se_of(s[0, 0]), se_of(sj[0, 0])
    if -127 < se and -127 < se + j <= 127 and float(np.abs(x).max()) > 0:
        assert sej == se + j and (qj == q).all()


@SETTINGS
@given(BLOCK)
def test_residual_pass_on_any_block(bits):
    x = block(bits)
    qx, sx, qr, sr = oracle.residual_quantize(x)
    d = oracle.dequantize(qx, sx)
    r = x - d
    # the residual of a bf16 block is exact in float32 as well as float64
    assert ((x.astype(np.float32) - d.astype(np.float32)).astype(np.float64) == r).all()
    # the second pass never adds error: zero is a grid value, and a saturated
    # element moves toward zero
    e2 = r - oracle.dequantize(qr, sr)
    assert (np.abs(e2) <= np.abs(r)).all()
    # error bounds of the floor scale rule when the scale is not clamped at
    # 2^-127: each pass leaves at most a quarter of its block maximum
    # (rounding error <= 2^se <= amax / 4; saturation error < amax / 4)
    if se_of(sx[0, 0]) > -127:
        assert float(np.abs(r).max()) <= float(np.abs(x).max()) / 4
    if se_of(sr[0, 0]) > -127:
        assert float(np.abs(e2).max()) <= float(np.abs(r).max()) / 4


MIDPOINTS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])   # halfway between grid neighbours
EVEN_WINNER = np.array([0, 2, 2, 4, 4, 6, 6])                   # index of the even neighbour


@SETTINGS
@given(st.lists(st.integers(0, 6), min_size=31, max_size=31), st.lists(st.booleans(), min_size=32, max_size=32),
       st.sampled_from([4.0, 6.0]), st.integers(-100, 100))
def test_ties_go_to_the_even_code(mids, signs, top, j):
    """Blocks of exact midpoints (times 2^j) with one element fixing the scale
    at 2^j: every midpoint takes the neighbour with the even magnitude index
    (round half to even on the 1-bit mantissa)."""
    v = np.concatenate([[top], MIDPOINTS[mids]])
    x = np.ldexp(np.where(signs, -v, v), j).reshape(1, 32)
    q, s = oracle.quantize_mxfp4(x)
    assert se_of(s[0, 0]) == j
    assert ((q[0, 1:] & 7) == EVEN_WINNER[mids]).all()
    assert ((q[0] >> 3) == np.array(signs, dtype=np.uint8)).all()
