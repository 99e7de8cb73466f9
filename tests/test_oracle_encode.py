"""Pins of the oracle's MXFP4 scale rule and E2M1 encoder.

* brute force: every E2M1 code is tried and the IEEE rule picked out by hand
  (nearest value of the operand's sign, ties to the code with a zero
  mantissa bit), for every finite bf16 pattern at every scale whose window
  matters;
* library rounding: inside each E2M1 binade the step is a power of two, so
  round-half-to-even onto the grid equals numpy's banker's rounding of
  v / step;
* the scale rule against the bit-field form max(biased_exponent - 2, 0).
"""
import numpy as np

import oracle

SPEC_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
ALL_BF16 = np.arange(65536, dtype=np.uint16)
X_ALL = oracle.bf16_bits_to_f64(ALL_BF16)
FINITE = np.isfinite(X_ALL)


def brute_force_codes(x, se):
    """Nearest E2M1 code among those carrying x's sign; ties to even mantissa.

    |v| is capped at 16 first: for any v >= 6 the nearest grid value is 6
    whatever v is, and the cap keeps every distance exact in float64.
    """
    v = np.clip(np.ldexp(x, -se), -16.0, 16.0)
    neg = np.signbit(x)
    vals = np.concatenate([SPEC_E2M1, -SPEC_E2M1])           # codes 0..15
    best = np.zeros(x.shape, np.uint8)
    bestd = np.full(x.shape, np.inf)
    for code in range(16):
        same_sign = (code >= 8) == neg
        d = np.where(same_sign, np.abs(v - vals[code]), np.inf)
        mant_even = (code & 1) == 0
        better = (d < bestd) | ((d == bestd) & mant_even)
        best = np.where(better, code, best)
        bestd = np.where(better, d, bestd)
    return best.astype(np.uint8)


def test_encoder_equals_brute_force_on_all_bf16_patterns():
    x = X_ALL[FINITE]
    ex = np.frexp(np.abs(x))[1] - 1                      # floor(log2 |x|), -inf guarded below
    for shift in range(-5, 6):                           # v = x / 2^se within [2^-5, 2^6)
        se = np.clip(ex - shift, -127, 125)
        got = oracle.encode_block_elements(x, se)
        want = brute_force_codes(x, se)
        assert (got == want).all(), shift
    for se in (-127, -126, -120, 0, 120, 125):           # extreme fixed scales, all patterns
        got = oracle.encode_block_elements(x, se)
        assert (got == brute_force_codes(x, se)).all(), se


def test_encoder_equals_per_binade_bankers_rounding():
    x = X_ALL[FINITE]
    for se in range(-3, 8):
        v = np.abs(np.ldexp(x, -se))
        a = np.minimum(v, 6.0)
        step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
        q = np.minimum(np.round(a / step) * step, 6.0)   # numpy rounds half to even
        want_mag = np.searchsorted(SPEC_E2M1, q)
        assert (SPEC_E2M1[want_mag] == q).all()
        got = oracle.encode_block_elements(x, se)
        assert ((got & 7) == want_mag).all(), se
        assert (((got >> 3) & 1) == np.signbit(x)).all()


def test_midpoint_ties_and_saturation():
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    want = [0, 2, 2, 4, 4, 6, 6]                         # even code wins every tie
    assert list(oracle.encode_block_elements(mids, 0)) == want
    assert list(oracle.encode_block_elements(-mids, 0)) == [c | 8 for c in want]
    sat = np.array([6.0, 6.5, 7.0, 7.99, 8.0, 1e30])
    assert (oracle.encode_block_elements(sat, 0) == 7).all()
    assert (oracle.encode_block_elements(-sat, 0) == 15).all()
    assert list(oracle.encode_block_elements(np.array([0.0, -0.0, -0.1, 0.1]), 0)) == [0, 8, 8, 0]


def test_scale_rule_matches_bitfield_form_for_every_bf16_amax():
    amax = np.abs(X_ALL[FINITE])
    bits = ALL_BF16[FINITE] & np.uint16(0x7FFF)
    biased = (bits >> 7).astype(np.int64)
    want = np.maximum(biased - 2, 0)
    _, code = oracle.scale_exponent(amax)
    assert (code.astype(np.int64) == want).all()


def test_scale_rule_over_fp32_exponent_sweep():
    for e in range(-149, 128):
        for f in (1.0, 1.5, 1.999999):
            amax = np.ldexp(f, e)
            if not np.isfinite(np.float32(amax)):
                continue
            se, code = oracle.scale_exponent(np.array([amax]))
            assert se[0] == max(e - 2, -127)
            assert code[0] == se[0] + 127


def test_scale_puts_amax_in_top_binade():
    # For amax >= 2^-125 (no clamp) amax / 2^se lies in [4, 8): the block maximum
    # lands in the top E2M1 binade, so only values in (6, 8) saturate.
    rng = np.random.default_rng(1)
    amax = np.abs(rng.standard_cauchy(10000)) + 1e-30
    se, _ = oracle.scale_exponent(amax)
    v = np.ldexp(amax, -se)
    keep = se > -127
    assert ((v[keep] >= 4) & (v[keep] < 8)).all()


def test_scale_special_cases():
    se, code = oracle.scale_exponent(np.array([0.0, np.inf, np.nan, 2.0 ** -140]))
    assert list(code) == [0, 255, 255, 0]
    assert se[0] == -127 and se[3] == -127


def test_encoder_on_float32_values_around_every_midpoint():
    """float32 inputs carry 24 significant bits (the rotated path quantizes
    them): values a few ulps either side of each E2M1 midpoint round to the
    nearer neighbour, the midpoint itself to the even code, in every scale
    window; checked against the brute-force rule and numpy's banker's rounding."""
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0], dtype=np.float32)
    vals = [mids]
    for k in range(1, 4):
        vals.append(np.nextafter(mids, np.float32(np.inf)) if k == 1 else
                    np.array([np.nextafter(np.nextafter(m, np.float32(np.inf)), np.float32(np.inf)) for m in mids],
                             dtype=np.float32) if k == 2 else
                    np.nextafter(mids, np.float32(0)))
    v = np.concatenate(vals).astype(np.float32)
    for se in (-10, -1, 0, 3, 50):
        x = np.ldexp(v.astype(np.float64), se)
        x = np.concatenate([x, -x])
        assert (x.astype(np.float32).astype(np.float64) == x).all()
        got = oracle.encode_block_elements(x, se)
        assert (got == brute_force_codes(x, se)).all(), se
        a = np.minimum(np.abs(np.ldexp(x, -se)), 6.0)
        step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
        q = np.minimum(np.round(a / step) * step, 6.0)
        assert (SPEC_E2M1[got & 7] == q).all(), se
