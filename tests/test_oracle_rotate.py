"""Pins of the block-Hadamard rotation in the oracle ("大模型量化中的双线性尾部问题与
QuaRot正交旋转解决方案", §3: an orthogonal +-1 rotation before quantization,
folded into the weight). Against the Sylvester matrix from scipy, exact
rational sums rounded to float32 by NumPy's own float32 conversion, closed-form
identities of H, and a layer built so that every quantization is exact."""
from fractions import Fraction

import numpy as np
import scipy.linalg

import oracle

H32 = scipy.linalg.hadamard(32).astype(np.float64)     # Sylvester order, H[i,j] = (-1)^popcount(i & j)


def test_transform_is_the_sylvester_matrix_on_exact_inputs():
    rng = np.random.default_rng(0)
    x = rng.integers(-8, 9, size=(7, 96)).astype(np.float64)     # every sum exact in float32
    got = oracle.hadamard32_rounded(x).astype(np.float64)
    want = (x.reshape(7, 3, 32) @ H32).reshape(7, 96)           # H symmetric: row blocks times H
    assert np.array_equal(got, want)


def exact_rounded(block, div32=False):
    """Each output of one 32-block: the exact rational sum with the Sylvester
    signs, rounded to float32 as a Python float is: NumPy's float32 cast of a
    float64 is a single rounding when the float64 holds the sum exactly,
    which the sums here are built to satisfy (checked)."""
    out = []
    for i in range(32):
        q = sum(Fraction(float(block[j])) * int(H32[j, i]) for j in range(32))
        if div32:
            q /= 32
        assert Fraction(float(q)) == q          # exact in float64
        out.append(np.float32(float(q)))
    return np.array(out, dtype=np.float32)


def test_each_output_is_the_exact_sum_rounded_once():
    """float32 inputs with 24-bit significands over a few binades: each output
    must be the exact sum rounded once, whatever order would have summed it.
    On these blocks a float32 butterfly (five roundings) gets some outputs
    wrong, so an oracle that summed in some float32 order would fail here."""
    rng = np.random.default_rng(1)
    x = (rng.uniform(1, 2, (40, 64)) * np.exp2(rng.integers(0, 12, (40, 64)))
         * rng.choice([-1, 1], (40, 64))).astype(np.float32).astype(np.float64)
    got = oracle.hadamard32_rounded(x)
    for w in (False, True):
        got = oracle.hadamard32_rounded(x, divide_by_32=w)
        for r in range(40):
            for b in range(2):
                assert np.array_equal(got[r, 32 * b:32 * b + 32], exact_rounded(x[r, 32 * b:32 * b + 32], w))
    # the float32 butterfly, for contrast: it differs from the exact rounding somewhere
    v = x.astype(np.float32).reshape(-1, 32).copy()
    for span in (1, 2, 4, 8, 16):
        lo = np.array([i for i in range(32) if not i & span])
        a, c = v[:, lo].copy(), v[:, lo + span].copy()
        v[:, lo], v[:, lo + span] = a + c, a - c
    assert not np.array_equal(v.reshape(x.shape), oracle.hadamard32_rounded(x))


def test_wide_blocks_take_the_rational_path():
    """Blocks whose terms span more than float64's 53 bits (a huge value, a
    tiny one and cancellation): the exact sum is formed as a rational and
    rounded to float32 directly (checked against an independent rounding of
    the same rationals: nearest of the float32 neighbours, ties to even)."""
    x = np.zeros((3, 32))
    x[0, 0], x[0, 1], x[0, 2] = 2.0 ** 100, -(2.0 ** 100), 1.5 * 2.0 ** -60
    x[1, :] = 1.0
    x[1, 5] = 2.0 ** 70
    x[1, 6] = 2.0 ** -20
    x[2, 0], x[2, 3] = 3.0 * 2.0 ** 80, 2.0 ** -80
    got = oracle.hadamard32_rounded(x)
    for r in range(3):
        for i in range(32):
            q = sum(Fraction(float(x[r, j])) * int(H32[j, i]) for j in range(32))
            f = np.float32(float(q))            # float64 first, then float32: may round twice
            cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
            dist = [abs(Fraction(float(c)) - q) for c in cands]
            best = min(dist)
            winners = [c for c, d in zip(cands, dist) if d == best]
            want = winners[0] if len(winners) == 1 else [c for c in winners
                                                        if not np.frombuffer(c.tobytes(), np.uint32)[0] & 1][0]
            assert got[r, i] == want, (r, i)
    # the cancellation survives: output 0 of row 0 is the small term, not 0
    assert got[0, 0] == np.float32(1.5 * 2.0 ** -60)


def test_fraction_to_f32_landmarks():
    assert oracle.fraction_to_f32(Fraction(1, 3)) == float(np.float32(1 / 3))
    assert oracle.fraction_to_f32(Fraction(2) ** -149) == 2.0 ** -149            # smallest subnormal
    assert oracle.fraction_to_f32(Fraction(2) ** -150) == 0.0                     # tie to even (0)
    assert oracle.fraction_to_f32(Fraction(3) * Fraction(2) ** -151) == 2.0 ** -149
    big = Fraction(2) ** 128 - Fraction(2) ** 103                                 # the overflow midpoint
    assert oracle.fraction_to_f32(big) == float("inf")
    assert oracle.fraction_to_f32(big - 1) == float(np.finfo(np.float32).max)
    assert oracle.fraction_to_f32(-Fraction(1) - Fraction(2) ** -24) == -1.0     # tie to even
    assert oracle.fraction_to_f32(Fraction(1) + Fraction(3) * Fraction(2) ** -25) == 1.0 + 2.0 ** -23


def test_twice_is_32_times_identity_and_energy_scales_by_32():
    rng = np.random.default_rng(2)
    x = rng.integers(-20, 21, size=(5, 64)).astype(np.float64)
    once = oracle.hadamard32_rounded(x).astype(np.float64)
    twice = oracle.hadamard32_rounded(once).astype(np.float64)
    assert np.array_equal(twice, 32 * x)
    assert np.array_equal((once ** 2).reshape(5, 2, 32).sum(axis=2), 32 * (x ** 2).reshape(5, 2, 32).sum(axis=2))


def test_a_spike_spreads_evenly_over_its_block_only():
    x = np.zeros((1, 64))
    x[0, 37] = 100.0
    v = oracle.hadamard32_rounded(x).astype(np.float64)
    assert (v[0, :32] == 0).all()
    assert (np.abs(v[0, 32:]) == 100.0).all()
    assert np.array_equal(np.sign(v[0, 32:]), H32[37 - 32])      # the spike's row of H


def grid_blocks(rng, rows, K):
    """Values that MXFP4 represents exactly with the scale the rule picks:
    random E2M1 codes times 2^se per block, each block holding a 4 or a 6."""
    mags = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    codes = rng.integers(0, 8, size=(rows, K))
    codes[:, ::32] = rng.choice([6, 7], size=(rows, K // 32))       # 4 or 6 somewhere in each block
    v = mags[codes] * rng.choice([-1.0, 1.0], size=(rows, K))
    se = rng.integers(-6, 4, size=(rows, K // 32))
    return v * np.repeat(2.0 ** se, 32, axis=1)


def test_rotation_cancels_in_the_layer_when_quantization_is_exact():
    """X = V H / 32 and W = U H with V, U on the MXFP4 grid: then X H = V and
    W H / 32 = U exactly, R = 0, and the rotated layer returns X W^T exactly."""
    rng = np.random.default_rng(3)
    M, N, K = 6, 5, 64
    V, U = grid_blocks(rng, M, K), grid_blocks(rng, N, K)
    X = (V.reshape(M, 2, 32) @ H32 / 32).reshape(M, K)
    W = (U.reshape(N, 2, 32) @ H32).reshape(N, K)
    assert np.array_equal(X.astype(np.float32).astype(np.float64), X)      # exact float32 inputs
    assert np.array_equal(W.astype(np.float32).astype(np.float64), W)
    y, s, (qx, sx, qr, sr), (wq, sw) = oracle.linear_rotated(X, W)
    assert np.array_equal(oracle.dequantize(qx, sx), V)
    assert np.array_equal(oracle.dequantize(wq, sw), U)
    assert (oracle.dequantize(qr, sr) == 0).all()
    assert np.array_equal(y, X @ W.T)


def test_weight_side_carries_the_one_over_32():
    rng = np.random.default_rng(4)
    w = rng.normal(0, 0.02, (3, 64)).astype(np.float32).astype(np.float64)
    wq, sw = oracle.rotate_quantize_weight(w)
    q0, s0 = oracle.quantize_mxfp4(oracle.hadamard32_rounded(w).astype(np.float64))
    assert np.array_equal(wq, q0)                     # same codes, scales 2^-5 apart
    assert np.array_equal(sw.astype(int), s0.astype(int) - 5)


def test_nonfinite_input_poisons_only_its_block():
    x = np.ones((1, 64))
    x[0, 3] = np.nan
    qx, sx, qr, sr = oracle.rotate_residual_quantize(x)
    assert sx[0, 0] == 255 and sr[0, 0] == 255 and (qx[0, :32] == 0).all()
    assert sx[0, 1] != 255


def test_an_exact_zero_sum_is_positive_zero():
    x = np.full((2, 32), -0.0)
    x[1, :2] = [1.0, 1.0]                        # output i is 1 + (-1)^i: 2 at even i, an exact 0 at odd i
    v = oracle.hadamard32_rounded(x)
    assert not np.signbit(v[0]).any() and (v[0] == 0).all()
    assert (v[1, ::2] == 2.0).all() and not np.signbit(v[1, 1::2]).any() and (v[1, 1::2] == 0).all()
    qx, sx, _, _ = oracle.rotate_residual_quantize(x)
    assert (qx[0] == 0).all()                    # +0 encodes as code 0, not 8


# ---- the 64-point rotation (the page's per-head size; two MX blocks) ----

H64 = scipy.linalg.hadamard(64).astype(np.float64)


def test_size64_is_the_sylvester_matrix_on_exact_inputs():
    rng = np.random.default_rng(10)
    x = rng.integers(-8, 9, size=(5, 192)).astype(np.float64)
    got = oracle.hadamard_rounded(x, 64).astype(np.float64)
    assert np.array_equal(got, (x.reshape(5, 3, 64) @ H64).reshape(5, 192))


def test_size64_is_two_32_point_transforms_combined():
    """Sylvester's block form H64 = [[H32, H32], [H32, -H32]]: with y0, y1
    the 32-point transforms of a block's halves, the 64-point transform is
    [y0 + y1, y0 - y1] (exact inputs, so every sum is exact)."""
    rng = np.random.default_rng(11)
    x = rng.integers(-50, 51, size=(4, 128)).astype(np.float64)
    y = oracle.hadamard_rounded(x, 32).astype(np.float64).reshape(4, 2, 2, 32)
    want = np.concatenate([y[:, :, 0] + y[:, :, 1], y[:, :, 0] - y[:, :, 1]], axis=2).reshape(4, 128)
    assert np.array_equal(oracle.hadamard_rounded(x, 64).astype(np.float64), want)


def test_size64_outputs_are_exact_sums_rounded_once():
    rng = np.random.default_rng(12)
    x = (rng.uniform(1, 2, (6, 64)) * np.exp2(rng.integers(0, 10, (6, 64)))
         * rng.choice([-1, 1], (6, 64))).astype(np.float32).astype(np.float64)
    for div in (False, True):
        got = oracle.hadamard_rounded(x, 64, divide=div)
        for r in range(6):
            for i in range(64):
                q = sum(Fraction(float(x[r, j])) * int(H64[j, i]) for j in range(64))
                if div:
                    q /= 64
                assert Fraction(float(q)) == q
                assert got[r, i] == np.float32(float(q)), (r, i)


def test_size64_twice_is_64_times_identity():
    rng = np.random.default_rng(13)
    x = rng.integers(-20, 21, size=(3, 128)).astype(np.float64)
    once = oracle.hadamard_rounded(x, 64).astype(np.float64)
    assert np.array_equal(oracle.hadamard_rounded(once, 64).astype(np.float64), 64 * x)


def test_size64_rotation_cancels_in_the_layer_when_quantization_is_exact():
    rng = np.random.default_rng(14)
    M, N, K = 5, 4, 128
    V, U = grid_blocks(rng, M, K), grid_blocks(rng, N, K)
    X = (V.reshape(M, 2, 64) @ H64 / 64).reshape(M, K)
    W = (U.reshape(N, 2, 64) @ H64).reshape(N, K)
    assert np.array_equal(X.astype(np.float32).astype(np.float64), X)
    assert np.array_equal(W.astype(np.float32).astype(np.float64), W)
    y, s, (qx, sx, qr, sr), (wq, sw) = oracle.linear_rotated(X, W, size=64)
    assert np.array_equal(oracle.dequantize(qx, sx), V)
    assert np.array_equal(oracle.dequantize(wq, sw), U)
    assert (oracle.dequantize(qr, sr) == 0).all()
    assert np.array_equal(y, X @ W.T)


def test_size64_weight_side_carries_the_one_over_64():
    rng = np.random.default_rng(15)
    w = rng.normal(0, 0.02, (3, 128)).astype(np.float32).astype(np.float64)
    wq, sw = oracle.rotate_quantize_weight(w, 64)
    q0, s0 = oracle.quantize_mxfp4(oracle.hadamard_rounded(w, 64).astype(np.float64))
    assert np.array_equal(wq, q0)
    assert np.array_equal(sw.astype(int), s0.astype(int) - 6)


def test_rotation_size_and_width_are_checked():
    import pytest
    with pytest.raises(ValueError):
        oracle.hadamard_rounded(np.zeros((1, 96)), 64)
    with pytest.raises(ValueError):
        oracle.hadamard_rounded(np.zeros((1, 96)), 48)
