"""Pins of the block-Hadamard rotation in the oracle ("大模型量化中的双线性尾部问题与
QuaRot正交旋转解决方案", §3: an orthogonal +-1 rotation before quantization,
folded into the weight). Against the Sylvester matrix from scipy, closed-form
identities of H, and a layer built so that every quantization is exact."""
import numpy as np
import scipy.linalg

import oracle

H32 = scipy.linalg.hadamard(32).astype(np.float64)     # Sylvester order, H[i,j] = (-1)^popcount(i & j)


def test_transform_is_the_sylvester_matrix_on_exact_inputs():
    rng = np.random.default_rng(0)
    x = rng.integers(-8, 9, size=(7, 96)).astype(np.float64)     # every partial sum exact in float32
    got = oracle.hadamard32_f32(x).astype(np.float64)
    want = (x.reshape(7, 3, 32) @ H32).reshape(7, 96)           # H symmetric: row blocks times H
    assert np.array_equal(got, want)


def test_transform_rounding_on_general_inputs():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((64, 256)) * np.exp(rng.uniform(-8, 8, (64, 256)))).astype(np.float32)
    got = oracle.hadamard32_f32(x).astype(np.float64)
    want = (x.astype(np.float64).reshape(64, 8, 32) @ H32).reshape(64, 256)
    scale = (np.abs(x.astype(np.float64)).reshape(64, 8, 32).sum(axis=2, keepdims=True) * np.ones((1, 1, 32))).reshape(64, 256)
    # five float32 roundings per output, each at most half an ulp of a partial sum bounded by sum |x|
    assert (np.abs(got - want) <= 5 * 2.0 ** -24 * scale).all()


def test_twice_is_32_times_identity_and_energy_scales_by_32():
    rng = np.random.default_rng(2)
    x = rng.integers(-20, 21, size=(5, 64)).astype(np.float64)
    once = oracle.hadamard32_f32(x).astype(np.float64)
    twice = oracle.hadamard32_f32(once).astype(np.float64)
    assert np.array_equal(twice, 32 * x)
    assert np.array_equal((once ** 2).reshape(5, 2, 32).sum(axis=2), 32 * (x ** 2).reshape(5, 2, 32).sum(axis=2))


def test_a_spike_spreads_evenly_over_its_block_only():
    x = np.zeros((1, 64))
    x[0, 37] = 100.0
    v = oracle.hadamard32_f32(x).astype(np.float64)
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
    q0, s0 = oracle.quantize_mxfp4(oracle.hadamard32_f32(w).astype(np.float64))
    assert np.array_equal(wq, q0)                     # same codes, scales 2^-5 apart
    assert np.array_equal(sw.astype(int), s0.astype(int) - 5)


def test_nonfinite_input_poisons_only_its_block():
    x = np.ones((1, 64))
    x[0, 3] = np.nan
    qx, sx, qr, sr = oracle.rotate_residual_quantize(x)
    assert sx[0, 0] == 255 and sr[0, 0] == 255 and (qx[0, :32] == 0).all()
    assert sx[0, 1] != 255
