"""Pins of the oracle's RFQ activation encoding (quantize, residual, second pass)."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "toy_block.json")


def _hex(s):
    return int(s, 16)


def test_toy_block_worked_example():
    g = json.load(open(GOLDEN))
    bits = np.zeros((1, 32), np.uint16)
    bits[0, :4] = [_hex(h) for h in g["x_bf16_bits_first4"]]
    x = oracle.bf16_bits_to_f64(bits)
    assert list(x[0, :4]) == g["x_values_first4"]
    qx, sx, qr, sr = oracle.residual_quantize(x)
    assert sx[0, 0] == _hex(g["qx_scale"]) and sr[0, 0] == _hex(g["qr_scale"])
    assert list(qx[0, :4]) == g["qx_codes_first4"] and (qx[0, 4:] == 0).all()
    assert list(qr[0, :4]) == g["qr_codes_first4"] and (qr[0, 4:] == 0).all()
    assert [int(b) for b in oracle.pack_codes(qx)[0, :2]] == [_hex(h) for h in g["qx_packed_first2"]]
    assert [int(b) for b in oracle.pack_codes(qr)[0, :2]] == [_hex(h) for h in g["qr_packed_first2"]]
    dqx = oracle.dequantize(qx, sx)[0, :4]
    assert list(dqx) == g["deq_qx_first4"] and np.signbit(dqx[0])
    assert list(x[0, :4] - dqx) == g["residual_first4"]
    assert list(oracle.dequantize(qr, sr)[0, :4]) == g["deq_qr_first4"]
    # the blog's qualitative point: the three small values share one level
    assert dqx[0] == dqx[1] == dqx[2] == 0.0


def test_grid_values_have_zero_residual():
    # Any block whose values are E2M1 grid values times one common 2^j, with its
    # largest magnitude in the top binade [4, 6] (so that se = j), is exact.
    rng = np.random.default_rng(2)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    for _ in range(50):
        j = int(rng.integers(-120, 120))
        vals = grid[rng.integers(0, 8, size=(4, 32))] * rng.choice([-1.0, 1.0], size=(4, 32))
        vals[:, 0] = rng.choice([4.0, 6.0], size=4)
        x = np.ldexp(vals, j)
        qx, sx, qr, sr = oracle.residual_quantize(x)
        assert (oracle.dequantize(qx, sx) == x).all()
        assert (sx == j + 127).all()           # amax in [4, 8) * 2^j -> se = j
        assert (qr == 0).all() and (sr == 0).all()


def _blocks(rng, rows=64, K=256):
    x = rng.standard_t(2.0, size=(rows, K))
    x[:, rng.integers(0, K, 3)] *= 80
    return workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(x.astype(np.float32))).astype(np.float64)


def test_residual_pass_never_increases_error_per_element_and_block():
    rng = np.random.default_rng(3)
    x = _blocks(rng)
    qx, sx, qr, sr = oracle.residual_quantize(x)
    r = x - oracle.dequantize(qx, sx)
    e2 = r - oracle.dequantize(qr, sr)
    assert (np.abs(e2) <= np.abs(r)).all()
    rb, eb, xb = (a.reshape(64, -1, 32) for a in (r, e2, x))
    assert (np.linalg.norm(eb, axis=2) <= np.linalg.norm(rb, axis=2)).all()
    assert (np.abs(eb).max(2) <= np.abs(rb).max(2)).all()
    # floor rule bounds: max rounding error is 2^se <= amax/4, and saturation
    # error is below amax/4 as well
    assert (np.abs(rb).max(2) <= np.abs(xb).max(2) / 4).all()
    assert (np.abs(eb).max(2) <= np.abs(rb).max(2) / 4).all()


def test_residual_is_exact_in_float32_for_bf16_inputs():
    rng = np.random.default_rng(4)
    x = _blocks(rng)
    qx, sx, _, _ = oracle.residual_quantize(x)
    d = oracle.dequantize(qx, sx)
    r64 = x - d
    r32 = (x.astype(np.float32) - d.astype(np.float32)).astype(np.float64)
    assert (r64 == r32).all()


def test_idempotence_sign_symmetry_and_power_of_two_covariance():
    rng = np.random.default_rng(5)
    x = _blocks(rng)
    qx, sx = oracle.quantize_mxfp4(x)
    d = oracle.dequantize(qx, sx)
    q2, s2 = oracle.quantize_mxfp4(d)
    assert (q2 == qx).all() and (s2 == sx).all()
    qn, sn = oracle.quantize_mxfp4(-x)
    assert (qn == (qx ^ 8)).all() and (sn == sx).all()
    for j in (-7, 3, 20):
        qj, sj = oracle.quantize_mxfp4(np.ldexp(x, j))
        assert (qj == qx).all() and (sj.astype(int) == sx.astype(int) + j).all()


def test_nonfinite_blocks():
    x = np.zeros((2, 64))
    x[0, 5] = np.nan
    x[1, 40] = np.inf
    x[1, 3] = 1.5
    qx, sx, qr, sr = oracle.residual_quantize(x)
    assert sx[0, 0] == 255 and sx[0, 1] == 0
    assert sx[1, 1] == 255 and sx[1, 0] == 125
    assert (qx[0, :32] == 0).all() and (qx[1, 32:] == 0).all()
    assert sr[0, 0] == 255 and sr[1, 1] == 255
    assert (qr[0, :32] == 0).all() and (qr[1, 32:] == 0).all()


def test_pack_unpack_roundtrip_and_nibble_order():
    rng = np.random.default_rng(6)
    c = rng.integers(0, 16, size=(5, 64)).astype(np.uint8)
    p = oracle.pack_codes(c)
    assert p.shape == (5, 32)
    assert (p[:, 0] == (c[:, 0] | (c[:, 1] << 4))).all()
    assert (oracle.unpack_codes(p) == c).all()


@pytest.mark.parametrize("name", ["tiny", "qwen3vl_attn_proj"])
def test_rfq_reduces_activation_error_on_config_inputs(name):
    cfg = workloads.CONFIGS[name]
    x = oracle.bf16_bits_to_f64(workloads.x_bf16(cfg, 0, 32))
    qx, sx, qr, sr = oracle.residual_quantize(x)
    e1 = x - oracle.dequantize(qx, sx)
    e2 = e1 - oracle.dequantize(qr, sr)
    assert np.linalg.norm(e2) < np.linalg.norm(e1) / 4
