"""GPU parity of the quantize and residual-quantize kernels: bit-exact codes
and scales against the oracle."""
import numpy as np
import pytest
import torch

import mxfp4_activation_gemm_amd as rfq
import oracle
import workloads
from gpu_helpers import assert_bytes_equal, dev_bf16, host, log, oracle_mx, oracle_rfq

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rfq.library()


def run_both(bits, what):
    log(f"[quantize] {what} shape={bits.shape}")
    x = dev_bf16(bits)
    c, s = rfq.quantize_mxfp4(x)
    qx, sx, qr, sr = rfq.residual_quantize(x)
    torch.cuda.synchronize()
    wc, ws = oracle_mx(bits)
    assert_bytes_equal(host(c), wc, what + " codes")
    assert_bytes_equal(host(s), ws, what + " scales")
    oqx, osx, oqr, osr = oracle_rfq(bits)
    assert_bytes_equal(host(qx), oqx, what + " Q(X) codes")
    assert_bytes_equal(host(sx), osx, what + " Q(X) scales")
    assert_bytes_equal(host(qr), oqr, what + " Q(R) codes")
    assert_bytes_equal(host(sr), osr, what + " Q(R) scales")


def test_every_bf16_pattern():
    # all 65536 patterns, NaN and Inf included: in order (neighbours share a
    # block), and shuffled (mixed magnitudes per block) in two row widths
    allp = np.arange(65536, dtype=np.uint16)
    run_both(allp.reshape(2048, 32), "all patterns, ordered")
    perm = np.random.default_rng(11).permutation(allp)
    run_both(perm.reshape(2048, 32), "all patterns, shuffled K=32")
    run_both(perm.reshape(128, 512), "all patterns, shuffled K=512")


def test_every_relative_position_below_the_block_max():
    # each block: one element sets amax = 2^j * f; the rest are random bf16
    # mantissas d binades below, for every bf16 exponent j and d in 0..12
    rng = np.random.default_rng(12)
    rows = []
    for e in range(1, 255):
        for d in range(13):
            blk = np.zeros(32, np.uint32)
            ee = max(e - d, 0)
            mant = rng.integers(0, 128, 32, dtype=np.uint32)
            sign = rng.integers(0, 2, 32, dtype=np.uint32)
            blk[:] = (sign << 15) | (np.uint32(ee) << 7) | mant
            blk[rng.integers(0, 32)] = (np.uint32(e) << 7) | np.uint32(rng.integers(0, 128))
            rows.append(blk.astype(np.uint16))
    bits = np.stack(rows)
    run_both(bits, "relative positions")


def test_rounding_ties_and_saturation_blocks():
    # exact midpoints and saturating values at many scales
    vals = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, 7.0, 7.5, 0.0, -0.0, 4.0, 6.0, 0.5, 3.0] * 2,
                    np.float32)
    rows = []
    for j in range(-133, 125, 3):
        v = np.ldexp(vals, j).astype(np.float32)
        v[31] = np.float32(np.ldexp(7.75, j))  # sets the scale to 2^j
        v[1::3] *= -1
        rows.append(workloads.f32_to_bf16_bits(v))
    run_both(np.stack(rows), "ties and saturation")


@pytest.mark.parametrize("name", ["tiny", "qwen3vl_attn_proj"])
def test_config_activations_full(name):
    cfg = workloads.CONFIGS[name]
    run_both(workloads.x_bf16(cfg), f"{name} X")


def test_weights_quantize():
    cfg = workloads.CONFIGS["tiny"]
    w = workloads.w_bf16(cfg)
    log("[quantize] tiny W")
    c, s = rfq.quantize_mxfp4(dev_bf16(w))
    wc, ws = oracle_mx(w)
    assert_bytes_equal(host(c), wc, "W codes")
    assert_bytes_equal(host(s), ws, "W scales")


def test_strided_rows_and_ragged_counts():
    rng = np.random.default_rng(13)
    for rows, K, ldx in [(1, 32, 32), (3, 96, 104), (5, 160, 256), (17, 480, 488), (33, 2080, 2080)]:
        full = workloads.f32_to_bf16_bits(rng.standard_t(3, size=(rows, ldx)).astype(np.float32) * 10)
        xd = dev_bf16(full)[:, :K]
        log(f"[quantize] strided rows={rows} K={K} ldx={ldx}")
        qx, sx, qr, sr = rfq.residual_quantize(xd)
        oqx, osx, oqr, osr = oracle_rfq(full[:, :K])
        assert_bytes_equal(host(qx), oqx, "strided Q(X)")
        assert_bytes_equal(host(sx), osx, "strided SX")
        assert_bytes_equal(host(qr), oqr, "strided Q(R)")
        assert_bytes_equal(host(sr), osr, "strided SR")


def test_empty_input():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    c, s = rfq.quantize_mxfp4(x)
    assert c.shape == (0, 32) and s.shape == (0, 2)


def _quantize_sweep():
    """Seeded (rows, K, row padding, input type) cases: whole and partial
    last waves (64 blocks per wave), rows shorter than a wave, padded rows."""
    rng = np.random.default_rng(77)
    cases = []
    for i in range(16):
        rows = int([rng.integers(1, 8), rng.integers(8, 300), rng.integers(300, 3000)][i % 3])
        K = int(32 * rng.integers(1, 80))
        pad = int(8 * rng.integers(0, 5)) if i % 4 else 0
        cases.append((rows, K, pad, "fp32" if i % 2 else "bf16"))
    return cases


@pytest.mark.parametrize("rows,K,pad,dtype", _quantize_sweep())
def test_quantize_sweep(rows, K, pad, dtype):
    """Both passes (Q(X) alone, and Q(X) with Q(R)) on dense and padded rows
    of bf16 and fp32 X, bit-exact against the oracle over the whole tensor."""
    rng = np.random.default_rng(rows * 31 + K + pad)
    ldx = K + pad
    full = (rng.standard_t(3, size=(rows, ldx)) * np.exp(rng.uniform(-8, 8, size=(rows, 1)))).astype(np.float32)
    log(f"[quantize] sweep rows={rows} K={K} ldx={ldx} {dtype}")
    if dtype == "bf16":
        bits = workloads.f32_to_bf16_bits(full)
        xd = dev_bf16(bits)[:, :K]
        x64 = oracle.bf16_bits_to_f64(bits[:, :K])
    else:
        xd = torch.from_numpy(full).cuda()[:, :K]
        x64 = full[:, :K].astype(np.float64)
    assert xd.stride(0) == ldx
    c, s = rfq.quantize_mxfp4(xd)
    qx, sx, qr, sr = rfq.residual_quantize(xd)
    torch.cuda.synchronize()
    wc, ws = oracle.quantize_mxfp4(x64)
    assert_bytes_equal(host(c), oracle.pack_codes(wc), "Q(X) alone codes")
    assert_bytes_equal(host(s), ws, "Q(X) alone scales")
    oqx, osx, oqr, osr = oracle.residual_quantize(x64)
    assert_bytes_equal(host(qx), oracle.pack_codes(oqx), "Q(X) codes")
    assert_bytes_equal(host(sx), osx, "Q(X) scales")
    assert_bytes_equal(host(qr), oracle.pack_codes(oqr), "Q(R) codes")
    assert_bytes_equal(host(sr), osr, "Q(R) scales")
