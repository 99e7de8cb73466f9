"""GPU parity of the fp32-input quantize paths and of the block-Hadamard
rotated paths (activation X H with the RFQ residual, weight W H / n, for
rotation sizes n = 32 and 64): codes and scales bit-exact against the
oracle, and the rotated layer's Y within the per-output tolerance."""
import numpy as np
import pytest
import torch

import mxfp4_activation_gemm_amd as rfq
import oracle
import workloads
from gpu_helpers import assert_bytes_equal, check_exact_where_covered, check_y, dev_bf16, host, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rfq.library()


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def check_mx(got, want, what):
    (gc, gs), (wc, ws) = got, want
    assert_bytes_equal(host(gc), oracle.pack_codes(wc), what + " codes")
    assert_bytes_equal(host(gs), ws, what + " scales")


def check_rfq(got, want, what):
    check_mx(got[:2], want[:2], what + " Q(X)")
    check_mx(got[2:], want[2:], what + " Q(R)")


def near_midpoints(rng, rows, K):
    """fp32 blocks that pin every E2M1 rounding decision: one element at
    4 * 2^se fixes the scale, the rest sit at midpoints and a few float32
    ulps either side of them (and of 6, the saturation edge), with random
    signs, scale exponents and positions."""
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.5, 3.0], dtype=np.float32)
    base = rng.choice(mids, size=(rows, K)).astype(np.float32)
    k = rng.integers(-3, 4, size=(rows, K))
    v = base.copy()
    for step in range(3):
        up, dn = k > step, k < -step
        v = np.where(up, np.nextafter(v, np.float32(np.inf)), v)
        v = np.where(dn, np.nextafter(v, np.float32(0)), v)
    v[:, ::32] = 4.0
    v *= rng.choice([-1.0, 1.0], size=(rows, K)).astype(np.float32)
    se = rng.integers(-20, 20, size=(rows, K // 32))
    return (v * np.repeat(np.exp2(se), 32, axis=1)).astype(np.float32)


def signed_zero_rows(rng, x, r0, zero, neg_zero, one):
    """Rows r0 and r0 + 1, first 64 columns (one 64-block, two 32-blocks):
    zeros of random sign, then the same with an equal nonzero pair at every
    position 4 i + 2, 4 i + 3, so that half of the Hadamard sums cancel
    exactly amid the signed zeros (every exact zero must come out as +0).
    Rows or columns past the array's are left out."""
    n = min(64, x.shape[1])
    for r in (r0, r0 + 1):
        if r < x.shape[0]:
            x[r, :n] = np.where(rng.random(n) < 0.5, neg_zero, zero)
    if r0 + 1 < x.shape[0]:
        x[r0 + 1, 2:n:4] = one
        x[r0 + 1, 3:n:4] = one


def heavy_f32(rng, rows, K):
    x = rng.standard_t(3, size=(rows, K)) * np.exp(rng.uniform(-6, 6, size=(rows, 1)))
    x[:, rng.choice(K, size=3, replace=False)] *= 80
    x = x.astype(np.float32)
    x[0, :32] = 0.0
    x[0, 32:64] = -0.0
    x[1, :16] = np.float32(1e-40)            # float32 subnormals
    signed_zero_rows(rng, x, 2, np.float32(0.0), np.float32(-0.0), np.float32(1.5))
    return x


@pytest.mark.parametrize("rows,K", [(96, 1024), (37, 224)])
@pytest.mark.parametrize("kind", ["midpoints", "heavy"])
def test_fp32_input_quantize_and_residual(kind, rows, K):
    """Dense fp32 X: whole waves (96 x 1024) and a ragged last wave
    (37 x 224, 259 blocks)."""
    rng = np.random.default_rng((31 if kind == "midpoints" else 32) + rows)
    x = near_midpoints(rng, rows, K) if kind == "midpoints" else heavy_f32(rng, rows, K)
    log(f"[rotate] fp32 input {kind} {rows}x{K}")
    xd = dev_f32(x)
    got_q = rfq.quantize_mxfp4(xd)
    got_r = rfq.residual_quantize(xd)
    torch.cuda.synchronize()
    x64 = x.astype(np.float64)
    check_mx(got_q, oracle.quantize_mxfp4(x64), f"fp32 {kind}")
    check_rfq(got_r, oracle.residual_quantize(x64), f"fp32 {kind}")


def fit_exactness(x, size):
    """Each rotation block's finite values snapped to multiples of
    2^(e_max - 29), e_max the exponent of the block's largest magnitude
    (zeros, NaN and infinities kept): every block's terms then lie within
    about 37 bits of each other, inside the 53 bits within which the
    kernel's fp64 sums are exact, whatever the input precision. Returns
    float32."""
    v = np.asarray(x, dtype=np.float64).reshape(-1, size).copy()
    fin = np.isfinite(v)
    mag = np.where(fin, np.abs(v), 0.0).max(axis=1, keepdims=True)
    _, e = np.frexp(np.where(mag > 0, mag, 1.0))            # mag < 2^e
    grid = np.exp2(e.astype(np.float64) - 30)
    v = np.where(fin, np.round(v / grid) * grid, v)
    return v.astype(np.float32).reshape(np.shape(x))


def assert_exactness(x64, size):
    """Every block with finite values has its terms within 53 bits (the
    kernel's exactness condition, as the oracle computes it)."""
    from oracle.rotate import _lsb_exponent
    b = np.asarray(x64, dtype=np.float64).reshape(-1, size)
    b = b[np.isfinite(b).all(axis=1)]
    mag = np.abs(b).sum(axis=1)
    L = _lsb_exponent(b).min(axis=1)
    U = np.floor(np.log2(np.where(mag > 0, mag, 1.0))) + 2
    spread = np.where(mag > 0, U - L, 0)
    assert spread.max() <= 53, f"a block spans {spread.max()} bits"


def spiky_bf16(rng, rows, K):
    x = rng.laplace(0, 1, size=(rows, K)).astype(np.float32)
    x[:, rng.choice(K, size=8, replace=False)] *= 80.0
    x[2, 5] = 3e38
    bits = workloads.f32_to_bf16_bits(fit_exactness(x, 64))
    bits[3, 40] = 0x7FC0          # NaN
    bits[4, 70] = 0xFF80          # -Inf
    bits[5, :32] = 0x8000         # -0.0 block
    signed_zero_rows(rng, bits, 6, 0x0000, 0x8000, 0x3FC0)   # 0x3FC0: 1.5
    return bits


@pytest.mark.parametrize("size", [32, 64])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_rotated_activation_and_weight_bit_exact(dtype, size):
    rng = np.random.default_rng(41)
    M, N, K = 200, 72, 640
    if dtype == "bf16":
        xb = spiky_bf16(rng, M, K)
        wb = workloads.f32_to_bf16_bits(fit_exactness(rng.normal(0, 0.02, (N, K)), 64))
        xd, wd = dev_bf16(xb), dev_bf16(wb)
        x64, w64 = oracle.bf16_bits_to_f64(xb), oracle.bf16_bits_to_f64(wb)
    else:
        x = heavy_f32(rng, M, K)
        x[1, :64] = np.float32(1e-40) * (1 + np.arange(64))   # blocks of fp32 subnormals
        x[7, 100] = np.nan
        x = fit_exactness(x, 64)
        w = fit_exactness(rng.normal(0, 0.02, (N, K)) * np.exp(rng.uniform(-30, 3, (N, 1))), 64)
        xd, wd = dev_f32(x), dev_f32(w)
        x64, w64 = x.astype(np.float64), w.astype(np.float64)
    assert_exactness(x64, size)
    assert_exactness(w64, size)
    log(f"[rotate] rotated quantize {dtype}, size {size}")
    got_x = rfq.rotate_residual_quantize(xd, size)
    got_w = rfq.rotate_quantize_weight(wd, size)
    torch.cuda.synchronize()
    check_rfq(got_x, oracle.rotate_residual_quantize(x64, size), f"rotated X {dtype} n={size}")
    check_mx(got_w, oracle.rotate_quantize_weight(w64, size), f"rotated W {dtype} n={size}")


def sylvester(n):
    return np.array([[-1.0 if bin(i & j).count("1") % 2 else 1.0 for j in range(n)] for i in range(n)])


def near_tie_blocks(rng, rows, K, weight=False, size=32):
    """Blocks whose rotated values sit within about an ulp of E2M1 rounding
    ties: V holds a 4 (which fixes the scale) and tie values (0.25, 0.75, ...,
    5) times 2^se, D perturbs them by up to 2^-21, and the input is
    (V + D) H / 32 (or (V + D) H for a weight, whose side divides by 32)
    rounded to float32, which leaves every value with a full significand.
    Rounding the rotated sums along the way (a float32 butterfly) moves
    thousands of them across a tie; only the exact sum rounded once lands
    where the oracle does."""
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    nb = rows * K // size
    V = rng.choice(ties, size=(nb, size)) * rng.choice([-1, 1], size=(nb, size))
    V[:, ::32] = 4.0                          # a 4 in each MX block fixes its scale
    se = rng.integers(-10, 10, size=(nb, 1)).astype(np.float64)
    D = rng.uniform(-1, 1, size=(nb, size)) * 2.0 ** -21
    X = ((V + D) @ sylvester(size)) * np.exp2(se) / (1.0 if weight else float(size))
    return fit_exactness(X, size).reshape(rows, K)


@pytest.mark.parametrize("size", [32, 64])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_rotation_is_the_exact_sum_rounded_once(dtype, size):
    """Every rotated value must be the exact block sum rounded once to
    float32: on near-tie blocks the codes of the order-free oracle differ in
    hundreds (bf16) to thousands (fp32) of bytes from those a float32
    butterfly gives (checked on the CPU), so only an exact-then-round kernel
    passes. Every block's terms lie within 53 bits, the kernel's exactness
    condition (asserted)."""
    rng = np.random.default_rng((45 if dtype == "fp32" else 46) + size)
    M, N, K = 96, 64, 512
    x, w = near_tie_blocks(rng, M, K, size=size), near_tie_blocks(rng, N, K, weight=True, size=size)
    if dtype == "fp32":
        xd, wd, x64, w64 = dev_f32(x), dev_f32(w), x.astype(np.float64), w.astype(np.float64)
    else:
        xb, wb = workloads.f32_to_bf16_bits(x), workloads.f32_to_bf16_bits(w)
        xd, wd, x64, w64 = dev_bf16(xb), dev_bf16(wb), oracle.bf16_bits_to_f64(xb), oracle.bf16_bits_to_f64(wb)
    assert_exactness(x64, size)
    assert_exactness(w64, size)
    log(f"[rotate] near-tie blocks, {dtype}, size {size}")
    got_x = rfq.rotate_residual_quantize(xd, size)
    got_w = rfq.rotate_quantize_weight(wd, size)
    torch.cuda.synchronize()
    check_rfq(got_x, oracle.rotate_residual_quantize(x64, size), f"rotated X {dtype} n={size}")
    check_mx(got_w, oracle.rotate_quantize_weight(w64, size), f"rotated W {dtype} n={size}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("size,rows,K,pad", [(32, 1, 32, 0), (32, 3, 32, 8), (32, 67, 32, 24), (32, 5, 96, 40),
                                             (32, 129, 224, 8), (64, 1, 64, 0), (64, 3, 64, 8), (64, 67, 64, 24),
                                             (64, 5, 192, 40), (64, 129, 256, 8), (64, 1001, 128, 0)])
def test_rotated_strided_and_ragged(dtype, size, rows, K, pad):
    """One block per lane, 64 per wave: fewer blocks than a wave, a ragged
    last wave, K = 32 (a wave's blocks spread over 64 rows), and rows
    padded past K (ldx = K + pad, pad a multiple of 8 elements)."""
    rng = np.random.default_rng(1000 + rows + K + pad)
    ldx = K + pad
    full = heavy_f32(rng, rows, ldx) if rows > 1 else rng.normal(0, 3, (1, ldx)).astype(np.float32)
    full = np.concatenate([fit_exactness(full[:, :K], size), full[:, K:]], axis=1)
    log(f"[rotate] strided {dtype} n={size} rows={rows} K={K} ldx={ldx}")
    if dtype == "bf16":
        bits = workloads.f32_to_bf16_bits(full)
        xd = dev_bf16(bits)
        x64 = oracle.bf16_bits_to_f64(bits[:, :K])
    else:
        xd = dev_f32(full)
        x64 = full[:, :K].astype(np.float64)
    view = xd[:, :K]
    assert view.stride(0) == ldx
    assert_exactness(x64, size)
    got_x = rfq.rotate_residual_quantize(view, size)
    got_w = rfq.rotate_quantize_weight(view, size)
    torch.cuda.synchronize()
    check_rfq(got_x, oracle.rotate_residual_quantize(x64, size), f"strided rotated X {dtype} n={size}")
    check_mx(got_w, oracle.rotate_quantize_weight(x64, size), f"strided rotated W {dtype} n={size}")


@pytest.mark.parametrize("size,M,N,K", [(32, 130, 200, 512), (32, 64, 96, 160), (64, 130, 200, 512), (64, 64, 96, 192)])
def test_rotated_layer_every_output(size, M, N, K):
    """Q(XH), Q(R) and Q(WH/32) from the GPU into the unchanged W4A4 GEMM;
    Y against the oracle's rotated layer, and the rotation's effect on the
    error against the float64 product X W^T logged beside plain RFQ's."""
    rng = np.random.default_rng(M + N + K)
    x = rng.standard_t(3, size=(M, K))
    x[:, rng.choice(K, size=4, replace=False)] *= 60
    xb = workloads.f32_to_bf16_bits(fit_exactness(x, 64))
    wb = workloads.f32_to_bf16_bits(fit_exactness(rng.normal(0, 0.02, (N, K)), 64))
    log(f"[rotate] rotated layer {M}x{N}x{K}, size {size}")
    xd, wd = dev_bf16(xb), dev_bf16(wb)
    qx, sx, qr, sr = rfq.rotate_residual_quantize(xd, size)
    wq, sw = rfq.rotate_quantize_weight(wd, size)
    y = host(rfq.gemm_w4a4(qx, sx, qr, sr, wq, sw, out_dtype=torch.float32)).astype(np.float64)
    x64, w64 = oracle.bf16_bits_to_f64(xb), oracle.bf16_bits_to_f64(wb)
    assert_exactness(x64, size)
    assert_exactness(w64, size)
    y_ref, s_ref, (_, osx, _, osr), (_, osw) = oracle.linear_rotated(x64, w64, size)
    worst = check_y(y, y_ref, s_ref, torch.float32, "rotated layer")
    cov = check_exact_where_covered(y, y_ref, s_ref, [(osx, osw), (osr, osw)], torch.float32, "rotated layer")
    log(f"   sums exact in fp32 at {100 * cov:.1f}% of the outputs, each bit-equal to the exact sum")
    exact = x64 @ w64.T
    y_plain, _, _, _ = oracle.linear(x64, w64)
    err = lambda a: float(np.linalg.norm(a - exact) / np.linalg.norm(exact))
    log(f"   max |dY|/S = {worst:.2e}; relative error vs X W^T: rotated RFQ {err(y):.3e}, plain RFQ {err(y_plain):.3e}")


_FULL_X = {}


def full_x(name):
    """The configuration's full bf16 X (generated once per module)."""
    if name not in _FULL_X:
        _FULL_X.clear()
        _FULL_X[name] = workloads.x_bf16(workloads.CONFIGS[name])
    return _FULL_X[name]


@pytest.mark.parametrize("name,size", [("wan22_ffn", 32), ("wan22_ffn", 64), ("dit_ffn_down", 32), ("dit_ffn_down", 64)])
def test_rotated_full_size_sampled(name, size):
    """A configuration's full X through the rotated activation pass (the
    launches the benchmark's rotated lines time: 4096 x 5120 and
    32768 x 13824) and its full W through the rotated weight pass; sampled
    rows bit-exact. The workload's own values, checked against the
    exactness condition, not adjusted."""
    cfg = workloads.CONFIGS[name]
    log(f"[rotate] full size {cfg.name}, size {size}")
    xb = full_x(name)
    qx, sx, qr, sr = rfq.rotate_residual_quantize(dev_bf16(xb), size)
    wb = workloads.w_bf16(cfg)
    wq, sw = rfq.rotate_quantize_weight(dev_bf16(wb), size)
    torch.cuda.synchronize()
    rows = workloads.sample_rows(cfg, n_random=62)
    x64 = oracle.bf16_bits_to_f64(xb[rows])
    assert_exactness(x64, size)
    want = oracle.rotate_residual_quantize(x64, size)
    got = tuple(t[torch.from_numpy(rows).cuda()] for t in (qx, sx, qr, sr))
    check_rfq(got, want, f"rotated {name} rows n={size}")
    wrows = np.unique(np.concatenate([[0, cfg.N - 1], np.random.default_rng(cfg.seed + 7).choice(cfg.N, 62, replace=False)]))
    w64 = oracle.bf16_bits_to_f64(wb[wrows])
    assert_exactness(w64, size)
    gw = tuple(t[torch.from_numpy(wrows).cuda()] for t in (wq, sw))
    check_mx(gw, oracle.rotate_quantize_weight(w64, size), f"rotated {name} W rows n={size}")
