"""MXFP8 (E4M3) quantization and the layer variants built on it (oracle; test use only).

"Activation Outliers Matter: Robust Recovery for Quantized Multimodal LLMs",
Abstract and §1 (contributions): MXFP8 is studied beside the 4-bit formats
and found close to lossless, while the 4-bit loss is traced mainly to the
activations. The pages name MXFP8 without defining it; the definitions here
are the OCP Microscaling Formats (MX) v1.0 ones for MXFP8 with E4M3 elements:

* E4M3 element: bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa.
  Exponent field 0 is subnormal: value = m/8 * 2^-6. Otherwise
  value = 2^(e - 7) * (1 + m/8), except e = 15, m = 7, which is NaN. No
  infinities. The largest normal is 448 = 1.75 * 2^8, so emax = 8.
* Block and scale as for MXFP4: 32 elements along K share an E8M0 scale,
  se = max(floor(log2 amax) - 8, -127).
* Element rule: v = x * 2^-se, rounded to the nearest E4M3 value with ties to
  the even code, saturating at +-448 (values past the largest normal clamp to
  it rather than becoming NaN).

Variants (readings of the pages; each keeps the weight in MXFP4):

* W4A8: the activation in MXFP8, no residual; Y = deq Q8(X) . deq Q4(W)^T.
* RFQ with an MXFP8 residual path: Q4(X) as in plain RFQ,
  R = X - deq Q4(X) (exact), and R quantized to MXFP8 by the second path;
  Y = deq Q4(X) . deq Q4(W)^T + deq Q8(R) . deq Q4(W)^T.

All arithmetic is float64 and exact for bfloat16/float32 inputs (scaling by
2^-se is exact, and every E4M3 value and every midpoint between neighbours
needs at most 5 significant bits).
"""

import numpy as np

from .formats import BLOCK, E8M0_BIAS, E8M0_NAN, e8m0_value
from .quantize import dequantize, quantize_mxfp4

E4M3_BIAS = 7
E4M3_EMAX = 8           # exponent of the largest normal, 448 = 1.75 * 2^8
E4M3_MAX = 448.0
E4M3_NAN_CODE = 0x7F    # S.1111.111


def e4m3_value(code: int) -> float:
    """Value of an 8-bit E4M3 code, from its sign/exponent/mantissa fields."""
    code = int(code) & 0xFF
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        mag = (m / 8.0) * 2.0 ** (1 - E4M3_BIAS)
    else:
        mag = 2.0 ** (e - E4M3_BIAS) * (1.0 + m / 8.0)
    return -mag if s else mag


# Magnitudes of the finite non-negative codes 0..126 (ascending in the code).
E4M3_MAGNITUDES = np.array([e4m3_value(c) for c in range(E4M3_NAN_CODE)], dtype=np.float64)


def scale_exponent_e4m3(amax):
    """Shared-scale exponent and E8M0 code for block maxima ``amax`` under
    MXFP8: se = max(floor(log2 amax) - 8, -127); amax == 0 gives -127; a
    non-finite amax gives code 255 (se returned as 0)."""
    amax = np.asarray(amax, dtype=np.float64)
    finite = np.isfinite(amax)
    safe = np.where(finite, amax, 1.0)
    _, e = np.frexp(safe)                        # safe = f * 2^e, f in [0.5, 1)
    se = np.maximum(e.astype(np.int64) - 1 - E4M3_EMAX, -E8M0_BIAS)
    se = np.where(safe == 0.0, -E8M0_BIAS, se)
    se = np.where(finite, se, 0)
    code = np.where(finite, se + E8M0_BIAS, E8M0_NAN).astype(np.uint8)
    return se, code


def encode_e4m3(x, se):
    """E4M3 codes (uint8) of float64 values ``x`` at scale exponents ``se``
    (broadcast against ``x``).

    v = x * 2^-se, a = min(|v|, 448); the two grid magnitudes around a are
    found by bisection of the ascending magnitude list, the nearer one is
    taken, and on a tie the even code (even mantissa) wins. The sign bit of x
    becomes bit 7, so -0.0 and negatives that round to zero give code 0x80.
    """
    x = np.asarray(x, dtype=np.float64)
    se = np.broadcast_to(np.asarray(se, dtype=np.int64), x.shape)
    a = np.minimum(np.abs(np.ldexp(x, -se)), E4M3_MAX)
    hi = np.minimum(np.searchsorted(E4M3_MAGNITUDES, a, side="left"), len(E4M3_MAGNITUDES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - E4M3_MAGNITUDES[lo]
    d_hi = E4M3_MAGNITUDES[hi] - a
    pick = np.where(d_hi < d_lo, hi, np.where(d_lo < d_hi, lo, np.where(hi % 2 == 0, hi, lo)))
    return ((np.signbit(x).astype(np.uint8) << 7) | pick.astype(np.uint8)).astype(np.uint8)


def quantize_mxfp8(x):
    """Quantize float64 ``x`` [rows, K] to MXFP8 (E4M3) along K.

    Returns (codes, scales): codes uint8 [rows, K], one E4M3 code per element;
    scales uint8 [rows, K/32] E8M0 codes. A block holding a NaN or an infinity
    gets scale code 255 and element codes 0.
    """
    x = np.asarray(x, dtype=np.float64)
    rows, K = x.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    xb = x.reshape(rows, K // BLOCK, BLOCK)
    finite = np.isfinite(xb).all(axis=2)
    amax = np.where(finite, np.abs(np.where(np.isfinite(xb), xb, 0.0)).max(axis=2), np.inf)
    se, scode = scale_exponent_e4m3(amax)
    codes = encode_e4m3(np.where(finite[:, :, None], xb, 0.0), se[:, :, None])
    codes = np.where(finite[:, :, None], codes, 0).astype(np.uint8)
    return codes.reshape(rows, K), scode


def dequantize_mxfp8(codes, scales):
    """float64 values of E4M3 codes [rows, K] with E8M0 scales [rows, K/32]."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows, K = codes.shape
    mag = np.append(E4M3_MAGNITUDES, np.nan)[codes & 0x7F]
    val = np.where((codes >> 7) & 1, -mag, mag)
    sc = e8m0_value(np.asarray(scales))
    return (val.reshape(rows, K // BLOCK, BLOCK) * sc[:, :, None]).reshape(rows, K)


def residual_quantize_fp8(x):
    """RFQ activation encoding with an MXFP8 residual path, on float64 ``x``
    [M, K]: returns (qx, sx, qr8, sr) with Q4(X) as unpacked E2M1 codes and
    E8M0 scales, and Q8(R) as E4M3 codes and E8M0 scales, for
    R = X - deq Q4(X) computed exactly in float64."""
    x = np.asarray(x, dtype=np.float64)
    qx, sx = quantize_mxfp4(x)
    r = x - dequantize(qx, sx)
    qr8, sr = quantize_mxfp8(r)
    return qx, sx, qr8, sr


def gemm_w4a8(qx8, sx, wq, sw):
    """Y and its condition scale S (float64 [M, N]) for MXFP8 activation codes
    qx8 [M, K] / sx and MXFP4 weight codes wq [N, K] (unpacked) / sw: a
    float64 library matmul of the decoded matrices (every product is exact in
    float64; S = sum of |terms|)."""
    a = dequantize_mxfp8(qx8, sx)
    w = dequantize(wq, sw)
    return a @ w.T, np.abs(a) @ np.abs(w).T


def gemm_w4a4_fp8_residual(qx, sx, qr8, sr, wq, sw):
    """Y and S for RFQ with an MXFP8 residual: one contraction of
    [deq Q4(X) | deq Q8(R)] against [deq W ; deq W] over the doubled K."""
    a = np.concatenate([dequantize(qx, sx), dequantize_mxfp8(qr8, sr)], axis=1)
    w = dequantize(wq, sw)
    w2 = np.concatenate([w, w], axis=1)
    return a @ w2.T, np.abs(a) @ np.abs(w2).T


def linear_w4a8(x, w):
    """W4A8 layer on float64 X [M, K], W [N, K]: returns (Y, S, (qx8, sx), (wq, sw))."""
    wq, sw = quantize_mxfp4(w)
    qx8, sx = quantize_mxfp8(x)
    y, s = gemm_w4a8(qx8, sx, wq, sw)
    return y, s, (qx8, sx), (wq, sw)


def linear_fp8_residual(x, w):
    """RFQ layer with an MXFP8 residual on float64 X, W: returns
    (Y, S, (qx, sx, qr8, sr), (wq, sw))."""
    wq, sw = quantize_mxfp4(w)
    enc = residual_quantize_fp8(x)
    y, s = gemm_w4a4_fp8_residual(*enc, wq, sw)
    return y, s, enc, (wq, sw)
