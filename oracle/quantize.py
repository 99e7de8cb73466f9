"""MXFP4 quantization and the RFQ residual pass (oracle; test use only).

Follows, in order:

1. per row, per 32-element block along K: amax = max |x|;
2. shared scale exponent se = floor(log2(amax)) - 2 (OCP MX v1.0 rule, 2 being
   the largest E2M1 exponent), clamped below at -127; amax == 0 gives -127;
   a non-finite amax gives the NaN scale code 255;
3. each element: v = x * 2^-se, saturate |v| to 6, round to the nearest E2M1
   magnitude with ties to the even code, keep the sign bit of x;
4. "Activation Outliers Matter: Robust Recovery for Quantized Multimodal
   LLMs", §1 (RFQ paragraph): the residual is the full quantization error
   R = X - deq(Q(X)), with nothing thresholded or dropped, and it is quantized
   by a second low-bit path of the same format: Q(R). One residual pass.

All arithmetic is float64. For bfloat16 or float32 inputs every step above is
exact in float64 (the scaling is by a power of two, and R needs at most 25
significant bits), so the codes do not depend on rounding in the oracle.
Distances |a - G[i]| are exact whenever a >= 2^-26; below that a is far
under the first midpoint 0.25 and the ordering of the distances is still
right.
"""

import numpy as np

from .formats import BLOCK, E2M1_EMAX, E2M1_MAGNITUDES, E8M0_BIAS, E8M0_NAN, e8m0_value

_MIN_SE = -E8M0_BIAS        # smallest E8M0 exponent, 2^-127
_CHUNK = 1 << 18            # elements per vectorised slice (bounds memory only)


def scale_exponent(amax):
    """Shared-scale exponent and E8M0 code for block maxima ``amax`` (float64, >= 0).

    Returns (se, code): se = max(floor(log2 amax) - 2, -127) with floor(log2)
    taken exactly from frexp (amax = f * 2^e, f in [0.5, 1) gives
    floor(log2 amax) = e - 1); amax == 0 gives se = -127; non-finite amax gives
    code 255 (se is then meaningless and returned as 0).
    """
    amax = np.asarray(amax, dtype=np.float64)
    finite = np.isfinite(amax)
    safe = np.where(finite, amax, 1.0)
    _, e = np.frexp(safe)
    se = np.maximum(e.astype(np.int64) - 1 - E2M1_EMAX, _MIN_SE)
    se = np.where(safe == 0.0, _MIN_SE, se)
    se = np.where(finite, se, 0)
    code = np.where(finite, se + E8M0_BIAS, E8M0_NAN).astype(np.uint8)
    return se, code


def encode_block_elements(x, se):
    """E2M1 codes (uint8, 0..15) for float64 values ``x`` at scale exponents ``se``.

    ``se`` broadcasts against ``x``. v = x * 2^-se; a = min(|v|, 6); the code
    magnitude is the index of the nearest entry of the E2M1 magnitude list,
    and when two entries are equally near (a midpoint) the even index wins
    (round half to even on the 1-bit mantissa). The sign bit of x becomes bit 3,
    so -0.0 and small negatives that round to zero give code 8.
    """
    x = np.asarray(x, dtype=np.float64)
    se = np.broadcast_to(np.asarray(se, dtype=np.int64), x.shape)
    flat_x = x.reshape(-1)
    flat_se = se.reshape(-1)
    out = np.empty(flat_x.shape, dtype=np.uint8)
    even = (np.arange(8) % 2) == 0
    for s in range(0, flat_x.size, _CHUNK):
        xv = flat_x[s:s + _CHUNK]
        v = np.ldexp(xv, -flat_se[s:s + _CHUNK])
        a = np.minimum(np.abs(v), 6.0)
        d = np.abs(a[:, None] - E2M1_MAGNITUDES[None, :])
        nearest = d == d.min(axis=1, keepdims=True)
        even_nearest = nearest & even[None, :]
        idx = np.where(even_nearest.any(axis=1), np.argmax(even_nearest, axis=1),
                       np.argmax(nearest, axis=1))
        out[s:s + _CHUNK] = (np.signbit(xv).astype(np.uint8) << 3) | idx.astype(np.uint8)
    return out.reshape(x.shape)


def quantize_mxfp4(x):
    """Quantize float64 ``x`` [rows, K] to MXFP4 along K.

    Returns (codes, scales): codes uint8 [rows, K] holding one 4-bit code per
    element (unpacked), scales uint8 [rows, K/32] E8M0 codes. A block holding a
    NaN or an infinity gets scale code 255 and element codes 0.
    """
    x = np.asarray(x, dtype=np.float64)
    rows, K = x.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    xb = x.reshape(rows, K // BLOCK, BLOCK)
    finite = np.isfinite(xb).all(axis=2)
    amax = np.where(finite, np.abs(np.where(np.isfinite(xb), xb, 0.0)).max(axis=2), np.inf)
    se, scode = scale_exponent(amax)
    codes = encode_block_elements(np.where(finite[:, :, None], xb, 0.0), se[:, :, None])
    codes = np.where(finite[:, :, None], codes, 0).astype(np.uint8)
    return codes.reshape(rows, K), scode


def dequantize(codes, scales):
    """float64 values of unpacked codes [rows, K] with E8M0 scales [rows, K/32]."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows, K = codes.shape
    mag = E2M1_MAGNITUDES[codes & 7]
    val = np.where((codes >> 3) & 1, -mag, mag)
    sc = e8m0_value(np.asarray(scales))
    return (val.reshape(rows, K // BLOCK, BLOCK) * sc[:, :, None]).reshape(rows, K)


def residual_quantize(x):
    """RFQ activation encoding of float64 ``x`` [M, K].

    Returns (qx, sx, qr, sr): Q(X) and Q(R) as unpacked codes and E8M0 scales,
    with R = X - deq(Q(X)) computed exactly in float64.
    """
    x = np.asarray(x, dtype=np.float64)
    qx, sx = quantize_mxfp4(x)
    r = x - dequantize(qx, sx)
    qr, sr = quantize_mxfp4(r)
    return qx, sx, qr, sr


def pack_codes(codes):
    """Pack unpacked codes [rows, K] into bytes [rows, K/2]: byte j holds element
    2j in its low nibble and element 2j+1 in its high nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] & 0xF) | ((c[:, 1::2] & 0xF) << 4)


def unpack_codes(packed):
    """Inverse of :func:`pack_codes`."""
    p = np.asarray(packed, dtype=np.uint8)
    rows, half = p.shape
    out = np.empty((rows, 2 * half), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out
