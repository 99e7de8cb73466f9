"""Block-Hadamard rotation before MXFP4 and the RFQ residual (oracle; test use only).

The rotation follows "大模型量化中的双线性尾部问题与QuaRot正交旋转解决方案" §3
(QuaRot): an orthogonal transform made of +1/-1 entries (a Hadamard matrix),
applied online to the activation right before it is quantized and folded into
the weight offline, spreads an outlier's magnitude over the coordinates it is
mixed with; being orthogonal, it leaves the layer's product unchanged, and it
needs only additions and subtractions.

Reading taken here (the page describes per-head rotations of size 64 for a
per-token INT4 scheme; MX quantization scales per 32-element block):

* the rotation is block diagonal along K with one n x n Sylvester Hadamard
  block, H[i, j] = (-1)^popcount(i & j), unnormalised, either n = 32 (one
  block per MX block, the default) or n = 64 (the page's per-head size; one
  block per two adjacent MX blocks, so K must be a multiple of 64);
* the activation side quantizes X H, the weight side W H / n, so that
  (X H)(W H / n)^T = X (H H^T / n) W^T = X W^T, because H H^T = n I; the
  1/n is a power of two and costs no rounding;
* each rotated value is the exact sum (x H)[i] = sum_j H[j, i] x[j] over its
  block (divided by n on the weight side), rounded once to the nearest
  float32, ties to even, an exact zero being +0 (the sum of zeros has no
  sign of its own): a definition with no summation order in it. The
  quantization codes are decided on these float32 values (the precision the
  quantize pass computes in), then everything is the plain oracle
  (``quantize_mxfp4`` / ``residual_quantize``); the residual is exact there.

Computing the exact sum: when every term is a multiple of 2^L and the sum of
magnitudes is below 2^U with U - L <= 53, every partial sum in any order is
exact in float64, so a float64 matrix product gives the exact value (for
bfloat16 inputs this holds whenever the block's nonzero values span at most
40 binades for n = 32 and 39 for n = 64, for float32 ones 24 and 23). Blocks
outside that are summed as exact rationals and rounded to float32 directly.
"""

from fractions import Fraction

import numpy as np

from .formats import BLOCK
from .quantize import quantize_mxfp4, residual_quantize

ROTATION_SIZES = (32, 64)


def _sylvester(n):
    """Sylvester order: H[i, j] = (-1)^popcount(i & j)."""
    return np.array([[-1.0 if bin(i & j).count("1") % 2 else 1.0 for j in range(n)] for i in range(n)])


_HS = {n: _sylvester(n) for n in ROTATION_SIZES}


def _lsb_exponent(v):
    """Exponent of the lowest set bit of each finite nonzero float64 value
    (v = m 2^L with m odd); +inf where v == 0."""
    bits = np.abs(v).view(np.uint64)
    exp_field = ((bits >> np.uint64(52)) & np.uint64(0x7FF)).astype(np.int64)
    mant = bits & np.uint64((1 << 52) - 1)
    mant = np.where(exp_field > 0, mant | np.uint64(1 << 52), mant)
    low = mant & (~mant + np.uint64(1))                     # lowest set bit of the integer significand
    _, e = np.frexp(low.astype(np.float64))                 # low = 2^(e - 1)
    unbiased = np.where(exp_field > 0, exp_field - 1075, -1074)   # value = mant * 2^unbiased
    return np.where(v == 0, np.inf, unbiased + e - 1)


def fraction_to_f32(q):
    """The float32 nearest the rational q (ties to even), as a float64;
    +-inf past the largest float32 (rounding as IEEE does)."""
    if q == 0:
        return 0.0
    sign = -1.0 if q < 0 else 1.0
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()   # 2^(e-1) <= a < 2^(e+1)
    if Fraction(2) ** e <= a:
        e += 1
    # now 2^(e-1) <= a < 2^e; float32 keeps 24 bits, or fewer below 2^-126
    ulp_exp = max(e - 24, -149)
    n = a / Fraction(2) ** ulp_exp
    lo = n.numerator // n.denominator
    rem = n - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    val = lo * 2.0 ** ulp_exp
    if val >= 2.0 ** 128:
        return sign * np.inf
    return sign * val


def hadamard_rounded(x, size=32, divide=False):
    """Per-`size`-block Walsh-Hadamard transform along the last axis (size 32
    or 64): each output the exact block sum (times 1/size if ``divide``)
    rounded once to float32. ``x`` [..., K] holds finite or non-finite
    float64 values; a block with a NaN or an infinity gives NaN/inf outputs
    as float32 sums would. Returns float32 of the same shape."""
    if size not in ROTATION_SIZES:
        raise ValueError("the rotation size must be 32 or 64")
    H = _HS[size]
    v = np.asarray(x, dtype=np.float64)
    if v.shape[-1] % size:
        raise ValueError(f"the last axis must be a multiple of {size}")
    lead = v.shape[:-1]
    b = v.reshape(-1, size)
    with np.errstate(invalid="ignore", over="ignore"):
        prod = b @ H                                          # H is symmetric: row block times H
    if divide:
        prod = prod / float(size)                             # exact: a power of two
    prod = prod + 0.0                                         # an exact zero is +0
    finite = np.isfinite(b).all(axis=1)
    mag = np.abs(np.where(np.isfinite(b), b, 0.0)).sum(axis=1)
    L = _lsb_exponent(np.where(np.isfinite(b), b, 0.0)).min(axis=1)
    with np.errstate(divide="ignore"):
        U = np.floor(np.log2(np.where(mag > 0, mag, 1.0))) + 2   # sum of magnitudes < 2^U, with margin
    exact = ~finite | (mag == 0) | (U - L <= 53)
    out = prod.astype(np.float32)                             # one rounding of an exact value
    for r in np.nonzero(~exact)[0]:
        terms = [Fraction(float(t)) for t in b[r]]
        for i in range(size):
            q = sum(terms[j] if H[j, i] > 0 else -terms[j] for j in range(size))
            if divide:
                q /= size
            out[r, i] = np.float32(fraction_to_f32(q))
    return out.reshape(*lead, v.shape[-1])


def hadamard32_rounded(x, divide_by_32=False):
    """The 32-point case of ``hadamard_rounded``."""
    return hadamard_rounded(x, 32, divide_by_32)


def rotate_residual_quantize(x, size=32):
    """RFQ encoding of the rotated activation X H (``x`` [M, K], values exactly
    representable in float32, e.g. decoded bfloat16; H of ``size`` 32 or 64):
    returns (qx, sx, qr, sr) as ``residual_quantize`` does."""
    v = hadamard_rounded(x, size).astype(np.float64)
    return residual_quantize(v)


def rotate_quantize_weight(w, size=32):
    """MXFP4 codes and scales of the rotated weight W H / size (``w`` [N, K])."""
    v = hadamard_rounded(w, size, divide=True).astype(np.float64)
    return quantize_mxfp4(v)


def linear_rotated(x, w, size=32):
    """The rotated RFQ linear layer on float64 X [M, K] and W [N, K] whose
    values are exact in float32: Y = Q(XH) Q(WH/n)^T + Q(R) Q(WH/n)^T with
    R = XH - deq Q(XH), n = ``size``. Returns (Y, S, (qx, sx, qr, sr), (wq, sw))."""
    from .gemm import gemm_w4a4
    wq, sw = rotate_quantize_weight(w, size)
    qx, sx, qr, sr = rotate_residual_quantize(x, size)
    y, s = gemm_w4a4(qx, sx, qr, sr, wq, sw)
    return y, s, (qx, sx, qr, sr), (wq, sw)
