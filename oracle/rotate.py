"""Block-Hadamard rotation before MXFP4 and the RFQ residual (oracle; test use only).

The rotation follows "大模型量化中的双线性尾部问题与QuaRot正交旋转解决方案" §3
(QuaRot): an orthogonal transform made of +1/-1 entries (a Hadamard matrix),
applied online to the activation right before it is quantized and folded into
the weight offline, spreads an outlier's magnitude over the coordinates it is
mixed with; being orthogonal, it leaves the layer's product unchanged, and it
needs only additions and subtractions.

Reading taken here (the page describes per-head rotations of size 64 for a
per-token INT4 scheme; MX quantization scales per 32-element block):

* the rotation is block diagonal along K with one 32 x 32 Sylvester Hadamard
  block per MX block, H[i, j] = (-1)^popcount(i & j), unnormalised;
* the activation side quantizes X H, the weight side W H / 32, so that
  (X H)(W H / 32)^T = X (H H^T / 32) W^T = X W^T, because H H^T = 32 I; the
  1/32 is a power of two and costs no rounding;
* X H is formed in float32 by the fast transform: five butterfly passes with
  spans 1, 2, 4, 8, 16, each replacing (a, b) at positions (i, i + span),
  i & span == 0, by (a + b, a - b). The quantization codes are decided on these
  float32 values, in the precision the kernel computes them, so the pass order
  is part of the definition. Everything after the rotation is the plain
  oracle (``quantize_mxfp4`` / ``residual_quantize``) on those values; the
  residual is exact there (see ``residual_quantize``).
"""

import numpy as np

from .formats import BLOCK
from .quantize import quantize_mxfp4, residual_quantize

_SPANS = (1, 2, 4, 8, 16)
_WEIGHT_SCALE = np.float32(1.0 / BLOCK)      # 2^-5, exact


def hadamard32_f32(x):
    """Per-32-block Walsh-Hadamard transform along the last axis, in float32.

    ``x`` [..., K] (K a multiple of 32) is converted to float32 and each block
    of 32 is transformed by the butterfly passes listed in the module
    docstring. Returns float32 of the same shape.
    """
    v = np.array(x, dtype=np.float32, copy=True)
    if v.shape[-1] % BLOCK:
        raise ValueError("the last axis must be a multiple of 32")
    lead = v.shape[:-1]
    b = v.reshape(*lead, v.shape[-1] // BLOCK, BLOCK)
    for span in _SPANS:
        # positions i with bit `span` clear pair with i + span
        lo = np.array([i for i in range(BLOCK) if not i & span])
        a, c = b[..., lo].copy(), b[..., lo + span].copy()
        b[..., lo] = a + c
        b[..., lo + span] = a - c
    return b.reshape(v.shape)


def rotate_residual_quantize(x):
    """RFQ encoding of the rotated activation X H (``x`` [M, K], values exactly
    representable in float32, e.g. decoded bfloat16): returns (qx, sx, qr, sr)
    as ``residual_quantize`` does."""
    v = hadamard32_f32(x).astype(np.float64)
    return residual_quantize(v)


def rotate_quantize_weight(w):
    """MXFP4 codes and scales of the rotated weight W H / 32 (``w`` [N, K])."""
    v = (hadamard32_f32(w) * _WEIGHT_SCALE).astype(np.float64)
    return quantize_mxfp4(v)


def linear_rotated(x, w):
    """The rotated RFQ linear layer on float64 X [M, K] and W [N, K] whose
    values are exact in float32: Y = Q(XH) Q(WH/32)^T + Q(R) Q(WH/32)^T with
    R = XH - deq Q(XH). Returns (Y, S, (qx, sx, qr, sr), (wq, sw))."""
    from .gemm import gemm_w4a4
    wq, sw = rotate_quantize_weight(w)
    qx, sx, qr, sr = rotate_residual_quantize(x)
    y, s = gemm_w4a4(qx, sx, qr, sr, wq, sw)
    return y, s, (qx, sx, qr, sr), (wq, sw)
