"""RFQ W4A4 GEMM and linear layer (oracle; test use only).

"Activation Outliers Matter: Robust Recovery for Quantized Multimodal LLMs",
§1 (contributions): the residual's quantized copy is multiplied during the
GEMM and its contribution accumulated with the primary product. Written as
one contraction over a doubled K:

    Y = [deq Q(X) | deq Q(R)] . [deq Wq | deq Wq]^T

with W [N, K] quantized to MXFP4 along K once (the weight gets no residual
pass). The contraction is a float64 library matmul of the decoded matrices;
every product of two E2M1 values times two E8M0 scales is exact in float64,
so the only rounding is float64 summation (relative 1e-12 of the condition
scale at these sizes), far below the 1e-5 comparison tolerance.
"""

import numpy as np

from .quantize import dequantize, quantize_mxfp4, residual_quantize


def gemm_w4a4(qx, sx, qr, sr, wq, sw):
    """Y and its condition scale S for MXFP4 operands (unpacked codes).

    qx [M, K], sx [M, K/32]: Q(X); qr, sr: Q(R), or None for plain W4A4;
    wq [N, K], sw [N, K/32]: the quantized weight. Returns (Y, S), float64
    [M, N], with S = sum over both products of |term|, the scale against
    which an fp32-accumulated result is compared.
    """
    a = dequantize(qx, sx)
    w = dequantize(wq, sw)
    if qr is not None:
        a = np.concatenate([a, dequantize(qr, sr)], axis=1)
        w = np.concatenate([w, w], axis=1)
    y = a @ w.T
    s = np.abs(a) @ np.abs(w).T
    return y, s


def linear(x, w):
    """Full RFQ linear on float64 X [M, K] and W [N, K]: returns
    (Y, S, (qx, sx, qr, sr), (wq, sw))."""
    wq, sw = quantize_mxfp4(w)
    qx, sx, qr, sr = residual_quantize(x)
    y, s = gemm_w4a4(qx, sx, qr, sr, wq, sw)
    return y, s, (qx, sx, qr, sr), (wq, sw)
