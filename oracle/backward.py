"""Backward pass of the RFQ linear layer under the straight-through estimator (oracle; test use only).

"Activation Outliers Matter: Robust Recovery for Quantized Multimodal LLMs",
§1: RFQ is meant for training ("fully differentiable and training-aware"
error modelling, low-bit training of MLLMs), but the pages do not write
out the backward pass. The reading taken here is the plain
straight-through one:

* the forward value is Y = Xh Wd^T with Xh = deq Q(X) + deq Q(R) and
  Wd = deq Q(W) (the RFQ layer's own operands);
* Q passes gradients through unchanged. Then d Xh / d X = I; and since
  R = X - deq Q(X), dR/dX = I - I = 0, so the residual path adds nothing
  beyond that identity;
* hence dX = dY Wd (contracting over the N outputs), and
  dW = dY^T Xh = dY^T deq Q(X) + dY^T deq Q(R) (contracting over the M
  tokens), the weight gradient taken at the quantized activations the
  forward pass used.

Both products are plain float64 library matmuls of the decoded operands;
for bfloat16 dY every product is exact in float64 and the only rounding is
float64 summation. S is the matching sum of |terms|.
"""

import numpy as np

from .quantize import dequantize, quantize_mxfp4, residual_quantize


def backward_dx(dy, wq, sw):
    """dX = dY deq(Wq) and its condition scale, for dy [M, N] float64 and the
    weight's MXFP4 codes wq [N, K] (unpacked) and scales sw [N, K/32]."""
    wd = dequantize(wq, sw)
    dy = np.asarray(dy, dtype=np.float64)
    return dy @ wd, np.abs(dy) @ np.abs(wd)


def backward_dw(dy, qx, sx, qr, sr):
    """dW = dY^T (deq Q(X) + deq Q(R)) as the K-doubled contraction
    [dY^T | dY^T] . [deq Q(X) ; deq Q(R)] over 2M, and its condition scale
    (sum of |terms| of both products)."""
    dy = np.asarray(dy, dtype=np.float64)
    xq, xr = dequantize(qx, sx), dequantize(qr, sr)
    dw = dy.T @ xq + dy.T @ xr
    s = np.abs(dy).T @ np.abs(xq) + np.abs(dy).T @ np.abs(xr)
    return dw, s


def linear_backward(dy, x, w):
    """The whole straight-through backward of the RFQ layer on float64 X
    [M, K], W [N, K] and dY [M, N]: returns (dX, S_dX, dW, S_dW), using the
    same encodings as the forward pass."""
    wq, sw = quantize_mxfp4(w)
    qx, sx, qr, sr = residual_quantize(x)
    dx, sdx = backward_dx(dy, wq, sw)
    dw, sdw = backward_dw(dy, qx, sx, qr, sr)
    return dx, sdx, dw, sdw
