"""RFQ W4A4 linear layer for MI355X: Python binding of librfq.

Residual Fallback Quantization ("Activation Outliers Matter: Robust
Recovery for Quantized Multimodal LLMs", §1): X is quantized to MXFP4, the
full error R = X - deq(Q(X)) is quantized to MXFP4 again, and
Y = Q(X) Wq^T + Q(R) Wq^T is one K-doubled block-scaled FP4 GEMM.

MXFP8 variants (E4M3 elements): W4A8 (activation in MXFP8, no residual) and
RFQ whose second path quantizes R to MXFP8; the weight stays MXFP4.

This module only marshals torch tensors (device memory and the current HIP
stream) into the C ABI of include/rfq.h; every step runs in the HIP kernels of
librfq.so. Nothing falls back to CPU or PyTorch compute: if the library is
missing, the calls raise.
"""
import ctypes

import torch

from ._lib import DTYPE_BF16, DTYPE_FP32, RfqError, check, load

__all__ = [
    "RfqError",
    "quantize_mxfp4",
    "residual_quantize",
    "gemm_w4a4",
    "rotate_residual_quantize",
    "rotate_quantize_weight",
    "quantize_mxfp8",
    "residual_quantize_mxfp8",
    "gemm_w4a8",
    "gemm_w4a4_mxfp8_residual",
    "backward_dx",
    "backward_dw",
    "linear",
    "linear_workspace_size",
    "library",
]


def library():
    """The loaded ctypes library (raises if librfq.so is not built)."""
    return load()


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _x_args(x):
    """(rows, K, ldx, dtype code) of a 2-D bf16 or fp32 CUDA tensor with unit stride along K."""
    if x.dtype not in (torch.bfloat16, torch.float32) or x.dim() != 2 or not x.is_cuda:
        raise ValueError("x must be a 2-D bfloat16 or float32 CUDA tensor")
    if x.stride(1) != 1:
        raise ValueError("x must have unit stride along K")
    return x.shape[0], x.shape[1], x.stride(0), (DTYPE_BF16 if x.dtype == torch.bfloat16 else DTYPE_FP32)


def _y_dtype(out_dtype):
    if out_dtype == torch.float32:
        return DTYPE_FP32
    if out_dtype == torch.bfloat16:
        return DTYPE_BF16
    raise ValueError("out_dtype must be torch.float32 or torch.bfloat16")


def _quantize(fn, x, bytes_per_element=0.5):
    rows, K, ldx, dt = _x_args(x)
    codes = torch.empty((rows, int(K * bytes_per_element)), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, K // 32), dtype=torch.uint8, device=x.device)
    check(fn(_ptr(x), dt, rows, K, ldx, _ptr(codes), _ptr(scales), _stream()))
    return codes, scales


def _residual(fn, x, r_bytes_per_element=0.5):
    M, K, ldx, dt = _x_args(x)
    qx = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    qr = torch.empty((M, int(K * r_bytes_per_element)), dtype=torch.uint8, device=x.device)
    sx = torch.empty((M, K // 32), dtype=torch.uint8, device=x.device)
    sr = torch.empty_like(sx)
    check(fn(_ptr(x), dt, M, K, ldx, _ptr(qx), _ptr(sx), _ptr(qr), _ptr(sr), _stream()))
    return qx, sx, qr, sr


def quantize_mxfp4(x):
    """MXFP4 along K of bf16 or fp32 X: returns (codes uint8 [rows, K/2], scales uint8 [rows, K/32])."""
    return _quantize(load().rfq_quantize_mxfp4, x)


def residual_quantize(x):
    """RFQ encoding of X: returns (qx, sx, qr, sr) = Q(X) codes/scales, Q(R) codes/scales."""
    return _residual(load().rfq_residual_quantize, x)


def rotate_residual_quantize(x):
    """RFQ encoding of X H (32-point block Hadamard along K): (qx, sx, qr, sr)."""
    return _residual(load().rfq_rotate_residual_quantize, x)


def rotate_quantize_weight(w):
    """MXFP4 codes and scales of W H / 32, the weight side of the rotated layer."""
    return _quantize(load().rfq_rotate_quantize_weight, w)


def _codes_ok(*ts):
    for t in ts:
        if t is not None and (t.dtype != torch.uint8 or not t.is_contiguous() or not t.is_cuda):
            raise ValueError("codes and scales must be contiguous uint8 CUDA tensors")


def _out(y, M, N, out_dtype, device):
    y = y if y is not None else torch.empty((M, N), dtype=out_dtype, device=device)
    if y.stride(1) != 1:
        raise ValueError("out must have unit stride along N")
    return y


def gemm_w4a4(qx, sx, qr, sr, wq, sw, out_dtype=torch.bfloat16, out=None):
    """Y = deq(QX) deq(W)^T + deq(QR) deq(W)^T (qr = sr = None: plain W4A4)."""
    M, N, K = qx.shape[0], wq.shape[0], qx.shape[1] * 2
    _codes_ok(qx, sx, qr, sr, wq, sw)
    if wq.shape[1] * 2 != K:
        raise ValueError("QX and W disagree on K")
    y = _out(out, M, N, out_dtype, qx.device)
    check(load().rfq_gemm_w4a4(_ptr(qx), _ptr(sx), _ptr(qr), _ptr(sr), _ptr(wq), _ptr(sw), M, N, K, _ptr(y),
                               _y_dtype(y.dtype), y.stride(0), _stream()))
    return y


def quantize_mxfp8(x):
    """MXFP8 (E4M3) along K of bf16 or fp32 X: (codes uint8 [rows, K], scales uint8 [rows, K/32])."""
    return _quantize(load().rfq_quantize_mxfp8, x, bytes_per_element=1)


def residual_quantize_mxfp8(x):
    """RFQ encoding with an MXFP8 second path: (qx [M, K/2], sx, qr8 [M, K], sr)."""
    return _residual(load().rfq_residual_quantize_mxfp8, x, r_bytes_per_element=1)


def gemm_w4a8(qx8, sx, wq, sw, out_dtype=torch.bfloat16, out=None):
    """Y = deq(QX8) deq(W)^T for MXFP8 activation codes and the MXFP4 weight."""
    M, N, K = qx8.shape[0], wq.shape[0], qx8.shape[1]
    _codes_ok(qx8, sx, wq, sw)
    if wq.shape[1] * 2 != K:
        raise ValueError("QX and W disagree on K")
    y = _out(out, M, N, out_dtype, qx8.device)
    check(load().rfq_gemm_w4a8(_ptr(qx8), _ptr(sx), _ptr(wq), _ptr(sw), M, N, K, _ptr(y), _y_dtype(y.dtype),
                               y.stride(0), _stream()))
    return y


def gemm_w4a4_mxfp8_residual(qx, sx, qr8, sr, wq, sw, out_dtype=torch.bfloat16, out=None):
    """Y = deq(QX) deq(W)^T + deq(QR8) deq(W)^T, QX MXFP4 and QR8 MXFP8."""
    M, N, K = qx.shape[0], wq.shape[0], qx.shape[1] * 2
    _codes_ok(qx, sx, qr8, sr, wq, sw)
    if wq.shape[1] * 2 != K or qr8.shape[1] != K:
        raise ValueError("operands disagree on K")
    y = _out(out, M, N, out_dtype, qx.device)
    check(load().rfq_gemm_w4a4_mxfp8_residual(_ptr(qx), _ptr(sx), _ptr(qr8), _ptr(sr), _ptr(wq), _ptr(sw), M, N, K,
                                              _ptr(y), _y_dtype(y.dtype), y.stride(0), _stream()))
    return y


def _dy_args(dy):
    if dy.dtype != torch.bfloat16 or dy.dim() != 2 or not dy.is_cuda or dy.stride(1) != 1:
        raise ValueError("dy must be a 2-D bfloat16 CUDA tensor with unit stride along N")
    return dy.shape[0], dy.shape[1], dy.stride(0)


def backward_dx(dy, wq, sw, out_dtype=torch.float32, out=None, workspace=None):
    """Straight-through dX = dY deq(Wq) for bf16 dY [M, N] (dense) and the
    weight's MXFP4 codes/scales; returns dX [M, K]."""
    M, N, lddy = _dy_args(dy)
    _codes_ok(wq, sw)
    K = wq.shape[1] * 2
    dx = _out(out, M, K, out_dtype, dy.device)
    need = int(load().rfq_backward_dx_workspace_size(N, K))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dy.device)
    check(load().rfq_backward_dx(_ptr(dy), DTYPE_BF16, M, N, lddy, _ptr(wq), _ptr(sw), K, _ptr(dx), _y_dtype(dx.dtype),
                                 dx.stride(0), _ptr(workspace), workspace.numel(), _stream()))
    return dx


def backward_dw(dy, qx, sx, qr, sr, out_dtype=torch.float32, out=None, workspace=None):
    """Straight-through dW = dY^T (deq Q(X) + deq Q(R)) for bf16 dY [M, N] and
    the forward's RFQ encoding of X; returns dW [N, K]."""
    M, N, lddy = _dy_args(dy)
    _codes_ok(qx, sx, qr, sr)
    K = qx.shape[1] * 2
    dw = _out(out, N, K, out_dtype, dy.device)
    need = int(load().rfq_backward_dw_workspace_size(M, N, K))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dy.device)
    check(load().rfq_backward_dw(_ptr(dy), DTYPE_BF16, M, N, lddy, _ptr(qx), _ptr(sx), _ptr(qr), _ptr(sr), K, _ptr(dw),
                                 _y_dtype(dw.dtype), dw.stride(0), _ptr(workspace), workspace.numel(), _stream()))
    return dw


def linear_workspace_size(M, K):
    return int(load().rfq_linear_workspace_size(M, K))


def linear(x, wq, sw, out_dtype=torch.bfloat16, out=None, workspace=None):
    """Whole RFQ W4A4 linear layer on bf16 X [M, K] and an MXFP4 weight."""
    M, K, ldx, dt = _x_args(x)
    N = wq.shape[0]
    y = out if out is not None else torch.empty((M, N), dtype=out_dtype, device=x.device)
    need = linear_workspace_size(M, K)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    check(load().rfq_linear(_ptr(x), dt, M, K, ldx, _ptr(wq), _ptr(sw), N, _ptr(y), _y_dtype(y.dtype),
                            y.stride(0), _ptr(workspace), workspace.numel(), _stream()))
    return y
