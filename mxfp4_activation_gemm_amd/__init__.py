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
    "linear_fused",
    "linear_noalloc",
    "linear_noalloc_max_workspace",
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


# Shape rules. The C ABI receives raw device pointers, so this binding is the
# only layer that can see a tensor's shape, dtype, strides and device: every
# operand is checked here, before any call into the library, and a mismatch
# raises ValueError with nothing launched and no output written. The rules
# below look only at tensor metadata (no device access), so they also run on
# CPU tensors.

def _fail(what, msg):
    raise ValueError(f"{what}: {msg}")


def _check_matrix(t, what, dtypes, rows=None, cols=None, dense=True):
    """A 2-D tensor of one of `dtypes`, [rows, cols] where given, unit stride
    along its last dimension, and (dense) fully contiguous."""
    if not isinstance(t, torch.Tensor):
        _fail(what, "must be a torch.Tensor")
    if t.dim() != 2:
        _fail(what, f"must be 2-D, got shape {tuple(t.shape)}")
    if t.dtype not in dtypes:
        _fail(what, f"dtype {t.dtype} not in {[str(d) for d in dtypes]}")
    if rows is not None and t.shape[0] != rows:
        _fail(what, f"has {t.shape[0]} rows, expected {rows}")
    if cols is not None and t.shape[1] != cols:
        _fail(what, f"has {t.shape[1]} columns, expected {cols}")
    if t.numel() and t.stride(1) != 1:
        _fail(what, f"must have unit stride along its last dimension, got strides {t.stride()}")
    if dense and t.numel() and not t.is_contiguous():
        _fail(what, "must be contiguous")


_U8 = (torch.uint8,)
_XTYPES = (torch.bfloat16, torch.float32)
_YTYPES = (torch.float32, torch.bfloat16)


def check_codes(codes, scales, rows, K, what, element_bytes=0.5):
    """MX codes [rows, K * element_bytes] (0.5: MXFP4 nibbles, 1: MXFP8 bytes)
    and scales [rows, K / 32], both contiguous uint8."""
    if K % 32:
        _fail(what, f"K = {K} is not a multiple of 32")
    _check_matrix(codes, f"{what} codes", _U8, rows, int(K * element_bytes))
    _check_matrix(scales, f"{what} scales", _U8, rows, K // 32)


def check_x(x, what="x"):
    """X [M, K] bf16 or fp32 with unit stride along K (any row stride); returns (M, K)."""
    _check_matrix(x, what, _XTYPES, dense=False)
    return x.shape[0], x.shape[1]


def check_out(out, rows, cols, what="out"):
    """An output [rows, cols] fp32 or bf16 with unit column stride and a row
    stride of at least cols (rows may be strided, as the ABI's ldy allows)."""
    _check_matrix(out, what, _YTYPES, rows, cols, dense=False)
    if rows > 1 and cols and out.stride(0) < cols:
        _fail(what, f"row stride {out.stride(0)} is below its {cols} columns")


def check_workspace(ws, need, what="workspace"):
    if not isinstance(ws, torch.Tensor) or ws.dtype != torch.uint8 or not ws.is_contiguous():
        _fail(what, "must be a contiguous uint8 tensor")
    if ws.numel() < need:
        _fail(what, f"holds {ws.numel()} bytes, needs {need}")


def check_device(device, **tensors):
    """Every tensor on `device`, a CUDA device."""
    if device.type != "cuda":
        raise ValueError(f"operands must be CUDA tensors, got device {device}")
    for name, t in tensors.items():
        if t is not None and t.device != device:
            _fail(name, f"is on {t.device}, expected {device}")


def _given_out(out, rows, cols):
    if out is not None:
        check_out(out, rows, cols)


def _new_out(out, rows, cols, out_dtype, device):
    if out is None:
        if out_dtype not in _YTYPES:
            raise ValueError("out_dtype must be torch.float32 or torch.bfloat16")
        out = torch.empty((rows, cols), dtype=out_dtype, device=device)
    check_out(out, rows, cols)
    return out


def _x_code(x):
    return DTYPE_BF16 if x.dtype == torch.bfloat16 else DTYPE_FP32


def _y_code(y):
    return DTYPE_FP32 if y.dtype == torch.float32 else DTYPE_BF16


def _quantize(name, x, bytes_per_element=0.5):
    """Entry point `name` on X after X's checks (the library is loaded only then)."""
    rows, K = check_x(x)
    check_device(x.device, x=x)
    fn = getattr(load(), name)
    codes = torch.empty((rows, int(K * bytes_per_element)), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, K // 32), dtype=torch.uint8, device=x.device)
    check(fn(_ptr(x), _x_code(x), rows, K, x.stride(0), _ptr(codes), _ptr(scales), _stream()))
    return codes, scales


def _residual(name, x, r_bytes_per_element=0.5):
    M, K = check_x(x)
    check_device(x.device, x=x)
    fn = getattr(load(), name)
    qx = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    qr = torch.empty((M, int(K * r_bytes_per_element)), dtype=torch.uint8, device=x.device)
    sx = torch.empty((M, K // 32), dtype=torch.uint8, device=x.device)
    sr = torch.empty_like(sx)
    check(fn(_ptr(x), _x_code(x), M, K, x.stride(0), _ptr(qx), _ptr(sx), _ptr(qr), _ptr(sr), _stream()))
    return qx, sx, qr, sr


def quantize_mxfp4(x):
    """MXFP4 along K of bf16 or fp32 X: returns (codes uint8 [rows, K/2], scales uint8 [rows, K/32])."""
    return _quantize("rfq_quantize_mxfp4", x)


def residual_quantize(x):
    """RFQ encoding of X: returns (qx, sx, qr, sr) = Q(X) codes/scales, Q(R) codes/scales."""
    return _residual("rfq_residual_quantize", x)


ROTATION_SIZES = (32, 64)


def _rotation_size(x, size):
    if size not in ROTATION_SIZES:
        raise ValueError(f"rotation size must be 32 or 64, got {size}")
    if x.dim() == 2 and x.shape[1] % size:
        raise ValueError(f"K = {x.shape[1]} must be a multiple of the rotation size {size}")


def rotate_residual_quantize(x, size=32):
    """RFQ encoding of X H (block Hadamard of `size` 32 or 64 along K): (qx, sx, qr, sr)."""
    _rotation_size(x, size)
    return _residual("rfq_rotate_residual_quantize" if size == 32 else "rfq_rotate64_residual_quantize", x)


def rotate_quantize_weight(w, size=32):
    """MXFP4 codes and scales of W H / size, the weight side of the rotated layer."""
    _rotation_size(w, size)
    return _quantize("rfq_rotate_quantize_weight" if size == 32 else "rfq_rotate64_quantize_weight", w)


def gemm_shapes(qx, sx, qr, sr, wq, sw, x_bytes=0.5, r_bytes=0.5):
    """(M, N, K) of a block-scaled GEMM's operands after checking them against
    each other: activation codes [M, K * x_bytes], residual codes [M, K * r_bytes]
    (or qr = sr = None), weight codes [N, K/2], every scale tensor [rows, K/32]."""
    _check_matrix(qx, "QX codes", _U8)
    M, K = qx.shape[0], int(round(qx.shape[1] / x_bytes))
    _check_matrix(wq, "W codes", _U8)
    N = wq.shape[0]
    check_codes(qx, sx, M, K, "QX", x_bytes)
    if (qr is None) != (sr is None):
        raise ValueError("QR codes and scales must be given together")
    if qr is not None:
        check_codes(qr, sr, M, K, "QR", r_bytes)
    check_codes(wq, sw, N, K, "W")
    return M, N, K


def gemm_w4a4(qx, sx, qr, sr, wq, sw, out_dtype=torch.bfloat16, out=None):
    """Y = deq(QX) deq(W)^T + deq(QR) deq(W)^T (qr = sr = None: plain W4A4)."""
    M, N, K = gemm_shapes(qx, sx, qr, sr, wq, sw)
    _given_out(out, M, N)
    check_device(qx.device, sx=sx, qr=qr, sr=sr, wq=wq, sw=sw, out=out)
    y = _new_out(out, M, N, out_dtype, qx.device)
    check(load().rfq_gemm_w4a4(_ptr(qx), _ptr(sx), _ptr(qr), _ptr(sr), _ptr(wq), _ptr(sw), M, N, K, _ptr(y),
                               _y_code(y), y.stride(0), _stream()))
    return y


def quantize_mxfp8(x):
    """MXFP8 (E4M3) along K of bf16 or fp32 X: (codes uint8 [rows, K], scales uint8 [rows, K/32])."""
    return _quantize("rfq_quantize_mxfp8", x, bytes_per_element=1)


def residual_quantize_mxfp8(x):
    """RFQ encoding with an MXFP8 second path: (qx [M, K/2], sx, qr8 [M, K], sr)."""
    return _residual("rfq_residual_quantize_mxfp8", x, r_bytes_per_element=1)


def gemm_w4a8(qx8, sx, wq, sw, out_dtype=torch.bfloat16, out=None):
    """Y = deq(QX8) deq(W)^T for MXFP8 activation codes and the MXFP4 weight."""
    M, N, K = gemm_shapes(qx8, sx, None, None, wq, sw, x_bytes=1)
    _given_out(out, M, N)
    check_device(qx8.device, sx=sx, wq=wq, sw=sw, out=out)
    y = _new_out(out, M, N, out_dtype, qx8.device)
    check(load().rfq_gemm_w4a8(_ptr(qx8), _ptr(sx), _ptr(wq), _ptr(sw), M, N, K, _ptr(y), _y_code(y),
                               y.stride(0), _stream()))
    return y


def gemm_w4a4_mxfp8_residual(qx, sx, qr8, sr, wq, sw, out_dtype=torch.bfloat16, out=None):
    """Y = deq(QX) deq(W)^T + deq(QR8) deq(W)^T, QX MXFP4 and QR8 MXFP8."""
    if qr8 is None or sr is None:
        raise ValueError("the MXFP8 residual term (qr8, sr) is required")
    M, N, K = gemm_shapes(qx, sx, qr8, sr, wq, sw, r_bytes=1)
    _given_out(out, M, N)
    check_device(qx.device, sx=sx, qr8=qr8, sr=sr, wq=wq, sw=sw, out=out)
    y = _new_out(out, M, N, out_dtype, qx.device)
    check(load().rfq_gemm_w4a4_mxfp8_residual(_ptr(qx), _ptr(sx), _ptr(qr8), _ptr(sr), _ptr(wq), _ptr(sw), M, N, K,
                                              _ptr(y), _y_code(y), y.stride(0), _stream()))
    return y


def check_dy(dy, dense):
    """dY [M, N] bf16 with unit stride along N; `dense` also requires rows
    back to back (row stride N), as rfq_backward_dx does. Returns (M, N)."""
    _check_matrix(dy, "dy", (torch.bfloat16,), dense=False)
    M, N = dy.shape
    if dense and M > 1 and dy.stride(0) != N:
        _fail("dy", f"must be dense (row stride {N}), got row stride {dy.stride(0)}")
    return M, N


def backward_dx(dy, wq, sw, out_dtype=torch.float32, out=None, workspace=None):
    """Straight-through dX = dY deq(Wq) for bf16 dY [M, N] (dense) and the
    weight's MXFP4 codes/scales [N, K/2], [N, K/32]; returns dX [M, K]."""
    M, N = check_dy(dy, dense=True)
    _check_matrix(wq, "W codes", _U8, rows=N)
    K = wq.shape[1] * 2
    check_codes(wq, sw, N, K, "W")
    _given_out(out, M, K)
    if workspace is not None:
        check_workspace(workspace, 0)
    check_device(dy.device, wq=wq, sw=sw, out=out, workspace=workspace)
    need = int(load().rfq_backward_dx_workspace_size(N, K))
    if workspace is not None:
        check_workspace(workspace, need)
    dx = _new_out(out, M, K, out_dtype, dy.device)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dy.device)
    check(load().rfq_backward_dx(_ptr(dy), DTYPE_BF16, M, N, dy.stride(0), _ptr(wq), _ptr(sw), K, _ptr(dx),
                                 _y_code(dx), dx.stride(0), _ptr(workspace), workspace.numel(), _stream()))
    return dx


def backward_dw(dy, qx, sx, qr, sr, out_dtype=torch.float32, out=None, workspace=None):
    """Straight-through dW = dY^T (deq Q(X) + deq Q(R)) for bf16 dY [M, N] and
    the forward's RFQ encoding of X ([M, K/2] codes, [M, K/32] scales each);
    returns dW [N, K]."""
    M, N = check_dy(dy, dense=False)
    _check_matrix(qx, "QX codes", _U8, rows=M)
    K = qx.shape[1] * 2
    check_codes(qx, sx, M, K, "QX")
    check_codes(qr, sr, M, K, "QR")
    _given_out(out, N, K)
    if workspace is not None:
        check_workspace(workspace, 0)
    check_device(dy.device, qx=qx, sx=sx, qr=qr, sr=sr, out=out, workspace=workspace)
    need = int(load().rfq_backward_dw_workspace_size(M, N, K))
    if workspace is not None:
        check_workspace(workspace, need)
    dw = _new_out(out, N, K, out_dtype, dy.device)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dy.device)
    check(load().rfq_backward_dw(_ptr(dy), DTYPE_BF16, M, N, dy.stride(0), _ptr(qx), _ptr(sx), _ptr(qr), _ptr(sr), K,
                                 _ptr(dw), _y_code(dw), dw.stride(0), _ptr(workspace), workspace.numel(), _stream()))
    return dw


def linear_workspace_size(M, K):
    return int(load().rfq_linear_workspace_size(M, K))


def linear_shapes(x, wq, sw):
    """(M, N, K) of the layer after checking X [M, K] against the weight's
    codes [N, K/2] and scales [N, K/32]."""
    M, K = check_x(x)
    _check_matrix(wq, "W codes", _U8)
    check_codes(wq, sw, wq.shape[0], K, "W")
    return M, wq.shape[0], K


def linear(x, wq, sw, out_dtype=torch.bfloat16, out=None, workspace=None):
    """Whole RFQ W4A4 linear layer on bf16 or fp32 X [M, K] and an MXFP4 weight."""
    M, N, K = linear_shapes(x, wq, sw)
    _given_out(out, M, N)
    if workspace is not None:
        check_workspace(workspace, 0)
    check_device(x.device, wq=wq, sw=sw, out=out, workspace=workspace)
    need = linear_workspace_size(M, K)
    if workspace is not None:
        check_workspace(workspace, need)
    y = _new_out(out, M, N, out_dtype, x.device)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    check(load().rfq_linear(_ptr(x), _x_code(x), M, K, x.stride(0), _ptr(wq), _ptr(sw), N, _ptr(y), _y_code(y),
                            y.stride(0), _ptr(workspace), workspace.numel(), _stream()))
    return y


def linear_fused(x, wq, sw, out_dtype=torch.bfloat16, out=None):
    """The layer with Q(X) and Q(R) formed inside the GEMM (rfq_linear_fused):
    bf16 X [M, K] with K a multiple of 512; no workspace; Y bit-equal to linear()."""
    M, N, K = linear_shapes(x, wq, sw)
    if x.dtype != torch.bfloat16:
        raise ValueError("x: the in-GEMM quantization takes bf16 X only")
    if K % 512:
        raise ValueError(f"K = {K}: the in-GEMM quantization needs K a multiple of 512")
    _given_out(out, M, N)
    check_device(x.device, wq=wq, sw=sw, out=out)
    y = _new_out(out, M, N, out_dtype, x.device)
    check(load().rfq_linear_fused(_ptr(x), DTYPE_BF16, M, K, x.stride(0), _ptr(wq), _ptr(sw), N, _ptr(y),
                                  _y_code(y), y.stride(0), _stream()))
    return y


def linear_noalloc_max_workspace():
    return int(load().rfq_linear_noalloc_max_workspace())


def linear_noalloc(x, wq, sw, out):
    """The layer through rfq_linear_noalloc, for callers that cannot allocate:
    `out` [M, N] (fp32 or bf16) is required, and Q(X), Q(R) are staged in the
    library's own device array (at most linear_noalloc_max_workspace() bytes)."""
    M, N, K = linear_shapes(x, wq, sw)
    if out is None:
        raise ValueError("out is required: this call allocates nothing")
    check_out(out, M, N)
    check_device(x.device, wq=wq, sw=sw, out=out)
    check(load().rfq_linear_noalloc(_ptr(x), _x_code(x), M, K, x.stride(0), _ptr(wq), _ptr(sw), N, _ptr(out),
                                    _y_code(out), out.stride(0), _stream()))
    return out
