"""The binding's shape rules, on CPU tensors (no GPU, no library call).

The C ABI receives raw device pointers, so a weight or output of the wrong
shape would be read or written past its end on the device; the binding is
the only layer that can see shapes, dtypes and strides. Each public call
checks its operands before anything reaches the library: here the library
loader is replaced by one that fails the test if it is ever reached."""
import pytest
import torch

import mxfp4_activation_gemm_amd as rfq

M, N, K = 8, 16, 64


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def forbidden():
        raise AssertionError("the library was reached before the operands were checked")
    monkeypatch.setattr(rfq, "load", forbidden)


def u8(*shape):
    return torch.zeros(shape, dtype=torch.uint8)


def good():
    return dict(x=torch.zeros((M, K), dtype=torch.bfloat16), qx=u8(M, K // 2), sx=u8(M, K // 32),
                qr=u8(M, K // 2), sr=u8(M, K // 32), wq=u8(N, K // 2), sw=u8(N, K // 32),
                out=torch.zeros((M, N), dtype=torch.float32))


def raises(fn, match):
    with pytest.raises(ValueError, match=match):
        fn()


def test_good_operands_pass_the_shape_rules():
    g = good()
    assert rfq.gemm_shapes(g["qx"], g["sx"], g["qr"], g["sr"], g["wq"], g["sw"]) == (M, N, K)
    assert rfq.gemm_shapes(g["qx"], g["sx"], None, None, g["wq"], g["sw"]) == (M, N, K)
    assert rfq.linear_shapes(g["x"], g["wq"], g["sw"]) == (M, N, K)
    rfq.check_out(g["out"], M, N)
    # strided rows (a column slice of a wider tensor) are allowed for X and out
    wide = torch.zeros((M, 3 * N), dtype=torch.bfloat16)
    rfq.check_out(wide[:, N:2 * N], M, N)
    assert rfq.check_x(torch.zeros((M, 2 * K), dtype=torch.float32)[:, :K]) == (M, K)
    # and the device rule rejects host tensors after the shapes pass
    raises(lambda: rfq.linear(g["x"], g["wq"], g["sw"], out=g["out"]), "CUDA")


@pytest.mark.parametrize("case,match", [
    ("w_codes_k", "W codes: has 16 columns, expected 32"),
    ("w_scales_rows", "W scales: has 15 rows, expected 16"),
    ("w_scales_k", "W scales: has 1 columns, expected 2"),
    ("w_dtype", "W codes: dtype"),
    ("w_noncontig", "W codes: must"),
    ("out_shape", "out: has 15 columns, expected 16"),
    ("out_rows", "out: has 9 rows, expected 8"),
    ("out_col_stride", "out: must have unit stride"),
    ("out_dtype", "out: dtype"),
    ("workspace_small", "workspace: holds"),
    ("x_col_stride", "x: must have unit stride"),
    ("x_dtype", "x: dtype"),
    ("x_3d", "x: must be 2-D"),
])
def test_linear_rejects(case, match):
    g = good()
    x, wq, sw, out, ws = g["x"], g["wq"], g["sw"], g["out"], None
    if case == "w_codes_k":
        wq = u8(N, K // 4)
    elif case == "w_scales_rows":
        sw = u8(N - 1, K // 32)
    elif case == "w_scales_k":
        sw = u8(N, K // 64)
    elif case == "w_dtype":
        wq = torch.zeros((N, K // 2), dtype=torch.int8)
    elif case == "w_noncontig":
        wq = u8(N, K)[:, ::2]
    elif case == "out_shape":
        out = torch.zeros((M, N - 1), dtype=torch.float32)
    elif case == "out_rows":
        out = torch.zeros((M + 1, N), dtype=torch.float32)
    elif case == "out_col_stride":
        out = torch.zeros((N, M), dtype=torch.float32).t()
    elif case == "out_dtype":
        out = torch.zeros((M, N), dtype=torch.float16)
    elif case == "workspace_small":
        ws = u8(10)
        rfq.check_workspace(u8(10), 10)          # the rule itself
        raises(lambda: rfq.check_workspace(ws, 11), match)
        return
    elif case == "x_col_stride":
        x = torch.zeros((K, M), dtype=torch.bfloat16).t()
    elif case == "x_dtype":
        x = torch.zeros((M, K), dtype=torch.float16)
    elif case == "x_3d":
        x = torch.zeros((1, M, K), dtype=torch.bfloat16)
    raises(lambda: rfq.linear(x, wq, sw, out=out, workspace=ws), match)
    raises(lambda: rfq.linear_noalloc(x, wq, sw, out), match)


@pytest.mark.parametrize("case,match", [
    ("sx_rows", "QX scales: has 7 rows"),
    ("qr_k", "QR codes: has 16 columns"),
    ("sr_missing", "given together"),
    ("sw_k", "W scales: has 4 columns"),
    ("wq_k", "W codes: has 33 columns"),
    ("k_not_32", "not a multiple of 32"),
    ("out_shape", "out: has 7 rows"),
])
def test_gemm_rejects(case, match):
    g = good()
    qx, sx, qr, sr, wq, sw, out = g["qx"], g["sx"], g["qr"], g["sr"], g["wq"], g["sw"], g["out"]
    if case == "sx_rows":
        sx = u8(M - 1, K // 32)
    elif case == "qr_k":
        qr = u8(M, K // 4)
    elif case == "sr_missing":
        sr = None
    elif case == "sw_k":
        sw = u8(N, 4)
    elif case == "wq_k":
        wq = u8(N, K // 2 + 1)
    elif case == "k_not_32":
        qx, qr = u8(M, 24), u8(M, 24)
    elif case == "out_shape":
        out = torch.zeros((M - 1, N), dtype=torch.float32)
    raises(lambda: rfq.gemm_w4a4(qx, sx, qr, sr, wq, sw, out=out), match)


def test_mxfp8_gemms_reject_wrong_code_widths():
    g = good()
    # W4A8: activation codes are one byte per element ([M, K]); [M, K/2] reads as K/2
    raises(lambda: rfq.gemm_w4a8(u8(M, K), g["sx"], g["wq"], u8(N, 1), out=g["out"]), "W scales")
    raises(lambda: rfq.gemm_w4a8(u8(M, K // 2), g["sx"], g["wq"], g["sw"], out=g["out"]), "columns")
    raises(lambda: rfq.gemm_w4a4_mxfp8_residual(g["qx"], g["sx"], u8(M, K // 2), g["sr"], g["wq"], g["sw"],
                                               out=g["out"]), "QR codes: has 32 columns, expected 64")
    raises(lambda: rfq.gemm_w4a4_mxfp8_residual(g["qx"], g["sx"], None, None, g["wq"], g["sw"]), "required")


def test_backward_rejects():
    g = good()
    dy = torch.zeros((M, N), dtype=torch.bfloat16)
    raises(lambda: rfq.backward_dx(dy, u8(N - 1, K // 2), g["sw"]), "W codes: has 15 rows")
    raises(lambda: rfq.backward_dx(dy, g["wq"], u8(N, 1)), "W scales")
    raises(lambda: rfq.backward_dx(torch.zeros((M, 2 * N), dtype=torch.bfloat16)[:, :N], g["wq"], g["sw"]),
           "must be dense")
    raises(lambda: rfq.backward_dx(dy, g["wq"], g["sw"], out=torch.zeros((M, K - 32))), "out: has 32 columns")
    raises(lambda: rfq.backward_dx(dy.float(), g["wq"], g["sw"]), "dy: dtype")
    raises(lambda: rfq.backward_dw(dy, u8(M + 1, K // 2), g["sx"], g["qr"], g["sr"]), "QX codes: has 9 rows")
    raises(lambda: rfq.backward_dw(dy, g["qx"], g["sx"], u8(M, K), g["sr"]), "QR codes")
    raises(lambda: rfq.backward_dw(dy, g["qx"], g["sx"], g["qr"], g["sr"], out=torch.zeros((N, K + 32))),
           "out: has 96 columns")
    raises(lambda: rfq.backward_dw(dy, g["qx"], g["sx"], g["qr"], g["sr"], workspace=torch.zeros(10)), "workspace")


@pytest.mark.parametrize("call", ["quantize_mxfp4", "residual_quantize", "rotate_residual_quantize",
                                  "rotate_quantize_weight", "quantize_mxfp8", "residual_quantize_mxfp8"])
def test_quantize_calls_check_x_before_the_library(call):
    fn = getattr(rfq, call)
    raises(lambda: fn(torch.zeros((M, K), dtype=torch.float16)), "dtype|bf16|fp32|float")     # unsupported dtype
    raises(lambda: fn(torch.zeros((M, K), dtype=torch.bfloat16)), "CUDA")                     # host tensor


def test_rotation_size_is_checked():
    x = torch.zeros((M, 96), dtype=torch.bfloat16)
    raises(lambda: rfq.rotate_residual_quantize(x, size=48), "32 or 64")
    raises(lambda: rfq.rotate_residual_quantize(x, size=64), "multiple of the rotation size 64")
    raises(lambda: rfq.rotate_quantize_weight(x, size=64), "multiple of the rotation size 64")
    raises(lambda: rfq.rotate_quantize_weight(torch.zeros((M, 128), dtype=torch.bfloat16), size=64), "CUDA")
