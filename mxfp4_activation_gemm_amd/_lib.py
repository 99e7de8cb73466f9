"""ctypes loader for librfq.so and its exported C ABI (include/rfq.h)."""
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librfq.so")

STATUS = {
    0: "RFQ_OK",
    1: "RFQ_ERR_NULL_POINTER",
    2: "RFQ_ERR_INVALID_SHAPE",
    3: "RFQ_ERR_INVALID_STRIDE",
    4: "RFQ_ERR_MISALIGNED",
    5: "RFQ_ERR_UNSUPPORTED_DTYPE",
    6: "RFQ_ERR_WORKSPACE_TOO_SMALL",
    7: "RFQ_ERR_HIP",
}
DTYPE_BF16 = 0
DTYPE_FP32 = 1

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i = ctypes.c_int
_sz = ctypes.c_size_t

# name -> (restype, argtypes), mirroring include/rfq.h
SIGNATURES = {
    "rfq_quantize_mxfp4": (_i, [_p, _i, _i64, _i64, _i64, _p, _p, _p]),
    "rfq_residual_quantize": (_i, [_p, _i, _i64, _i64, _i64, _p, _p, _p, _p, _p]),
    "rfq_rotate_residual_quantize": (_i, [_p, _i, _i64, _i64, _i64, _p, _p, _p, _p, _p]),
    "rfq_rotate_quantize_weight": (_i, [_p, _i, _i64, _i64, _i64, _p, _p, _p]),
    "rfq_rotate64_residual_quantize": (_i, [_p, _i, _i64, _i64, _i64, _p, _p, _p, _p, _p]),
    "rfq_rotate64_quantize_weight": (_i, [_p, _i, _i64, _i64, _i64, _p, _p, _p]),
    "rfq_gemm_w4a4": (_i, [_p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _p, _i, _i64, _p]),
    "rfq_linear_workspace_size": (_sz, [_i64, _i64]),
    "rfq_linear": (_i, [_p, _i, _i64, _i64, _i64, _p, _p, _i64, _p, _i, _i64, _p, _sz, _p]),
    "rfq_linear_fused": (_i, [_p, _i, _i64, _i64, _i64, _p, _p, _i64, _p, _i, _i64, _p]),
    "rfq_linear_noalloc": (_i, [_p, _i, _i64, _i64, _i64, _p, _p, _i64, _p, _i, _i64, _p]),
    "rfq_linear_noalloc_max_workspace": (_sz, []),
    "rfq_status_string": (ctypes.c_char_p, [_i]),
    "rfq_last_error_detail": (ctypes.c_char_p, []),
    "rfq_abi_version": (_i, []),
    "rfq_quantize_mxfp8": (_i, [_p, _i, _i64, _i64, _i64, _p, _p, _p]),
    "rfq_residual_quantize_mxfp8": (_i, [_p, _i, _i64, _i64, _i64, _p, _p, _p, _p, _p]),
    "rfq_gemm_w4a8": (_i, [_p, _p, _p, _p, _i64, _i64, _i64, _p, _i, _i64, _p]),
    "rfq_gemm_w4a4_mxfp8_residual": (_i, [_p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _p, _i, _i64, _p]),
    "rfq_backward_dx_workspace_size": (_sz, [_i64, _i64]),
    "rfq_backward_dw_workspace_size": (_sz, [_i64, _i64, _i64]),
    "rfq_backward_dx": (_i, [_p, _i, _i64, _i64, _i64, _p, _p, _i64, _p, _i, _i64, _p, _sz, _p]),
    "rfq_backward_dw": (_i, [_p, _i, _i64, _i64, _i64, _p, _p, _p, _p, _i64, _p, _i, _i64, _p, _sz, _p]),
}

_LIB = None


class RfqError(RuntimeError):
    """A non-OK status returned by librfq."""

    def __init__(self, status, detail):
        self.status = status
        self.status_name = STATUS.get(status, str(status))
        super().__init__(f"{self.status_name}: {detail}")


def load():
    """Loads librfq.so (built by mxfp4_activation_gemm_amd.build); raises if absent."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m mxfp4_activation_gemm_amd.build` "
                               "or __graft_entry__.build() first")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def check(status):
    if status != 0:
        detail = load().rfq_last_error_detail().decode()
        raise RfqError(status, detail)
