"""The C ABI boundary without a GPU: the library loads, exports every entry
point include/*.h declares, and rejects bad arguments on the host with the
documented status before anything is launched. Only calls that fail
validation (or are zero-sized no-ops) are made here."""
import os
import re

import pytest

from mxfp4_activation_gemm_amd import _lib

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include")
FAKE = 0x10000000          # a well-aligned non-null address; never dereferenced here

# These calls pass fake device addresses that validation must reject before
# any launch; where a GPU is visible a validation slip would launch a kernel on
# them, so the module runs only on GPU-less hosts (the GPU tests cover the
# same entry points with real buffers).
pytestmark = pytest.mark.skipif(__import__("torch").cuda.device_count() > 0,
                                reason="fake-pointer validation checks run on hosts without a GPU")


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def declared_functions():
    names = set()
    for h in sorted(os.listdir(INCLUDE)):
        if h.endswith(".h"):
            text = re.sub(r"/\*.*?\*/", "", open(os.path.join(INCLUDE, h)).read(), flags=re.S)
            names |= set(re.findall(r"\b(rfq_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_header_declarations_are_exported_and_bound(lib):
    names = declared_functions()
    assert len(names) == 23
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, n
    assert lib.rfq_abi_version() == 8


def status_name(st):
    return _lib.STATUS[st]


def q(lib, x=FAKE, dt=0, rows=4, K=64, ldx=64, codes=FAKE, scales=FAKE):
    return status_name(lib.rfq_quantize_mxfp4(x, dt, rows, K, ldx, codes, scales, None))


def test_quantize_validation(lib):
    assert q(lib, x=None) == "RFQ_ERR_NULL_POINTER"
    assert "x is NULL" in lib.rfq_last_error_detail().decode()
    assert q(lib, codes=None) == "RFQ_ERR_NULL_POINTER"
    assert q(lib, K=48, ldx=48) == "RFQ_ERR_INVALID_SHAPE"
    assert q(lib, K=0, ldx=0) == "RFQ_ERR_INVALID_SHAPE"
    assert q(lib, K=1 << 23, ldx=1 << 23) == "RFQ_ERR_INVALID_SHAPE"
    assert q(lib, rows=-1) == "RFQ_ERR_INVALID_SHAPE"
    assert q(lib, rows=1 << 31) == "RFQ_ERR_INVALID_SHAPE"
    assert q(lib, rows=1 << 22, K=1 << 15, ldx=1 << 15) == "RFQ_ERR_INVALID_SHAPE"   # 2^37 elements
    assert q(lib, dt=2) == "RFQ_ERR_UNSUPPORTED_DTYPE"
    assert q(lib, dt=-1) == "RFQ_ERR_UNSUPPORTED_DTYPE"
    assert q(lib, ldx=32) == "RFQ_ERR_INVALID_STRIDE"
    assert q(lib, ldx=68) == "RFQ_ERR_INVALID_STRIDE"              # bf16 rows need a multiple of 8
    assert q(lib, dt=1, ldx=66) == "RFQ_ERR_INVALID_STRIDE"        # fp32 rows need a multiple of 4
    assert q(lib, x=FAKE + 8) == "RFQ_ERR_MISALIGNED"
    assert q(lib, codes=FAKE + 4) == "RFQ_ERR_MISALIGNED"
    assert q(lib, x=None, rows=0) == "RFQ_OK"              # empty input: no-op, pointers unused
    assert lib.rfq_last_error_detail().decode() == ""


def test_residual_quantize_validation(lib):
    f = lib.rfq_residual_quantize
    assert status_name(f(FAKE, 0, 4, 64, 64, FAKE, FAKE, None, FAKE, None)) == "RFQ_ERR_NULL_POINTER"
    assert status_name(f(FAKE, 0, 4, 64, 64, FAKE, FAKE, FAKE + 1, FAKE, None)) == "RFQ_ERR_MISALIGNED"
    assert status_name(f(FAKE, 0, 4, 96, 100, FAKE, FAKE, FAKE, FAKE, None)) == "RFQ_ERR_INVALID_STRIDE"
    assert status_name(f(None, 0, 0, 64, 64, None, None, None, None, None)) == "RFQ_OK"


def g(lib, qx=FAKE, sx=FAKE, qr=FAKE, sr=FAKE, w=FAKE, sw=FAKE, M=8, N=8, K=64, y=FAKE, yd=0, ldy=8):
    return status_name(lib.rfq_gemm_w4a4(qx, sx, qr, sr, w, sw, M, N, K, y, yd, ldy, None))


def test_gemm_validation(lib):
    assert g(lib, qr=FAKE, sr=None) == "RFQ_ERR_NULL_POINTER"
    assert g(lib, qr=None, sr=FAKE) == "RFQ_ERR_NULL_POINTER"
    assert g(lib, w=None) == "RFQ_ERR_NULL_POINTER"
    assert g(lib, y=None) == "RFQ_ERR_NULL_POINTER"
    assert g(lib, K=40) == "RFQ_ERR_INVALID_SHAPE"
    assert g(lib, N=-3) == "RFQ_ERR_INVALID_SHAPE"
    assert g(lib, M=1 << 20, N=1 << 20, K=32) == "RFQ_ERR_INVALID_SHAPE"   # Y of 2^40 elements
    assert g(lib, yd=7) == "RFQ_ERR_UNSUPPORTED_DTYPE"
    assert g(lib, ldy=4) == "RFQ_ERR_INVALID_STRIDE"
    assert g(lib, y=FAKE + 1, yd=0) == "RFQ_ERR_MISALIGNED"
    assert g(lib, y=FAKE + 2, yd=1) == "RFQ_ERR_MISALIGNED"
    assert g(lib, w=FAKE + 8) == "RFQ_ERR_MISALIGNED"
    assert g(lib, M=0, qx=None, y=None) == "RFQ_OK"
    assert g(lib, N=0, w=None, y=None) == "RFQ_OK"


def test_linear_workspace_rule_and_validation(lib):
    ws = lib.rfq_linear_workspace_size
    r256 = lambda b: (b + 255) // 256 * 256
    for M, K in [(1, 32), (64, 256), (4096, 5120), (32768, 13824), (3, 96)]:
        assert ws(M, K) == 2 * (r256(M * K // 2) + r256(M * K // 32))
    assert ws(4, 48) == 0 and ws(-1, 64) == 0 and ws(0, 64) == 0
    f = lib.rfq_linear
    need = ws(8, 64)
    assert status_name(f(FAKE, 0, 8, 64, 64, FAKE, FAKE, 8, FAKE, 0, 8, FAKE, need - 1, None)) == \
        "RFQ_ERR_WORKSPACE_TOO_SMALL"
    assert status_name(f(FAKE, 0, 8, 64, 64, FAKE, FAKE, 8, FAKE, 0, 8, None, need, None)) == "RFQ_ERR_NULL_POINTER"
    assert status_name(f(FAKE, 0, 8, 64, 64, FAKE, FAKE, 8, FAKE, 0, 8, FAKE + 16, need, None)) == \
        "RFQ_ERR_MISALIGNED"
    assert status_name(f(FAKE, 5, 8, 64, 64, FAKE, FAKE, 8, FAKE, 0, 8, FAKE, need, None)) == \
        "RFQ_ERR_UNSUPPORTED_DTYPE"
    assert status_name(f(FAKE, 1, 8, 64, 62, FAKE, FAKE, 8, FAKE, 0, 8, FAKE, need, None)) == \
        "RFQ_ERR_INVALID_STRIDE"                                   # fp32 X, row stride not a multiple of 4
    assert status_name(f(None, 0, 0, 64, 64, None, None, 8, None, 0, 8, None, 0, None)) == "RFQ_OK"


def test_status_strings(lib):
    assert lib.rfq_status_string(0) == b"success"
    for code in range(1, 8):
        assert lib.rfq_status_string(code) not in (b"", b"unknown status")
    assert lib.rfq_status_string(99) == b"unknown status"


def test_rotated_quantize_validation(lib):
    f, w = lib.rfq_rotate_residual_quantize, lib.rfq_rotate_quantize_weight
    assert status_name(f(FAKE, 0, 4, 64, 64, FAKE, FAKE, None, FAKE, None)) == "RFQ_ERR_NULL_POINTER"
    assert status_name(f(FAKE, 3, 4, 64, 64, FAKE, FAKE, FAKE, FAKE, None)) == "RFQ_ERR_UNSUPPORTED_DTYPE"
    assert status_name(f(FAKE, 0, 4, 48, 48, FAKE, FAKE, FAKE, FAKE, None)) == "RFQ_ERR_INVALID_SHAPE"
    assert status_name(f(None, 0, 0, 64, 64, None, None, None, None, None)) == "RFQ_OK"
    assert status_name(w(FAKE, 1, 4, 64, 62, FAKE, FAKE, None)) == "RFQ_ERR_INVALID_STRIDE"
    assert status_name(w(FAKE + 4, 1, 4, 64, 64, FAKE, FAKE, None)) == "RFQ_ERR_MISALIGNED"
    assert status_name(w(FAKE, 0, 4, 64, 64, None, FAKE, None)) == "RFQ_ERR_NULL_POINTER"
    assert status_name(w(None, 0, 0, 64, 64, None, None, None)) == "RFQ_OK"


def test_rotated64_quantize_validation(lib):
    f, w = lib.rfq_rotate64_residual_quantize, lib.rfq_rotate64_quantize_weight
    # K a multiple of 32 but not of 64: rejected, also with no rows
    assert status_name(f(FAKE, 0, 4, 96, 96, FAKE, FAKE, FAKE, FAKE, None)) == "RFQ_ERR_INVALID_SHAPE"
    assert status_name(f(None, 0, 0, 96, 96, None, None, None, None, None)) == "RFQ_ERR_INVALID_SHAPE"
    assert status_name(w(FAKE, 0, 4, 160, 160, FAKE, FAKE, None)) == "RFQ_ERR_INVALID_SHAPE"
    assert status_name(f(FAKE, 0, 4, 48, 48, FAKE, FAKE, FAKE, FAKE, None)) == "RFQ_ERR_INVALID_SHAPE"
    assert status_name(f(FAKE, 0, 4, 128, 128, FAKE, FAKE, None, FAKE, None)) == "RFQ_ERR_NULL_POINTER"
    assert status_name(f(FAKE, 3, 4, 128, 128, FAKE, FAKE, FAKE, FAKE, None)) == "RFQ_ERR_UNSUPPORTED_DTYPE"
    assert status_name(f(None, 0, 0, 128, 128, None, None, None, None, None)) == "RFQ_OK"
    assert status_name(w(FAKE, 1, 4, 128, 126, FAKE, FAKE, None)) == "RFQ_ERR_INVALID_STRIDE"
    assert status_name(w(FAKE + 4, 1, 4, 128, 128, FAKE, FAKE, None)) == "RFQ_ERR_MISALIGNED"
    assert status_name(w(None, 0, 0, 128, 128, None, None, None)) == "RFQ_OK"


def test_mxfp8_entry_points_validation(lib):
    q8, r8 = lib.rfq_quantize_mxfp8, lib.rfq_residual_quantize_mxfp8
    assert status_name(q8(None, 0, 4, 64, 64, FAKE, FAKE, None)) == "RFQ_ERR_NULL_POINTER"
    assert status_name(q8(FAKE, 2, 4, 64, 64, FAKE, FAKE, None)) == "RFQ_ERR_UNSUPPORTED_DTYPE"
    assert status_name(q8(FAKE, 0, 4, 80, 80, FAKE, FAKE, None)) == "RFQ_ERR_INVALID_SHAPE"
    assert status_name(q8(FAKE, 0, 4, 64, 64, FAKE + 8, FAKE, None)) == "RFQ_ERR_MISALIGNED"
    assert status_name(q8(None, 0, 0, 64, 64, None, None, None)) == "RFQ_OK"
    assert status_name(r8(FAKE, 0, 4, 64, 64, FAKE, FAKE, FAKE, None, None)) == "RFQ_ERR_NULL_POINTER"
    assert status_name(r8(FAKE, 1, 4, 64, 66, FAKE, FAKE, FAKE, FAKE, None)) == "RFQ_ERR_INVALID_STRIDE"
    assert status_name(r8(FAKE, 0, 4, 64, 64, FAKE, FAKE, FAKE + 4, FAKE, None)) == "RFQ_ERR_MISALIGNED"
    assert status_name(r8(None, 0, 0, 64, 64, None, None, None, None, None)) == "RFQ_OK"

    g8, gr8 = lib.rfq_gemm_w4a8, lib.rfq_gemm_w4a4_mxfp8_residual
    assert status_name(g8(None, FAKE, FAKE, FAKE, 8, 8, 64, FAKE, 0, 8, None)) == "RFQ_ERR_NULL_POINTER"
    assert status_name(g8(FAKE, FAKE, FAKE, FAKE, 8, 8, 40, FAKE, 0, 8, None)) == "RFQ_ERR_INVALID_SHAPE"
    assert status_name(g8(FAKE, FAKE, FAKE, FAKE, 8, 8, 64, FAKE, 3, 8, None)) == "RFQ_ERR_UNSUPPORTED_DTYPE"
    assert status_name(g8(FAKE, FAKE, FAKE, FAKE, 8, 8, 64, FAKE, 0, 4, None)) == "RFQ_ERR_INVALID_STRIDE"
    assert status_name(g8(FAKE + 8, FAKE, FAKE, FAKE, 8, 8, 64, FAKE, 0, 8, None)) == "RFQ_ERR_MISALIGNED"
    assert status_name(g8(None, None, None, None, 0, 8, 64, None, 0, 8, None)) == "RFQ_OK"
    assert status_name(gr8(FAKE, FAKE, None, None, FAKE, FAKE, 8, 8, 64, FAKE, 0, 8, None)) == \
        "RFQ_ERR_NULL_POINTER"                                     # the residual term is required here
    assert status_name(gr8(FAKE, FAKE, FAKE + 8, FAKE, FAKE, FAKE, 8, 8, 64, FAKE, 0, 8, None)) == "RFQ_ERR_MISALIGNED"
    assert status_name(gr8(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 8, 64, FAKE + 1, 1, 8, None)) == "RFQ_ERR_MISALIGNED"
    assert status_name(gr8(None, None, None, None, None, None, 8, 0, 64, None, 0, 8, None)) == "RFQ_OK"


def test_backward_validation(lib):
    dx, dw = lib.rfq_backward_dx, lib.rfq_backward_dw
    wsx = lib.rfq_backward_dx_workspace_size(64, 96)
    assert wsx == (96 * 64 * 2 + 255) // 256 * 256
    assert lib.rfq_backward_dx_workspace_size(60, 96) == 0          # N not a multiple of 8
    mp = 104
    assert lib.rfq_backward_dw_workspace_size(100, 40, 96) == ((40 * mp * 2 + 255) // 256 * 256
                                                                 + 2 * ((96 * mp * 2 + 255) // 256 * 256))
    def bx(dy=FAKE, dt=0, M=8, N=64, ld=64, w=FAKE, sw=FAKE, K=96, out=FAKE, od=1, ldo=96, ws=FAKE, n=wsx):
        return status_name(dx(dy, dt, M, N, ld, w, sw, K, out, od, ldo, ws, n, None))
    assert bx(N=60, ld=60) == "RFQ_ERR_INVALID_SHAPE"
    assert bx(K=80) == "RFQ_ERR_INVALID_SHAPE"
    assert bx(dt=1) == "RFQ_ERR_UNSUPPORTED_DTYPE"
    assert bx(ld=72) == "RFQ_ERR_INVALID_STRIDE"
    assert bx(dy=None) == "RFQ_ERR_NULL_POINTER"
    assert bx(dy=FAKE + 2) == "RFQ_ERR_MISALIGNED"
    assert bx(n=wsx - 1) == "RFQ_ERR_WORKSPACE_TOO_SMALL"
    assert bx(ws=FAKE + 16) == "RFQ_ERR_MISALIGNED"
    assert bx(ldo=90) == "RFQ_ERR_INVALID_STRIDE"
    assert bx(M=0, dy=None, w=None, out=None, ws=None) == "RFQ_OK"
    wsw = lib.rfq_backward_dw_workspace_size(8, 40, 96)
    def bw(dy=FAKE, M=8, N=40, ld=40, qx=FAKE, qr=FAKE, K=96, out=FAKE, od=0, ldo=96, ws=FAKE, n=wsw):
        return status_name(dw(dy, 0, M, N, ld, qx, FAKE, qr, FAKE, K, out, od, ldo, ws, n, None))
    assert bw(M=0) == "RFQ_ERR_INVALID_SHAPE"
    assert bw(ld=30) == "RFQ_ERR_INVALID_STRIDE"
    assert bw(qr=None) == "RFQ_ERR_NULL_POINTER"
    assert bw(qx=FAKE + 4) == "RFQ_ERR_MISALIGNED"
    assert bw(n=wsw - 1) == "RFQ_ERR_WORKSPACE_TOO_SMALL"
    assert bw(od=3) == "RFQ_ERR_UNSUPPORTED_DTYPE"
    assert bw(N=0, dy=None, qx=None, qr=None, out=None, ws=None) == "RFQ_OK"


def test_linear_noalloc_validation(lib):
    f = lib.rfq_linear_noalloc
    cap = lib.rfq_linear_noalloc_max_workspace()
    assert cap == 64 << 20

    def na(x=FAKE, dt=0, M=8, K=64, ldx=64, w=FAKE, sw=FAKE, N=8, y=FAKE, yd=1, ldy=8):
        return status_name(f(x, dt, M, K, ldx, w, sw, N, y, yd, ldy, None))
    assert na(x=None) == "RFQ_ERR_NULL_POINTER"
    assert na(w=None) == "RFQ_ERR_NULL_POINTER"
    assert na(K=48, ldx=48) == "RFQ_ERR_INVALID_SHAPE"
    assert na(ldx=60) == "RFQ_ERR_INVALID_STRIDE"
    assert na(ldy=4) == "RFQ_ERR_INVALID_STRIDE"
    assert na(yd=7) == "RFQ_ERR_UNSUPPORTED_DTYPE"
    assert na(x=FAKE + 8) == "RFQ_ERR_MISALIGNED"
    # a shape whose staging exceeds the library's array is refused on the host
    # (12400 x 5120 needs 67.5 MB > 64 MiB) before the device is touched
    assert lib.rfq_linear_workspace_size(12400, 5120) > cap
    assert na(M=12400, K=5120, ldx=5120) == "RFQ_ERR_WORKSPACE_TOO_SMALL"
    assert "allocation-free" in lib.rfq_last_error_detail().decode()
    assert na(M=0, x=None, w=None, sw=None, y=None) == "RFQ_OK"


def test_linear_fused_validation(lib):
    f = lib.rfq_linear_fused

    def lf(x=FAKE, dt=0, M=8, K=512, ldx=512, w=FAKE, sw=FAKE, N=8, y=FAKE, yd=1, ldy=8):
        return status_name(f(x, dt, M, K, ldx, w, sw, N, y, yd, ldy, None))
    assert lf(dt=1) == "RFQ_ERR_UNSUPPORTED_DTYPE"                # fp32 X is not taken
    assert lf(K=256, ldx=256) == "RFQ_ERR_INVALID_SHAPE"          # K must be a multiple of 512
    assert lf(K=96, ldx=96) == "RFQ_ERR_INVALID_SHAPE"
    assert lf(ldx=1 << 24) == "RFQ_ERR_INVALID_STRIDE"
    assert lf(x=None) == "RFQ_ERR_NULL_POINTER"
    assert lf(ldy=4) == "RFQ_ERR_INVALID_STRIDE"
    assert lf(x=FAKE + 2) == "RFQ_ERR_MISALIGNED"
    assert lf(M=0, x=None, w=None, sw=None, y=None) == "RFQ_OK"
