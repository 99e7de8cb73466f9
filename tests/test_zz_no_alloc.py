"""rfq_linear_noalloc through the C ABI: the allocation-free variant of
rfq_linear (Q(X) and Q(R) staged in the library's own device array) gives
the same Y as rfq_linear with a caller workspace, bit for bit, on two calls
in a row, the second smaller than the first; Y also matches the oracle
within 1e-5 of the condition scale. Shapes beyond the array are refused
before anything is launched, leaving Y untouched."""
import ctypes

import numpy as np
import pytest
import torch

import mxfp4_activation_gemm_amd as rfq
import oracle
import workloads
from gpu_helpers import check_y, dev_bf16, host, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rfq.library()


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def noalloc(lib, x, wq, sw, y):
    M, K = x.shape
    return lib.rfq_linear_noalloc(x.data_ptr(), 0, M, K, x.stride(0), wq.data_ptr(), sw.data_ptr(), wq.shape[0],
                                  y.data_ptr(), 1 if y.dtype == torch.float32 else 0, y.stride(0), stream())


def operands(M, N, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3, size=(M, K)).astype(np.float32)
    x[:, rng.choice(K, size=4, replace=False)] *= 60
    xb = workloads.f32_to_bf16_bits(x)
    wb = workloads.f32_to_bf16_bits(rng.normal(0, 0.02, (N, K)).astype(np.float32))
    return xb, wb


def test_noalloc_matches_linear_on_two_calls_second_smaller():
    lib = rfq.library()
    cap = int(lib.rfq_linear_noalloc_max_workspace())
    assert cap == 64 << 20
    # first call near the array's size (12288 x 5120: 66.8 MB of staging),
    # then a smaller, ragged one that reuses the array
    for (M, N, K, out_dtype, seed) in [(12288, 512, 5120, torch.bfloat16, 1), (200, 300, 1024, torch.float32, 2)]:
        log(f"[noalloc] M={M} N={N} K={K} {out_dtype}")
        assert rfq.linear_workspace_size(M, K) <= cap
        xb, wb = operands(M, N, K, seed)
        x = dev_bf16(xb)
        wq, sw = rfq.quantize_mxfp4(dev_bf16(wb))
        y0 = torch.full((M, N), 3.0, dtype=out_dtype, device="cuda")
        st = noalloc(lib, x, wq, sw, y0)
        assert st == 0, lib.rfq_last_error_detail().decode()
        y1 = rfq.linear(x, wq, sw, out_dtype=out_dtype)
        torch.cuda.synchronize()
        if out_dtype == torch.bfloat16:
            a, b = host(y0.view(torch.int16)), host(y1.view(torch.int16))
        else:
            a, b = host(y0), host(y1)
        assert np.array_equal(a, b), "rfq_linear_noalloc differs from rfq_linear"
        rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(seed).choice(M, 62, replace=False)]))
        xq = oracle.bf16_bits_to_f64(xb[rows])
        y_ref, s_ref, _, _ = oracle.linear(xq, oracle.bf16_bits_to_f64(wb))
        yh = y0[torch.from_numpy(rows).cuda()].float()
        worst = check_y(host(yh).astype(np.float64), y_ref, s_ref, out_dtype, f"noalloc {M}x{N}x{K}")
        log(f"   bit-equal to rfq_linear; max |dY|/S = {worst:.2e}")


def test_noalloc_refuses_shapes_beyond_its_array():
    lib = rfq.library()
    cap = int(lib.rfq_linear_noalloc_max_workspace())
    K = 5120
    M = 12400                                   # 5440 bytes of staging per row: 67.5 MB > 64 MiB
    assert rfq.linear_workspace_size(M, K) > cap
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    wq = torch.zeros((64, K // 2), dtype=torch.uint8, device="cuda")
    sw = torch.full((64, K // 32), 127, dtype=torch.uint8, device="cuda")
    y = torch.full((M, 64), 5.0, dtype=torch.float32, device="cuda")
    st = noalloc(lib, x, wq, sw, y)
    assert rfq._lib.STATUS[st] == "RFQ_ERR_WORKSPACE_TOO_SMALL"
    assert "allocation-free" in lib.rfq_last_error_detail().decode()
    torch.cuda.synchronize()
    assert bool((y == 5.0).all()), "Y was written by a refused call"
    # M = 0 is a no-op
    assert noalloc(lib, x[:0], wq, sw, y[:0]) == 0
