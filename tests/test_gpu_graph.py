"""The RFQ linear layer on a side stream and inside a captured HIP graph.

The library's entry points only enqueue kernels on the caller's stream (no
allocation, memset or synchronization), so the layer's three launches can be
captured once and replayed. Each replay is checked against the eager result,
with the program's own eager work and a synchronization between replays, and
the input rewritten between replays so that a replay must read it again."""
import numpy as np
import pytest
import torch

import mxfp4_activation_gemm_amd as rfq
import workloads
from gpu_helpers import dev_bf16, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rfq.library()


@pytest.mark.parametrize("M,N,K", [(64, 128, 256), (300, 520, 1024), (512, 768, 2048)])
def test_side_stream_and_graph_replays_match_eager(M, N, K):
    rng = np.random.default_rng(M + N + K)
    xs = [dev_bf16(workloads.f32_to_bf16_bits(rng.standard_t(3, size=(M, K)).astype(np.float32)))
          for _ in range(2)]
    w = dev_bf16(workloads.f32_to_bf16_bits(rng.normal(0, 0.02, (N, K)).astype(np.float32)))
    log(f"[graph] M={M} N={N} K={K}")
    wq, sw = rfq.quantize_mxfp4(w)
    ws = torch.empty(rfq.linear_workspace_size(M, K), dtype=torch.uint8, device="cuda")
    eager = []
    for x in xs:
        y = torch.empty(M, N, dtype=torch.float32, device="cuda")
        rfq.linear(x, wq, sw, out=y, workspace=ws)
        eager.append(y)
    x_in = xs[0].clone()
    y = torch.empty(M, N, dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        rfq.linear(x_in, wq, sw, out=y, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(y, eager[0]), "side stream"
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        rfq.linear(x_in, wq, sw, out=y, workspace=ws)
    for rep in range(6):
        k = rep % 2
        x_in.copy_(xs[k])
        y.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager[k]), f"replay {rep}"
