#!/usr/bin/env python3
"""Benchmark of the RFQ W4A4 linear layer on one MI355X.

One step = one pass of the whole hot path on one batch: quantize X to MXFP4,
form the fp32 residual and quantize it (one kernel), then the K-doubled
block-scaled FP4 GEMM into Y (one kernel). The weight is quantized once
before timing (setup). Inputs are seeded synthetic tensors already resident
in HBM when the timed region starts.

Workload: the Wan2.2-DiT-style FFN layer, X [4096, 5120] bf16 (Laplace(0,1)
with 8 outlier channels x80), W [13824, 5120] quantized to MXFP4, Y bf16.

Prints one JSON line (rank 0) with the effective TFLOP/s of the step
(4 M N K per step: the contraction over the doubled K), the per-kernel
rooflines measured with HIP events on the launch stream, and the CPU oracle
timed on a bounded sample of the same workload. Beside the layer it times,
on the same X and weight: the block-Hadamard-rotated quantize passes (32- and
64-point), the
plain W4A4 GEMM, and the MXFP8 variants (W4A8; RFQ with an MXFP8 residual),
each with its own quantize pass.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
FP4_PEAK_TFLOPS = 10100.0        # MI355X dense MXFP4 MFMA, TFLOP/s
FP8_PEAK_TFLOPS = 5000.0         # MI355X dense FP8 / MXFP8 MFMA, TFLOP/s
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense BF16 MFMA, TFLOP/s
ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "RFQ W4A4 linear effective TFLOP/s (% MXFP4 peak); quantize GB/s (% HBM)"
QUANT_BYTES_PER_ELEM = 2 + 2 * (0.5 + 1.0 / 32)      # bf16 in, Q(X) and Q(R) codes + scales out
QUANT8_BYTES_PER_ELEM = 2 + 1 + 1.0 / 32              # bf16 in, MXFP8 codes + scales out
QUANT_R8_BYTES_PER_ELEM = 2 + (0.5 + 1.0 / 32) + (1 + 1.0 / 32)   # bf16 in, Q4(X), Q8(R) out
CPU_GEMM_ROWS = 4096                                  # rows of X in the oracle GEMM sample


def progress(msg):
    """A progress line on stderr (the JSON line alone goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="wan22_ffn")
    ap.add_argument("--ramp-seconds", type=float, default=1.0,
                    help="untimed steps run for this long before the warmup steps, so that the GPU has left its "
                         "idle clock state (reported as clock_ramp in the JSON)")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing (profiling runs)")
    ap.add_argument("--no-hbm-quantize", action="store_true",
                    help="skip the extra quantize measurement on the long-sequence layer")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the per-configuration layer timings (the other four shapes)")
    return ap.parse_args()


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "mxfp4_activation_gemm_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_traffic(workload, kernel_hash):
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"gemm_counters_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != kernel_hash:
        return None
    return float(t.group(1))


def cpu_baseline(cfg):
    """The oracle, as it stands, on the workload: the residual quantization
    of the whole X (one thread) and the K-doubled float64 GEMM on the first
    CPU_GEMM_ROWS rows (all of them at the default size) against every
    column of W (BLAS threads). With fewer rows the step time is the
    quantize time plus the GEMM time scaled by M / CPU_GEMM_ROWS, labelled
    as extrapolated."""
    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = os.cpu_count() or 1
    g_rows = min(CPU_GEMM_ROWS, cfg.M)
    x = oracle.bf16_bits_to_f64(workloads.x_bf16(cfg))
    w = oracle.bf16_bits_to_f64(workloads.w_bf16(cfg))
    wq, sw = oracle.quantize_mxfp4(w)                      # setup, as on the GPU
    del w
    t0 = time.perf_counter()
    qx, sx, qr, sr = oracle.residual_quantize(x)
    t_q = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.gemm_w4a4(qx[:g_rows], sx[:g_rows], qr[:g_rows], sr[:g_rows], wq, sw)
    t_g = time.perf_counter() - t0
    t_full = t_q + t_g * cfg.M / g_rows
    value = 4.0 * cfg.M * cfg.N * cfg.K / t_full / 1e12
    whole = g_rows == cfg.M
    return {
        "value": value,
        "unit": "TFLOP/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": (f"oracle residual_quantize on all {cfg.M} rows of X ({t_q:.2f} s, 1 thread) and oracle "
                   f"K-doubled float64 GEMM (Y and its condition scale) on "
                   + (f"all {cfg.M} x {cfg.N} outputs" if whole else f"rows 0..{g_rows - 1} x all {cfg.N} columns")
                   + f" ({t_g:.2f} s, {blas_threads} BLAS threads): "
                   + ("the whole step, " if whole else "full step extrapolated to ")
                   + f"{t_full:.1f} s"),
    }


def oracle_config_timings():
    """The oracle on a bounded sample of every configuration: the residual
    quantization of up to 1024 rows of X (one thread: GB/s of the pass's
    algorithmic bytes), and the K-doubled float64 GEMM of those rows against
    up to 2048 rows of W on all BLAS threads and, on 128 rows, on one thread.
    The step time is extrapolated from the sample's rates (a small GEMM
    sample runs BLAS less efficiently than the full layer would)."""
    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threadpool_limits = None
        blas_threads = os.cpu_count() or 1
    out = {}
    for name, c in workloads.CONFIGS.items():
        q_rows, g_rows, n_cols = min(c.M, 1024), min(c.M, 1024), min(c.N, 2048)
        x = oracle.bf16_bits_to_f64(workloads.x_bf16(c, 0, q_rows))
        w = oracle.bf16_bits_to_f64(workloads.w_bf16(c)[:n_cols])
        wq, sw = oracle.quantize_mxfp4(w)
        t0 = time.perf_counter()
        qx, sx, qr, sr = oracle.residual_quantize(x)
        t_q = time.perf_counter() - t0
        t0 = time.perf_counter()
        oracle.gemm_w4a4(qx[:g_rows], sx[:g_rows], qr[:g_rows], sr[:g_rows], wq, sw)
        t_g = time.perf_counter() - t0
        r1 = min(g_rows, 128)
        t1 = None
        if threadpool_limits is not None:
            with threadpool_limits(limits=1):
                t0 = time.perf_counter()
                oracle.gemm_w4a4(qx[:r1], sx[:r1], qr[:r1], sr[:r1], wq, sw)
                t1 = time.perf_counter() - t0
        gbs = QUANT_BYTES_PER_ELEM * q_rows * c.K / t_q / 1e9
        tf = 4.0 * g_rows * n_cols * c.K / t_g / 1e12
        t_step = QUANT_BYTES_PER_ELEM * c.M * c.K / (gbs * 1e9) + 4.0 * c.M * c.N * c.K / (tf * 1e12)
        out[name] = {
            "quantize_GB_per_s_1_thread": round(gbs, 4),
            "gemm_TFLOP_per_s": round(tf, 5),
            "gemm_TFLOP_per_s_1_thread": round(4.0 * r1 * n_cols * c.K / t1 / 1e12, 5) if t1 else None,
            "step_s_extrapolated": round(t_step, 2),
            "sample": f"quantize {q_rows} rows; GEMM {g_rows} x {n_cols} outputs ({blas_threads} threads), "
                      f"{r1} x {n_cols} (1 thread)",
        }
    return out


def mfma_ceiling(rfq, torch, qx, qr, wq, stream, sp, iters=2000, reps=5, e4m3=None):
    """The power-limited ceiling of the GEMM's instruction on this workload's
    own operand bytes: rfq_probe_mfma_ceiling runs only scaled FP4 MFMAs (no
    memory traffic in the loop), one 8-wave workgroup per CU; the A operands
    interleave Q(X) and Q(R) codes, the B operands are weight codes. With
    `e4m3` (MXFP8 activation codes) it times the E2M1 x E4M3 instruction of
    the W4A8 GEMM instead (rfq_probe_mfma_ceiling_e4m3: weight codes first,
    E4M3 codes second)."""
    import bench_probe
    lib = bench_probe.load()
    props = torch.cuda.get_device_properties(0)
    wgs = props.multi_processor_count
    if e4m3 is None:
        n = min(qx.numel(), qr.numel(), wq.numel(), 1 << 23) // 32 * 16
        a = torch.stack([qx.view(-1)[:n].view(-1, 16), qr.view(-1)[:n].view(-1, 16)], 1).reshape(-1).contiguous()
        b = wq.view(-1)[:2 * n].contiguous()
        fn = lib.rfq_probe_mfma_ceiling
    else:
        a = wq.view(-1)[:1 << 22].contiguous()
        b = e4m3.view(-1)[:1 << 23].contiguous()
        fn = lib.rfq_probe_mfma_ceiling_e4m3
    stamps = torch.zeros(2 * wgs, dtype=torch.int64, device=qx.device)
    sink = torch.empty(512 * wgs, dtype=torch.float32, device=qx.device)
    call = lambda: bench_probe.check(fn(a.data_ptr(), a.numel(), b.data_ptr(), b.numel(), wgs, iters,
                                        stamps.data_ptr(), sink.data_ptr(), sp))
    call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = 2.0 * 32 * 32 * 64 * 32 * 8 * iters * wgs
    st = stamps.cpu().numpy().reshape(-1, 2).astype(np.float64)
    clock = float(np.median(st[:, 0] / (st[:, 1] * 10.0)))      # cycles per 100 MHz tick -> GHz
    tf = flops / (ms * 1e-3) / 1e12
    if e4m3 is not None:
        return {"TFLOP_per_s": round(tf, 1), "pct_of_datasheet_fp8_peak": round(100 * tf / FP8_PEAK_TFLOPS, 2),
                "shader_clock_GHz": round(clock, 3),
                "what": "scaled E2M1 x E4M3 16x16x128 MFMA loop (the W4A8 GEMM's instruction) on this workload's W "
                        "and MXFP8 X codes, no memory traffic, one 8-wave workgroup per CU "
                        "(rfq_probe_mfma_ceiling_e4m3)"}
    return {"TFLOP_per_s": round(tf, 1), "pct_of_datasheet_peak": round(100 * tf / FP4_PEAK_TFLOPS, 2),
            "shader_clock_GHz": round(clock, 3),
            "what": "scaled FP4 16x16x128 MFMA loop (the GEMM's instruction) on this workload's Q(X)/Q(R) and W codes, no memory traffic, "
                    "one 8-wave workgroup per CU (rfq_probe_mfma_ceiling)"}


def library_reference(rfq, torch, qx, qr, wq, M, N, K, batch_ms, gemm_ms, w4a4_ms, w4a8_ms, bdx_ms):
    """The vendor library's GEMMs on this layer's operands, for context (not
    part of the path): torch._scaled_mm (hipBLASLt) with MXFP4 operands, as
    one call on [Q(X) | Q(R)] against [Wq | Wq] (the K-doubled contraction;
    the concatenations are made outside the timed region) and as the plain
    W4A4 product; its block-scaled MXFP8 GEMM with both operands in E4M3 (the
    nearest library operation to W4A8, whose instruction runs at the same
    rate) and its FP8 GEMM with one scale per tensor; and a bf16 torch.matmul
    of the dX shape. Unit scales (E8M0
    code 127) in the MXFP4 calls: the time does not depend on the scale
    values, and with unit scales every output is a sum of E2M1 products that
    fp32 holds exactly (|Y| < 36 K, in steps of 1/4): rfq_gemm_w4a4's fp32 Y
    is that exact sum, and the library's bf16 Y (it takes bf16 or fp16
    output with block scales) is checked bit for bit against it cut to bf16
    (the library truncates to bf16 where this GEMM rounds to nearest even),
    which shows that both read the codes alike."""
    if not (hasattr(torch, "float4_e2m1fn_x2") and hasattr(torch, "float8_e8m0fnu")):
        return {"available": False, "reason": "this torch build has no float4_e2m1fn_x2 / float8_e8m0fnu dtypes"}
    dev = qx.device
    fp4, e8 = torch.float4_e2m1fn_x2, torch.float8_e8m0fnu

    def unit(rows, k):
        return torch.full((rows, k // 32), 127, dtype=torch.uint8, device=dev)

    try:
        ua, ub = unit(M, K), unit(N, K)
        y_lib = torch._scaled_mm(qx.view(fp4), wq.view(fp4).t(), ua.view(e8), ub.view(e8), out_dtype=torch.bfloat16)
        y_own = rfq.gemm_w4a4(qx, ua, None, None, wq, ub, out_dtype=torch.float32)
        cut = (y_own.view(torch.int32) >> 16).to(torch.int16)
        same = float((y_lib.view(torch.int16) == cut).float().mean())
        del y_lib, y_own, cut
        a2, b2 = torch.cat([qx, qr], dim=1), torch.cat([wq, wq], dim=1)
        ua2, ub2 = unit(M, 2 * K), unit(N, 2 * K)
        lib_k2_ms = batch_ms(lambda: torch._scaled_mm(a2.view(fp4), b2.view(fp4).t(), ua2.view(e8), ub2.view(e8),
                                                      out_dtype=torch.bfloat16), 30, warm=5)
        lib_k_ms = batch_ms(lambda: torch._scaled_mm(qx.view(fp4), wq.view(fp4).t(), ua.view(e8), ub.view(e8),
                                                     out_dtype=torch.bfloat16), 30, warm=5)
        del a2, b2, ua2, ub2
    except Exception as e:   # a torch build without MXFP4 support in _scaled_mm
        return {"available": False, "reason": f"{type(e).__name__}: {str(e)[:200]}"}
    gen = torch.Generator(device=dev)
    gen.manual_seed(1)
    try:
        a8 = torch.randn((M, K), generator=gen, device=dev).to(torch.float8_e4m3fn)
        b8 = torch.randn((N, K), generator=gen, device=dev).to(torch.float8_e4m3fn)
        ua, ub = unit(M, K), unit(N, K)
        one = torch.ones((), device=dev)
        mx8_ms = batch_ms(lambda: torch._scaled_mm(a8, b8.t(), ua.view(e8), ub.view(e8), out_dtype=torch.bfloat16),
                          20, warm=5)
        fp8_ms = batch_ms(lambda: torch._scaled_mm(a8, b8.t(), one, one, out_dtype=torch.bfloat16), 20, warm=5)
        del a8, b8
    except Exception:
        mx8_ms = fp8_ms = None
    dy = torch.randn((M, N), generator=gen, device=dev).to(torch.bfloat16)
    wd = torch.randn((N, K), generator=gen, device=dev).to(torch.bfloat16)
    mm_ms = batch_ms(lambda: torch.matmul(dy, wd), 10, warm=3)
    del dy, wd
    return {
        "available": True,
        "what": "torch._scaled_mm (hipBLASLt) with MXFP4 operands, with E4M3 operands (block scales, or one scale per "
                "tensor), bf16 Y; torch.matmul in bf16",
        "mxfp4_k_doubled_us": round(lib_k2_ms * 1e3, 2),
        "rfq_gemm_us": round(gemm_ms * 1e3, 2),
        "rfq_gemm_speedup_over_library": round(lib_k2_ms / gemm_ms, 3),
        "mxfp4_plain_w4a4_us": round(lib_k_ms * 1e3, 2),
        "plain_w4a4_us": round(w4a4_ms * 1e3, 2),
        "plain_w4a4_speedup_over_library": round(lib_k_ms / w4a4_ms, 3),
        "library_bf16_y_equal_to_exact_y_truncated": round(same, 6),
        "mxfp8_e4m3_us": round(mx8_ms * 1e3, 2) if mx8_ms else None,
        "fp8_per_tensor_scale_us": round(fp8_ms * 1e3, 2) if fp8_ms else None,
        "w4a8_us": round(w4a8_ms * 1e3, 2),
        "bf16_matmul_dx_shape_us": round(mm_ms * 1e3, 2),
        "backward_dx_call_us": round(bdx_ms * 1e3, 2),
    }


def layer_timings(rfq, torch, cfg, x, wq, sw, batch_ms, reps):
    """Quantize pass, GEMM and the whole step (both, back to back) of one
    configuration's layer, each averaged over `reps` back-to-back launches
    between two events on the launch stream."""
    M, N, K = cfg.M, cfg.N, cfg.K
    dev = x.device
    lib = rfq.library()
    sp = rfq._stream()
    qx = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    qr = torch.empty_like(qx)
    sx = torch.empty((M, K // 32), dtype=torch.uint8, device=dev)
    sr = torch.empty_like(sx)
    yd = rfq._lib.DTYPE_FP32 if cfg.y_dtype == "fp32" else rfq._lib.DTYPE_BF16
    y = torch.empty((M, N), dtype=torch.float32 if cfg.y_dtype == "fp32" else torch.bfloat16, device=dev)

    def quantize():
        rfq._lib.check(lib.rfq_residual_quantize(x.data_ptr(), 0, M, K, x.stride(0), qx.data_ptr(), sx.data_ptr(),
                                                 qr.data_ptr(), sr.data_ptr(), sp))

    def gemm():
        rfq._lib.check(lib.rfq_gemm_w4a4(qx.data_ptr(), sx.data_ptr(), qr.data_ptr(), sr.data_ptr(), wq.data_ptr(),
                                         sw.data_ptr(), M, N, K, y.data_ptr(), yd, N, sp))

    def step():
        quantize()
        gemm()

    def fused():
        rfq._lib.check(lib.rfq_linear_fused(x.data_ptr(), 0, M, K, x.stride(0), wq.data_ptr(), sw.data_ptr(), N,
                                            y.data_ptr(), yd, N, sp))
    # a short ramp of steps first: the kernels timed before the sweep (the
    # backward pass, the MXFP8 GEMMs) leave the clock in a state that takes a
    # few hundred steps to settle, which showed up as a step slower than its
    # two kernels' sum
    torch.cuda.synchronize()
    t_ramp = time.perf_counter()
    while time.perf_counter() - t_ramp < 0.3:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
    s_ms, q_ms, g_ms = batch_ms(step, reps), batch_ms(quantize, reps), batch_ms(gemm, reps)
    f_ms = batch_ms(fused, reps) if K % 512 == 0 else None
    flops = 4.0 * M * N * K
    return {
        "M": M, "K": K, "N": N, "y_dtype": cfg.y_dtype,
        "step_us": round(s_ms * 1e3, 2),
        "step_TFLOP_per_s": round(flops / (s_ms * 1e-3) / 1e12, 1),
        "gemm_us": round(g_ms * 1e3, 2),
        "gemm_TFLOP_per_s": round(flops / (g_ms * 1e-3) / 1e12, 1),
        "gemm_pct_fp4_peak": round(100 * flops / (g_ms * 1e-3) / 1e12 / FP4_PEAK_TFLOPS, 2),
        "quantize_us": round(q_ms * 1e3, 2),
        "quantize_GB_per_s": round(QUANT_BYTES_PER_ELEM * M * K / (q_ms * 1e-3) / 1e9, 1),
        "fused_step_us": round(f_ms * 1e3, 2) if f_ms else None,
        "fused_over_two_kernel_step": round(f_ms / s_ms, 3) if f_ms else None,
        "reps": reps,
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the layer would shard by rows of X, with no exchange between GPUs)", file=sys.stderr)
        return 2

    import torch
    import mxfp4_activation_gemm_amd as rfq
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    rfq.library()
    cfg = workloads.CONFIGS[args.workload]
    M, N, K = cfg.M, cfg.N, cfg.K
    dev = torch.device("cuda:0")

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    progress(f"generating {cfg.name} inputs")
    x = to_dev(workloads.x_bf16(cfg))
    w = to_dev(workloads.w_bf16(cfg))
    wq, sw = rfq.quantize_mxfp4(w)                 # setup: the weight is quantized once
    del w
    qx = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    qr = torch.empty_like(qx)
    sx = torch.empty((M, K // 32), dtype=torch.uint8, device=dev)
    sr = torch.empty_like(sx)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    lib = rfq.library()
    stream = torch.cuda.current_stream()
    sp = rfq._stream()

    def quantize():
        rfq._lib.check(lib.rfq_residual_quantize(x.data_ptr(), 0, M, K, x.stride(0), qx.data_ptr(), sx.data_ptr(),
                                                 qr.data_ptr(), sr.data_ptr(), sp))

    def gemm():
        rfq._lib.check(lib.rfq_gemm_w4a4(qx.data_ptr(), sx.data_ptr(), qr.data_ptr(), sr.data_ptr(), wq.data_ptr(),
                                         sw.data_ptr(), M, N, K, y.data_ptr(), rfq._lib.DTYPE_BF16, N, sp))

    def step(ev=None):
        # the two launches of rfq_linear; events around the GEMM call
        quantize()
        if ev is not None:
            ev[0].record(stream)
        gemm()
        if ev is not None:
            ev[1].record(stream)

    # Clock ramp: generating the inputs on the host leaves the GPU idle for
    # several seconds, and a few warmup steps (~0.3 ms each) are not enough
    # for it to leave its idle clock state; so untimed steps run for
    # --ramp-seconds first, then the --warmup steps, then the timed steps.
    progress("clock ramp, warmup and timed steps")
    torch.cuda.synchronize()
    ramp_steps, t_ramp = 0, time.perf_counter()
    while time.perf_counter() - t_ramp < args.ramp_seconds:
        for _ in range(50):
            step()
        ramp_steps += 50
        torch.cuda.synchronize()
    ramp_s = time.perf_counter() - t_ramp
    for _ in range(args.warmup):
        step()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    gemm_times = np.array([e[0].elapsed_time(e[1]) for e in events])
    gemm_ms = float(gemm_times.mean())
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def batch_ms(fn, reps, warm=3):
        # back-to-back launches between two events: the per-launch time
        # without an event between launches
        for _ in range(warm):
            fn()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    progress("kernel timings")
    quant_ms = batch_ms(quantize, 100)

    # the same pass with its inputs and outputs rotated over 8 buffer sets
    # (514 MB, more than the 256 MB last-level cache), so that each launch
    # reads X from HBM
    cold_sets = [(x.clone(), torch.empty_like(qx), torch.empty_like(sx), torch.empty_like(qr), torch.empty_like(sr))
                 for _ in range(8)]
    cold_i = [0]

    def quantize_cold():
        xc, a, b, c, d = cold_sets[cold_i[0] % 8]
        cold_i[0] += 1
        rfq._lib.check(lib.rfq_residual_quantize(xc.data_ptr(), 0, M, K, xc.stride(0), a.data_ptr(), b.data_ptr(),
                                                 c.data_ptr(), d.data_ptr(), sp))
    cold_ms = batch_ms(quantize_cold, 96)
    del cold_sets

    def rotated_quantize():
        rfq._lib.check(lib.rfq_rotate_residual_quantize(x.data_ptr(), 0, M, K, x.stride(0), qx.data_ptr(), sx.data_ptr(),
                                                        qr.data_ptr(), sr.data_ptr(), sp))
    rot_ms = batch_ms(rotated_quantize, 100)

    def rotated64_quantize():
        rfq._lib.check(lib.rfq_rotate64_residual_quantize(x.data_ptr(), 0, M, K, x.stride(0), qx.data_ptr(),
                                                          sx.data_ptr(), qr.data_ptr(), sr.data_ptr(), sp))
    rot64_ms = batch_ms(rotated64_quantize, 100)

    flops = 4.0 * M * N * K
    value = flops / (ms_per_step * 1e-3) / 1e12
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    quant_gbs = QUANT_BYTES_PER_ELEM * M * K / (quant_ms * 1e-3) / 1e9

    # the layer with the quantization inside the GEMM (rfq_linear_fused: one
    # launch, Q(X) and Q(R) never leave the GEMM) beside the two-kernel step
    def fused_step():
        rfq._lib.check(lib.rfq_linear_fused(x.data_ptr(), 0, M, K, x.stride(0), wq.data_ptr(), sw.data_ptr(), N,
                                            y.data_ptr(), rfq._lib.DTYPE_BF16, N, sp))
    fused_ms = batch_ms(fused_step, 50, warm=10) if K % 512 == 0 else None
    two_kernel_ms = batch_ms(step, 50, warm=10)

    # plain W4A4 GEMM (no residual operand) on the same operands, for the
    # overhead of the residual path
    w4a4_ms = batch_ms(lambda: rfq.gemm_w4a4(qx, sx, None, None, wq, sw, out=y), 50)

    ceiling = mfma_ceiling(rfq, torch, qx, qr, wq, stream, sp)

    # MXFP8 variants on the same layer: W4A8 (X in MXFP8) and RFQ whose
    # second path quantizes R to MXFP8; the weight stays MXFP4
    qx8 = torch.empty((M, K), dtype=torch.uint8, device=dev)
    qr8 = torch.empty((M, K), dtype=torch.uint8, device=dev)

    def quantize8():
        rfq._lib.check(lib.rfq_quantize_mxfp8(x.data_ptr(), 0, M, K, x.stride(0), qx8.data_ptr(), sx.data_ptr(), sp))

    def quantize_r8():
        rfq._lib.check(lib.rfq_residual_quantize_mxfp8(x.data_ptr(), 0, M, K, x.stride(0), qx.data_ptr(),
                                                       sx.data_ptr(), qr8.data_ptr(), sr.data_ptr(), sp))
    q8_ms = batch_ms(quantize8, 100)
    qr8_ms = batch_ms(quantize_r8, 100)
    quantize8()
    w4a8_ms = batch_ms(lambda: rfq._lib.check(lib.rfq_gemm_w4a8(
        qx8.data_ptr(), sx.data_ptr(), wq.data_ptr(), sw.data_ptr(), M, N, K, y.data_ptr(), rfq._lib.DTYPE_BF16, N,
        sp)), 50)
    ceiling8 = mfma_ceiling(rfq, torch, qx, qr, wq, stream, sp, e4m3=qx8)
    quantize_r8()
    rfq8_ms = batch_ms(lambda: rfq._lib.check(lib.rfq_gemm_w4a4_mxfp8_residual(
        qx.data_ptr(), sx.data_ptr(), qr8.data_ptr(), sr.data_ptr(), wq.data_ptr(), sw.data_ptr(), M, N, K,
        y.data_ptr(), rfq._lib.DTYPE_BF16, N, sp)), 50)
    w4a8_tf = 2.0 * M * N * K / (w4a8_ms * 1e-3) / 1e12
    # instruction time of the MXFP8-residual GEMM in E2M1-MFMA units: one
    # E2M1 x E2M1 MFMA per X term, one E2M1 x E4M3 (twice the cycles) per R term
    rfq8_tf = 4.0 * M * N * K / (rfq8_ms * 1e-3) / 1e12
    del qx8, qr8

    # straight-through backward pass of the same layer: dX = dY deq(Wq) and
    # dW = dY^T (deq Q(X) + deq Q(R)), each one entry-point call (operand
    # staging + bf16 GEMM); dY is a seeded N(0, 1) bf16 tensor. (10 untimed
    # calls first: the first few calls of a new kernel mix run up to 10%
    # slower than the steady state.)
    quantize()
    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg.seed)
    dy = torch.randn((M, N), generator=gen, device=dev).to(torch.bfloat16)
    ws_dx = torch.empty(lib.rfq_backward_dx_workspace_size(N, K), dtype=torch.uint8, device=dev)
    ws_dw = torch.empty(lib.rfq_backward_dw_workspace_size(M, N, K), dtype=torch.uint8, device=dev)
    g_dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    g_dw = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    bdx_ms = batch_ms(lambda: rfq._lib.check(lib.rfq_backward_dx(
        dy.data_ptr(), 0, M, N, N, wq.data_ptr(), sw.data_ptr(), K, g_dx.data_ptr(), rfq._lib.DTYPE_BF16, K,
        ws_dx.data_ptr(), ws_dx.numel(), sp)), 20, warm=10)
    bdw_ms = batch_ms(lambda: rfq._lib.check(lib.rfq_backward_dw(
        dy.data_ptr(), 0, M, N, N, qx.data_ptr(), sx.data_ptr(), qr.data_ptr(), sr.data_ptr(), K, g_dw.data_ptr(),
        rfq._lib.DTYPE_BF16, K, ws_dw.data_ptr(), ws_dw.numel(), sp)), 20, warm=10)
    del dy, ws_dx, ws_dw, g_dx, g_dw
    progress("library reference")
    library = library_reference(rfq, torch, qx, qr, wq, M, N, K, batch_ms, gemm_ms, w4a4_ms, w4a8_ms, bdx_ms)

    kernel_hash = source_hash("gemm.hip")
    traffic = counter_traffic(args.workload, kernel_hash)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "clock_ramp": {"untimed_steps": ramp_steps, "seconds": round(ramp_s, 3),
                       "note": "untimed steps before the warmup steps, so that the GPU leaves its idle clock state "
                               "after the host-side input generation"},
        "dtype": "fp4",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: {cfg.description}",
            "M": M, "N": N, "K": K,
            "x_dtype": "bf16", "y_dtype": "bf16",
            "flops_per_step": flops,
            "pct_fp4_peak_whole_step": round(100 * value / FP4_PEAK_TFLOPS, 2),
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "rfq_gemm_w4a4 (K-doubled FP4 GEMM)",
            "achieved": round(gemm_tflops, 2),
            "peak": FP4_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(gemm_tflops / FP4_PEAK_TFLOPS, 4),
            "traffic": traffic,
            "avg_launch_us": round(gemm_ms * 1e3, 2),
            "median_launch_us": round(float(np.median(gemm_times)) * 1e3, 2),
            "iqr_launch_us": [round(float(np.percentile(gemm_times, 25)) * 1e3, 2),
                              round(float(np.percentile(gemm_times, 75)) * 1e3, 2)],
            "first_launches_us": [round(float(t) * 1e3, 2) for t in gemm_times[:5]],
            "last_launches_us": [round(float(t) * 1e3, 2) for t in gemm_times[-5:]],
            "measured_mfma_ceiling": dict(ceiling, frac_of_ceiling=round(gemm_tflops / ceiling["TFLOP_per_s"], 4)),
        },
        "kernels": {
            "quantize_residual_cache_resident": {
                "avg_launch_us": round(quant_ms * 1e3, 2),
                "GB_per_s": round(quant_gbs, 1),
                "pct_of_hbm_peak_rate": round(100 * quant_gbs / HBM_PEAK_GBS, 2),
                "algorithmic_bytes": QUANT_BYTES_PER_ELEM * M * K,
                "note": "100 back-to-back launches on the same buffers: the 64 MB working set is partly served by the "
                        "256 MB last-level cache, so this is not an HBM figure (see quantize_residual_cold and the "
                        "top-level quantize_hbm)",
            },
            "quantize_residual_cold": {
                "avg_launch_us": round(cold_ms * 1e3, 2),
                "GB_per_s": round(QUANT_BYTES_PER_ELEM * M * K / (cold_ms * 1e-3) / 1e9, 1),
                "pct_hbm_peak": round(100 * QUANT_BYTES_PER_ELEM * M * K / (cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                "note": "96 launches rotating over 8 input/output buffer sets (514 MB): X comes from HBM",
            },
            "quantize_residual_rotated": {
                "avg_launch_us": round(rot_ms * 1e3, 2),
                "GB_per_s": round(QUANT_BYTES_PER_ELEM * M * K / (rot_ms * 1e-3) / 1e9, 1),
                "pct_hbm_peak": round(100 * QUANT_BYTES_PER_ELEM * M * K / (rot_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                "what": "32-point block Hadamard of X fused before the RFQ pass (rfq_rotate_residual_quantize)",
            },
            "quantize_residual_rotated64": {
                "avg_launch_us": round(rot64_ms * 1e3, 2),
                "GB_per_s": round(QUANT_BYTES_PER_ELEM * M * K / (rot64_ms * 1e-3) / 1e9, 1),
                "pct_hbm_peak": round(100 * QUANT_BYTES_PER_ELEM * M * K / (rot64_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                "what": "64-point block Hadamard (two MX blocks) of X fused before the RFQ pass "
                        "(rfq_rotate64_residual_quantize)",
            },
            "gemm_rfq": {
                "avg_launch_us": round(gemm_ms * 1e3, 2),
                "TFLOP_per_s": round(gemm_tflops, 1),
                "pct_fp4_peak": round(100 * gemm_tflops / FP4_PEAK_TFLOPS, 2),
            },
            "quantize_mxfp8": {
                "avg_launch_us": round(q8_ms * 1e3, 2),
                "GB_per_s": round(QUANT8_BYTES_PER_ELEM * M * K / (q8_ms * 1e-3) / 1e9, 1),
                "pct_hbm_peak": round(100 * QUANT8_BYTES_PER_ELEM * M * K / (q8_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                "algorithmic_bytes": QUANT8_BYTES_PER_ELEM * M * K,
                "what": "X to MXFP8 (E4M3) for W4A8 (rfq_quantize_mxfp8)",
            },
            "quantize_residual_mxfp8": {
                "avg_launch_us": round(qr8_ms * 1e3, 2),
                "GB_per_s": round(QUANT_R8_BYTES_PER_ELEM * M * K / (qr8_ms * 1e-3) / 1e9, 1),
                "pct_hbm_peak": round(100 * QUANT_R8_BYTES_PER_ELEM * M * K / (qr8_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                "algorithmic_bytes": QUANT_R8_BYTES_PER_ELEM * M * K,
                "what": "Q4(X) and the residual to MXFP8 (rfq_residual_quantize_mxfp8)",
            },
            "gemm_w4a8": {
                "avg_launch_us": round(w4a8_ms * 1e3, 2),
                "TFLOP_per_s_2MNK": round(w4a8_tf, 1),
                "pct_fp8_peak": round(100 * w4a8_tf / FP8_PEAK_TFLOPS, 2),
                "measured_mfma_ceiling": dict(ceiling8, frac_of_ceiling=round(w4a8_tf / ceiling8["TFLOP_per_s"], 4)),
            },
            "gemm_rfq_mxfp8_residual": {
                "avg_launch_us": round(rfq8_ms * 1e3, 2),
                "TFLOP_per_s_4MNK": round(rfq8_tf, 1),
                "over_rfq_time": round(rfq8_ms / gemm_ms, 3),
                "note": "128 x 256 tiles; per output tile the E2M1 x E4M3 residual MFMAs take twice the cycles of the "
                        "E2M1 ones, so the instruction-time floor is 1.5x the RFQ GEMM's",
            },
            "backward_dx": {
                "avg_call_us": round(bdx_ms * 1e3, 2),
                "TFLOP_per_s_2MNK": round(2.0 * M * N * K / (bdx_ms * 1e-3) / 1e12, 1),
                "pct_bf16_peak": round(100 * 2.0 * M * N * K / (bdx_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 2),
                "what": "dX = dY deq(Wq) (rfq_backward_dx: decode-transpose of Wq, then the bf16 GEMM), bf16 dX",
            },
            "backward_dw": {
                "avg_call_us": round(bdw_ms * 1e3, 2),
                "TFLOP_per_s_4MNK": round(4.0 * M * N * K / (bdw_ms * 1e-3) / 1e12, 1),
                "pct_bf16_peak": round(100 * 4.0 * M * N * K / (bdw_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 2),
                "what": "dW = dY^T (deq Q(X) + deq Q(R)) (rfq_backward_dw: transposes of dY, Q(X), Q(R), then the "
                        "K-doubled bf16 GEMM with transposed store), bf16 dW",
            },
            "rfq_linear_fused": {
                "avg_call_us": round(fused_ms * 1e3, 2) if fused_ms else None,
                "TFLOP_per_s": round(flops / (fused_ms * 1e-3) / 1e12, 1) if fused_ms else None,
                "two_kernel_step_us": round(two_kernel_ms * 1e3, 2),
                "fused_over_two_kernel": round(fused_ms / two_kernel_ms, 3) if fused_ms else None,
                "what": "the layer with Q(X), Q(R) formed inside the GEMM from bf16 X tiles (one launch, 128 x 256 "
                        "tiles), against the quantize pass + GEMM step, same launches back to back",
            },
            "gemm_plain_w4a4": {
                "avg_launch_us": round(w4a4_ms * 1e3, 2),
                "TFLOP_per_s_2MNK": round(2.0 * M * N * K / (w4a4_ms * 1e-3) / 1e12, 1),
                "rfq_over_w4a4_time": round(gemm_ms / w4a4_ms, 3),
            },
        },
        "library_reference": library,
    }
    sweep = {}
    progress("configuration sweep")
    if not args.no_sweep:
        sweep[cfg.name] = layer_timings(rfq, torch, cfg, x, wq, sw, batch_ms, 50)
    del qx, qr, sx, sr, y, x

    if not args.no_sweep:
        for name in ("tiny", "qwen3vl_attn_proj", "qwen3vl_ffn_up", "wan22_ffn"):
            if name in sweep:
                continue
            c = workloads.CONFIGS[name]
            xc = to_dev(workloads.x_bf16(c))
            wqc, swc = rfq.quantize_mxfp4(to_dev(workloads.w_bf16(c)))
            sweep[name] = layer_timings(rfq, torch, c, xc, wqc, swc, batch_ms, 50)
            del xc, wqc, swc

    if not args.no_hbm_quantize or not args.no_sweep:
        # the quantize pass on the long-sequence layer, whose traffic (1.39 GB)
        # exceeds the 256 MB last-level cache, so the figure is HBM-bound
        c5 = workloads.CONFIGS["dit_ffn_down"]
        x5 = to_dev(workloads.x_bf16(c5))
        q5 = [torch.empty((c5.M, c5.K // 2), dtype=torch.uint8, device=dev) for _ in range(2)]
        s5 = [torch.empty((c5.M, c5.K // 32), dtype=torch.uint8, device=dev) for _ in range(2)]

        def q5_step():
            rfq._lib.check(lib.rfq_residual_quantize(x5.data_ptr(), 0, c5.M, c5.K, c5.K, q5[0].data_ptr(),
                                                     s5[0].data_ptr(), q5[1].data_ptr(), s5[1].data_ptr(), sp))
        # (each pass gets 20 untimed launches first: the first few dozen
        # launches of a new kernel on this 1.4 GB working set run up to 20%
        # slower than the steady state)
        q5_ms = batch_ms(q5_step, 40, warm=20)
        gbs = QUANT_BYTES_PER_ELEM * c5.M * c5.K / (q5_ms * 1e-3) / 1e9

        def q5_rot():
            rfq._lib.check(lib.rfq_rotate_residual_quantize(x5.data_ptr(), 0, c5.M, c5.K, c5.K, q5[0].data_ptr(),
                                                            s5[0].data_ptr(), q5[1].data_ptr(), s5[1].data_ptr(), sp))
        q5r_ms = batch_ms(q5_rot, 40, warm=20)
        gbs_rot = QUANT_BYTES_PER_ELEM * c5.M * c5.K / (q5r_ms * 1e-3) / 1e9

        def q5_rot64():
            rfq._lib.check(lib.rfq_rotate64_residual_quantize(x5.data_ptr(), 0, c5.M, c5.K, c5.K, q5[0].data_ptr(),
                                                              s5[0].data_ptr(), q5[1].data_ptr(), s5[1].data_ptr(), sp))
        q5r64_ms = batch_ms(q5_rot64, 40, warm=20)
        gbs_rot64 = QUANT_BYTES_PER_ELEM * c5.M * c5.K / (q5r64_ms * 1e-3) / 1e9
        if not args.no_sweep and "dit_ffn_down" not in sweep:
            w5q, w5s = rfq.quantize_mxfp4(to_dev(workloads.w_bf16(c5)))
            sweep["dit_ffn_down"] = layer_timings(rfq, torch, c5, x5, w5q, w5s, batch_ms, 10)
            del w5q, w5s
        del x5, q5, s5
        # what a plain device-to-device copy reaches on this HBM (read + write)
        ca = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        cb = torch.empty_like(ca)
        copy_ms = batch_ms(lambda: cb.copy_(ca), 10)
        copy_gbs = 2.0 * ca.numel() / (copy_ms * 1e-3) / 1e9
        del ca, cb
        out["kernels"]["quantize_residual_dit_ffn_down"] = {
            "shape": [c5.M, c5.K],
            "avg_launch_us": round(q5_ms * 1e3, 2),
            "GB_per_s": round(gbs, 1),
            "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "pct_of_device_copy": round(100 * gbs / copy_gbs, 2),
        }
        # the quantize half of the metric: the pass's HBM-bound rate, on the
        # layer whose traffic (1.39 GB) is larger than the last-level cache
        out["quantize_hbm"] = {
            "kernel": "rfq_residual_quantize (Q(X), R in fp32, Q(R); one pass)",
            "workload": f"{c5.name}: X [{c5.M}, {c5.K}] bf16",
            "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "algorithmic_bytes_per_launch": QUANT_BYTES_PER_ELEM * c5.M * c5.K,
            "avg_launch_us": round(q5_ms * 1e3, 2),
        }
        out["kernels"]["quantize_residual_rotated_dit_ffn_down"] = {
            "shape": [c5.M, c5.K],
            "avg_launch_us": round(q5r_ms * 1e3, 2),
            "GB_per_s": round(gbs_rot, 1),
            "pct_hbm_peak": round(100 * gbs_rot / HBM_PEAK_GBS, 2),
        }
        out["kernels"]["quantize_residual_rotated64_dit_ffn_down"] = {
            "shape": [c5.M, c5.K],
            "avg_launch_us": round(q5r64_ms * 1e3, 2),
            "GB_per_s": round(gbs_rot64, 1),
            "pct_hbm_peak": round(100 * gbs_rot64 / HBM_PEAK_GBS, 2),
        }
        out["kernels"]["hbm_device_copy_reference"] = {
            "bytes_moved": 2 * (1 << 30), "GB_per_s": round(copy_gbs, 1),
            "pct_hbm_peak": round(100 * copy_gbs / HBM_PEAK_GBS, 2),
        }

    if sweep:
        out["configs"] = dict(sweep, note="RFQ layer on each configuration: quantize + residual pass, K-doubled GEMM, "
                                          "and the step (both back to back), averaged over back-to-back launches; "
                                          "TFLOP/s count 4 M N K")

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = a.numel()

    if not args.no_cpu_baseline:
        progress("oracle timing on the host")
        out["cpu_baseline"] = cpu_baseline(cfg)
        if not args.no_sweep:
            out["cpu_baseline"]["per_config"] = oracle_config_timings()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
