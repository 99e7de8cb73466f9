"""Shared helpers for the GPU parity tests: device transfer and the
comparison rules. Expected values always come from the CPU oracle."""
import json
import os
import sys

import numpy as np
import torch

import oracle

# Tolerance on each output, relative to its condition scale S = sum |terms|:
# fp32 accumulation of the K-doubled sum in an order the oracle does not fix.
REL_TOL = 1e-5
BF16_HALF_ULP = 2.0 ** -8          # RNE to bfloat16: |error| <= 2^-8 |value|


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits):
    """uint16 bf16 bits (numpy) -> CUDA bfloat16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def host(t):
    return t.cpu().numpy()


def host_bf16_as_f64(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16).astype(np.uint32).__lshift__(16).view(np.float32).astype(
        np.float64)


def oracle_mx(x_bits):
    """Oracle Q(X) for bf16 bits: packed codes and scales."""
    codes, scales = oracle.quantize_mxfp4(oracle.bf16_bits_to_f64(x_bits))
    return oracle.pack_codes(codes), scales


def oracle_rfq(x_bits):
    qx, sx, qr, sr = oracle.residual_quantize(oracle.bf16_bits_to_f64(x_bits))
    return oracle.pack_codes(qx), sx, oracle.pack_codes(qr), sr


def assert_bytes_equal(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{what}: {len(bad)} mismatching bytes, first at {bad[:5].tolist()}: " \
                          f"got {got[tuple(bad[0])]} want {want[tuple(bad[0])]}"


def e4m3_group_bound(a, w):
    """Bound on what the scaled MFMA's E4M3 arithmetic drops from Y = a w^T
    (a [M, K] decoded E4M3 operand values with their scales, w [N, K] the
    decoded E2M1 weight).

    Measured on gfx950 with single-output probes (one-hot and two-term
    operands; the two-term facts are pinned in test_gpu_mxfp8): within every
    aligned group of 8 consecutive K positions, products far below the
    group's largest come back truncated toward zero to a multiple of
    2^(E - 13), E the largest sum of the two operands' binary exponents in
    the group, while products in different groups add without that loss.
    With at most 7 truncated products per group and 2^E <= max|a| max|w|
    over the group, a group loses less than 7 * 2^-13 * max|a| max|w|.
    Returns that sum over groups, [M, N]."""
    M, K = a.shape
    ag = np.abs(a).reshape(M, K // 8, 8).max(axis=2)
    wg = np.abs(w).reshape(w.shape[0], K // 8, 8).max(axis=2)
    return 7.0 * 2.0 ** -13 * (ag @ wg.T)


def record_stats(**fields):
    """Appends one JSON line of parity statistics to the file named by the
    RFQ_PARITY_STATS environment variable, if set (a run artefact to read
    back; the tests' verdicts do not depend on it)."""
    path = os.environ.get("RFQ_PARITY_STATS")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(fields) + "\n")


def check_y(y_gpu, y_ref, s_ref, out_dtype, what="", extra=None):
    """Per-output check: fp32 |dY| <= 1e-5 S (+ `extra`, a per-output bound on
    what the instruction itself drops); bf16 adds the RNE half-ulp. Returns
    the largest |dY| / S; with `extra`, also records how close the outputs
    come to the plain 1e-5 S gate and to the widened bound."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    gate = REL_TOL * s_ref + 2.0 ** -126
    tol = gate if extra is None else gate + extra
    if out_dtype == torch.bfloat16:
        tol = tol * (1 + BF16_HALF_ULP) + BF16_HALF_ULP * np.abs(y_ref) + 2.0 ** -133
    err = np.abs(y_gpu - y_ref)
    bad = np.argwhere(~(err <= tol))
    worst = float(np.max(err / np.maximum(s_ref, 1e-300)))
    stats = dict(what=what, out=str(out_dtype).replace("torch.", ""), outputs=int(err.size),
                 max_err_over_S=worst, max_err_over_tol=float(np.max(err / tol)))
    if extra is not None:
        plain = gate if out_dtype != torch.bfloat16 else \
            gate * (1 + BF16_HALF_ULP) + BF16_HALF_ULP * np.abs(y_ref) + 2.0 ** -133
        stats.update(outputs_over_plain_gate=int(np.sum(err > plain)),
                     max_err_over_plain_gate=float(np.max(err / plain)))
    record_stats(**stats)
    assert bad.size == 0, f"{what}: {len(bad)} outputs out of tolerance, first {bad[:3].tolist()}, " \
                          f"max |dY|/S = {worst:.3e}"
    return worst


def exact_cover(s_ref, pairs, chunk=64):
    """Outputs of an E2M1 x E2M1 contraction whose fp32 accumulation is exact
    in any order of additions. A term of output (r, c) in K-block b is a
    multiple of 2^(sa[r, b] + sw[c, b] - 256) (E2M1 magnitudes are multiples
    of 1/2, E8M0 code e is 2^(e - 127)); where S is below 2^24 times the
    smallest such unit over the output's blocks and products, and that unit
    is not below fp32's smallest denormal 2^-149, every partial sum is a
    multiple of the unit below 2^24 of it, so exact in fp32, and so is Y.
    pairs: [(sa [rows, K/32], sw [cols, K/32]), ...], the E8M0 codes of each
    product's operands. Returns a boolean [rows, cols] mask."""
    rows, cols = s_ref.shape
    unit = np.full((rows, cols), 1 << 20, np.int64)
    for sa, sw in pairs:
        sa, sw = np.asarray(sa, np.int32), np.asarray(sw, np.int32)
        for r0 in range(0, rows, chunk):
            m = np.min(sa[r0:r0 + chunk, None, :] + sw[None, :, :], axis=2)
            unit[r0:r0 + chunk] = np.minimum(unit[r0:r0 + chunk], m)
    unit -= 256
    with np.errstate(invalid="ignore"):
        return (s_ref < np.ldexp(1.0, unit + 24)) & (unit >= -149)


def rne_bf16(v):
    """float64 values exactly representable in fp32, rounded to bfloat16 by
    round to nearest even (integer arithmetic on the fp32 bits)."""
    u = np.asarray(v, np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    h = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32)
    return (h << 16).view(np.float32).astype(np.float64)


def check_exact_where_covered(y_gpu, y_ref, s_ref, pairs, out_dtype, what=""):
    """Where exact_cover holds, Y must be the exact sum itself (fp32 Y) or
    its round-to-nearest-even to bfloat16 (bf16 Y), bit for bit. Returns the
    covered fraction."""
    cov = exact_cover(s_ref, pairs)
    y_gpu = np.asarray(y_gpu, np.float64)
    want = y_ref if out_dtype != torch.bfloat16 else rne_bf16(y_ref)
    bad = np.argwhere(cov & ~(y_gpu == want))
    assert bad.size == 0, (f"{what}: {len(bad)} outputs whose sums are exact in fp32 differ from the exact sum"
                           f"{' rounded to bf16' if out_dtype == torch.bfloat16 else ''}, first {bad[:3].tolist()}")
    return float(cov.mean())


def check_grad(g_gpu, g_ref, s_ref, contraction, out_dtype, what=""):
    """Per-output check of a straight-through gradient computed with bf16
    matrix instructions: products of bf16 dY and decoded MXFP4 values are
    exact in fp32, each instruction adds 16 of them, and its result goes into
    the fp32 accumulator with one rounding (measured on gfx950: the sum
    comes back within an fp32 ulp of exact, sometimes truncated), so
    |dG| <= (ceil(P / 16) + 1) 2^-23 S over a contraction of length P; bf16
    output adds the RNE half-ulp."""
    g_gpu = np.asarray(g_gpu, dtype=np.float64)
    steps = -(-int(contraction) // 16) + 1
    tol = steps * 2.0 ** -23 * s_ref + 2.0 ** -126
    if out_dtype == torch.bfloat16:
        tol = tol * (1 + BF16_HALF_ULP) + BF16_HALF_ULP * np.abs(g_ref) + 2.0 ** -133
    err = np.abs(g_gpu - g_ref)
    bad = np.argwhere(~(err <= tol))
    worst = float(np.max(err / np.maximum(s_ref, 1e-300)))
    assert bad.size == 0, f"{what}: {len(bad)} outputs out of tolerance, first {bad[:3].tolist()}, " \
                          f"max |dG|/S = {worst:.3e}"
    return worst
