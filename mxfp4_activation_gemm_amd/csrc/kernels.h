// Internal launch interface between the C ABI layer (api.cpp) and the HIP
// kernels. Arguments here are already validated by the caller.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rfq {

// MX quantization of a bf16 (or, x_f32, fp32) matrix along K into format
// x_fmt (4: MXFP4, 8: MXFP8 E4M3), optionally with the RFQ residual pass
// (qr/sr non-null; Q(X) must be MXFP4, Q(R) in format r_fmt) and a
// block-Hadamard rotation first (rotate 1: X H, with an MXFP4 residual pass;
// rotate 2: X H / 32, plain MXFP4). Other combinations return
// hipErrorInvalidValue. rows * (K/32) must be < 2^32.
hipError_t launch_quantize(const void* x, bool x_f32, int rotate, int x_fmt, int r_fmt, int64_t rows, int64_t K,
                           int64_t ldx, uint8_t* qx, uint8_t* sx, uint8_t* qr, uint8_t* sr, hipStream_t stream);

// Block-scaled GEMM against an MXFP4 weight, Y = QX.W^T (+ QR.W^T when
// qr != nullptr), with QX in format x_fmt and QR in r_fmt (4: MXFP4, 8:
// MXFP8 E4M3). Supported: (4, -), (4, 4), (4, 8), (8, -); others return
// hipErrorInvalidValue.
hipError_t launch_gemm(int x_fmt, int r_fmt, const uint8_t* qx, const uint8_t* sx, const uint8_t* qr,
                       const uint8_t* sr, const uint8_t* w, const uint8_t* sw, int64_t M, int64_t N, int64_t K,
                       void* y, bool y_bf16, int64_t ldy, hipStream_t stream);

// Measurement probe: the scaled MFMA loop on caller-supplied operands (first
// operand E2M1, second E2M1 or, b_fmt 8, E4M3).
hipError_t launch_mfma_ceiling(const uint8_t* a, size_t a_bytes, const uint8_t* b, size_t b_bytes, int b_fmt,
                               int workgroups, int iters, uint64_t* stamps, float* sink, hipStream_t stream);

}  // namespace rfq
