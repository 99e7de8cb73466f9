// Internal launch interface between the C ABI layer (api.cpp) and the HIP
// kernels. Arguments here are already validated by the caller.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rfq {

// MXFP4 quantization of a bf16 (or, x_f32, fp32) matrix along K, optionally
// with the RFQ residual pass (qr/sr non-null) and a block-Hadamard rotation
// first (rotate 1: X H, with the residual pass; rotate 2: X H / 32, without).
// rows * (K/32) must be < 2^32.
hipError_t launch_quantize(const void* x, bool x_f32, int rotate, int64_t rows, int64_t K, int64_t ldx,
                           uint8_t* qx, uint8_t* sx, uint8_t* qr, uint8_t* sr, hipStream_t stream);

// Block-scaled FP4 GEMM, Y = QX.W^T (+ QR.W^T when qr != nullptr).
hipError_t launch_gemm(const uint8_t* qx, const uint8_t* sx, const uint8_t* qr, const uint8_t* sr,
                       const uint8_t* w, const uint8_t* sw, int64_t M, int64_t N, int64_t K,
                       void* y, bool y_bf16, int64_t ldy, hipStream_t stream);

// Measurement probe: the scaled FP4 MFMA loop on caller-supplied operands.
hipError_t launch_mfma_ceiling(const uint8_t* a, size_t a_bytes, const uint8_t* b, size_t b_bytes, int workgroups,
                               int iters, uint64_t* stamps, float* sink, hipStream_t stream);

}  // namespace rfq
