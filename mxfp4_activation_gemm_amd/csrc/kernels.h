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
//
// x_fmt 16: bfloat16 operands throughout, no scales (r_fmt 0 or 16, the second
// pair sharing w); K then counts four per bf16 element (bytes per row = K/2),
// and y_trans (required with r_fmt 16, refused otherwise) stores the result
// transposed: element (m, n) to y[n * ldy + m].
hipError_t launch_gemm(int x_fmt, int r_fmt, const uint8_t* qx, const uint8_t* sx, const uint8_t* qr,
                       const uint8_t* sr, const uint8_t* w, const uint8_t* sw, int64_t M, int64_t N, int64_t K,
                       void* y, bool y_bf16, int64_t ldy, hipStream_t stream, bool y_trans = false);

// The RFQ GEMM that quantizes its own activation: Y = Q(X) W^T + Q(R) W^T
// for bf16 X [M, K] (row stride ldx elements) and the MXFP4 weight, with Q(X)
// and Q(R) formed tile by tile inside the GEMM and never written to memory.
// K must be a multiple of 512 (hipErrorInvalidValue otherwise); 128 * ldx * 2
// must stay below 2^32.
hipError_t launch_gemm_fused(const uint16_t* x, int64_t ldx, const uint8_t* w, const uint8_t* sw, int64_t M, int64_t N,
                             int64_t K, void* y, bool y_bf16, int64_t ldy, hipStream_t stream);

// Backward-pass operand staging (csrc/backward.hip): MXFP4 codes [rows,
// cols/2] + scales to bf16 [cols, ld_out] transposed, and a bf16 transpose
// [rows, cols] (stride ld_in) to [cols, ld_out]; columns past `rows` are
// zero-filled. ld_out a multiple of 8, pointers 16-byte aligned.
hipError_t launch_decode_transpose(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                                   uint16_t* out, int64_t ld_out, hipStream_t stream);
hipError_t launch_transpose_bf16(const uint16_t* in, int64_t rows, int64_t cols, int64_t ld_in, uint16_t* out,
                                 int64_t ld_out, hipStream_t stream);

// Staging memory of the allocation-free linear entry point (noalloc.hip):
// the device address, on the current device, of a library-owned array of
// kNoallocScratchBytes (looked up once per device and kept).
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
hipError_t noalloc_scratch(uint8_t** ptr);

}  // namespace rfq
