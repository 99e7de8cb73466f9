// Operand staging for the straight-through backward pass of the RFQ layer
// ("Activation Outliers Matter", §1: RFQ for training; the gradients
// dX = dY deq(Wq) and dW = dY^T (deq Q(X) + deq Q(R)) taken with Q passed
// through unchanged). Both products run on the GEMM kernel's bf16 mode,
// which contracts two row-major operands along their rows, so the operands
// whose contraction index is their row index are transposed first:
//
//  * decode_transpose: MXFP4 codes [rows, cols/2] with scales [rows, cols/32]
//    to bf16 [cols, ld] holding the decoded values transposed (element
//    (r, c) at out[c * ld + r]); columns r in [rows, ld) are written as
//    zeros. E2M1 times a power of two is exact in bf16 for scale exponents
//    up to 125 (those of any bf16 or fp32 input's quantization but the very
//    largest fp32 blocks).
//  * transpose_bf16: bf16 [rows, cols] (row stride ld_in) to [cols, ld_out],
//    zero columns past `rows` likewise.
//
// Both move 64 x 64 tiles through LDS: a workgroup of 256 threads reads the
// tile row-wise (coalesced), and writes it out row-wise after the transpose
// in LDS. HBM-bound: 2.5 B per element for the decode (0.5 + 1/32 read,
// 2 written), 4 B for the bf16 transpose.

#include "kernels.h"

namespace rfq {
namespace {

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kTile = 64;
constexpr int kPad = 2;                 // u16 elements of row padding in LDS (bank spread)
constexpr int kThreads = 256;

__device__ __forceinline__ uint16_t f32_to_bf16_exact(float v) {
  return (uint16_t)(__builtin_bit_cast(uint32_t, v) >> 16);   // exact: E2M1 values have two significant bits
}

// Writes the LDS tile t[c][r] (c: output row within the tile, r: output
// column) to out rows c0 + c (those below `cols`), columns r0 .. r0 + 63
// (those below ld_cols).
__device__ __forceinline__ void store_tile_rows(const uint16_t (&t)[kTile][kTile + kPad], uint16_t* out, int64_t ld,
                                                int c0, int cols, int r0, int ld_cols) {
  const int c = threadIdx.x / 4, part = threadIdx.x % 4;    // 16 elements each
  if (c0 + c >= cols) return;
  uint16_t* dst = out + (int64_t)(c0 + c) * ld + r0 + 16 * part;
  const int n = min(16, ld_cols - (r0 + 16 * part));
  if (n == 16) {
    u32x4_t lo, hi;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo[j] = t[c][16 * part + 2 * j] | ((uint32_t)t[c][16 * part + 2 * j + 1] << 16);
      hi[j] = t[c][16 * part + 8 + 2 * j] | ((uint32_t)t[c][16 * part + 8 + 2 * j + 1] << 16);
    }
    reinterpret_cast<u32x4_t*>(dst)[0] = lo;
    reinterpret_cast<u32x4_t*>(dst)[1] = hi;
  } else {
    for (int j = 0; j < n; ++j) dst[j] = t[c][16 * part + j];
  }
}

// One workgroup per 64 x 64 tile, blockIdx.x = ty * tiles_r + tx over
// tiles_r = ceil(ld_out / 64) tile rows: the tile covers input rows
// r0 = 64 tx .. and input columns c0 = 64 ty ...
__global__ __launch_bounds__(kThreads) void decode_transpose_kernel(const uint8_t* codes, const uint8_t* scales,
                                                                   int rows, int cols, uint16_t* out, int64_t ld_out,
                                                                   int tiles_r) {
  __shared__ uint16_t t[kTile][kTile + kPad];
  const int r0 = (blockIdx.x % tiles_r) * kTile, c0 = (blockIdx.x / tiles_r) * kTile;
  const int r = threadIdx.x / 4, part = threadIdx.x % 4;   // input row, 16 columns (8 code bytes) each
  const int row = r0 + r, col = c0 + 16 * part;
  float v[16];
  if (row < rows && col < cols) {
    const int64_t cb = (int64_t)cols / 2;
    const u32x2_t w = *reinterpret_cast<const u32x2_t*>(codes + (int64_t)row * cb + col / 2);
    const uint32_t sc = scales[(int64_t)row * (cols / 32) + col / 32];
    const float s = __builtin_bit_cast(float, sc << 23);   // E8M0 code in the exponent field
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t word = h ? w.y : w.x;
      const f32x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, s, 0);
      const f32x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, s, 1);
      const f32x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, s, 2);
      const f32x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, s, 3);
      v[8 * h + 0] = p0.x; v[8 * h + 1] = p0.y; v[8 * h + 2] = p1.x; v[8 * h + 3] = p1.y;
      v[8 * h + 4] = p2.x; v[8 * h + 5] = p2.y; v[8 * h + 6] = p3.x; v[8 * h + 7] = p3.y;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) t[16 * part + j][r] = f32_to_bf16_exact(v[j]);
  __syncthreads();
  store_tile_rows(t, out, ld_out, c0, cols, r0, (int)ld_out);
}

__global__ __launch_bounds__(kThreads) void transpose_bf16_kernel(const uint16_t* in, int rows, int cols, int64_t ld_in,
                                                                 uint16_t* out, int64_t ld_out, int tiles_r) {
  __shared__ uint16_t t[kTile][kTile + kPad];
  const int r0 = (blockIdx.x % tiles_r) * kTile, c0 = (blockIdx.x / tiles_r) * kTile;
  const int r = threadIdx.x / 4, part = threadIdx.x % 4;
  const int row = r0 + r, col = c0 + 16 * part;
  uint16_t v[16];
  if (row < rows && col + 16 <= cols && (ld_in % 8) == 0) {
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(in + (int64_t)row * ld_in + col);
    const u32x4_t a = src[0], b = src[1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = (uint16_t)a[j]; v[2 * j + 1] = (uint16_t)(a[j] >> 16);
      v[8 + 2 * j] = (uint16_t)b[j]; v[8 + 2 * j + 1] = (uint16_t)(b[j] >> 16);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = (row < rows && col + j < cols) ? in[(int64_t)row * ld_in + col + j] : (uint16_t)0;
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) t[16 * part + j][r] = v[j];
  __syncthreads();
  store_tile_rows(t, out, ld_out, c0, cols, r0, (int)ld_out);
}

}  // namespace

hipError_t launch_decode_transpose(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                                   uint16_t* out, int64_t ld_out, hipStream_t stream) {
  const int64_t tr = (ld_out + kTile - 1) / kTile, tc = (cols + kTile - 1) / kTile;
  hipLaunchKernelGGL(decode_transpose_kernel, dim3((unsigned)(tr * tc)), dim3(kThreads), 0, stream, codes, scales,
                     (int)rows, (int)cols, out, ld_out, (int)tr);
  return hipGetLastError();
}

hipError_t launch_transpose_bf16(const uint16_t* in, int64_t rows, int64_t cols, int64_t ld_in, uint16_t* out,
                                 int64_t ld_out, hipStream_t stream) {
  const int64_t tr = (ld_out + kTile - 1) / kTile, tc = (cols + kTile - 1) / kTile;
  hipLaunchKernelGGL(transpose_bf16_kernel, dim3((unsigned)(tr * tc)), dim3(kThreads), 0, stream, in, (int)rows,
                     (int)cols, ld_in, out, ld_out, (int)tr);
  return hipGetLastError();
}

}  // namespace rfq
