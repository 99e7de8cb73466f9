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
// Both transpose in registers, without LDS: a wave owns a tile of 64 input
// rows, and lane l = 8 g + c of it the 8 rows r0 + 8 g .. r0 + 8 g + 7 of
// column chunk c. It loads its chunk of each of its 8 rows (the 8 lanes of a
// row group read 128 contiguous bytes of one row per instruction), and for
// each column of the chunk writes the 8 row values as one 16-byte store into
// that column's output row (the 8 row groups' lanes cover 128 contiguous
// bytes of it). A chunk is 32 columns (16 code bytes, one scale block) for
// the decode and 8 columns (16 bytes of bf16) for the bf16 transpose, so a
// wave's tile is 64 x 256 or 64 x 64 input elements. HBM-bound: 2.53 B per
// element for the decode (0.5 + 1/32 read, 2 written), 4 B for the bf16
// transpose.

#include "kernels.h"

namespace rfq {
namespace {

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;            // 4 waves, one tile each
constexpr int kTileRows = 64;

// (lo16(a), lo16(b)) and (hi16(a), hi16(b)) packed into one word, a low
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

// Byte kSel of code words wa (row k) and wb (row k + 1) decoded: the two
// columns 2 kSel and 2 kSel + 1 of the word, each as (row k, row k + 1) bf16
// pairs. E2M1 times a power of two is exact in bf16: the top half of the
// fp32 value. (Elements are copied to scalars before the bit casts: a bit
// cast of an ext-vector element has been seen to read element 0.)
template <int kSel>
__device__ __forceinline__ void decode_pair(uint32_t wa, uint32_t wb, float sa, float sb, uint32_t& even,
                                            uint32_t& odd) {
  const f32x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wa, sa, kSel);
  const f32x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wb, sb, kSel);
  const float a0 = a.x, a1 = a.y, b0 = b.x, b1 = b.y;
  even = pack_hi(__builtin_bit_cast(uint32_t, a0), __builtin_bit_cast(uint32_t, b0));
  odd = pack_hi(__builtin_bit_cast(uint32_t, a1), __builtin_bit_cast(uint32_t, b1));
}

// MXFP4 [rows, cols] -> decoded bf16 transposed, [cols, ld_out]; tile t of
// `tiles` covers rows 64 (t % tiles_r) .. and columns 256 (t / tiles_r) ...
__global__ __launch_bounds__(kThreads) void decode_transpose_kernel(const uint8_t* codes, const uint8_t* scales,
                                                                   int rows, int cols, uint16_t* out, int64_t ld_out,
                                                                   int tiles_r, int tiles) {
  const int tile = (int)blockIdx.x * (kThreads / 64) + (int)(threadIdx.x >> 6);
  if (tile >= tiles) return;
  const int lane = threadIdx.x & 63;
  const int r0 = (tile % tiles_r) * kTileRows + 8 * (lane >> 3);   // first of this lane's 8 rows
  const int col = (tile / tiles_r) * 256 + 32 * (lane & 7);          // first of its 32 columns
  if (col >= cols || r0 >= ld_out) return;                          // (cols is a multiple of 32)
  const int64_t cb = cols / 2, nb = cols / 32;
  u32x4_t w[8];
  float s[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int row = r0 + k;
    if (row < rows) {
      w[k] = *reinterpret_cast<const u32x4_t*>(codes + (int64_t)row * cb + col / 2);
      s[k] = __builtin_bit_cast(float, (uint32_t)scales[(int64_t)row * nb + col / 32] << 23);
    } else {
      w[k] = u32x4_t{0u, 0u, 0u, 0u};   // rows past the input: zeros
      s[k] = 1.0f;
    }
  }
  // columns in two halves of 16 (code words 2 h and 2 h + 1)
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t o[16][4];
#pragma unroll
    for (int k = 0; k < 8; k += 2) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint32_t wa = w[k][2 * h + q], wb = w[k + 1][2 * h + q];
        decode_pair<0>(wa, wb, s[k], s[k + 1], o[8 * q + 0][k / 2], o[8 * q + 1][k / 2]);
        decode_pair<1>(wa, wb, s[k], s[k + 1], o[8 * q + 2][k / 2], o[8 * q + 3][k / 2]);
        decode_pair<2>(wa, wb, s[k], s[k + 1], o[8 * q + 4][k / 2], o[8 * q + 5][k / 2]);
        decode_pair<3>(wa, wb, s[k], s[k + 1], o[8 * q + 6][k / 2], o[8 * q + 7][k / 2]);
      }
    }
#pragma unroll
    for (int j = 0; j < 16; ++j)
      *reinterpret_cast<u32x4_t*>(out + (int64_t)(col + 16 * h + j) * ld_out + r0) =
          u32x4_t{o[j][0], o[j][1], o[j][2], o[j][3]};
  }
}

// bf16 [rows, cols] (row stride ld_in) -> [cols, ld_out]; tile t covers rows
// 64 (t % tiles_r) .. and columns 64 (t / tiles_r) ... `vec`: rows start
// 16-byte aligned (base and ld_in), so whole 8-column chunks load as one.
__global__ __launch_bounds__(kThreads) void transpose_bf16_kernel(const uint16_t* in, int rows, int cols, int64_t ld_in,
                                                                 uint16_t* out, int64_t ld_out, int tiles_r, int tiles,
                                                                 int vec) {
  const int tile = (int)blockIdx.x * (kThreads / 64) + (int)(threadIdx.x >> 6);
  if (tile >= tiles) return;
  const int lane = threadIdx.x & 63;
  const int r0 = (tile % tiles_r) * kTileRows + 8 * (lane >> 3);
  const int col = (tile / tiles_r) * 64 + 8 * (lane & 7);
  if (col >= cols || r0 >= ld_out) return;
  u32x4_t v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int row = r0 + k;
    const uint16_t* src = in + (int64_t)row * ld_in + col;
    if (row < rows && vec && col + 8 <= cols) {
      v[k] = *reinterpret_cast<const u32x4_t*>(src);
    } else {
      uint32_t e[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) e[j] = (row < rows && col + j < cols) ? src[j] : 0u;
      v[k] = u32x4_t{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (col + j >= cols) break;
    uint32_t o[4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
      o[p] = (j & 1) ? pack_hi(v[2 * p][j / 2], v[2 * p + 1][j / 2]) : pack_lo(v[2 * p][j / 2], v[2 * p + 1][j / 2]);
    *reinterpret_cast<u32x4_t*>(out + (int64_t)(col + j) * ld_out + r0) = u32x4_t{o[0], o[1], o[2], o[3]};
  }
}

}  // namespace

hipError_t launch_decode_transpose(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                                   uint16_t* out, int64_t ld_out, hipStream_t stream) {
  const int64_t tr = (ld_out + kTileRows - 1) / kTileRows, tc = (cols + 255) / 256;
  const int64_t tiles = tr * tc;
  hipLaunchKernelGGL(decode_transpose_kernel, dim3((unsigned)((tiles + 3) / 4)), dim3(kThreads), 0, stream, codes,
                     scales, (int)rows, (int)cols, out, ld_out, (int)tr, (int)tiles);
  return hipGetLastError();
}

hipError_t launch_transpose_bf16(const uint16_t* in, int64_t rows, int64_t cols, int64_t ld_in, uint16_t* out,
                                 int64_t ld_out, hipStream_t stream) {
  const int64_t tr = (ld_out + kTileRows - 1) / kTileRows, tc = (cols + 63) / 64;
  const int64_t tiles = tr * tc;
  const int vec = ((uintptr_t)in % 16 == 0 && ld_in % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL(transpose_bf16_kernel, dim3((unsigned)((tiles + 3) / 4)), dim3(kThreads), 0, stream, in,
                     (int)rows, (int)cols, ld_in, out, ld_out, (int)tr, (int)tiles, vec);
  return hipGetLastError();
}

}  // namespace rfq
