// MXFP4 quantization and the RFQ residual pass on gfx950.
//
// What is computed ("Activation Outliers Matter: Robust Recovery for
// Quantized Multimodal LLMs", §1, RFQ paragraph; formats per OCP MX v1.0):
// for each 32-element block of a row of bf16 X,
//   se   = max(floor(log2 amax) - 2, -127)      (E8M0 code max(e_bf16 - 2, 0))
//   Q(X) = E2M1 RNE-with-saturation codes of x / 2^se
//   R    = x - deq(Q(X))                         (exact in fp32 for bf16 x)
//   Q(R) = the same encoding applied to R        (second low-bit path)
// A block holding NaN/Inf gets scale 255 and zero codes, and so does its
// residual block.
//
// Mapping: 4 lanes own one block (8 bf16 = one 16-byte load each), so a wave
// reads 1 KB of X per load instruction, fully contiguous when rows are dense.
// The block amax is a max over the lane's 8 values then a DPP quad exchange.
// The bf16 values are widened to fp32 (exact), and element encoding and
// decoding use gfx950's fp32 <-> FP4 scaled converters, which
// take the E8M0 code in the exponent field of an fp32 scale operand, divide
// by 2^se on the way to FP4 (round to nearest even, saturating) and multiply
// on the way back. The residual never leaves fp32 registers.
//
// Traffic per element: 2 B read, 2 x (0.5 + 1/32) B written = 3.0625 B.

#include "kernels.h"

namespace rfq {
namespace {

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;          // 4 waves per workgroup
constexpr int kUnits = 4;              // 16-block units per wave
constexpr int kBlocksPerWave = 16 * kUnits;

// DPP quad permutations: lane ^ 1 and lane ^ 2 within each group of 4 lanes.
constexpr int kQuadXor1 = 0xB1;        // quad_perm:[1,0,3,2]
constexpr int kQuadXor2 = 0x4E;        // quad_perm:[2,3,0,1]

__device__ __forceinline__ unsigned quad_max_u32(unsigned v) {
  v = max(v, (unsigned)__builtin_amdgcn_mov_dpp((int)v, kQuadXor1, 0xF, 0xF, true));
  v = max(v, (unsigned)__builtin_amdgcn_mov_dpp((int)v, kQuadXor2, 0xF, 0xF, true));
  return v;
}

// max over 8 bf16 magnitudes, as the 15-bit magnitude pattern (monotone in
// the value for non-NaN inputs; any pattern >= 0x7F80 is Inf or NaN).
// (Each word is copied to a scalar before the bit cast: a bit cast applied
// directly to an ext-vector element has been seen to read element 0.)
__device__ __forceinline__ unsigned bf16x8_absmax_bits(u32x4_t w) {
  const u16x2_t mask = {0x7FFF, 0x7FFF};
  const unsigned w0 = w.x, w1 = w.y, w2 = w.z, w3 = w.w;
  u16x2_t a = __builtin_bit_cast(u16x2_t, w0) & mask;
  u16x2_t b = __builtin_bit_cast(u16x2_t, w1) & mask;
  u16x2_t c = __builtin_bit_cast(u16x2_t, w2) & mask;
  u16x2_t d = __builtin_bit_cast(u16x2_t, w3) & mask;
  u16x2_t m = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
  return max((unsigned)m.x, (unsigned)m.y);
}

__device__ __forceinline__ float scale_operand(unsigned code) {
  return __builtin_bit_cast(float, code << 23);  // exponent field = E8M0 code
}

// The 8 bf16 values of `w` widened to fp32 (exact): element 2j is the low
// half of word j.
__device__ __forceinline__ void widen_bf16x8(u32x4_t w, float* f) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = __builtin_bit_cast(float, w[j] << 16);
    f[2 * j + 1] = __builtin_bit_cast(float, w[j] & 0xFFFF0000u);
  }
}

// E2M1 codes of 8 fp32 values at scale code s (exponent field of `s`): byte j
// holds element 2j in its low nibble and 2j+1 in its high nibble.
__device__ __forceinline__ unsigned encode_f32x8(const float* f, float s) {
  unsigned c = 0;
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, f[0], f[1], s, 0);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, f[2], f[3], s, 1);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, f[4], f[5], s, 2);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, f[6], f[7], s, 3);
  return c;
}

// r[2J], r[2J+1] = x[2J], x[2J+1] minus their decoded codes (byte J of
// `codes`), in fp32.
template <int J>
__device__ __forceinline__ void residual_pair(const float* x, unsigned codes, float s, float* r) {
  const f32x2_t d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, s, J);
  r[2 * J] = x[2 * J] - d.x;
  r[2 * J + 1] = x[2 * J + 1] - d.y;
}

struct QuantParams {
  const uint16_t* x;
  int64_t ldx;            // elements
  uint8_t* qx;
  uint8_t* sx;
  uint8_t* qr;
  uint8_t* sr;
  uint32_t nblk_row;      // K / 32
  uint32_t total_blocks;  // rows * K / 32
};

template <bool kResidual>
__global__ __launch_bounds__(kThreads) void quantize_kernel(QuantParams p) {
  const unsigned lane = threadIdx.x & 63;
  const unsigned wave = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const uint32_t g0 = wave * kBlocksPerWave;   // first block of this wave
  if (g0 >= p.total_blocks) return;
  const uint32_t quad = lane >> 2, part = lane & 3;

  // row/column of each unit's block for this lane
  uint32_t row0 = g0 / p.nblk_row;
  uint32_t col0 = g0 - row0 * p.nblk_row;

  u32x4_t w[kUnits];
  uint32_t gblk[kUnits];
#pragma unroll
  for (int u = 0; u < kUnits; ++u) {
    uint32_t g = g0 + u * 16 + quad;
    uint32_t b = col0 + u * 16 + quad, r = row0;
    while (b >= p.nblk_row) { b -= p.nblk_row; ++r; }
    gblk[u] = g;
    const uint16_t* src = p.x + (int64_t)r * p.ldx + (int64_t)b * 32 + part * 8;
    w[u] = (g < p.total_blocks) ? *reinterpret_cast<const u32x4_t*>(src) : u32x4_t{0, 0, 0, 0};
  }

#pragma unroll
  for (int u = 0; u < kUnits; ++u) {
    const uint32_t g = gblk[u];
    const bool valid = g < p.total_blocks;
    const unsigned amax = quad_max_u32(bf16x8_absmax_bits(w[u]));
    const unsigned e = amax >> 7;                      // bf16 biased exponent of amax
    const bool nonfinite = e == 255;
    const unsigned sxc = nonfinite ? 255u : (e > 2 ? e - 2 : 0u);
    const float s = scale_operand(sxc);
    float xf[8];
    widen_bf16x8(w[u], xf);
    unsigned cx = encode_f32x8(xf, s);
    if (nonfinite) cx = 0;

    unsigned cr = 0, src = 255u;
    if (kResidual) {
      // deq(Q(X)) and R = X - deq(Q(X)) in fp32
      float r[8];
      residual_pair<0>(xf, cx, s, r);
      residual_pair<1>(xf, cx, s, r);
      residual_pair<2>(xf, cx, s, r);
      residual_pair<3>(xf, cx, s, r);
      float m = fmaxf(fmaxf(fmaxf(fabsf(r[0]), fabsf(r[1])), fmaxf(fabsf(r[2]), fabsf(r[3]))),
                      fmaxf(fmaxf(fabsf(r[4]), fabsf(r[5])), fmaxf(fabsf(r[6]), fabsf(r[7]))));
      const unsigned ramax = quad_max_u32(__builtin_bit_cast(unsigned, m));
      const unsigned er = ramax >> 23;                 // fp32 biased exponent
      const unsigned rc = er > 2 ? er - 2 : 0u;
      const float sr = scale_operand(rc);
      cr = encode_f32x8(r, sr);
      if (nonfinite) cr = 0;
      src = nonfinite ? 255u : rc;
    }

    if (valid) {
      const uint64_t cofs = (uint64_t)g * 16 + part * 4;
      *reinterpret_cast<unsigned*>(p.qx + cofs) = cx;
      if (kResidual) *reinterpret_cast<unsigned*>(p.qr + cofs) = cr;
      if (part == 0) {
        p.sx[g] = (uint8_t)sxc;
        if (kResidual) p.sr[g] = (uint8_t)src;
      }
    }
  }
}

}  // namespace

hipError_t launch_quantize(const uint16_t* x, int64_t rows, int64_t K, int64_t ldx,
                           uint8_t* qx, uint8_t* sx, uint8_t* qr, uint8_t* sr,
                           hipStream_t stream) {
  QuantParams p;
  p.x = x;
  p.ldx = ldx;
  p.qx = qx;
  p.sx = sx;
  p.qr = qr;
  p.sr = sr;
  p.nblk_row = (uint32_t)(K / 32);
  p.total_blocks = (uint32_t)(rows * (K / 32));
  const uint64_t waves = (p.total_blocks + kBlocksPerWave - 1) / kBlocksPerWave;
  const uint64_t groups = (waves + kThreads / 64 - 1) / (kThreads / 64);
  if (qr != nullptr)
    hipLaunchKernelGGL(quantize_kernel<true>, dim3((unsigned)groups), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(quantize_kernel<false>, dim3((unsigned)groups), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace rfq
