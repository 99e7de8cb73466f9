// Per-lane MXFP4 encoding primitives shared by the quantize pass
// (quantize.hip) and the GEMM that quantizes its own activation tiles
// (gemm.hip, fused variant), so that both produce the same bytes.
//
// Formats ("Activation Outliers Matter: Robust Recovery for Quantized
// Multimodal LLMs", §1 names MXFP4; the encodings are OCP MX v1.0's): a
// block is 32 elements along K held by four consecutive lanes (a DPP quad),
// 8 elements per lane; the E8M0 scale code is max(e_amax - 2, 0) for the
// biased exponent e_amax of the block maximum; elements are E2M1 codes of
// x / 2^se, rounded to nearest even and saturating, produced by gfx950's
// scaled fp32 -> FP4 converter (v_cvt_scalef32_pk_fp4_f32), which takes the
// E8M0 code in the exponent field of its fp32 scale operand.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rfq {
namespace mx {

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

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

// The RFQ encoding of one lane's 8 bf16 elements of a block (its quad holds
// the other 24): Q(X) codes and scale code, then R = x - deq(Q(X)) in fp32
// (exact for bf16 x) and Q(R) codes and scale code. A block holding NaN or
// Inf gets scale 255 and zero codes in both. Every lane of the quad must
// call this together (DPP exchanges).
struct RfqLane {
  unsigned cx, sx, cr, sr;   // 4 code bytes and the scale code, for Q(X) and Q(R)
};
__device__ __forceinline__ RfqLane rfq_encode_bf16x8(u32x4_t w) {
  const unsigned e = quad_max_u32(bf16x8_absmax_bits(w)) >> 7;   // biased exponent of the block amax
  float xf[8];
  widen_bf16x8(w, xf);
  const bool nonfinite = e == 255;
  const unsigned sxc = nonfinite ? 255u : (e > 2u ? e - 2u : 0u);
  const float s = scale_operand(sxc);
  unsigned cx = encode_f32x8(xf, s);
  if (nonfinite) cx = 0u;
  float r[8];
  residual_pair<0>(xf, cx, s, r);
  residual_pair<1>(xf, cx, s, r);
  residual_pair<2>(xf, cx, s, r);
  residual_pair<3>(xf, cx, s, r);
  const float m = fmaxf(fmaxf(fmaxf(fabsf(r[0]), fabsf(r[1])), fmaxf(fabsf(r[2]), fabsf(r[3]))),
                        fmaxf(fmaxf(fabsf(r[4]), fabsf(r[5])), fmaxf(fabsf(r[6]), fabsf(r[7]))));
  const unsigned er = quad_max_u32(__builtin_bit_cast(unsigned, m)) >> 23;   // fp32 biased exponent
  const unsigned rc = er > 2u ? er - 2u : 0u;
  unsigned cr = encode_f32x8(r, scale_operand(rc));
  if (nonfinite) cr = 0u;
  return RfqLane{cx, sxc, cr, nonfinite ? 255u : rc};
}

}  // namespace mx
}  // namespace rfq
