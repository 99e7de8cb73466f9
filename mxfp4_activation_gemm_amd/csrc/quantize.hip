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
// X is read and the codes written with non-temporal accesses: each byte is
// touched once, and streaming it past the caches measured 8% faster on a
// layer larger than the last-level cache (75% of HBM peak against 69%).
//
// Variants of the same pass:
//  * fp32 input (8 values = 32 bytes per lane);
//  * rotation before quantization ("大模型量化中的双线性尾部问题与QuaRot正交旋转
//    解决方案" §3, QuaRot: an orthogonal +-1 matrix applied online to the
//    activation and folded into the weight): each 32-block is multiplied by
//    the unnormalised 32 x 32 Sylvester Hadamard matrix H in fp32, by five
//    butterfly passes of spans 1, 2, 4 (inside a lane) and 8, 16 (across the
//    block's four lanes, DPP), each taking (a, b) at (i, i + span) to
//    (a + b, a - b). Activations quantize X H; weights W H / 32 (an exact
//    power of two), so the GEMM returns X W^T unchanged. Codes are decided
//    on the rotated fp32 values; the residual stays exact (|R| is at most
//    half an E2M1 step, so R = v - deq(v) loses no bits in fp32);
//  * MXFP8 output ("Activation Outliers Matter", Abstract and §1 study MXFP8
//    beside MXFP4; elements per OCP MX v1.0): E4M3 codes, one byte per
//    element, with se = max(floor(log2 amax) - 8, -127), either for X itself
//    (W4A8) or for the residual R of an MXFP4 Q(X) (RFQ with an MXFP8 second
//    path). Values are clamped to +-448 * 2^se before the scaled fp32 -> FP8
//    conversion (round to nearest even), which is the saturation rule: from
//    448 up to the 464 midpoint the nearest value is 448 anyway.

#include "kernels.h"

namespace rfq {
namespace {

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x2_t __attribute__((ext_vector_type(2)));

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

// E4M3 codes of 8 fp32 values at E8M0 scale code `code` (not 255): byte j of
// the 8 holds element j. Each value is first clamped to +-448 * 2^se (whose
// fp32 pattern has exponent field code + 8 and the mantissa of 1.75).
__device__ __forceinline__ u32x2_t encode_e4m3_f32x8(const float* f, unsigned code) {
  const float s = scale_operand(code);
  const float lim = __builtin_bit_cast(float, ((code + 8u) << 23) | 0x00600000u);
  float c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_fmed3f(f[j], -lim, lim);
  i16x2_t lo = {0, 0}, hi = {0, 0};
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, c[0], c[1], s, false);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, c[2], c[3], s, true);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hi, c[4], c[5], s, false);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hi, c[6], c[7], s, true);
  return u32x2_t{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
}

// The largest element exponent of a format: 2 for E2M1 (6 = 1.5 * 2^2), 8 for
// E4M3 (448 = 1.75 * 2^8). The block scale code is max(e_amax - emax, 0) for
// the biased fp32 exponent e_amax of the block maximum.
template <int kFmt>
constexpr unsigned kEmax = kFmt == 8 ? 8u : 2u;

// A lane's 8 elements of one block in format kFmt (4: E2M1, 8: E4M3) at scale
// code `code`: 4 bytes of packed nibbles (in .x) or 8 bytes.
template <int kFmt>
__device__ __forceinline__ u32x2_t encode_part(const float* f, unsigned code) {
  if constexpr (kFmt == 8)
    return encode_e4m3_f32x8(f, code);
  else
    return u32x2_t{encode_f32x8(f, scale_operand(code)), 0u};
}

// Stores a lane's part of block g (codes of 32 elements: 16 bytes for E2M1,
// 32 for E4M3, of which this lane holds a quarter).
template <int kFmt>
__device__ __forceinline__ void store_part(uint8_t* q, uint32_t g, uint32_t part, u32x2_t c) {
  if constexpr (kFmt == 8)
    __builtin_nontemporal_store(c, reinterpret_cast<u32x2_t*>(q + (uint64_t)g * 32 + part * 8));
  else
    __builtin_nontemporal_store(c.x, reinterpret_cast<unsigned*>(q + (uint64_t)g * 16 + part * 4));
}

// r[2J], r[2J+1] = x[2J], x[2J+1] minus their decoded codes (byte J of
// `codes`), in fp32.
template <int J>
__device__ __forceinline__ void residual_pair(const float* x, unsigned codes, float s, float* r) {
  const f32x2_t d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, s, J);
  r[2 * J] = x[2 * J] - d.x;
  r[2 * J + 1] = x[2 * J + 1] - d.y;
}

// One butterfly pass across lanes: this lane's element pairs with the same
// element of lane (lane ^ kXor) in its quad; the lane with the span bit clear
// keeps a + b, the other a - b (a = the clear lane's value).
// (o - a is formed as (-a) + o: negation is exact, so the result is the same
// IEEE sum, and the partner's value can feed the add through DPP directly.)
template <int kDpp>
__device__ __forceinline__ void butterfly_across(float* v, bool upper) {
  const unsigned flip = upper ? 0x80000000u : 0u;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float o = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v[j]), kDpp, 0xF, 0xF, true));
    v[j] = __builtin_bit_cast(float, __builtin_bit_cast(unsigned, v[j]) ^ flip) + o;
  }
}

// Walsh-Hadamard transform of the 32-block held by a quad of lanes (lane part
// p holds elements 8 p .. 8 p + 7), unnormalised, in the pass order above.
__device__ __forceinline__ void hadamard32(float* v, unsigned part) {
#pragma unroll
  for (int span = 1; span < 8; span *= 2)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (!(j & span)) {
        const float a = v[j], b = v[j + span];
        v[j] = a + b;
        v[j + span] = a - b;
      }
  butterfly_across<kQuadXor1>(v, part & 1);   // span 8
  butterfly_across<kQuadXor2>(v, part & 2);   // span 16
}

// max over 8 fp32 magnitudes as a bit pattern (monotone in the value for
// non-NaN inputs; >= 0x7F800000 means Inf or NaN)
__device__ __forceinline__ unsigned f32x8_absmax_bits(const float* v) {
  unsigned m = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) m = max(m, __builtin_bit_cast(unsigned, v[j]) & 0x7FFFFFFFu);
  return m;
}

struct QuantParams {
  const void* x;
  int64_t ldx;            // elements
  uint8_t* qx;
  uint8_t* sx;
  uint8_t* qr;
  uint8_t* sr;
  uint32_t nblk_row;      // K / 32
  uint32_t total_blocks;  // rows * K / 32
};

// kXFmt: format of Q(X), 4 (E2M1) or 8 (E4M3). kRFmt: format of Q(R), 0 for
// no residual pass (the residual needs an E2M1 Q(X)). kF32In: X is fp32
// (else bf16). kRotate: 0 none, 1 X H (activations), 2 X H / 32 (weights).
template <int kXFmt, int kRFmt, bool kF32In, int kRotate>
__global__ __launch_bounds__(kThreads) void quantize_kernel(QuantParams p) {
  constexpr bool kResidual = kRFmt != 0;
  static_assert(kXFmt == 4 || (kXFmt == 8 && !kResidual && kRotate == 0), "format combination");
  const unsigned lane = threadIdx.x & 63;
  const unsigned wave = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const uint32_t g0 = wave * kBlocksPerWave;   // first block of this wave
  if (g0 >= p.total_blocks) return;
  const uint32_t quad = lane >> 2, part = lane & 3;

  // row/column of each unit's block for this lane
  uint32_t row0 = g0 / p.nblk_row;
  uint32_t col0 = g0 - row0 * p.nblk_row;

  // the lane's 8 values of each unit: one 16-byte load of bf16, or two of fp32
  constexpr int kLoads = kF32In ? 2 : 1;
  u32x4_t w[kUnits][kLoads];
  uint32_t gblk[kUnits];
#pragma unroll
  for (int u = 0; u < kUnits; ++u) {
    uint32_t g = g0 + u * 16 + quad;
    uint32_t b = col0 + u * 16 + quad, r = row0;
    while (b >= p.nblk_row) { b -= p.nblk_row; ++r; }
    gblk[u] = g;
    const int64_t elem = (int64_t)r * p.ldx + (int64_t)b * 32 + part * 8;
    const u32x4_t* src = kF32In ? reinterpret_cast<const u32x4_t*>(static_cast<const float*>(p.x) + elem)
                                : reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(p.x) + elem);
#pragma unroll
    for (int h = 0; h < kLoads; ++h) w[u][h] = (g < p.total_blocks) ? __builtin_nontemporal_load(src + h) : u32x4_t{0, 0, 0, 0};
  }

#pragma unroll
  for (int u = 0; u < kUnits; ++u) {
    const uint32_t g = gblk[u];
    const bool valid = g < p.total_blocks;
    float xf[8];
    unsigned e;                                        // biased exponent of the block amax (fp32/bf16 field)
    if (!kF32In && kRotate == 0) {
      const unsigned amax = quad_max_u32(bf16x8_absmax_bits(w[u][0]));
      e = amax >> 7;
      widen_bf16x8(w[u][0], xf);
    } else {
      if (kF32In) {
        // (whole-vector bit casts: a bit cast of a single ext-vector element
        // has been seen to read element 0)
        const f32x4_t lo = __builtin_bit_cast(f32x4_t, w[u][0]), hi = __builtin_bit_cast(f32x4_t, w[u][kLoads - 1]);
        xf[0] = lo.x; xf[1] = lo.y; xf[2] = lo.z; xf[3] = lo.w;
        xf[4] = hi.x; xf[5] = hi.y; xf[6] = hi.z; xf[7] = hi.w;
      } else {
        widen_bf16x8(w[u][0], xf);
      }
      if (kRotate != 0) {
        hadamard32(xf, part);
        if (kRotate == 2) {
#pragma unroll
          for (int j = 0; j < 8; ++j) xf[j] *= 0.03125f;   // 1/32, exact
        }
      }
      e = quad_max_u32(f32x8_absmax_bits(xf)) >> 23;
    }
    const bool nonfinite = e == 255;
    const unsigned sxc = nonfinite ? 255u : (e > kEmax<kXFmt> ? e - kEmax<kXFmt> : 0u);
    const float s = scale_operand(sxc);
    u32x2_t cx = encode_part<kXFmt>(xf, sxc);
    if (nonfinite) cx = u32x2_t{0u, 0u};

    u32x2_t cr = {0u, 0u};
    unsigned src = 255u;
    if constexpr (kResidual) {
      // deq(Q(X)) and R = X - deq(Q(X)) in fp32
      float r[8];
      residual_pair<0>(xf, cx.x, s, r);
      residual_pair<1>(xf, cx.x, s, r);
      residual_pair<2>(xf, cx.x, s, r);
      residual_pair<3>(xf, cx.x, s, r);
      float m = fmaxf(fmaxf(fmaxf(fabsf(r[0]), fabsf(r[1])), fmaxf(fabsf(r[2]), fabsf(r[3]))),
                      fmaxf(fmaxf(fabsf(r[4]), fabsf(r[5])), fmaxf(fabsf(r[6]), fabsf(r[7]))));
      const unsigned ramax = quad_max_u32(__builtin_bit_cast(unsigned, m));
      const unsigned er = ramax >> 23;                 // fp32 biased exponent
      const unsigned rc = er > kEmax<kRFmt> ? er - kEmax<kRFmt> : 0u;
      cr = encode_part<kRFmt>(r, rc);
      if (nonfinite) cr = u32x2_t{0u, 0u};
      src = nonfinite ? 255u : rc;
    }

    if (valid) {
      store_part<kXFmt>(p.qx, g, part, cx);
      if constexpr (kResidual) store_part<kRFmt>(p.qr, g, part, cr);
      if (part == 0) {
        p.sx[g] = (uint8_t)sxc;
        if (kResidual) p.sr[g] = (uint8_t)src;
      }
    }
  }
}

}  // namespace

namespace {

template <int kXFmt, int kRFmt, int kRotate>
void launch_one(bool x_f32, dim3 grid, dim3 block, hipStream_t stream, const QuantParams& p) {
  if (x_f32)
    hipLaunchKernelGGL((quantize_kernel<kXFmt, kRFmt, true, kRotate>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((quantize_kernel<kXFmt, kRFmt, false, kRotate>), grid, block, 0, stream, p);
}

}  // namespace

hipError_t launch_quantize(const void* x, bool x_f32, int rotate, int x_fmt, int r_fmt, int64_t rows, int64_t K,
                           int64_t ldx, uint8_t* qx, uint8_t* sx, uint8_t* qr, uint8_t* sr, hipStream_t stream) {
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
  const dim3 grid((unsigned)groups), block(kThreads);
  if (qr == nullptr) r_fmt = 0;
  // rotation 1 goes with the E2M1 residual pass (activations), rotation 2
  // with plain E2M1 (weights); E4M3 output only without rotation
  const int key = rotate * 100 + x_fmt * 10 + r_fmt;
  switch (key) {
    case 40: launch_one<4, 0, 0>(x_f32, grid, block, stream, p); break;
    case 44: launch_one<4, 4, 0>(x_f32, grid, block, stream, p); break;
    case 48: launch_one<4, 8, 0>(x_f32, grid, block, stream, p); break;
    case 80: launch_one<8, 0, 0>(x_f32, grid, block, stream, p); break;
    case 144: launch_one<4, 4, 1>(x_f32, grid, block, stream, p); break;
    case 240: launch_one<4, 0, 2>(x_f32, grid, block, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rfq
