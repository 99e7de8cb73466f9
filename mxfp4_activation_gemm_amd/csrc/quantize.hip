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
//    activation and folded into the weight): each n-block along K (n = 32,
//    one MX block, or 64, two) is multiplied by the unnormalised n x n
//    Sylvester Hadamard matrix H, and each output, the exact sum of the
//    block's n values with signs (over n for the weight), is rounded once
//    to fp32. Here one lane owns a whole MX block (a wave's blocks are
//    loaded contiguously and transposed through LDS), so the 32-point
//    transform needs no cross-lane moves: five in-lane fp64 butterfly
//    passes of spans 1, 2, 4, 8, 16, each taking (a, b) at (i, i + span) to
//    (a + b, a - b); the 64-point one adds a sixth pass across the lane
//    pair that holds its two MX blocks. The sums are exact whenever the
//    block's terms span at most 53 bits (a bf16 block whose nonzero values
//    span at most 40 binades for n = 32, 39 for n = 64; fp32: 24, 23), and
//    then the one fp64 -> fp32 conversion is the only rounding. Activations
//    quantize X H; weights W H / n (an exact power of two), so the GEMM
//    returns X W^T unchanged. Codes are decided on the rotated fp32 values;
//    the residual stays exact (|R| is at most half an E2M1 step, so
//    R = v - deq(v) loses no bits in fp32);
//  * MXFP8 output ("Activation Outliers Matter", Abstract and §1 study MXFP8
//    beside MXFP4; elements per OCP MX v1.0): E4M3 codes, one byte per
//    element, with se = max(floor(log2 amax) - 8, -127), either for X itself
//    (W4A8) or for the residual R of an MXFP4 Q(X) (RFQ with an MXFP8 second
//    path). Values are clamped to +-448 * 2^se before the scaled fp32 -> FP8
//    conversion (round to nearest even), which is the saturation rule: from
//    448 up to the 464 midpoint the nearest value is 448 anyway.

#include "kernels.h"
#include "mx_encode.h"

namespace rfq {
namespace {

using namespace mx;

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x2_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;          // 4 waves per workgroup
constexpr int kUnits = 4;              // 16-block units per wave
constexpr int kBlocksPerWave = 16 * kUnits;

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

// Walsh-Hadamard sums of one 32-block held whole by this lane,
// unnormalised, in fp64: five butterfly passes.
//
// A sum that is exactly zero comes out as +0, whatever the signs of the
// zeros summed. Rounding to nearest gives -0 for a + b only when a and b
// are both -0, and for a - b only when a is -0 and b is +0; so when no
// first operand a of a butterfly is -0, no output of it is either. The first
// pass's first operands are turned from -0 to +0 (a + 0.0), and every later
// first operand is an output of an earlier pass.
__device__ __forceinline__ void hadamard32_sums(double* v) {
#pragma unroll
  for (int j = 0; j < 32; j += 2) v[j] = v[j] + 0.0;
#pragma unroll
  for (int span = 1; span < 32; span *= 2)
#pragma unroll
    for (int j = 0; j < 32; ++j)
      if (!(j & span)) {
        const double a = v[j], b = v[j + span];
        v[j] = a + b;
        v[j + span] = a - b;
      }
}

// The span-32 pass of a 64-point transform over lanes 2m and 2m + 1, which
// hold the 32-point sums of the two halves of one 64-block (Sylvester's
// H64 = [[H32, H32], [H32, -H32]]): the even lane keeps a + b, the odd one
// a - b, a the even lane's value and b the odd one's. The partner's fp64
// value comes over as two 32-bit DPP moves; fma(-1, b, a) is a - b with one
// rounding, as the sum of a and -b. (Neither lane's first operand, its own
// sum on the even lane and the partner's on the odd one, is -0, so neither
// output is.)
__device__ __forceinline__ void hadamard64_pair_pass(double* v, unsigned lane) {
  const double sign = (lane & 1) ? -1.0 : 1.0;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v[j]);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)u, kQuadXor1, 0xF, 0xF, true);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), kQuadXor1, 0xF, 0xF, true);
    const double o = __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
    v[j] = __builtin_fma(sign, v[j], o);
  }
}

// One rounding of each fp64 sum to fp32, after an exact power-of-two
// scaling (1, or 1 / n on the weight side). (The passes leave no exact zero
// as -0; a nonzero sum too small for fp32 keeps its sign.)
__device__ __forceinline__ void round_sums(const double* v, float* f, double scale) {
#pragma unroll
  for (int j = 0; j < 32; ++j) f[j] = (float)(v[j] * scale);
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
// (else bf16).
template <int kXFmt, int kRFmt, bool kF32In>
__global__ __launch_bounds__(kThreads) void quantize_kernel(QuantParams p) {
  constexpr bool kResidual = kRFmt != 0;
  static_assert(kXFmt == 4 || (kXFmt == 8 && !kResidual), "format combination");
  const unsigned lane = threadIdx.x & 63;
  const unsigned wave = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  // first block of this wave, and how many blocks are left from it (64-bit
  // first: the block count may come close to 2^32)
  if ((uint64_t)wave * kBlocksPerWave >= p.total_blocks) return;
  const uint32_t g0 = wave * kBlocksPerWave;
  const uint32_t left = p.total_blocks - g0;
  const uint32_t quad = lane >> 2, part = lane & 3;

  // the lane's 8 values of each unit: one 16-byte load of bf16, or two of fp32
  constexpr int kLoads = kF32In ? 2 : 1;
  u32x4_t w[kUnits][kLoads];
  uint32_t gblk[kUnits];
  if (kF32In && left >= kBlocksPerWave && p.ldx == (int64_t)p.nblk_row * 32) {
    // fp32 X, a whole wave of dense rows: unit u is 16 consecutive blocks
    // from block g0 + 16 u on, and lane l takes their elements 8 l .. 8 l + 7.
    // (This path gains 7% on fp32 X of 32768 x 13824, 389 against 414 us;
    // for bf16 X the same path measured 2% slower than the general one, 223
    // against 219 us, so bf16 takes the general path.)
    const u32x4_t* src = static_cast<const u32x4_t*>(p.x) + (uint64_t)g0 * (4 * kLoads) + kLoads * lane;
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      gblk[u] = g0 + u * 16 + quad;
#pragma unroll
      for (int h = 0; h < kLoads; ++h) w[u][h] = __builtin_nontemporal_load(src + 64 * kLoads * u + h);
    }
  } else {
    // row/column of each unit's block for this lane
    const uint32_t row0 = g0 / p.nblk_row, col0 = g0 - row0 * p.nblk_row;
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      const uint32_t g = g0 + u * 16 + quad;
      uint32_t b = col0 + u * 16 + quad, r = row0;
      while (b >= p.nblk_row) { b -= p.nblk_row; ++r; }
      gblk[u] = g;
      const bool valid = u * 16 + quad < left;
      const int64_t elem = (int64_t)r * p.ldx + (int64_t)b * 32 + part * 8;
      const u32x4_t* src = kF32In ? reinterpret_cast<const u32x4_t*>(static_cast<const float*>(p.x) + elem)
                                  : reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(p.x) + elem);
#pragma unroll
      for (int h = 0; h < kLoads; ++h) w[u][h] = valid ? __builtin_nontemporal_load(src + h) : u32x4_t{0, 0, 0, 0};
    }
  }

#pragma unroll
  for (int u = 0; u < kUnits; ++u) {
    const uint32_t g = gblk[u];
    const bool valid = u * 16 + quad < left;
    float xf[8];
    unsigned e;                                        // biased exponent of the block amax (fp32/bf16 field)
    if (!kF32In) {
      const unsigned amax = quad_max_u32(bf16x8_absmax_bits(w[u][0]));
      e = amax >> 7;
      widen_bf16x8(w[u][0], xf);
    } else {
      // (whole-vector bit casts: a bit cast of a single ext-vector element
      // has been seen to read element 0)
      const f32x4_t lo = __builtin_bit_cast(f32x4_t, w[u][0]), hi = __builtin_bit_cast(f32x4_t, w[u][kLoads - 1]);
      xf[0] = lo.x; xf[1] = lo.y; xf[2] = lo.z; xf[3] = lo.w;
      xf[4] = hi.x; xf[5] = hi.y; xf[6] = hi.z; xf[7] = hi.w;
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

// max |f[j]| over 32 fp32 values as a float (a NaN operand of max is dropped
// unless both are NaN).
__device__ __forceinline__ float absmax32(const float* f) {
  float m[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) m[j] = fmaxf(fmaxf(fabsf(f[4 * j]), fabsf(f[4 * j + 1])), fmaxf(fabsf(f[4 * j + 2]), fabsf(f[4 * j + 3])));
#pragma unroll
  for (int k = 4; k >= 1; k /= 2)
#pragma unroll
    for (int j = 0; j < k; ++j) m[j] = fmaxf(m[j], m[j + k]);
  return m[0];
}

// The rotated passes, one 32-block per lane: X H with the E2M1 residual
// pass (kRotate 1, activations) or W H / n to plain E2M1 (kRotate 2,
// weights), H of size kSize = 32 (one MX block) or 64 (two adjacent MX
// blocks of a row, held by lanes 2m and 2m + 1: K is a multiple of 64, so a
// row has an even number of blocks and every even block starts a pair). A
// wave covers 64 consecutive blocks; each lane transforms and encodes one
// block and writes its 16 code bytes and its scale byte, so the code and
// scale stores of a wave are contiguous.
template <bool kF32In, int kRotate, int kSize>
__global__ __launch_bounds__(kThreads) void rotate_quantize_kernel(QuantParams p) {
  constexpr bool kResidual = kRotate == 1;
  const unsigned lane = threadIdx.x & 63;
  // (the wave index as a scalar, so that the choice of load path below is a
  // scalar branch)
  const unsigned wave = __builtin_amdgcn_readfirstlane(blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6));
  // (64-bit first: the block count may come close to 2^32; waves past the
  // end stay to the barrier below and skip their loads and stores)
  const bool wave_live = (uint64_t)wave * 64 < p.total_blocks;
  const uint32_t g0 = wave * 64;
  const uint32_t left = wave_live ? p.total_blocks - g0 : 0u;
  const uint32_t g = g0 + lane;
  const bool valid = lane < left;

  // A block's bytes as 16-byte chunks (4 for bf16, 8 for fp32). The wave
  // loads its 64 blocks contiguously (1 KB per instruction, lane l taking
  // chunk l) and transposes them through LDS to one block per lane, with one
  // padding chunk per block so that the per-lane reads are free of bank
  // conflicts. Loading each lane's own block directly (4 or 8 loads that
  // each take 16 bytes of every 64 or 128 across the wave) measured 232
  // against 253 us on one box and 280 against 239 us on another for bf16 X
  // on a 32768 x 13824 layer, and 519 against 374 us for fp32 X.
  constexpr int kLoads = kF32In ? 8 : 4;
  constexpr int kStride = kLoads * 16 + 16;
  __shared__ __attribute__((aligned(16))) uint8_t stage[kThreads / 64][64 * kStride];
  uint8_t* ws = stage[threadIdx.x >> 6];
  u32x4_t w[kLoads];
  if (left >= 64 && p.ldx == (int64_t)p.nblk_row * 32) {
    // the common case, a whole wave of a dense X: its 64 blocks are
    // 64 kLoads consecutive chunks from block g0 on
    const u32x4_t* src = static_cast<const u32x4_t*>(p.x) + (uint64_t)g0 * kLoads + lane;
#pragma unroll
    for (int h = 0; h < kLoads; ++h) w[h] = __builtin_nontemporal_load(src + h * 64);
  } else {
    // rows with a stride, or the last wave: each chunk's row and column,
    // from those of g0 (computed in every wave, so that the row walks take
    // at most 1 + 63 / nblk_row steps, in waves past the end too)
    const uint32_t row0 = g0 / p.nblk_row, col0 = g0 - row0 * p.nblk_row;
#pragma unroll
    for (int h = 0; h < kLoads; ++h) {
      const uint32_t c = h * 64 + lane, blk = c / kLoads, chunk = c % kLoads;
      uint32_t b = col0 + blk, r = row0;
      while (b >= p.nblk_row) { b -= p.nblk_row; ++r; }
      const bool ok = blk < left;
      const int64_t eo = ok ? (int64_t)r * p.ldx + (int64_t)b * 32 + chunk * (kF32In ? 4 : 8) : 0;
      const u32x4_t* src = kF32In ? reinterpret_cast<const u32x4_t*>(static_cast<const float*>(p.x) + eo)
                                  : reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(p.x) + eo);
      w[h] = ok ? __builtin_nontemporal_load(src) : u32x4_t{0, 0, 0, 0};
    }
  }
#pragma unroll
  for (int h = 0; h < kLoads; ++h) {
    const uint32_t c = h * 64 + lane;
    *reinterpret_cast<u32x4_t*>(ws + (c / kLoads) * kStride + (c % kLoads) * 16) = w[h];
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < kLoads; ++h) w[h] = *reinterpret_cast<const u32x4_t*>(ws + lane * kStride + h * 16);

  double v[32];
#pragma unroll
  for (int h = 0; h < kLoads; ++h) {
    if constexpr (kF32In) {
      const f32x4_t q = __builtin_bit_cast(f32x4_t, w[h]);
      v[4 * h] = q.x; v[4 * h + 1] = q.y; v[4 * h + 2] = q.z; v[4 * h + 3] = q.w;
    } else {
      float f[8];
      widen_bf16x8(w[h], f);
#pragma unroll
      for (int j = 0; j < 8; ++j) v[8 * h + j] = f[j];
    }
  }
  float xf[32];
  hadamard32_sums(v);
  if constexpr (kSize == 64) hadamard64_pair_pass(v, lane);
  round_sums(v, xf, kRotate == 2 ? 1.0 / kSize : 1.0);

  // Block amax by float max over magnitudes. Max drops a NaN operand, but
  // here non-finite values never mix with finite ones in a block: a NaN or
  // an infinity among the inputs reaches every one of the 32 sums, as a
  // NaN or an infinity, and an fp32 overflow of a sum gives an infinity
  // that the max keeps; a block of NaNs gives a NaN. Either way the
  // exponent field reads 255.
  const unsigned e = __builtin_bit_cast(unsigned, absmax32(xf)) >> 23;
  const bool nonfinite = e == 255;
  const unsigned sxc = nonfinite ? 255u : (e > 2u ? e - 2u : 0u);
  const float s = scale_operand(sxc);
  u32x4_t cx;
#pragma unroll
  for (int q = 0; q < 4; ++q) cx[q] = nonfinite ? 0u : encode_f32x8(xf + 8 * q, s);

  u32x4_t cr = {0u, 0u, 0u, 0u};
  unsigned src_code = 255u;
  if constexpr (kResidual) {
    float rr[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const unsigned c = cx[q];
      residual_pair<0>(xf + 8 * q, c, s, rr + 8 * q);
      residual_pair<1>(xf + 8 * q, c, s, rr + 8 * q);
      residual_pair<2>(xf + 8 * q, c, s, rr + 8 * q);
      residual_pair<3>(xf + 8 * q, c, s, rr + 8 * q);
    }
    const unsigned er = __builtin_bit_cast(unsigned, absmax32(rr)) >> 23;   // (R is finite when X is)
    const unsigned rc = er > 2u ? er - 2u : 0u;
    const float sr = scale_operand(rc);
#pragma unroll
    for (int q = 0; q < 4; ++q) cr[q] = nonfinite ? 0u : encode_f32x8(rr + 8 * q, sr);
    src_code = nonfinite ? 255u : rc;
  }

  if (valid) {
    __builtin_nontemporal_store(cx, reinterpret_cast<u32x4_t*>(p.qx + (uint64_t)g * 16));
    p.sx[g] = (uint8_t)sxc;
    if constexpr (kResidual) {
      __builtin_nontemporal_store(cr, reinterpret_cast<u32x4_t*>(p.qr + (uint64_t)g * 16));
      p.sr[g] = (uint8_t)src_code;
    }
  }
}

}  // namespace

namespace {

template <int kXFmt, int kRFmt>
void launch_one(bool x_f32, dim3 grid, dim3 block, hipStream_t stream, const QuantParams& p) {
  if (x_f32)
    hipLaunchKernelGGL((quantize_kernel<kXFmt, kRFmt, true>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((quantize_kernel<kXFmt, kRFmt, false>), grid, block, 0, stream, p);
}

template <int kRotate, int kSize>
void launch_rotated(bool x_f32, hipStream_t stream, const QuantParams& p) {
  const uint64_t waves = ((uint64_t)p.total_blocks + 63) / 64;
  const dim3 grid((unsigned)((waves + kThreads / 64 - 1) / (kThreads / 64))), block(kThreads);
  if (x_f32)
    hipLaunchKernelGGL((rotate_quantize_kernel<true, kRotate, kSize>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((rotate_quantize_kernel<false, kRotate, kSize>), grid, block, 0, stream, p);
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
  const uint64_t waves = ((uint64_t)p.total_blocks + kBlocksPerWave - 1) / kBlocksPerWave;
  const uint64_t groups = (waves + kThreads / 64 - 1) / (kThreads / 64);
  const dim3 grid((unsigned)groups), block(kThreads);
  if (qr == nullptr) r_fmt = 0;
  // rotation 1 (3) goes with the E2M1 residual pass (activations), rotation
  // 2 (4) with plain E2M1 (weights), 32-point (64-point); E4M3 output only
  // without rotation
  const int key = rotate * 100 + x_fmt * 10 + r_fmt;
  switch (key) {
    case 40: launch_one<4, 0>(x_f32, grid, block, stream, p); break;
    case 44: launch_one<4, 4>(x_f32, grid, block, stream, p); break;
    case 48: launch_one<4, 8>(x_f32, grid, block, stream, p); break;
    case 80: launch_one<8, 0>(x_f32, grid, block, stream, p); break;
    case 144: launch_rotated<1, 32>(x_f32, stream, p); break;
    case 240: launch_rotated<2, 32>(x_f32, stream, p); break;
    case 344: launch_rotated<1, 64>(x_f32, stream, p); break;
    case 440: launch_rotated<2, 64>(x_f32, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rfq
