// RFQ W4A4 GEMM on gfx950 block-scaled FP4 MFMA.
//
// What is computed ("Activation Outliers Matter: Robust Recovery for
// Quantized Multimodal LLMs", §1 contributions: the quantized residual is
// multiplied during the GEMM and its contribution accumulated):
//   Y[m, n] = sum_k deq(QX)[m,k] deq(W)[n,k] + deq(QR)[m,k] deq(W)[n,k]
// i.e. one contraction of [QX | QR] (M x 2K) against [W ; W] over a doubled
// K, every term landing in the same fp32 accumulator.
//
// Instruction: v_mfma_scale_f32_32x32x64_f8f6f4 with both operands FP4
// (E2M1). Operand lane layout (checked on hardware): lane l holds row l % 32
// and the 32 elements of K-block l / 32 of the 64-wide K step, as 16 bytes,
// element 2j in the low nibble of byte j; its 32-bit scale operand supplies
// the E8M0 code of that (row, block) in the byte chosen by op_sel. Output
// lane l holds column l % 32, rows 8 (i / 4) + 4 (l / 32) + i % 4.
//
// Tiling: a 256 x 256 output tile per workgroup of 4 waves (2 x 2), each
// wave 128 x 128 = 4 x 4 MFMA tiles (256 fp32 accumulators per lane).
// K advances 128 elements (64 bytes of codes per row) per stage, two MFMA
// steps.
//
// Data movement, per stage:
//  * Code tiles (QX, QR, W; 256 rows x 64 B each) go global -> LDS with
//    buffer loads that write LDS directly. Four consecutive lanes fetch one
//    row's 64 contiguous bytes, so each quad touches one cache line. In LDS a
//    row is 4 chunks of 16 B (one K-block each); chunk c of row r sits at
//    position c ^ f(r), f(r) = (r >> 2) & 3, which makes the MFMA operand
//    reads (32 rows, same chunk) free of LDS bank conflicts on gfx950
//    (measured with the LDS bank-conflict counter; swizzles that are
//    conflict-free under a plain 32- or 64-bank model were not). The swizzle
//    is applied by choosing which chunk each lane fetches; the LDS slot of a
//    lane is fixed by the hardware.
//  * Scales are fetched 16 B per row (16 blocks = 4 stages) into a separate
//    LDS area every fourth stage; each stage reads its 4-byte word per row.
//  * Buffer loads return zero outside the tensor, which covers partial M
//    and N tiles; partial K is masked per 16-byte chunk.
// Two LDS stages: stage s + 1 is loaded while stage s's 64 MFMAs run.

#include "kernels.h"

namespace rfq {
namespace {

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kThreads = 256;               // 4 waves per workgroup
constexpr int kBK = 128;                    // K elements per stage
constexpr int kSteps = kBK / 64;            // 2 MFMA K-steps per stage
constexpr int kRowBytes = kBK / 2;          // 64 bytes of codes per row per stage
constexpr int kScaleGroup = 4;              // stages per scale fetch (16 blocks)
constexpr int kScaleRowBytes = 16;
constexpr uint32_t kOOB = 0x80000000u;      // voffset that is always out of range
constexpr int kGroupM = 4;                  // tile rows swept together (L2 reuse)

// Output tile BM x BN on a kWavesM x kWavesN grid of waves; kOcc workgroups
// are meant to share a CU (LDS and registers are sized for that).
template <int BM_, int BN_, int WavesM_, int WavesN_, int Occ_>
struct TileCfg {
  static constexpr int kBM = BM_, kBN = BN_, kWavesM = WavesM_, kWavesN = WavesN_, kOcc = Occ_;
  static_assert(kWavesM * kWavesN * 64 == kThreads, "4 waves");
  static constexpr int kTM = kBM / kWavesM / 32;   // MFMA tiles along M per wave
  static constexpr int kTN = kBN / kWavesN / 32;   // along N
  static constexpr int kTileBytesA = kBM * kRowBytes;
  static constexpr int kTileBytesB = kBN * kRowBytes;
  static constexpr int kStageBytes = 2 * kTileBytesA + kTileBytesB;     // X, R, W
  static constexpr int kScaleBytesA = kBM * kScaleRowBytes;
  static constexpr int kScaleBytes = 2 * kScaleBytesA + kBN * kScaleRowBytes;
  static constexpr int kLdsBytes = 2 * kStageBytes + 2 * kScaleBytes;
  static constexpr int kLoadsA = kBM / 4 / 16;     // 16-row load instructions per wave for X (and R)
  static constexpr int kLoadsB = kBN / 4 / 16;     // for W
  static constexpr int kScaleLoadsA = kBM / 64;    // 64-row scale instructions per operand
  static constexpr int kScaleLoadsB = kBN / 64;
  static constexpr int kScaleLoads = 2 * kScaleLoadsA + kScaleLoadsB;
  static_assert(kScaleLoads % 4 == 0, "scale loads spread evenly over 4 waves");
  static_assert(kLdsBytes * kOcc <= 160 * 1024, "LDS budget per CU");
};
using Tile256 = TileCfg<256, 256, 2, 2, 1>;   // one workgroup per CU, 128x128 per wave
using Tile128 = TileCfg<128, 256, 2, 2, 2>;   // two workgroups per CU, 64x128 per wave

struct GemmParams {
  const uint8_t* qx;
  const uint8_t* sx;
  const uint8_t* qr;
  const uint8_t* sr;
  const uint8_t* w;
  const uint8_t* sw;
  void* y;
  int64_t ldy;
  int32_t M, N, K;
  int32_t tiles_m, tiles_n;
};

__device__ __forceinline__ uint32_t swz(uint32_t r) { return (r >> 2) & 3u; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // gfx9 raw buffer: stride 0, num_records in bytes, dword3 = 32-bit data format
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ void load16_to_lds(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, voff, 0, 0, 0);
}

__device__ __forceinline__ i32x8_t read_frag(const uint8_t* p) {
  const i32x4_t v = *reinterpret_cast<const i32x4_t*>(p);
  return i32x8_t{v.x, v.y, v.z, v.w, 0, 0, 0, 0};
}

// Maps a workgroup id to an output tile: first spread consecutive tiles of
// one XCD's share over its workgroups (ids are dealt round-robin to the 8
// XCDs), then walk tiles in groups of kGroupM tile rows so that concurrently
// running workgroups share activation rows and weight columns in L2.
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  const int xcd = bid % 8, idx = bid / 8;
  const int base = total / 8, rem = total % 8;
  const int logical = xcd < rem ? xcd * (base + 1) + idx : rem * (base + 1) + (xcd - rem) * base + idx;
  const int per_group = kGroupM * tiles_n;
  const int group = logical / per_group;
  const int first_m = group * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int in_group = logical - group * per_group;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

template <int S, bool kResid, int kTM, int kTN>
__device__ __forceinline__ void mfma_step(f32x16_t (&acc)[kTM][kTN], const i32x8_t (&ax)[kTM],
                                          const i32x8_t (&ar)[kTM], const i32x8_t (&b)[kTN],
                                          const uint32_t (&scx)[kTM], const uint32_t (&scr)[kTM],
                                          const uint32_t (&scw)[kTN]) {
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ax[i], b[j], acc[i][j], 4, 4, 2 * S,
                                                                  (int)scx[i], 2 * S, (int)scw[j]);
  if (kResid) {
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ar[i], b[j], acc[i][j], 4, 4, 2 * S,
                                                                    (int)scr[i], 2 * S, (int)scw[j]);
  }
}

// kFast: K % 512 == 0 (whole stages and whole 16-block scale groups).
template <class C, bool kResid, bool kOutBf16, bool kFast>
__global__ __launch_bounds__(kThreads, C::kOcc) void gemm_kernel(GemmParams p) {
  constexpr int kBM = C::kBM, kBN = C::kBN, kWavesM = C::kWavesM, kWavesN = C::kWavesN;
  constexpr int kTM = C::kTM, kTN = C::kTN;
  constexpr int kTileBytesA = C::kTileBytesA, kStageBytes = C::kStageBytes;
  constexpr int kScaleBytesA = C::kScaleBytesA, kScaleBytes = C::kScaleBytes;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::kLdsBytes];
  uint8_t* const tiles = lds;
  uint8_t* const scales = lds + 2 * kStageBytes;

  const unsigned lane = threadIdx.x & 63;
  const unsigned wave = threadIdx.x >> 6;
  const unsigned wm = wave / kWavesN, wn = wave % kWavesN;
  int tm, tn;
  tile_of(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  const int m0 = tm * kBM, n0 = tn * kBN;
  const uint32_t kbytes = (uint32_t)p.K / 2, kblocks = (uint32_t)p.K / 32;
  const uint32_t rows_a = (uint32_t)min(kBM, p.M - m0), rows_b = (uint32_t)min(kBN, p.N - n0);

  const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.qx + (int64_t)m0 * kbytes, rows_a * kbytes);
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(kResid ? p.qr + (int64_t)m0 * kbytes : p.qx, rows_a * kbytes);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.w + (int64_t)n0 * kbytes, rows_b * kbytes);
  const __amdgpu_buffer_rsrc_t rsx = make_rsrc(p.sx + (int64_t)m0 * kblocks, rows_a * kblocks);
  const __amdgpu_buffer_rsrc_t rsr = make_rsrc(kResid ? p.sr + (int64_t)m0 * kblocks : p.sx, rows_a * kblocks);
  const __amdgpu_buffer_rsrc_t rsw = make_rsrc(p.sw + (int64_t)n0 * kblocks, rows_b * kblocks);

  // Code-tile loads: this wave fetches tile rows [BM/4 wave, BM/4 (wave+1))
  // of X and R and [BN/4 wave, BN/4 (wave+1)) of W, 16 rows per instruction;
  // lane l takes row 16 n + l / 4 and chunk (l % 4) ^ f(row) of it.
  const unsigned lrow = lane & 31, lhalf = lane >> 5;
  uint32_t lda_voff[C::kLoadsA], lda_chunk[C::kLoadsA], ldb_voff[C::kLoadsB], ldb_chunk[C::kLoadsB];
#pragma unroll
  for (int n = 0; n < C::kLoadsA; ++n) {
    const uint32_t row = kBM / 4 * wave + 16 * n + (lane >> 2);
    lda_chunk[n] = (lane & 3) ^ swz(row);
    lda_voff[n] = row * kbytes + 16 * lda_chunk[n];
  }
#pragma unroll
  for (int n = 0; n < C::kLoadsB; ++n) {
    const uint32_t row = kBN / 4 * wave + 16 * n + (lane >> 2);
    ldb_chunk[n] = (lane & 3) ^ swz(row);
    ldb_voff[n] = row * kbytes + 16 * ldb_chunk[n];
  }

  auto issue_stage = [&](int st, uint8_t* buf) {
    const uint32_t kb = (uint32_t)st * kRowBytes;
#pragma unroll
    for (int n = 0; n < C::kLoadsA; ++n) {
      uint32_t vo = lda_voff[n] + kb;
      if (!kFast && (uint32_t)st * (kBK / 32) + lda_chunk[n] >= kblocks) vo = kOOB;
      uint8_t* dst = buf + (kBM / 4 * wave + 16 * n) * kRowBytes;
      load16_to_lds(rx, dst, vo);
      if (kResid) load16_to_lds(rr, dst + kTileBytesA, vo);
    }
#pragma unroll
    for (int n = 0; n < C::kLoadsB; ++n) {
      uint32_t vo = ldb_voff[n] + kb;
      if (!kFast && (uint32_t)st * (kBK / 32) + ldb_chunk[n] >= kblocks) vo = kOOB;
      load16_to_lds(rw, buf + 2 * kTileBytesA + (kBN / 4 * wave + 16 * n) * kRowBytes, vo);
    }
  };

  // Scale loads for group g (stages 4g .. 4g + 3): 16 bytes per row, lane l
  // of instruction j takes row 64 (j % 4) + l of operand j / 4 (X, R, W);
  // wave w issues j = 3w, 3w + 1, 3w + 2.
  auto issue_scale_rows = [&](__amdgpu_buffer_rsrc_t r, int g, uint8_t* dst, uint32_t row) {
      if (kFast) {
        load16_to_lds(r, dst, row * kblocks + 16 * g);
      } else {
        // gather byte by byte; blocks past K get a finite scale (their codes are zero)
        uint32_t wv[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          uint32_t v = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t blk = 16 * g + 4 * d + e;
            const uint32_t b = blk < kblocks ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, row * kblocks + blk, 0, 0)
                                             : 127u;
            v |= b << (8 * e);
          }
          wv[d] = v;
        }
        *reinterpret_cast<i32x4_t*>(dst + lane * kScaleRowBytes) =
            i32x4_t{(int)wv[0], (int)wv[1], (int)wv[2], (int)wv[3]};
      }
  };
  // Instruction j of a group covers 64 rows: j < A loads X rows, then R rows,
  // then W rows (A = BM / 64); wave w issues j = w q .. w q + q - 1.
  auto issue_scales = [&](int g, uint8_t* sbuf) {
    constexpr int kA = C::kScaleLoadsA, kPerWave = C::kScaleLoads / 4;
#pragma unroll
    for (int q = 0; q < kPerWave; ++q) {
      const int j = kPerWave * (int)wave + q;   // wave-uniform: plain branches, no descriptor select
      if (j < kA) {
        issue_scale_rows(rsx, g, sbuf + 64 * j * kScaleRowBytes, 64 * j + lane);
      } else if (j < 2 * kA) {
        if (kResid) issue_scale_rows(rsr, g, sbuf + kScaleBytesA + 64 * (j - kA) * kScaleRowBytes, 64 * (j - kA) + lane);
      } else {
        issue_scale_rows(rsw, g, sbuf + 2 * kScaleBytesA + 64 * (j - 2 * kA) * kScaleRowBytes, 64 * (j - 2 * kA) + lane);
      }
    }
  };

  // Per-lane LDS read offsets. A fragment of 32 rows starting at tile row
  // 32 t: lane (lhalf, lrow) reads chunk (2 s + lhalf) of row 32 t + lrow.
  uint32_t rd_off[kSteps];
#pragma unroll
  for (int s = 0; s < kSteps; ++s) rd_off[s] = lrow * kRowBytes + 16 * ((2 * s + lhalf) ^ swz(lrow));
  const uint32_t a_row0 = kBM / kWavesM * wm, b_row0 = kBN / kWavesN * wn;

  f32x16_t acc[kTM][kTN];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  const int nstages = (p.K + kBK - 1) / kBK;
  i32x4_t gx[kTM], gr[kTM], gw[kTN];     // scale rows of the current group
  issue_scales(0, scales);
  issue_stage(0, tiles);

  for (int st = 0; st < nstages; ++st) {
    const uint8_t* buf = tiles + (st & 1) * kStageBytes;
    const uint8_t* sbuf = scales + ((st / kScaleGroup) & 1) * kScaleBytes;
    __builtin_amdgcn_s_waitcnt(0);      // this stage's tiles and scales have landed in LDS
    __syncthreads();

    i32x8_t ax[kSteps][kTM], ar[kSteps][kTM], bw[kSteps][kTN];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
#pragma unroll
      for (int i = 0; i < kTM; ++i) {
        const uint8_t* src = buf + (a_row0 + 32 * i) * kRowBytes + rd_off[s];
        ax[s][i] = read_frag(src);
        if (kResid) ar[s][i] = read_frag(src + kTileBytesA);
      }
#pragma unroll
      for (int j = 0; j < kTN; ++j) bw[s][j] = read_frag(buf + 2 * kTileBytesA + (b_row0 + 32 * j) * kRowBytes + rd_off[s]);
    }
    // Scale words: every fourth stage each lane reads the 16 bytes (16
    // blocks = 4 stages) of each of its rows in one ds_read_b128; word
    // (st % 4) of them serves stage st, and byte 2 s of (word >> 8 lhalf) is
    // the scale of block 4 st + 2 s + lhalf of the row.
    if (st % kScaleGroup == 0) {
#pragma unroll
      for (int i = 0; i < kTM; ++i) {
        const uint8_t* s0 = sbuf + (a_row0 + 32 * i + lrow) * kScaleRowBytes;
        gx[i] = *reinterpret_cast<const i32x4_t*>(s0);
        if (kResid) gr[i] = *reinterpret_cast<const i32x4_t*>(s0 + kScaleBytesA);
      }
#pragma unroll
      for (int j = 0; j < kTN; ++j)
        gw[j] = *reinterpret_cast<const i32x4_t*>(sbuf + 2 * kScaleBytesA + (b_row0 + 32 * j + lrow) * kScaleRowBytes);
    }
    const int sw_idx = st % kScaleGroup;
    uint32_t cx[kTM], cr[kTM], cw[kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      cx[i] = (uint32_t)gx[i][sw_idx] >> (8 * lhalf);
      cr[i] = kResid ? (uint32_t)gr[i][sw_idx] >> (8 * lhalf) : 0u;
    }
#pragma unroll
    for (int j = 0; j < kTN; ++j) cw[j] = (uint32_t)gw[j][sw_idx] >> (8 * lhalf);

    if (st + 1 < nstages) {
      if ((st + 1) % kScaleGroup == 0) issue_scales((st + 1) / kScaleGroup, scales + (((st + 1) / kScaleGroup) & 1) * kScaleBytes);
      issue_stage(st + 1, tiles + ((st + 1) & 1) * kStageBytes);
    }
    mfma_step<0, kResid, kTM, kTN>(acc, ax[0], ar[0], bw[0], cx, cr, cw);
    mfma_step<1, kResid, kTM, kTN>(acc, ax[1], ar[1], bw[1], cx, cr, cw);
  }

  // Epilogue: fp32 accumulators to Y.
  const int row_base = m0 + (int)a_row0 + 4 * (int)lhalf;
  const int col_base = n0 + (int)b_row0 + (int)lrow;
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
      const int col = col_base + 32 * j;
      if (col >= p.N) continue;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = row_base + 32 * i + 8 * (q / 4) + (q % 4);
        if (row >= p.M) continue;
        const float v = acc[i][j][q];
        if (kOutBf16) {
          uint32_t u = __builtin_bit_cast(uint32_t, v);
          u = (v != v) ? 0x7FC00000u : u + 0x7FFFu + ((u >> 16) & 1u);
          reinterpret_cast<uint16_t*>(p.y)[(int64_t)row * p.ldy + col] = (uint16_t)(u >> 16);
        } else {
          reinterpret_cast<float*>(p.y)[(int64_t)row * p.ldy + col] = v;
        }
      }
    }
}

template <class C, bool kResid, bool kOutBf16>
hipError_t launch_variant(GemmParams p, bool fast, hipStream_t stream) {
  p.tiles_m = (p.M + C::kBM - 1) / C::kBM;
  p.tiles_n = (p.N + C::kBN - 1) / C::kBN;
  const int grid = p.tiles_m * p.tiles_n;
  if (fast)
    hipLaunchKernelGGL((gemm_kernel<C, kResid, kOutBf16, true>), dim3(grid), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm_kernel<C, kResid, kOutBf16, false>), dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <class C>
hipError_t launch_cfg(const GemmParams& p, bool resid, bool y_bf16, bool fast, hipStream_t stream) {
  if (resid)
    return y_bf16 ? launch_variant<C, true, true>(p, fast, stream) : launch_variant<C, true, false>(p, fast, stream);
  return y_bf16 ? launch_variant<C, false, true>(p, fast, stream) : launch_variant<C, false, false>(p, fast, stream);
}

}  // namespace

hipError_t launch_gemm(const uint8_t* qx, const uint8_t* sx, const uint8_t* qr, const uint8_t* sr,
                       const uint8_t* w, const uint8_t* sw, int64_t M, int64_t N, int64_t K,
                       void* y, bool y_bf16, int64_t ldy, hipStream_t stream) {
  GemmParams p;
  p.qx = qx; p.sx = sx; p.qr = qr; p.sr = sr; p.w = w; p.sw = sw;
  p.y = y; p.ldy = ldy;
  p.M = (int32_t)M; p.N = (int32_t)N; p.K = (int32_t)K;
  const bool fast = (K % (kBK * kScaleGroup)) == 0;
  return launch_cfg<Tile128>(p, qr != nullptr, y_bf16, fast, stream);
}

}  // namespace rfq
