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
// K advances 128 elements per stage (two MFMA steps). Per stage the QX, QR
// and W tiles go global -> LDS by buffer loads that write LDS directly,
// already in MFMA lane order (one 1 KB fragment per load instruction), so
// every LDS read is a contiguous, conflict-free ds_read_b128. Buffer loads
// return zero outside the tensor, which covers partial M, N and K tiles.
// Scales (4 bytes per row per stage) are loaded straight into registers.
// Two LDS stages; the next stage's loads are issued after this stage's
// fragments are in registers and overlap its 64 MFMAs.

#include "kernels.h"

namespace rfq {
namespace {

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kThreads = 256;
constexpr int kBM = 256, kBN = 256, kBK = 128;
constexpr int kWavesM = 2, kWavesN = 2;
constexpr int kTM = kBM / kWavesM / 32;     // 4 MFMA tiles along M per wave
constexpr int kTN = kBN / kWavesN / 32;     // 4 along N
constexpr int kSteps = kBK / 64;            // 2 MFMA K-steps per stage
constexpr int kFrag = 1024;                 // 32 rows x 32 bytes
constexpr int kTileBytesA = kBM / 32 * kSteps * kFrag;   // 16 KB
constexpr int kTileBytesB = kBN / 32 * kSteps * kFrag;   // 16 KB
constexpr int kStageBytes = 2 * kTileBytesA + kTileBytesB;  // X, R, W
constexpr uint32_t kOOB = 0x80000000u;      // voffset that is always out of range
constexpr int kGroupM = 4;                  // tile rows swept together (L2 reuse)

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

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // gfx9 raw buffer: stride 0, num_records in bytes, dword3 = 32-bit data format
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ void load_frag_to_lds(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, voff, 0, 0, 0);
}

__device__ __forceinline__ i32x8_t read_frag(const uint8_t* lds_frag, unsigned lane) {
  const i32x4_t v = *reinterpret_cast<const i32x4_t*>(lds_frag + lane * 16);
  return i32x8_t{v.x, v.y, v.z, v.w, 0, 0, 0, 0};
}

// One 32-bit word = the E8M0 scales of 4 consecutive blocks of one row.
__device__ __forceinline__ uint32_t load_scale_word(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0);
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

template <int S, bool kResid>
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

template <bool kResid, bool kOutBf16, bool kKAligned>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2][kStageBytes];

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

  // This wave loads fragments (row-frag f, step s) for f in {2 wave, 2 wave + 1}
  // of each of X, R and W; lane l fetches row 32 f + l % 32, bytes 32 s + 16 (l / 32).
  const unsigned lrow = lane & 31, lhalf = lane >> 5;
  uint32_t frag_voff[2][kSteps];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
      frag_voff[f][s] = (32 * (2 * wave + f) + lrow) * kbytes + 32 * s + 16 * lhalf;

  // Scale words: the 4 consecutive block scales (one stage) of this lane's rows.
  uint32_t sc_voff_a[kTM], sc_voff_b[kTN];
#pragma unroll
  for (int i = 0; i < kTM; ++i) sc_voff_a[i] = (kBM / kWavesM * wm + 32 * i + lrow) * kblocks;
#pragma unroll
  for (int j = 0; j < kTN; ++j) sc_voff_b[j] = (kBN / kWavesN * wn + 32 * j + lrow) * kblocks;

  f32x16_t acc[kTM][kTN];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  const int nstages = (p.K + kBK - 1) / kBK;

  auto issue_stage = [&](int st, uint8_t* buf) {
    const uint32_t kb = (uint32_t)st * (kBK / 2);        // byte offset of the stage in a row
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        uint32_t vo = frag_voff[f][s] + kb;
        if (!kKAligned) {
          const uint32_t blk = (uint32_t)st * (kBK / 32) + 2 * s + lhalf;
          if (blk >= kblocks) vo = kOOB;
        }
        const int frag = (2 * wave + f) * kSteps + s;
        load_frag_to_lds(rx, buf + frag * kFrag, vo);
        if (kResid) load_frag_to_lds(rr, buf + kTileBytesA + frag * kFrag, vo);
        load_frag_to_lds(rw, buf + 2 * kTileBytesA + frag * kFrag, vo);
      }
  };

  auto load_scales = [&](int st, uint32_t (&scx)[kTM], uint32_t (&scr)[kTM], uint32_t (&scw)[kTN]) {
    const uint32_t kb = (uint32_t)st * (kBK / 32);
    if (kKAligned) {
#pragma unroll
      for (int i = 0; i < kTM; ++i) {
        scx[i] = load_scale_word(rsx, sc_voff_a[i] + kb);
        if (kResid) scr[i] = load_scale_word(rsr, sc_voff_a[i] + kb);
      }
#pragma unroll
      for (int j = 0; j < kTN; ++j) scw[j] = load_scale_word(rsw, sc_voff_b[j] + kb);
    } else {
      // K not a multiple of 128: gather the bytes one by one into the same
      // word layout; blocks past K read as zero codes with a finite scale.
      auto byte_at = [&](__amdgpu_buffer_rsrc_t r, uint32_t row_off, uint32_t blk) -> uint32_t {
        if (blk >= kblocks) return 127u;
        return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, row_off + blk, 0, 0);
      };
      auto word_at = [&](__amdgpu_buffer_rsrc_t r, uint32_t row_off) -> uint32_t {
        return byte_at(r, row_off, kb) | (byte_at(r, row_off, kb + 1) << 8) |
               (byte_at(r, row_off, kb + 2) << 16) | (byte_at(r, row_off, kb + 3) << 24);
      };
#pragma unroll
      for (int i = 0; i < kTM; ++i) {
        scx[i] = word_at(rsx, sc_voff_a[i]);
        if (kResid) scr[i] = word_at(rsr, sc_voff_a[i]);
      }
#pragma unroll
      for (int j = 0; j < kTN; ++j) scw[j] = word_at(rsw, sc_voff_b[j]);
    }
  };

  uint32_t scx[kTM], scr[kTM], scw[kTN];
  issue_stage(0, lds[0]);
  load_scales(0, scx, scr, scw);

  for (int st = 0; st < nstages; ++st) {
    uint8_t* buf = lds[st & 1];
    __builtin_amdgcn_s_waitcnt(0);      // this stage's LDS writes and scale words have landed
    __syncthreads();

    i32x8_t ax[kSteps][kTM], ar[kSteps][kTM], bw[kSteps][kTN];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
#pragma unroll
      for (int i = 0; i < kTM; ++i) {
        const int frag = (kTM * wm + i) * kSteps + s;
        ax[s][i] = read_frag(buf + frag * kFrag, lane);
        if (kResid) ar[s][i] = read_frag(buf + kTileBytesA + frag * kFrag, lane);
      }
#pragma unroll
      for (int j = 0; j < kTN; ++j)
        bw[s][j] = read_frag(buf + 2 * kTileBytesA + ((kTN * wn + j) * kSteps + s) * kFrag, lane);
    }
    // Byte 2s of each shifted word is the scale of block (4 st + 2 s + lhalf).
    uint32_t cx[kTM], cr[kTM], cw[kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i) { cx[i] = scx[i] >> (8 * lhalf); cr[i] = scr[i] >> (8 * lhalf); }
#pragma unroll
    for (int j = 0; j < kTN; ++j) cw[j] = scw[j] >> (8 * lhalf);

    if (st + 1 < nstages) {
      issue_stage(st + 1, lds[(st + 1) & 1]);
      load_scales(st + 1, scx, scr, scw);
    }
    mfma_step<0, kResid>(acc, ax[0], ar[0], bw[0], cx, cr, cw);
    mfma_step<1, kResid>(acc, ax[1], ar[1], bw[1], cx, cr, cw);
  }

  // Epilogue: fp32 accumulators to Y.
  const int row_base = m0 + kBM / kWavesM * wm + 4 * lhalf;
  const int col_base = n0 + kBN / kWavesN * wn + lrow;
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

template <bool kResid, bool kOutBf16>
hipError_t launch_variant(const GemmParams& p, bool kaligned, int grid, hipStream_t stream) {
  if (kaligned)
    hipLaunchKernelGGL((gemm_kernel<kResid, kOutBf16, true>), dim3(grid), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm_kernel<kResid, kOutBf16, false>), dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const uint8_t* qx, const uint8_t* sx, const uint8_t* qr, const uint8_t* sr,
                       const uint8_t* w, const uint8_t* sw, int64_t M, int64_t N, int64_t K,
                       void* y, bool y_bf16, int64_t ldy, hipStream_t stream) {
  GemmParams p;
  p.qx = qx; p.sx = sx; p.qr = qr; p.sr = sr; p.w = w; p.sw = sw;
  p.y = y; p.ldy = ldy;
  p.M = (int32_t)M; p.N = (int32_t)N; p.K = (int32_t)K;
  p.tiles_m = (int32_t)((M + kBM - 1) / kBM);
  p.tiles_n = (int32_t)((N + kBN - 1) / kBN);
  const int grid = p.tiles_m * p.tiles_n;
  const bool kaligned = (K % kBK) == 0;
  const bool resid = qr != nullptr;
  if (resid)
    return y_bf16 ? launch_variant<true, true>(p, kaligned, grid, stream)
                  : launch_variant<true, false>(p, kaligned, grid, stream);
  return y_bf16 ? launch_variant<false, true>(p, kaligned, grid, stream)
                : launch_variant<false, false>(p, kaligned, grid, stream);
}

}  // namespace rfq
