// RFQ W4A4 GEMM on gfx950 block-scaled FP4 MFMA.
//
// What is computed ("Activation Outliers Matter: Robust Recovery for
// Quantized Multimodal LLMs", §1 contributions: the quantized residual is
// multiplied during the GEMM and its contribution accumulated):
//   Y[m, n] = sum_k deq(QX)[m,k] deq(W)[n,k] + deq(QR)[m,k] deq(W)[n,k]
// i.e. one contraction of [QX | QR] (M x 2K) against [W ; W] over a doubled
// K, every term landing in the same fp32 accumulator.
//
// Instruction: the scaled MFMA v_mfma_scale_f32_*_f8f6f4. E2M1 x E2M1
// products (RFQ, plain W4A4) use its 16 x 16 x 128 form (lane layout and the
// reason at mfma16_group below); E4M3 activations use the 32 x 32 x 64 form:
// lane l holds row l % 32 and K-block l / 32 of the 64-wide K step (E2M1: 16
// bytes, element 2j in the low nibble of byte j; E4M3: see Fmts), its 32-bit
// scale operand supplies the E8M0 code of that (row, block) in the byte
// chosen by op_sel, and output lane l holds column l % 32, rows
// 8 (i / 4) + 4 (l / 32) + i % 4 (checked on hardware). W is the first
// operand and X (or R) the second, so an output tile is a tile of Y^T: each
// lane holds one row of Y and, per group of four accumulators, four
// consecutive columns, which leave as one vector store.
//
// Tiling: a 256 x 256 output tile per workgroup of 8 waves on a 4 x 2 grid
// (two waves per SIMD, one workgroup per CU); each wave owns 64 x 128
// outputs = 4 x 8 tiles of 16 x 16, or 2 x 4 of 32 x 32 (128 fp32
// accumulators per lane either way). K advances
// 128 elements (64 bytes of codes per row) per stage, as two MFMA steps of
// 64. When the tile count leaves a last partial round on the CUs, that
// round's tiles are split into upper and lower halves (128 x 256 on 8 waves
// of 32 x 128, one workgroup per CU), or, when they form a rectangle that
// such pieces cover in one round, into 128 x 192 pieces (8 waves of
// 32 x 96); when the whole rounds stream, either goes in the same launch
// (see gemm_pair_kernel). Formats whose main tile is already 128 rows split
// it into quadrants (4 waves, two workgroups per CU, in a second launch). The bf16 product of the backward pass's dX also
// has 256 x 320 tiles (8 waves of 64 x 160), used alone when they cover Y
// in whole rounds and 256 x 256 tiles would not.
//
// Data movement:
//  * Code tiles (QX, QR, W; 256 rows x 64 B each per stage) go global ->
//    LDS with buffer loads that write LDS directly. Four consecutive lanes
//    fetch one row's 64 contiguous bytes, so each quad touches one cache
//    line. In LDS a row is 4 chunks of 16 B (one K-block each); chunk c of
//    row r sits at position c ^ f(r), f(r) = (r >> 1) & 3. Any 8 lanes that
//    read one chunk of 8 consecutive rows (the 32 x 32 operand reads) or
//    one chunk of 8 of 16 consecutive rows (the 16 x 16 ones) then hit
//    distinct banks of gfx950's 256-byte-wide LDS. (Measured: a loop of the
//    16 x 16 reads runs at the linear-read rate with this f and 8% below it
//    with f(r) = (r >> 2) & 3; the whole RFQ GEMM is 2.6% faster.) The
//    swizzle is applied by choosing which chunk each lane fetches.
//  * Stages live in a ring of three LDS buffers and are fetched two stages
//    ahead, so a fetch that misses L2 has two stages of MFMA work to land.
//    A stage's loads go out in two halves, one behind each MFMA step, so the
//    memory pipeline gets an even stream rather than one burst per stage.
//    Each wait names exactly the loads it needs (s_waitcnt vmcnt(N) with N =
//    the loads issued after them), never "everything outstanding".
//  * Scales: 16 bytes per row (16 blocks = 4 stages) per scale group, in one
//    LDS buffer; each lane copies its rows into registers once per group, and
//    the next group is fetched as soon as every wave has done so.
//  * Within a stage, the second MFMA step's fragments are read while the
//    first step's MFMAs run, and the next stage's first-step fragments while
//    the second step's run; one barrier per stage sits between the two.
//  * Buffer loads return zero outside the tensor, which covers partial M
//    and N tiles; partial K is masked per 16-byte chunk.

#include "kernels.h"
#include "mx_encode.h"

#include <algorithm>
#include <type_traits>

namespace rfq {
namespace {

typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kBK = 128;                            // K elements per stage
constexpr int kWavesN = 2;                          // wave grid (waves / 2) x 2
constexpr int kRowBytes = kBK / 2;                  // 64 bytes of codes per row per stage
constexpr int kRing = 3;                            // LDS stages in flight
constexpr int kScaleGroup = 4;                      // stages per scale fetch (16 blocks)
constexpr int kScaleRowBytes = 16;
constexpr uint32_t kOOB = 0x80000000u;              // voffset that is always out of range
constexpr int kGroupM = 4;                          // tile rows swept together (L2 reuse)

// Operand formats of one GEMM variant. The activation side has one or two
// terms, X and (for RFQ) the residual R, each E2M1 (4) or E4M3 (8); the
// weight is E2M1. In LDS a stage row of an E2M1 term is one 64-byte sub-tile
// (128 elements); an E4M3 term's 128 bytes are two sub-tiles.
//
// E4M3 operand layouts of the instruction (checked on hardware with one-hot
// operands and distinct per-lane scales):
//  * 16 x 16 x 128 form: lane group g (lanes 16 g .. 16 g + 15, row l % 16)
//    holds elements 16 g .. 16 g + 15 of each 64-wide half of the step, the
//    first half's in bytes 0..15 and the second's in bytes 16..31, and the
//    scale of K-block g is the one that lane group supplies (as for E2M1,
//    whose lane group g holds K-block g whole). So the two sub-tiles of an
//    E4M3 term are the two 64-byte halves of the stage row, each read like
//    an E2M1 sub-tile, and the operand is the two fragments side by side.
//  * 32 x 32 x 64 form: per row and 64-wide K step, lane half h holds
//    elements 16 h .. 16 h + 15 of K-block 0 in its bytes 0..15 and the same
//    elements of K-block 1 in bytes 16..31; the scale of K-block b is the
//    one supplied by lane half b. So the two sub-tiles hold, at LDS chunk
//    c = 2 s + lhalf (the chunk an MFMA lane reads in step s), the 16-byte
//    row chunks 4 s + lhalf (first sub-tile) and 4 s + 2 + lhalf (second):
//    row chunk 4 (c / 2) + (c % 2), plus 2 for the second sub-tile.
//
// Format 16 is bfloat16 for every operand (the weight operand too), with no
// scales: the straight-through backward's products of decoded values. A
// stage row is then 64 bytes = 32 elements, two K-steps of the bf16
// 32x32x16 MFMA, whose 16-byte fragments are read exactly like the E2M1
// ones. kT: the result is stored transposed (element (r, c) of the tile to
// y[c * ldy + r]).
//
// kQ: the activation arrives as bf16 X and the GEMM quantizes it itself (X
// and its residual R to MXFP4, the RFQ encoding), stage by stage, into the
// LDS ring; the weight side is unchanged. Each stage slot then also holds
// the activation's scale bytes of that stage ([rows, 4] per term).
template <int kX, int kR, bool kT = false, bool kQ = false>
struct Fmts {
  static constexpr int kXFmt = kX, kRFmt = kR;
  static constexpr bool kResid = kR != 0;
  static constexpr bool kBf16 = kX == 16;
  static constexpr bool kOutT = kT;
  static constexpr bool kFusedQ = kQ;
  static constexpr int kXSub = kX == 8 ? 2 : 1;
  static constexpr int kRSub = kR == 8 ? 2 : (kR != 0 ? 1 : 0);
  static constexpr int kSubA = kXSub + kRSub;          // activation sub-tiles per stage
  static constexpr int kScalesA = (kBf16 || kQ) ? 0 : (kResid ? 2 : 1);   // activation scale streams (group-wise)
  static constexpr int kScalesB = kBf16 ? 0 : 1;       // weight scale stream
  static constexpr int kTerms = kResid ? 2 : 1;        // MFMAs per output tile per step
  // E2M1 weights against E2M1 or E4M3 activations (one term) run on the
  // 16 x 16 x 128 form of the scaled MFMA (see the kernel); an E4M3 residual
  // term and bf16 operands on the 32 x 32 forms.
  static constexpr bool kM16 = (kX == 4 && (kR == 0 || kR == 4)) || (kX == 8 && kR == 0);
  static_assert((kX == 4 && (kR == 0 || kR == 4 || kR == 8)) || (kX == 8 && kR == 0) ||
                    (kX == 16 && (kR == 0 || kR == 16)),
                "formats");
  static_assert(!kT || kBf16, "transposed stores are for the bf16 products");
  static_assert(!kQ || (kX == 4 && kR == 4 && !kT), "in-GEMM quantization is of the RFQ operands");
};
using FmtW4A4 = Fmts<4, 0>;
using FmtRfq = Fmts<4, 4>;
using FmtW4A8 = Fmts<8, 0>;
using FmtRfq8 = Fmts<4, 8>;
using FmtBf16 = Fmts<16, 0>;                // dX = dY Wd: bf16 x bf16
using FmtBf16PairT = Fmts<16, 16, true>;    // dW^T = Xq dY^T + Xr dY^T, stored as dW
using FmtRfqFused = Fmts<4, 4, false, true>;  // RFQ from bf16 X, quantized inside the GEMM

// MFMA format code of an element format: E4M3 is 0, E2M1 is 4.
template <int kFmt>
constexpr int kMfmaFmt = kFmt == 8 ? 0 : 4;

// An output tile of BM x BN on `Waves` waves (grid Waves/2 x 2) for the
// operand formats F; Occ workgroups are meant to share a CU, and LDS and
// registers are sized so.
template <int BM_, int BN_, int Waves_, int Occ_, class F>
struct TileCfg {
  static constexpr int kBM = BM_, kBN = BN_, kWaves = Waves_, kOcc = Occ_;
  static constexpr int kWavesM = kWaves / kWavesN;
  static constexpr int kWaveM = kBM / kWavesM, kWaveN = kBN / kWavesN;
  static constexpr int kTM = kWaveM / 32, kTN = kWaveN / 32;           // MFMA tiles per wave
  static constexpr int kT16M = kWaveM / 16, kT16N = kWaveN / 16;       // the same in 16 x 16 tiles
  static constexpr int kTileBytesA = kBM * kRowBytes, kTileBytesB = kBN * kRowBytes;   // one sub-tile
  // in-GEMM quantization: the stage's activation scale bytes, [kBM, 4] for
  // X then for R, after the code sub-tiles
  static constexpr int kStageScaleOff = F::kSubA * kTileBytesA + kTileBytesB;
  static constexpr int kStageScaleBytes = F::kFusedQ ? 2 * kBM * 4 : 0;
  static constexpr int kStageBytes = kStageScaleOff + kStageScaleBytes;
  // in-GEMM quantization: 16-byte loads of bf16 X per lane per stage (4
  // lanes per 32-block, 4 blocks per stage row), 4 rows per wave per load
  static constexpr int kLoadsX = F::kFusedQ ? kBM * 16 / (64 * kWaves) : 0;
  static constexpr int kScaleBytesA = kBM * kScaleRowBytes;
  static constexpr int kScaleBytes = F::kScalesA * kScaleBytesA + F::kScalesB * kBN * kScaleRowBytes;
  static constexpr int kLdsBytes = kRing * kStageBytes + kScaleBytes;
  static constexpr int kLoadsA = kBM / 16 / kWaves;    // 16-row DMA instructions per wave per sub-tile of X / R
  // for W; when the 16-row groups do not divide evenly among the waves,
  // load n of wave w takes group (w + kWaves n) mod (kBN / 16), so a few
  // groups are fetched twice (identical bytes to the same place)
  static constexpr int kGroupsB = kBN / 16;
  static constexpr bool kWrapB = kGroupsB % kWaves != 0;
  static constexpr int kLoadsB = (kGroupsB + kWaves - 1) / kWaves;
  static_assert(kTM >= 1 && kTN >= 1 && kLoadsA >= 1 && kLoadsB >= 1, "tile shape");
  static_assert(!F::kM16 || (kT16M % 2 == 0 && kT16N % 2 == 0), "16 x 16 tiles come in halves");
  static_assert(kLdsBytes * kOcc <= 160 * 1024, "LDS budget per CU");
  static_assert(kStageBytes % 16 == 0, "stage slots 16-byte aligned");
  static_assert(!F::kFusedQ || (kLoadsX * 4 * kWaves == kBM && kBM % (4 * kWaves) == 0), "X load mapping");
};
// Main tiles: 256 x 256 outputs, 8 waves of 64 x 128 (128 accumulators
// each), one workgroup per CU (up to 156 KB of LDS); for the last partial
// round of a launch, halves of 128 x 256 on 8 waves of 32 x 128, one per
// CU, pieces of 128 x 192 on 8 waves of 32 x 96 over the round's
// rectangle, or quadrants of 128 x 128 on 4 waves, two per CU. With an E4M3
// residual (three activation sub-tiles) the stage would not fit three deep,
// so that variant uses 128 x 256 tiles (8 waves of 32 x 128) and 64 x 128
// quadrants.
template <class F, bool kNarrow = (F::kSubA > 2 || F::kFusedQ)>
struct Tiles {
  using Big = TileCfg<256, 256, 8, 1, F>;
  using Quad = TileCfg<128, 128, 4, 2, F>;
  using Half = TileCfg<128, 256, 8, 1, F>;   // upper or lower half of a big tile
  using Piece = TileCfg<128, 192, 8, 1, F>;  // tiles the last round's rectangle (8 waves of 32 x 96)
  static constexpr bool kHasHalf = true;
};
template <class F>
struct Tiles<F, true> {
  // (in-GEMM quantization needs registers for the bf16 X tiles in flight, so
  // it also runs 128-row tiles)
  using Big = TileCfg<128, 256, 8, 1, F>;
  using Quad = TileCfg<64, 128, 4, 2, F>;
  using Half = Big;                          // (not used)
  using Piece = Big;                         // (not used)
  static constexpr bool kHasHalf = false;
};

struct GemmParams {
  const uint8_t* qx;      // X codes: K/2 bytes per row (E2M1) or K (E4M3)
  const uint8_t* sx;
  const uint8_t* qr;      // R codes, likewise by format (RFQ variants)
  const uint8_t* sr;
  const uint8_t* w;
  const uint8_t* sw;
  void* y;
  int64_t ldy;
  int64_t ldx;            // in-GEMM quantization: row stride of bf16 X (at qx), elements
  int32_t M, N, K;
  // Tile map: `grid` work items; tiles of gm x gn form a tiles_m x tiles_n
  // grid walked in a fixed logical order; item ids map to logical tile
  // first + (0 .. grid - 1), or, split into `pieces` (4: quadrants, 2: upper
  // and lower halves), to piece id % pieces of logical tile first + id /
  // pieces. With pieces == 3 the items are instead the tiles_m x tiles_n
  // blocks of gm x gn of the rectangle at (rm0, rn0), item i at block row
  // i % tiles_m, column i / tiles_m. The launch has `wg` workgroups;
  // workgroup b runs items b, b + wg, b + 2 wg, ... back to back.
  int32_t tiles_m, tiles_n, gm, gn;
  int32_t first, grid, pieces, wg;
  int32_t vec_out;   // Y base and row stride allow 4-element vector stores
  int32_t rm0, rn0;
};

__device__ __forceinline__ uint32_t swz(uint32_t r) { return (r >> 1) & 3u; }

// The kernel's parameter block, read again from the kernel-argument segment.
// Code that runs once per tile uses it instead of values held since the
// kernel started, so those do not occupy scalar registers through the loop.
// It must be inlined into the kernel itself: in a called function the
// segment pointer is not passed along (the compiler substitutes 0), which is
// why every lambda of the kernel body is marked always_inline.
// kSlot picks the block: 0 for a one-tile-shape launch, 0 or 1 for the two
// blocks of a launch that runs two tile shapes (GemmPairParams).
typedef __attribute__((address_space(4))) const GemmParams* const_params_ptr;
template <int kSlot>
__device__ __forceinline__ GemmParams fresh_params() {
  const_params_ptr q = (const_params_ptr)__builtin_amdgcn_kernarg_segment_ptr() + kSlot;
  asm volatile("" : "+s"(q));
  GemmParams r;
  __builtin_memcpy(&r, (const GemmParams*)q, sizeof(r));
  return r;
}

// Two parameter blocks back to back: a launch whose first `a.wg` workgroups
// run one tile shape and the rest another.
struct GemmPairParams {
  GemmParams a, b;
};
static_assert(offsetof(GemmPairParams, b) == sizeof(GemmParams), "parameter blocks back to back");

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // gfx9 raw buffer: stride 0, num_records in bytes, dword3 = 32-bit data format
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// soff: a wave-uniform byte offset added to every lane's (it goes in the
// instruction's scalar offset, not in the lanes' offset registers)
__device__ __forceinline__ void load16_to_lds(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voff, uint32_t soff = 0) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, voff, (int)soff, 0, 0);
}

__device__ __forceinline__ i32x4_t read_frag(const uint8_t* p) { return *reinterpret_cast<const i32x4_t*>(p); }

// Two fp32 values to bfloat16, packed (a in the low half): gfx950's
// v_cvt_pk_bf16_f32, which rounds to nearest even under the kernel's default
// round mode and keeps fp32 denormals (the kernels run with denormals
// preserved); a NaN stays a NaN.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// FP4 operands use the low 4 of the instruction's 8 operand registers.
__device__ __forceinline__ i32x8_t widen(i32x4_t v) { return i32x8_t{v.x, v.y, v.z, v.w, 0, 0, 0, 0}; }

// s_waitcnt vmcnt(n) only (expcnt and lgkmcnt left at their maxima); gfx9
// encoding: vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }   // lgkmcnt(0)

// Barrier without the workgroup memory fence that __syncthreads implies (that
// fence would also wait for the loads of later stages still in flight). LDS
// reads and writes of this wave are complete before it (lgkmcnt(0) above the
// call sites); the compiler barriers keep memory accesses from moving across.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Maps a workgroup id to the origin of its output tile. Ids are dealt
// round-robin to the 8 XCDs, so consecutive logical tiles are first spread
// over one XCD's share of ids; logical tiles are then walked in groups of
// kGroupM tile rows, so that concurrently running workgroups share
// activation rows and weight columns in that XCD's L2.
__device__ __forceinline__ void tile_origin(const GemmParams& p, int bid, int& m0, int& n0) {
  const int total = p.grid;
  const int xcd = bid % 8, idx = bid / 8;
  const int base = total / 8, rem = total % 8;
  const int local = xcd < rem ? xcd * (base + 1) + idx : rem * (base + 1) + (xcd - rem) * base + idx;
  if (p.pieces == 3) {
    m0 = p.rm0 + (local % p.tiles_m) * p.gm;
    n0 = p.rn0 + (local / p.tiles_m) * p.gn;
    return;
  }
  const int logical = p.first + local / p.pieces;
  const int q = local % p.pieces;
  const int per_group = kGroupM * p.tiles_n;
  const int group = logical / per_group;
  const int first_m = group * kGroupM;
  const int gsize = min(p.tiles_m - first_m, kGroupM);
  const int in_group = logical - group * per_group;
  const int tm = first_m + in_group % gsize, tn = in_group / gsize;
  if (p.pieces == 4) {
    m0 = tm * p.gm + (q / 2) * (p.gm / 2);
    n0 = tn * p.gn + (q % 2) * (p.gn / 2);
  } else {
    m0 = tm * p.gm + q * (p.gm / 2);
    n0 = tn * p.gn;
  }
}

// The MFMA operand of one activation term for fragment row group i: an E2M1
// term is one 16-byte fragment (the low half of the operand registers), an
// E4M3 term the fragments of its first and second sub-tiles, in that order.
template <int kFmt, int kSub, int kSubA, int kTM>
__device__ __forceinline__ i32x8_t term_operand(const i32x4_t (&a)[kSubA][kTM], int i) {
  if constexpr (kFmt == 8)
    return i32x8_t{a[kSub][i].x, a[kSub][i].y, a[kSub][i].z, a[kSub][i].w,
                   a[kSub + 1][i].x, a[kSub + 1][i].y, a[kSub + 1][i].z, a[kSub + 1][i].w};
  else
    return widen(a[kSub][i]);
}

template <int S, class F, int kTM, int kTN>
__device__ __forceinline__ void mfma_step(f32x16_t (&acc)[kTM][kTN], const i32x4_t (&a)[F::kSubA][kTM],
                                          const i32x4_t (&b)[kTN], const uint32_t (&scx)[kTM],
                                          const uint32_t (&scr)[kTM], const uint32_t (&scw)[kTN]) {
  if constexpr (F::kBf16) {
#pragma unroll
    for (int t = 0; t < F::kSubA; ++t)
#pragma unroll
      for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, b[j]),
                                                              __builtin_bit_cast(bf16x8_t, a[t][i]), acc[i][j], 0, 0, 0);
    return;
  }
#pragma unroll
  for (int i = 0; i < kTM; ++i) {
    const i32x8_t ax = term_operand<F::kXFmt, 0, F::kSubA, kTM>(a, i);
#pragma unroll
    for (int j = 0; j < kTN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(b[j]), ax, acc[i][j], 4, kMfmaFmt<F::kXFmt>,
                                                                  2 * S, (int)scw[j], 2 * S, (int)scx[i]);
  }
  if constexpr (F::kResid) {
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      const i32x8_t ar = term_operand<F::kRFmt, F::kXSub, F::kSubA, kTM>(a, i);
#pragma unroll
      for (int j = 0; j < kTN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(b[j]), ar, acc[i][j], 4, kMfmaFmt<F::kRFmt>,
                                                                    2 * S, (int)scw[j], 2 * S, (int)scr[i]);
    }
  }
}

// Scheduling hint for one MFMA step (group) of kMfma MFMAs: its LDS reads
// (kReads) go two behind each MFMA from the first one on, so that they have
// the rest of the group to land, and its LDS-DMA loads (kVmem) one behind
// each of the last kVmem MFMAs; both issue while the MFMA pipe is busy.
// Fragments read in one group feed the next group's MFMAs in two of a
// stage's four groups. Same-box A/B against spreading both evenly over the
// group: 261.6 against 265.1 us on 4096 x 5120 x 13824, 181.9 against
// 184.3 us on 4096 x 4096 x 12288, 36.4 against 36.6 us on 2048 x 4096 x
// 4096; Y bit-identical.
template <int kSlot, int kMfma, int kVmem, int kReads>
__device__ __forceinline__ void interleave_slots() {
  if constexpr (kSlot < kMfma) {
    constexpr int vm = kSlot >= kMfma - kVmem ? 1 : 0;
    constexpr int done = 2 * kSlot < kReads ? 2 * kSlot : kReads;
    constexpr int ds = (kReads - done) < 2 ? (kReads - done) : 2;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);               // MFMA
    if constexpr (ds > 0) __builtin_amdgcn_sched_group_barrier(0x100, ds, 0);   // DS read
    if constexpr (vm > 0) __builtin_amdgcn_sched_group_barrier(0x010, vm, 0);   // any VMEM (the LDS-DMA loads)
    interleave_slots<kSlot + 1, kMfma, kVmem, kReads>();
  }
}
template <int kReads, int kVmem, int kMfma>
__device__ __forceinline__ void interleave_hint() {
  static_assert(kVmem <= kMfma, "one load behind each of the last kVmem MFMAs");
  interleave_slots<0, kMfma, kVmem, kReads>();
}

// The 16 x 16 x 128 form of the instruction, for E2M1 x E2M1 (lane layout
// checked on hardware with random operands and per-lane scales): lane l
// holds row l % 16 and the 32 elements of K-block l / 16 of the 128-wide
// step (16 bytes, element 2j in the low nibble of byte j), and its scale
// operand supplies that (row, block)'s E8M0 code in the byte op_sel picks;
// output lane l holds column l % 16, rows 4 (l / 16) + 0..3. A stage (128 K
// elements) is one step. On this workload's codes its power-limited rate
// measured 13% above the 32 x 32 x 64 form's (7.45 against 6.6 PFLOP/s in
// an MFMA-only loop): a quarter of the accumulator reads and writes per
// instruction for half the products.
//
// A lane's scale bytes for the four stages of a scale group, gathered from
// its row's 16 group bytes (stage s's four blocks at bytes 4 s .. 4 s + 3)
// into one word whose byte s is the lane's block (lane / 16) of stage s;
// sel01 = b | (4 + b) << 8 for that block b. (Elements are copied to
// scalars first: a bit cast of an ext-vector element has been seen to read
// element 0.)
__device__ __forceinline__ uint32_t gather_stage_bytes(i32x4_t w, uint32_t sel01) {
  const int e0 = w.x, e1 = w.y, e2 = w.z, e3 = w.w;
  const uint32_t t01 = __builtin_amdgcn_perm((uint32_t)e1, (uint32_t)e0, sel01);
  const uint32_t t23 = __builtin_amdgcn_perm((uint32_t)e3, (uint32_t)e2, sel01);
  return __builtin_amdgcn_perm(t23, t01, 0x05040100u);
}

// One group of 16 x 16 x 128 MFMAs: weight half HW (kHN fragments of 16
// rows) against activation half HX (kHM row tiles, kTerms terms each), at
// stage P of the scale group (the weight scale byte op_sel picks; PX for the
// activation's, which is byte 0 when the GEMM quantizes the activation
// itself and holds per-stage scale bytes). Terms outermost, so MFMAs into
// one accumulator are kHM x kHN instructions apart.
template <int P, int PX, int HW, int HX, int kTerms, int kSubA, int kXFmt, int kHM, int kHN, int kT16M, int kT16N>
__device__ __forceinline__ void mfma16_group(f32x4_t (&acc)[kT16M][kT16N], const i32x4_t (&wf)[2][kHN],
                                             const i32x4_t (&xf)[2][kHM * kSubA], const uint32_t (&ws)[2][kHN],
                                             const uint32_t (&xs)[2][kHM * kTerms]) {
#pragma unroll
  for (int t = 0; t < kTerms; ++t)
#pragma unroll
    for (int m = 0; m < kHM; ++m)
#pragma unroll
      for (int n = 0; n < kHN; ++n) {
        // an E4M3 activation (one term, two sub-tiles) is its two fragments
        // side by side; an E2M1 term is one fragment
        const i32x4_t& f0 = xf[HX][m * kSubA + (kXFmt == 8 ? 0 : t)];
        const i32x4_t& f1 = xf[HX][m * kSubA + (kXFmt == 8 ? 1 : t)];
        const i32x8_t xop = kXFmt == 8 ? i32x8_t{f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w} : widen(f0);
        acc[HX * kHM + m][HW * kHN + n] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            widen(wf[HW][n]), xop, acc[HX * kHM + m][HW * kHN + n], 4, kMfmaFmt<kXFmt>, P, (int)ws[HW][n], PX,
            (int)xs[HX][m * kTerms + t]);
      }
}

// kFast: K % 512 == 0 (whole stages and whole 16-block scale groups); the
// other instantiation masks partial K and waits for all loads at each stage.
// kStream (needs kFast): every tile of the launch lies inside Y and Y takes
// vector stores, and each workgroup streams several tiles; otherwise each
// workgroup computes one tile and stores it with per-element bounds checks.
template <class C, class F, bool kOutBf16, bool kFast, bool kStream, int kSlot>
__device__ __forceinline__ void gemm_body(const GemmParams& p, const int bid, uint8_t* const lds) {
  static_assert(kFast || !kStream, "streaming needs whole scale groups");
  constexpr bool kResid = F::kResid;
  constexpr bool kM16 = F::kM16;
  constexpr int kSubA = F::kSubA;
  constexpr int kBM = C::kBM, kBN = C::kBN, kWaves = C::kWaves;
  constexpr int kWaveM = C::kWaveM, kWaveN = C::kWaveN, kTM = C::kTM, kTN = C::kTN;
  constexpr int kTileBytesA = C::kTileBytesA, kStageBytes = C::kStageBytes;
  constexpr int kScaleBytesA = C::kScaleBytesA;
  uint8_t* const ring = lds;
  uint8_t* const sbuf = lds + kRing * kStageBytes;

  // (the lane from mbcnt, not from the thread index: the thread index then
  // dies once the wave index is in a scalar register, instead of holding a
  // VGPR through the loop for the epilogue)
  const unsigned lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  // wave index as a scalar: everything derived from it (row ranges, which
  // operand a scale piece belongs to) stays in SGPRs and scalar branches
  const unsigned wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const unsigned wm = wave / kWavesN, wn = wave % kWavesN;
  const unsigned lrow = lane & 31, lhalf = lane >> 5;
  // This workgroup's items (tiles) run as one stream of K stages: while the
  // last stages of one tile are computed, the first stages of the next are
  // already being fetched, and the finished tile's stores drain behind the
  // next tile's MFMAs. (Streaming needs whole scale groups per tile, kFast;
  // otherwise the launch gives each workgroup one item.)
  const int ntiles = (p.grid - bid + p.wg - 1) / p.wg;
  int cm0, cn0;                                  // origin of the tile being computed
  tile_origin(p, bid, cm0, cn0);
  if (cm0 >= p.M || cn0 >= p.N) return;          // a quadrant past the edge (whole workgroup)
  const int nstages = (p.K + kBK - 1) / kBK;
  const int ngroups = (nstages + kScaleGroup - 1) / kScaleGroup;
  const int total_stages = ntiles * nstages;

  // Byte offset of stage st's ring slot (slot st mod 3). The K loop advances
  // by a scale group (4 stages, 1 mod 3) per iteration, so instead of
  // reducing st mod 3 at every use it keeps the offsets of the slots of
  // stages st0, st0 + 1 and st0 + 2 (st0 the iteration's first stage) and
  // rotates them once per iteration; every use names its stage as st0 plus a
  // distance known at compile time. (Same-box A/B against st mod 3 at every
  // use: 283.7 against 284.8 us on the 4096 x 5120 x 13824 layer, 39.8
  // against 40.7 us on 2048 x 4096 x 4096; Y bit-identical.)
  int loop_st0 = 0;
  uint32_t rot[3] = {0u, (uint32_t)kStageBytes, 2u * kStageBytes};
  auto slot_off = [&](int st) __attribute__((always_inline)) -> uint32_t {
    return rot[(st - loop_st0) % kRing];
  };

  // Buffer descriptors of the tile being fetched (rows past the tensor read
  // as zero), one per activation sub-tile: an E4M3 term's second sub-tile
  // starts 32 bytes (two chunks) into the row, so the same offsets fetch it.
  const uint32_t kbytes = (uint32_t)p.K / 2, kblocks = (uint32_t)p.K / 32;
  // where an E4M3 term's second sub-tile starts in a 128-byte stage row: the
  // second 64-byte half for the 16 x 16 x 128 form, 32 bytes in (two chunks,
  // interleaved with the first sub-tile's) for the 32 x 32 x 64 form
  constexpr uint32_t kE4Second = kM16 ? 64u : 32u;
  __amdgpu_buffer_rsrc_t ra[kSubA], rw, rsx, rsr, rsw, rx;
  auto set_load_tile = [&](const GemmParams& q, int m0, int n0) __attribute__((always_inline)) {
    const uint32_t rows_a = (uint32_t)min(kBM, q.M - m0), rows_b = (uint32_t)min(kBN, q.N - n0);
    if constexpr (F::kFusedQ) {
      // bf16 X rows [m0, m0 + rows_a): the extent ends at the last row's K-th
      // element, so a lane offset that carries a row past the tile's last
      // reads zeros
      rx = make_rsrc(q.qx + (int64_t)m0 * q.ldx * 2, (uint32_t)(((int64_t)(rows_a - 1) * q.ldx + q.K) * 2));
    } else {
      const uint32_t xrow = F::kXFmt == 8 ? 2 * kbytes : kbytes, rrow = F::kRFmt == 8 ? 2 * kbytes : kbytes;
      ra[0] = make_rsrc(q.qx + (int64_t)m0 * xrow, rows_a * xrow);
      // (an E4M3 second sub-tile's extent is the tile's bytes past its start,
      // none when the tile holds fewer: a wrapped extent would let the
      // out-of-range offset kOOB through)
      [[maybe_unused]] const uint32_t xbytes = rows_a * xrow, rbytes = rows_a * rrow;
      if constexpr (F::kXFmt == 8)
        ra[1] = make_rsrc(q.qx + (int64_t)m0 * xrow + kE4Second, xbytes > kE4Second ? xbytes - kE4Second : 0u);
      if constexpr (F::kResid) {
        ra[F::kXSub] = make_rsrc(q.qr + (int64_t)m0 * rrow, rows_a * rrow);
        if constexpr (F::kRFmt == 8)
          ra[F::kXSub + 1] = make_rsrc(q.qr + (int64_t)m0 * rrow + kE4Second, rbytes > kE4Second ? rbytes - kE4Second : 0u);
      }
    }
    rw = make_rsrc(q.w + (int64_t)n0 * kbytes, rows_b * kbytes);
    if constexpr (!F::kBf16) {
      if constexpr (!F::kFusedQ) {
        rsx = make_rsrc(q.sx + (int64_t)m0 * kblocks, rows_a * kblocks);
        rsr = make_rsrc(kResid ? q.sr + (int64_t)m0 * kblocks : q.sx, rows_a * kblocks);
      }
      rsw = make_rsrc(q.sw + (int64_t)n0 * kblocks, rows_b * kblocks);
    }
  };
  set_load_tile(p, cm0, cn0);
  int load_tile = 0, load_base = 0;              // tile being fetched and its first stream stage

  // Code-tile loads: wave w fetches rows [BM/waves w, BM/waves (w + 1)) of
  // each activation sub-tile and the matching range of W's BN rows, 16 rows
  // per instruction; lane l takes row 16 n + l / 4 of them and LDS chunk
  // c = (l % 4) ^ f(row), which is row chunk c of an E2M1 sub-tile; of an
  // E4M3 term, row chunk c (+ 4 in the second sub-tile) on the 16 x 16 x 128
  // form and row chunk 4 (c / 2) + c % 2 (+ 2 in the second) on the
  // 32 x 32 x 64 form.
  uint32_t lda_chunk[C::kLoadsA], lda_row[C::kLoadsA], ldb_voff[C::kLoadsB], ldb_chunk[C::kLoadsB];
#pragma unroll
  for (int n = 0; n < C::kLoadsA; ++n) {
    lda_row[n] = kBM / kWaves * wave + 16 * n + (lane >> 2);
    lda_chunk[n] = (lane & 3) ^ swz(lda_row[n]);
  }
  // first row of the 16-row group of W that load n of this wave fetches
  auto ldb_group_row = [&](int n) __attribute__((always_inline)) -> uint32_t {
    return C::kWrapB ? 16 * ((wave + kWaves * n) % C::kGroupsB) : kBN / kWaves * wave + 16 * n;
  };
#pragma unroll
  for (int n = 0; n < C::kLoadsB; ++n) {
    const uint32_t row = ldb_group_row(n) + (lane >> 2);
    ldb_chunk[n] = (lane & 3) ^ swz(row);
    ldb_voff[n] = row * kbytes + 16 * ldb_chunk[n];
  }
  // byte offset of a lane's chunk in stage 0 of an activation term of format kFmt
  auto lda_voff = [&](auto fmt_c, int n) __attribute__((always_inline)) -> uint32_t {
    constexpr int fmt = decltype(fmt_c)::value;
    return fmt == 8 ? lda_row[n] * (2 * kbytes) + (kM16 ? 16 * lda_chunk[n] : 64 * (lda_chunk[n] >> 1) + 16 * (lda_chunk[n] & 1))
                    : lda_row[n] * kbytes + 16 * lda_chunk[n];
  };
  constexpr int kDmaPerStage = (F::kFusedQ ? 0 : kSubA * C::kLoadsA) + C::kLoadsB;
  constexpr int kLoadsX = C::kLoadsX;
  constexpr int kMfmaPerStep = kTM * kTN * F::kTerms;
  constexpr int kReadsPerStep = kTM * kSubA + kTN;
  constexpr int kScaleRowReads = kTM * F::kScalesA + kTN;
  // scale pieces (64 rows x 16 B) per group: BM/64 for X and for R, BN/64
  // for W, dealt round the waves; when they do not divide evenly the spare
  // slots repeat pieces (identical bytes to the same place), so every wave
  // issues as many loads
  constexpr int kPiecesA = kBM / 64, kPiecesB = kBN / 64;
  constexpr int kPieces = F::kScalesA * kPiecesA + F::kScalesB * kPiecesB;
  constexpr int kScaleLoadsPerWave = (kPieces + kWaves - 1) / kWaves;   // 0 without scales

  // Stream stage st (stage st - load_base of the tile being fetched). A
  // stage past the end of the stream is still issued, so that the number of
  // loads per stage stays constant; it fills a slot nothing reads again. In
  // the kFast variant a stage's K offset is the loads' scalar offset and each
  // lane's offset is the same in every stage (no per-stage lane arithmetic),
  // and a stage past the end re-reads the tile's stage 0; otherwise the lane
  // offsets carry the stage and a chunk past K, or a stage past the end, is
  // aimed out of range (zeros). The loads go out in two parts.
  constexpr int kPart0 = (kDmaPerStage + 1) / 2;
  auto issue_stage = [&](int st, auto part_c) __attribute__((always_inline)) {
    constexpr int part = decltype(part_c)::value;   // 0: first kPart0 loads, 1: the rest, 2: all
    uint8_t* buf = ring + slot_off(st);
    const int kst = st - load_base;
    const bool past_end = st >= total_stages;
    const uint32_t kst_s = past_end ? 0u : (uint32_t)kst;   // kFast: stage in the scalar offset
#pragma unroll
    for (int n = 0; n < (F::kFusedQ ? 0 : C::kLoadsA); ++n) {
      uint8_t* dst = buf + (kBM / kWaves * wave + 16 * n) * kRowBytes;
#pragma unroll
      for (int t = 0; t < kSubA; ++t) {
        const bool is_x = t < F::kXSub;
        const bool fp8 = is_x ? F::kXFmt == 8 : F::kRFmt == 8;
        const bool second = fp8 && t == (is_x ? 1 : F::kXSub + 1);
        // K-block (within the stage) of this lane's chunk: c for E2M1; for
        // E4M3 c / 2, + 2 in the second sub-tile (16 x 16 x 128 form), or
        // 2 (c / 2), + 1 in the second sub-tile (32 x 32 x 64 form)
        const uint32_t blk = !fp8 ? lda_chunk[n]
                             : kM16 ? 2 * (second ? 1 : 0) + (lda_chunk[n] >> 1)
                                    : 2 * (lda_chunk[n] >> 1) + (second ? 1 : 0);
        const uint32_t base = fp8 ? lda_voff(std::integral_constant<int, 8>{}, n) : lda_voff(std::integral_constant<int, 4>{}, n);
        const uint32_t step = fp8 ? 2 * kRowBytes : kRowBytes;
        uint32_t vo = base, so = kst_s * step;
        if (!kFast) {
          vo = base + (uint32_t)kst * step;
          so = 0;
          if ((uint32_t)kst * (kBK / 32) + blk >= kblocks || past_end) vo = kOOB;
        }
        const int ix = kSubA * n + t;
        if (part == 2 || (ix < kPart0) == (part == 0)) load16_to_lds(ra[t], dst + t * kTileBytesA, vo, so);
      }
    }
#pragma unroll
    for (int n = 0; n < C::kLoadsB; ++n) {
      uint32_t vo = ldb_voff[n], so = kst_s * kRowBytes;
      if (!kFast) {
        vo = ldb_voff[n] + (uint32_t)kst * kRowBytes;
        so = 0;
        if ((uint32_t)kst * (kBK / 32) + ldb_chunk[n] >= kblocks || past_end) vo = kOOB;
      }
      const int ix = (F::kFusedQ ? 0 : kSubA * C::kLoadsA) + n;
      if (part == 2 || (ix < kPart0) == (part == 0))
        load16_to_lds(rw, buf + kSubA * kTileBytesA + ldb_group_row(n) * kRowBytes, vo, so);
    }
  };

  // Scale group g of the tile being fetched: 16 bytes (blocks 16 g .. 16 g +
  // 15) of every row of X, R and W, as 64-row pieces.
  auto issue_scale_piece = [&](__amdgpu_buffer_rsrc_t r, int g, int op, int q) __attribute__((always_inline)) {
    // (the lane index is re-read here so that the row offset is recomputed
    // once per group instead of occupying a register through the loop)
    uint32_t lane_now = lane;
    asm volatile("" : "+v"(lane_now));
    const uint32_t row = 64 * q + lane_now;
    uint8_t* dst = sbuf + op * kScaleBytesA + 64 * q * kScaleRowBytes;
    if (kFast) {
      load16_to_lds(r, dst, g < ngroups ? row * kblocks + 16 * g : kOOB);
    } else {
      // gather byte by byte; blocks past K get a finite scale (their codes are zero)
      uint32_t wv[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        uint32_t v = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t blk = 16 * g + 4 * d + e;
          const uint32_t b =
              blk < kblocks ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, row * kblocks + blk, 0, 0) : 127u;
          v |= b << (8 * e);
        }
        wv[d] = v;
      }
      *reinterpret_cast<i32x4_t*>(dst + lane * kScaleRowBytes) = i32x4_t{(int)wv[0], (int)wv[1], (int)wv[2], (int)wv[3]};
    }
  };
  auto issue_scales = [&](int stream_g) __attribute__((always_inline)) {
    if constexpr (kPieces == 0) return;
    const int g = stream_g - load_base / kScaleGroup;   // past the stream end: g >= ngroups
#pragma unroll
    for (int t = 0; t < kScaleLoadsPerWave; ++t) {
      const int j = (kScaleLoadsPerWave * (int)wave + t) % (kPieces > 0 ? kPieces : 1);   // wave-uniform
      // pieces 0 .. kScalesA kPiecesA - 1 are the activation's (none when the
      // GEMM quantizes the activation itself), the rest the weight's
      if (F::kScalesA >= 1 && j < kPiecesA)
        issue_scale_piece(rsx, g, 0, j);
      else if (F::kScalesA >= 2 && j < 2 * kPiecesA)
        issue_scale_piece(rsr, g, 1, j - kPiecesA);
      else
        issue_scale_piece(rsw, g, F::kScalesA, j - F::kScalesA * kPiecesA);
    }
  };

  // In-GEMM quantization of the activation (F::kFusedQ). Stage st + 2's
  // bf16 X tile (kBM rows x 128 elements) is loaded into registers at the
  // start of stage st, beside that stage's second weight part, and quantized
  // after stage st's barrier (spread over its last two MFMA groups) into its
  // ring slot, which is free since the barrier of stage st - 1: RFQ codes of
  // X and of R = X - deq(Q(X)) in the layout the DMA would have written
  // (chunk c of row r at c ^ f(r)), and the stage's scale bytes; the barrier
  // of stage st + 1 makes them visible before stage st + 2's first reads.
  // Lane (quad q = lane / 4, part p = lane % 4) of wave w takes, in load u,
  // row (kBM / kWaves) w + 4 u + q / 4 of the tile, block q % 4 of the stage
  // and its elements 8 p .. 8 p + 7, so each quad holds one 32-block (the
  // DPP block maxima need that).
  mx::u32x4_t xin[kLoadsX > 0 ? kLoadsX : 1];      // bf16 X of the stage being quantized
  uint32_t xld_off[kLoadsX > 0 ? kLoadsX : 1];
  if constexpr (F::kFusedQ) {
#pragma unroll
    for (int u = 0; u < kLoadsX; ++u) {
      const uint32_t row = kBM / kWaves * wave + 4 * u + (lane >> 4);
      xld_off[u] = (uint32_t)(row * p.ldx * 2) + (32 * ((lane >> 2) & 3) + 8 * (lane & 3)) * 2;
    }
  }
  auto issue_x = [&](int st) __attribute__((always_inline)) {
    if constexpr (F::kFusedQ) {
      // the stage's K offset in the scalar offset; past the end of the stream,
      // the tile's stage 0 again (nothing reads what it becomes)
      const uint32_t so = st >= total_stages ? 0u : (uint32_t)(st - load_base) * (kBK * 2);
#pragma unroll
      for (int u = 0; u < kLoadsX; ++u)
        xin[u] = __builtin_bit_cast(mx::u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rx, xld_off[u], so, 0));
    }
  };
  // units [u0, u1) of stage st's X (register set `set`)
  auto quantize_units = [&](int st, auto u0_c, auto u1_c) __attribute__((always_inline)) {
    if constexpr (F::kFusedQ) {
      constexpr int u0 = decltype(u0_c)::value, u1 = decltype(u1_c)::value;
      uint8_t* slot = ring + slot_off(st);
      const uint32_t blk = (lane >> 2) & 3, part = lane & 3;
#pragma unroll
      for (int u = u0; u < u1; ++u) {
        const mx::RfqLane e = mx::rfq_encode_bf16x8(xin[u]);
        const uint32_t row = kBM / kWaves * wave + 4 * u + (lane >> 4);
        const uint32_t off = row * kRowBytes + 16 * (blk ^ swz(row)) + 4 * part;
        *reinterpret_cast<uint32_t*>(slot + off) = e.cx;
        *reinterpret_cast<uint32_t*>(slot + kTileBytesA + off) = e.cr;
        if (part == 0) {
          slot[C::kStageScaleOff + row * 4 + blk] = (uint8_t)e.sx;
          slot[C::kStageScaleOff + kBM * 4 + row * 4 + blk] = (uint8_t)e.sr;
        }
      }
    }
  };
  auto quantize_x = [&](int st) __attribute__((always_inline)) {
    quantize_units(st, std::integral_constant<int, 0>{}, std::integral_constant<int, kLoadsX>{});
  };
  // half h of stage st's units (the loop spreads a stage's quantization over
  // two MFMA groups)
  auto quantize_half = [&](int st, auto h_c) __attribute__((always_inline)) {
    constexpr int h = decltype(h_c)::value;
    quantize_units(st, std::integral_constant<int, h * kLoadsX / 2>{},
                   std::integral_constant<int, (h + 1) * kLoadsX / 2>{});
  };

  // Per-lane LDS read offsets: lane (lhalf, lrow) of a 32-row fragment reads
  // chunk 2 s + lhalf of its row.
  uint32_t rd_off[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) rd_off[s] = lrow * kRowBytes + 16 * ((2 * s + lhalf) ^ swz(lrow));
  const uint32_t a_row0 = kWaveM * wm, b_row0 = kWaveN * wn;

  auto read_step = [&](int st, int s, i32x4_t (&a)[kSubA][kTM], i32x4_t (&bw)[kTN]) {
    // one lane offset per step plus a scalar slot base; every fragment then
    // sits at a constant distance from it (an instruction offset). (The lane
    // offset is re-read here so that the compiler does not keep a separate
    // precomputed address per ring slot and fragment through the loop.)
    uint32_t off = rd_off[s];
    asm volatile("" : "+v"(off));
    const uint8_t* buf = ring + slot_off(st) + off;
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      const uint8_t* src = buf + (a_row0 + 32 * i) * kRowBytes;
#pragma unroll
      for (int t = 0; t < kSubA; ++t) a[t][i] = read_frag(src + t * kTileBytesA);
    }
#pragma unroll
    for (int j = 0; j < kTN; ++j) bw[j] = read_frag(buf + kSubA * kTileBytesA + (b_row0 + 32 * j) * kRowBytes);
  };
  // this lane's scale words for two stages (a pair of the group's four)
  i32x2_t gx[kTM], gr[kTM], gw[kTN];
  auto read_scale_pair = [&](int pair) __attribute__((always_inline)) {
    if constexpr (F::kBf16) return;
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      const uint8_t* s0 = sbuf + (a_row0 + 32 * i + lrow) * kScaleRowBytes + 8 * pair;
      gx[i] = *reinterpret_cast<const i32x2_t*>(s0);
      if (kResid) gr[i] = *reinterpret_cast<const i32x2_t*>(s0 + kScaleBytesA);
    }
#pragma unroll
    for (int j = 0; j < kTN; ++j)
      gw[j] = *reinterpret_cast<const i32x2_t*>(sbuf + F::kScalesA * kScaleBytesA + (b_row0 + 32 * j + lrow) * kScaleRowBytes +
                                                8 * pair);
  };

  // 16 x 16 x 128 path: fragments and scale words in two halves each (the
  // weight's kT16N row tiles, the activation's kT16M row tiles with their
  // terms). A stage's MFMAs go in four groups, (W0, A0), (W0, A1), (W1, A0),
  // (W1, A1), and each half is re-read for the next stage right after its
  // last use in this one: W0 after the second group (past the barrier, where
  // the next stage has landed), A0 after the third, W1 and A1 after the
  // fourth (during the next stage's first group). So one set of fragment
  // registers serves, as in the 32 x 32 path. Scale words hold a whole
  // scale group (byte s = stage s) and roll over at its last stage the same
  // way.
  constexpr int kHM = C::kT16M / 2, kHN = C::kT16N / 2;
  constexpr int kXH = kHM * F::kTerms;          // activation scale words per half
  constexpr int kXF = kHM * kSubA;              // activation fragments per half (two per E4M3 term)
  i32x4_t wf[2][kHN], xf[2][kXF];
  uint32_t ws[2][kHN], xs[2][kXH];
  // lane offset of a 16-row fragment: row lane % 16, chunk lane / 16
  // (swizzled by the row; fragment bases are multiples of 16 rows)
  const uint32_t rd16 = (lane & 15) * kRowBytes + 16 * ((lane >> 4) ^ swz(lane & 15));
  const uint32_t sel01 = (lane >> 4) | ((4 + (lane >> 4)) << 8);
  auto read_w16 = [&](int st, auto h_c) __attribute__((always_inline)) {
    constexpr int h = decltype(h_c)::value;
    uint32_t off = rd16;
    asm volatile("" : "+v"(off));
    const uint8_t* buf = ring + slot_off(st) + kSubA * kTileBytesA + off;
#pragma unroll
    for (int n = 0; n < kHN; ++n) wf[h][n] = read_frag(buf + (b_row0 + 16 * (h * kHN + n)) * kRowBytes);
  };
  auto read_x16 = [&](int st, auto h_c) __attribute__((always_inline)) {
    constexpr int h = decltype(h_c)::value;
    uint32_t off = rd16;
    asm volatile("" : "+v"(off));
    const uint8_t* buf = ring + slot_off(st) + off;
#pragma unroll
    for (int m = 0; m < kHM; ++m)
#pragma unroll
      for (int t = 0; t < kSubA; ++t)
        xf[h][m * kSubA + t] = read_frag(buf + t * kTileBytesA + (a_row0 + 16 * (h * kHM + m)) * kRowBytes);
  };
  auto read_ws16 = [&](auto h_c) __attribute__((always_inline)) {
    constexpr int h = decltype(h_c)::value;
    if constexpr (!F::kBf16) {
#pragma unroll
      for (int n = 0; n < kHN; ++n) {
        const uint32_t row = b_row0 + 16 * (h * kHN + n) + (lane & 15);
        ws[h][n] = gather_stage_bytes(
            *reinterpret_cast<const i32x4_t*>(sbuf + F::kScalesA * kScaleBytesA + row * kScaleRowBytes), sel01);
      }
    }
  };
  auto read_xs16 = [&](auto h_c) __attribute__((always_inline)) {
    constexpr int h = decltype(h_c)::value;
    if constexpr (!F::kBf16 && !F::kFusedQ) {
#pragma unroll
      for (int m = 0; m < kHM; ++m) {
        const uint32_t row = a_row0 + 16 * (h * kHM + m) + (lane & 15);
#pragma unroll
        for (int t = 0; t < F::kTerms; ++t)
          xs[h][m * F::kTerms + t] = gather_stage_bytes(
              *reinterpret_cast<const i32x4_t*>(sbuf + t * kScaleBytesA + row * kScaleRowBytes), sel01);
      }
    }
  };

  // In-GEMM quantization: the activation scale bytes of stage st, one byte
  // per fragment (row lane % 16, block lane / 16 of the stage), for op_sel 0.
  auto read_xs16f = [&](int st, auto h_c) __attribute__((always_inline)) {
    constexpr int h = decltype(h_c)::value;
    if constexpr (F::kFusedQ) {
      const uint8_t* sc = ring + slot_off(st) + C::kStageScaleOff + (lane >> 4);
#pragma unroll
      for (int m = 0; m < kHM; ++m) {
        const uint32_t row = a_row0 + 16 * (h * kHM + m) + (lane & 15);
#pragma unroll
        for (int t = 0; t < F::kTerms; ++t) xs[h][m * F::kTerms + t] = sc[t * kBM * 4 + row * 4];
      }
    }
  };

  f32x16_t acc[kTM][kTN];
  f32x4_t acc16[C::kT16M][C::kT16N];
  auto zero_acc = [&]() __attribute__((always_inline)) {
    if constexpr (kM16) {
#pragma unroll
      for (int i = 0; i < C::kT16M; ++i)
#pragma unroll
        for (int j = 0; j < C::kT16N; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) acc16[i][j][q] = 0.f;
    } else {
#pragma unroll
      for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j)
#pragma unroll
          for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
    }
  };
  zero_acc();

  // Prologue: scales of group 0, then stages 0..2; wait for stage 0 (and the
  // scales issued before it), make it visible, read its first step. With
  // in-GEMM quantization, X of stages 0..2 is loaded beside them and stages
  // 0 and 1 are quantized here (the loop quantizes stage st + 2 in stage st).
  static_assert(!F::kFusedQ || kFast, "in-GEMM quantization runs on whole scale groups");
  issue_scales(0);
  if constexpr (F::kFusedQ) {
    issue_stage(0, std::integral_constant<int, 2>{});
    issue_stage(1, std::integral_constant<int, 2>{});
    issue_x(0);
    wait_vmcnt<0>();
    quantize_x(0);
    issue_x(1);
    wait_vmcnt<0>();
    quantize_x(1);
    issue_stage(2, std::integral_constant<int, 0>{});
  } else {
#pragma unroll
    for (int st = 0; st < kRing - 1; ++st) issue_stage(st, std::integral_constant<int, 2>{});
    issue_stage(kRing - 1, std::integral_constant<int, 0>{});
  }
  if (F::kFusedQ)
    wait_vmcnt<kPart0>();
  else if (kFast)
    wait_vmcnt<kDmaPerStage + kPart0>();
  else
    wait_vmcnt<0>();
  wait_lgkmcnt0();
  stage_barrier();
  i32x4_t a0[kSubA][kTM], bw0[kTN], a1[kSubA][kTM], bw1[kTN];
  if constexpr (kM16) {
    // stage 0's first halves and the group's first-half scale words; the
    // second halves are read in stage 0's first group, as in every stage
    read_ws16(std::integral_constant<int, 0>{});
    read_xs16(std::integral_constant<int, 0>{});
    read_xs16f(0, std::integral_constant<int, 0>{});
    read_w16(0, std::integral_constant<int, 0>{});
    read_x16(0, std::integral_constant<int, 0>{});
  } else {
    read_scale_pair(0);
    read_step(0, 0, a0, bw0);
  }

  // One stage; P = st % 4 is a compile-time constant so that every wait count
  // and scale-word index below is one.
  // The middle of stage st: stage st + 1 must have landed, and at the end of
  // a group also the next group's scales. The only loads issued after those
  // are stage st + 2's (scales go out before the stage loads of the same
  // sync point, and every stage issues the same loads, see issue_stage).
  // After the barrier every wave is past its reads of stage st, so its slot
  // takes stage st + 3; at P == 2 every wave also holds the group's scale
  // words for its remaining stages, so the scale buffer takes the next group
  // (issued first, see the wait).
  auto sync_and_refill = [&](auto pc, int st) __attribute__((always_inline)) {
    constexpr int P = decltype(pc)::value;
    // (with in-GEMM quantization the X loads of stage st + 2 went out after
    // the second weight part of stage st + 2, and those of stage st + 1,
    // older than the scales, are already in)
    if (kFast)
      wait_vmcnt<kDmaPerStage + kLoadsX>();
    else
      wait_vmcnt<0>();
    wait_lgkmcnt0();
    stage_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (kStream && P == 1 && st + kRing - load_base == nstages && load_tile + 1 < ntiles) {
      // the stream reaches the next tile with this stage's fetch (stage
      // st + 3 = 4 g + 4, a tile start; every earlier fetch of the old tile
      // has been issued, and none of the new one)
      ++load_tile;
      load_base += nstages;
      const GemmParams q = fresh_params<kSlot>();
      int m0, n0;
      tile_origin(q, bid + load_tile * q.wg, m0, n0);
      set_load_tile(q, m0, n0);
    }
    if (P == 2) issue_scales(st / kScaleGroup + 1);
    issue_stage(st + kRing, std::integral_constant<int, 0>{});
    if constexpr (F::kFusedQ) {
      // X of stage st + 2 (loaded at the start of this stage) must be in
      // before it is quantized: only the loads just issued went out after it
      wait_vmcnt<kPart0 + (P == 2 ? kScaleLoadsPerWave : 0)>();
    }
  };

  auto stage = [&](auto pc, int st) __attribute__((always_inline)) {
    constexpr int P = decltype(pc)::value;
    __builtin_amdgcn_sched_barrier(0);   // keep each stage's schedule to itself
    // scale words of this stage: byte 2 s of (word >> 8 lhalf) is block 4 st + 2 s + lhalf
    // (the empty asm pins each extraction in its own stage, so the compiler
    // does not compute all four stages' words up front and hold them)
    uint32_t cx[kTM], cr[kTM], cw[kTN];
    if constexpr (!F::kBf16) {
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      cx[i] = (uint32_t)gx[i][P % 2];
      asm volatile("" : "+v"(cx[i]));
      cx[i] >>= 8 * lhalf;
      if (kResid) {
        cr[i] = (uint32_t)gr[i][P % 2];
        asm volatile("" : "+v"(cr[i]));
        cr[i] >>= 8 * lhalf;
      } else {
        cr[i] = 0u;
      }
    }
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
      cw[j] = (uint32_t)gw[j][P % 2];
      asm volatile("" : "+v"(cw[j]));
      cw[j] >>= 8 * lhalf;
    }
    }

    // first MFMA step; meanwhile read the second step's fragments and issue
    // the second part of stage st + 2's loads
    issue_stage(st + kRing - 1, std::integral_constant<int, 1>{});
    read_step(st, 1, a1, bw1);
    mfma_step<0, F, kTM, kTN>(acc, a0, bw0, cx, cr, cw);
    interleave_hint<kReadsPerStep, kFast ? kDmaPerStage - kPart0 : 0, kMfmaPerStep>();

    sync_and_refill(pc, st);

    // second MFMA step; meanwhile read stage st + 1's first step and, after
    // stages 1 and 3 of a group, the scale words of the next two stages (this
    // stage's words were taken out of the registers above). Past the end
    // these reads fetch values nobody uses.
    if (P == 1) read_scale_pair(1);
    if (P == 3) read_scale_pair(0);
    read_step(st + 1, 0, a0, bw0);
    mfma_step<1, F, kTM, kTN>(acc, a1, bw1, cx, cr, cw);
    interleave_hint<kReadsPerStep + (P % 2 == 1 ? kScaleRowReads : 0),
                    kFast ? kPart0 + (P == 2 ? kScaleLoadsPerWave : 0) : 0, kMfmaPerStep>();
    __builtin_amdgcn_sched_barrier(0);
  };

  // One stage on the 16 x 16 x 128 path: four MFMA groups, the barrier
  // after the second; the reads beside each group are the halves freed by
  // the groups before it (see the register note above).
  // One group of 16 x 16 x 128 MFMAs, (weight half HW, activation half HX),
  // with the LDS reads (kReads) and loads (kVmem) issued before it in
  // program order spread among its MFMAs. (The scheduler places the two
  // MFMAs into one accumulator next to each other in some groups; fencing
  // the X terms from the R terms so that they stay kHM x kHN apart measured
  // 1% slower, so the hardware's result forwarding covers that.)
  auto group16 = [&](auto pc, auto hw_c, auto hx_c, auto reads_c, auto vmem_c) __attribute__((always_inline)) {
    constexpr int P = decltype(pc)::value;
    constexpr int PX = F::kFusedQ ? 0 : P;
    constexpr int HW = decltype(hw_c)::value, HX = decltype(hx_c)::value;
    constexpr int kReads = decltype(reads_c)::value, kVmem = decltype(vmem_c)::value;
    constexpr int kG = kHM * kHN * F::kTerms;
    mfma16_group<P, PX, HW, HX, F::kTerms, kSubA, F::kXFmt, kHM, kHN, C::kT16M, C::kT16N>(acc16, wf, xf, ws, xs);
    if constexpr (kReads + kVmem > 0) interleave_hint<kReads, kVmem, kG>();
  };

  auto stage16 = [&](auto pc, int st) __attribute__((always_inline)) {
    constexpr int P = decltype(pc)::value;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    __builtin_amdgcn_sched_barrier(0);
    // (W0, A0): meanwhile stage st's second halves (and, at a group's first
    // stage, its second-half scale words) and the second part of stage
    // st + 2's loads
    constexpr int kXsReads = F::kFusedQ ? kXH : 0;   // per-stage scale bytes (in-GEMM quantization)
    issue_stage(st + kRing - 1, I1{});
    issue_x(st + kRing - 1);
    read_w16(st, I1{});
    read_x16(st, I1{});
    read_xs16f(st, I1{});
    if (P == 0) {
      read_ws16(I1{});
      read_xs16(I1{});
    }
    group16(pc, I0{}, I0{}, std::integral_constant<int, kHN + kXF + kXsReads + (P == 0 ? kHN + (F::kFusedQ ? 0 : kXH) : 0)>{},
            std::integral_constant<int, kFast ? kDmaPerStage - kPart0 + kLoadsX : 0>{});
    __builtin_amdgcn_sched_barrier(0);
    // (W0, A1)
    group16(pc, I0{}, I1{}, I0{}, I0{});
    __builtin_amdgcn_sched_barrier(0);
    sync_and_refill(pc, st);
    // (W1, A0): meanwhile stage st + 1's W0 (and at the group's last stage
    // the next group's W0 scale words); with in-GEMM quantization also the
    // first half of stage st + 2's quantization
    read_w16(st + 1, I0{});
    if (P == 3) read_ws16(I0{});
    quantize_half(st + 2, I0{});
    group16(pc, I1{}, I0{}, std::integral_constant<int, kHN + (P == 3 ? kHN : 0)>{},
            std::integral_constant<int, kFast ? kPart0 + (P == 2 ? kScaleLoadsPerWave : 0) : 0>{});
    __builtin_amdgcn_sched_barrier(0);
    // (W1, A1): meanwhile stage st + 1's A0 (and the next group's A0 scale
    // words), and the rest of stage st + 2's quantization
    read_x16(st + 1, I0{});
    read_xs16f(st + 1, I0{});
    if (P == 3) read_xs16(I0{});
    quantize_half(st + 2, I1{});
    group16(pc, I1{}, I1{}, std::integral_constant<int, kXF + kXsReads + (P == 3 && !F::kFusedQ ? kXH : 0)>{}, I0{});
    __builtin_amdgcn_sched_barrier(0);
  };
  auto run_stage = [&](auto pc, int st) __attribute__((always_inline)) {
    if constexpr (kM16)
      stage16(pc, st);
    else
      stage(pc, st);
  };

  // Epilogue of a tile: fp32 accumulators to Y. The weight is the MFMA's
  // first operand, so tile (i, j) holds Y^T: lane (lhalf, lrow) has row m of
  // Y and, in accumulator group q / 4, the four consecutive columns
  // 8 (q / 4) + 4 lhalf + (0..3), stored together (8 bytes of bf16 or 16 of
  // fp32) when the host found Y's base and row stride aligned for it.
  auto store_tile = [&](int em0, int en0) __attribute__((always_inline)) {
    const GemmParams q = fresh_params<kSlot>();
    if constexpr (kM16) {
      // 16 x 16 tiles: lane (lane / 16, lane % 16) has row m of Y and the
      // four consecutive columns 16 n + 4 (lane / 16) + (0..3) of tile n
      const int row16 = em0 + (int)a_row0 + (int)(lane & 15);
      const int col16 = en0 + (int)b_row0 + 4 * (int)(lane >> 4);
#pragma unroll
      for (int i = 0; i < C::kT16M; ++i) {
        const int row = row16 + 16 * i;
        if (row >= q.M) continue;
#pragma unroll
        for (int j = 0; j < C::kT16N; ++j) {
          const int col = col16 + 16 * j;
          const f32x4_t& a = acc16[i][j];
          const float v[4] = {a[0], a[1], a[2], a[3]};
          if (kOutBf16) {
            const uint32_t h01 = bf16_pair(v[0], v[1]), h23 = bf16_pair(v[2], v[3]);
            const uint16_t h[4] = {(uint16_t)h01, (uint16_t)(h01 >> 16), (uint16_t)h23, (uint16_t)(h23 >> 16)};
            uint16_t* dst = reinterpret_cast<uint16_t*>(q.y) + (int64_t)row * q.ldy + col;
            if (q.vec_out && col + 3 < q.N) {
              *reinterpret_cast<i32x2_t*>(dst) = i32x2_t{(int)h01, (int)h23};
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (col + e < q.N) dst[e] = h[e];
            }
          } else {
            float* dst = reinterpret_cast<float*>(q.y) + (int64_t)row * q.ldy + col;
            if (q.vec_out && col + 3 < q.N) {
              *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{v[0], v[1], v[2], v[3]};
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (col + e < q.N) dst[e] = v[e];
            }
          }
        }
      }
      return;
    }
    const int row_base = em0 + (int)a_row0 + (int)lrow;
    const int col_base = en0 + (int)b_row0 + 4 * (int)lhalf;
    if constexpr (F::kOutT) {
      // element (row, col) to y[col * ldy + row]: for one (i, j, g, e) the 32
      // lanes of a half write 32 consecutive rows of one output row
#pragma unroll
      for (int i = 0; i < kTM; ++i) {
        const int row = row_base + 32 * i;
        if (row >= q.M) continue;
#pragma unroll
        for (int j = 0; j < kTN; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int col = col_base + 32 * j + 8 * g + e;
              if (col >= q.N) continue;
              const float v = acc[i][j][4 * g + e];
              const int64_t at = (int64_t)col * q.ldy + row;
              if (kOutBf16) {
                reinterpret_cast<uint16_t*>(q.y)[at] = (uint16_t)bf16_pair(v, 0.f);
              } else {
                reinterpret_cast<float*>(q.y)[at] = v;
              }
            }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      const int row = row_base + 32 * i;
      if (row >= q.M) continue;
#pragma unroll
      for (int j = 0; j < kTN; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = col_base + 32 * j + 8 * g;
          const float v[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
          if (kOutBf16) {
            const uint32_t h01 = bf16_pair(v[0], v[1]), h23 = bf16_pair(v[2], v[3]);
            const uint16_t h[4] = {(uint16_t)h01, (uint16_t)(h01 >> 16), (uint16_t)h23, (uint16_t)(h23 >> 16)};
            uint16_t* dst = reinterpret_cast<uint16_t*>(q.y) + (int64_t)row * q.ldy + col;
            if (q.vec_out && col + 3 < q.N) {
              *reinterpret_cast<i32x2_t*>(dst) = i32x2_t{(int)h01, (int)h23};
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (col + e < q.N) dst[e] = h[e];
            }
          } else {
            float* dst = reinterpret_cast<float*>(q.y) + (int64_t)row * q.ldy + col;
            if (q.vec_out && col + 3 < q.N) {
              *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{v[0], v[1], v[2], v[3]};
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (col + e < q.N) dst[e] = v[e];
            }
          }
        }
      }
    }
  };

  // The same for a tile that lies inside Y, with vector stores allowed. Each
  // store is scheduled on its own (sched_barrier), so that only one group of
  // converted values is live at a time: this runs inside the K loop, beside
  // the next tile's fragments.
  auto store_full_tile = [&](int em0, int en0) __attribute__((always_inline)) {
    if constexpr (F::kOutT) {
      store_tile(em0, en0);
      return;
    }
    const GemmParams q = fresh_params<kSlot>();
    if constexpr (kM16) {
      // (the lane recomputed here, so that nothing derived from it has to
      // stay live through the K loop for this epilogue)
      uint32_t sl = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
      asm volatile("" : "+v"(sl));
#pragma unroll
      for (int i = 0; i < C::kT16M; ++i) {
        const int64_t at =
            (int64_t)(em0 + (int)a_row0 + (int)(sl & 15) + 16 * i) * q.ldy + en0 + (int)b_row0 + 4 * (int)(sl >> 4);
        uint16_t* yb = reinterpret_cast<uint16_t*>(q.y) + at;
        float* yf = reinterpret_cast<float*>(q.y) + at;
#pragma unroll
        for (int j = 0; j < C::kT16N; ++j) {
          const f32x4_t& a = acc16[i][j];
          if (kOutBf16) {
            *reinterpret_cast<i32x2_t*>(yb + 16 * j) = i32x2_t{(int)bf16_pair(a[0], a[1]), (int)bf16_pair(a[2], a[3])};
          } else {
            *reinterpret_cast<f32x4_t*>(yf + 16 * j) = f32x4_t{a[0], a[1], a[2], a[3]};
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      const int64_t at = (int64_t)(em0 + (int)a_row0 + (int)lrow + 32 * i) * q.ldy + en0 + (int)b_row0 + 4 * (int)lhalf;
      uint16_t* yb = reinterpret_cast<uint16_t*>(q.y) + at;
      float* yf = reinterpret_cast<float*>(q.y) + at;
#pragma unroll
      for (int j = 0; j < kTN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16_t& a = acc[i][j];
          if (kOutBf16) {
            *reinterpret_cast<i32x2_t*>(yb + 32 * j + 8 * g) =
                i32x2_t{(int)bf16_pair(a[4 * g], a[4 * g + 1]), (int)bf16_pair(a[4 * g + 2], a[4 * g + 3])};
          } else {
            *reinterpret_cast<f32x4_t*>(yf + 32 * j + 8 * g) = f32x4_t{a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
          }
          __builtin_amdgcn_sched_barrier(0);
        }
    }
  };

  // (the per-stage guards also keep each stage in its own block, which the
  // register allocator needs to fit this loop without spills)
  int comp_base = 0, comp_tile = 0;
  for (int st = 0; st < total_stages; st += kScaleGroup) {
    loop_st0 = st;
    run_stage(std::integral_constant<int, 0>{}, st);
    if (st + 1 < total_stages) run_stage(std::integral_constant<int, 1>{}, st + 1);
    if (st + 2 < total_stages) run_stage(std::integral_constant<int, 2>{}, st + 2);
    if (st + 3 < total_stages) run_stage(std::integral_constant<int, 3>{}, st + 3);
    if (kStream && st + kScaleGroup - comp_base == nstages && st + kScaleGroup < total_stages) {
      // a tile ends here and another follows in the stream: store it, then
      // start the next from zero (its first fragments are already read)
      store_full_tile(cm0, cn0);
      zero_acc();
      ++comp_tile;
      comp_base += nstages;
      const GemmParams q = fresh_params<kSlot>();
      tile_origin(q, bid + comp_tile * q.wg, cm0, cn0);
    }
    const uint32_t r0 = rot[0];
    rot[0] = rot[1];
    rot[1] = rot[2];
    rot[2] = r0;
  }
  if (kStream)
    store_full_tile(cm0, cn0);
  else
    store_tile(cm0, cn0);
}

template <class C, class F, bool kOutBf16, bool kFast, bool kStream>
__global__ __launch_bounds__(64 * C::kWaves, C::kOcc) void gemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::kLdsBytes];
  gemm_body<C, F, kOutBf16, kFast, kStream, 0>(p, (int)blockIdx.x, lds);
}

// The streamed whole rounds of big tiles and the last partial round (as
// halves or rectangle pieces) in one launch: workgroups 0 .. a.wg - 1
// stream big tiles (one per CU), the rest take one piece each, so each
// piece starts on a CU as soon as that CU's stream ends (no workgroup waits
// for another).
template <class CB, class CH, class F, bool kOutBf16>
__global__ __launch_bounds__(64 * CB::kWaves, 1) void gemm_pair_kernel(GemmPairParams pp) {
  static_assert(CB::kWaves == CH::kWaves, "one workgroup size");
  constexpr int kLds = CB::kLdsBytes > CH::kLdsBytes ? CB::kLdsBytes : CH::kLdsBytes;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLds];
  if ((int)blockIdx.x < pp.a.wg)
    gemm_body<CB, F, kOutBf16, true, true, 0>(pp.a, (int)blockIdx.x, lds);
  else
    gemm_body<CH, F, kOutBf16, true, false, 1>(pp.b, (int)blockIdx.x - pp.a.wg, lds);
}

template <class C, class F, bool kOutBf16, bool kCanStream>
hipError_t launch_tiles(const GemmParams& p, bool fast, bool stream_tiles, hipStream_t stream) {
  if (p.grid <= 0) return hipSuccess;
  if (kCanStream && stream_tiles)
    hipLaunchKernelGGL((gemm_kernel<C, F, kOutBf16, true, kCanStream>), dim3(p.wg), dim3(64 * C::kWaves), 0, stream, p);
  else if (fast)
    hipLaunchKernelGGL((gemm_kernel<C, F, kOutBf16, true, false>), dim3(p.wg), dim3(64 * C::kWaves), 0, stream, p);
  else if constexpr (!F::kFusedQ)
    hipLaunchKernelGGL((gemm_kernel<C, F, kOutBf16, false, false>), dim3(p.wg), dim3(64 * C::kWaves), 0, stream, p);
  else
    return hipErrorInvalidValue;   // in-GEMM quantization needs K % 512 == 0 (checked by the caller)
  return hipGetLastError();
}

// Plans the launch: big tiles, one workgroup per CU, in whole rounds of
// `cus` tiles; a last partial round of `rest` tiles goes out in whichever of
// these shapes is priced lowest (in units of one big-tile round):
//  - big tiles on `rest` CUs: 1;
//  - quadrants (128 x 128 on 4 waves, two workgroups per CU): kQuadRound per
//    ceil(4 rest / (2 cus)) rounds;
//  - halves (128 x 256 on 8 waves, one per CU): kHalfRound per
//    ceil(2 rest / cus) rounds.
// Quadrants run in a second launch after the whole rounds, and so do halves
// when the whole rounds do not stream; behind streamed rounds the halves go
// in the same launch (gemm_pair_kernel: each CU takes a half as soon as its
// stream ends, and the gap between two launches goes away; same-box A/B on
// the 4096 x 5120 x 13824 layer 275.0 against 281.8 us, W4A8 236.8 against
// 243.3 us; Y bit-identical). The prices are measured: on the 4096 x 13824 x 5120 layer (96 tiles left after
// three rounds) 384 quadrants took 0.55 of a big round and 192 halves 0.44;
// on 2048 x 4096 x 4096 (128 tiles, no whole round) one round of halves ran
// in 0.70 of the big-tile time and of quadrants in 0.84. Halves have the
// 8-wave workgroup's operand reuse (half the fragment reads per MFMA of a
// 4-wave quadrant) and fill one CU each. The same holds for plain W4A4 and
// W4A8. Behind streamed rounds, when the last partial round's tiles form a
// rectangle that 128 x 192 pieces cover in at most one round, the pieces
// (8 waves of 32 x 96) run there instead of halves. On the 4096 x 5120 x
// 13824 layer (96 tiles left: a 1024 x 6144 rectangle, 256 pieces on all
// CUs, where 192 halves leave 64 idle)
// same-box A/B measured the RFQ GEMM at 275.4 against 276.0 us (equal) and
// W4A8 at 236.7 against 241.0 us, Y bit-identical; their price is set just
// below the halves'. The bf16 mode of the backward products is the other way round: its
// stages are short (32 K elements), and two quadrant workgroups per CU hide
// each other's barriers better (dX on the 4096 x 5120 x 13824 layer: 554-558
// us with quadrants, 595-599 us with halves; dW 892-896 against 909-912 us).
constexpr double kQuadRound = 0.55, kHalfRound = 0.48, kPieceRound = 0.47;
constexpr double kQuadRoundBf16 = 0.50, kHalfRoundBf16 = 0.60;

// The launch plan of every variant but in-GEMM quantization (below): big
// tiles in whole rounds, the rest as halves or quadrants.
template <class F, bool kOutBf16>
hipError_t launch_tiled_impl(GemmParams p, bool fast, int cus, int tiles, hipStream_t stream) {
  using Big = typename Tiles<F>::Big;
  using Quad = typename Tiles<F>::Quad;
  using Half = typename Tiles<F>::Half;
  using Piece = typename Tiles<F>::Piece;
  if constexpr (F::kBf16 && !F::kOutT) {
    // The bf16 product dY Wd: when 256 x 320 tiles (8 waves of 64 x 160)
    // cover Y in whole rounds and 256 x 256 tiles would leave a partial
    // one, the wide tiles run alone (dX of a layer with K = 5120: 16 x 16
    // tiles per 4096 rows). They also do a quarter more MFMA work per stage
    // and barrier.
    using Wide = TileCfg<256, 320, 8, 1, F>;
    const int wm = p.M / Wide::kBM, wn = p.N / Wide::kBN;
    if (fast && p.vec_out && p.M % Wide::kBM == 0 && p.N % Wide::kBN == 0 && (int64_t)wm * wn % cus == 0 &&
        tiles % cus != 0) {
      p.gm = Wide::kBM;
      p.gn = Wide::kBN;
      p.tiles_m = wm;
      p.tiles_n = wn;
      p.first = 0;
      p.grid = wm * wn;
      p.pieces = 1;
      const bool stream_tiles = p.grid > cus;
      p.wg = stream_tiles ? cus : p.grid;
      return launch_tiles<Wide, F, kOutBf16, true>(p, fast, stream_tiles, stream);
    }
  }
  const int rounds = tiles / cus, rest = tiles % cus;
  enum { kTailBig = 1, kTailQuad = 2, kTailHalf = 3 };
  int tail = kTailBig;
  double best = 1.0;
  if (rest != 0) {
    const double quad_round = F::kBf16 ? kQuadRoundBf16 : kQuadRound;
    const double half_round = F::kBf16 ? kHalfRoundBf16 : kHalfRound;
    const double t_quad = quad_round * ((4 * rest + 2 * cus - 1) / (2 * cus));
    const double t_half = Tiles<F>::kHasHalf ? half_round * ((2 * rest + cus - 1) / cus) : 1e30;
    if (t_quad < best) { best = t_quad; tail = kTailQuad; }
    if (t_half < best) { best = t_half; tail = kTailHalf; }
  }
  const int big = tail == kTailBig ? tiles : rounds * cus;
  p.first = 0;
  p.grid = big;
  p.pieces = 1;
  // When every tile lies inside Y and Y takes vector stores, one workgroup
  // per CU streams its tiles back to back; otherwise every tile gets its own
  // workgroup.
  const bool stream_tiles = fast && p.vec_out && p.M % Big::kBM == 0 && p.N % Big::kBN == 0 && big > cus;
  p.wg = stream_tiles ? cus : big;
  if constexpr (Tiles<F>::kHasHalf && !F::kFusedQ && !F::kBf16) {
    // The last partial round as one round of 128 x 192 pieces, when its
    // tiles form a rectangle that such pieces cover exactly: the logical
    // order walks groups of kGroupM tile rows column by column, so the
    // leftover tiles are whole columns of the last group when they start at
    // a column boundary of it.
    const int per_group = kGroupM * p.tiles_n;
    const int g_last = big / per_group, g_start = g_last * per_group;
    const int g_rows = min(p.tiles_m - g_last * kGroupM, kGroupM);
    const int off = big - g_start;
    if (stream_tiles && rest != 0 && kPieceRound < best && g_start + g_rows * p.tiles_n == tiles && off % g_rows == 0) {
      const int tn0 = off / g_rows;
      const int rows = g_rows * Big::kBM, cols = (p.tiles_n - tn0) * Big::kBN;
      const int pm = rows / Piece::kBM, pn = cols / Piece::kBN;
      if (rows % Piece::kBM == 0 && cols % Piece::kBN == 0 && pm * pn <= cus) {
        GemmPairParams pp;
        pp.a = p;
        pp.b = p;
        pp.b.pieces = 3;
        pp.b.gm = Piece::kBM;
        pp.b.gn = Piece::kBN;
        pp.b.tiles_m = pm;
        pp.b.tiles_n = pn;
        pp.b.rm0 = g_last * kGroupM * Big::kBM;
        pp.b.rn0 = tn0 * Big::kBN;
        pp.b.first = 0;
        pp.b.grid = pp.b.wg = pm * pn;
        hipLaunchKernelGGL((gemm_pair_kernel<Big, Piece, F, kOutBf16>), dim3(pp.a.wg + pp.b.wg),
                           dim3(64 * Big::kWaves), 0, stream, pp);
        return hipGetLastError();
      }
    }
  }
  if constexpr (Tiles<F>::kHasHalf && !F::kFusedQ) {
    if (stream_tiles && tail == kTailHalf && Big::kWaves == Half::kWaves) {
      GemmPairParams pp;
      pp.a = p;
      pp.b = p;
      pp.b.first = big;
      pp.b.pieces = 2;
      pp.b.grid = pp.b.wg = 2 * (tiles - big);
      hipLaunchKernelGGL((gemm_pair_kernel<Big, Half, F, kOutBf16>), dim3(pp.a.wg + pp.b.wg), dim3(64 * Big::kWaves), 0,
                         stream, pp);
      return hipGetLastError();
    }
  }
  hipError_t e = launch_tiles<Big, F, kOutBf16, true>(p, fast, stream_tiles, stream);
  if (e != hipSuccess || big == tiles) return e;
  p.first = big;
  if (tail == kTailHalf) {
    p.pieces = 2;
    p.grid = p.wg = 2 * (tiles - big);
    return launch_tiles<Half, F, kOutBf16, false>(p, fast, false, stream);
  }
  p.pieces = 4;
  p.grid = p.wg = 4 * (tiles - big);
  return launch_tiles<Quad, F, kOutBf16, false>(p, fast, false, stream);
}

template <class F, bool kOutBf16>
hipError_t launch_variant(GemmParams p, bool fast, int cus, hipStream_t stream) {
  using Big = typename Tiles<F>::Big;
  p.gm = Big::kBM;
  p.gn = Big::kBN;
  p.tiles_m = (p.M + p.gm - 1) / p.gm;
  p.tiles_n = (p.N + p.gn - 1) / p.gn;
  const int tiles = p.tiles_m * p.tiles_n;
  if constexpr (F::kFusedQ) {
    // In-GEMM quantization: one launch of 128 x 256 tiles. When they lie
    // inside Y, one workgroup per CU streams items b, b + wg, ... (a last
    // partial round just gives some workgroups one tile more); otherwise one
    // workgroup per tile.
    const bool stream_tiles = fast && p.vec_out && p.M % Big::kBM == 0 && p.N % Big::kBN == 0 && tiles > cus;
    p.first = 0;
    p.grid = tiles;
    p.pieces = 1;
    p.wg = stream_tiles ? cus : tiles;
    return launch_tiles<Big, F, kOutBf16, true>(p, fast, stream_tiles, stream);
  } else {
    return launch_tiled_impl<F, kOutBf16>(p, fast, cus, tiles, stream);
  }
}

int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace

hipError_t launch_gemm(int x_fmt, int r_fmt, const uint8_t* qx, const uint8_t* sx, const uint8_t* qr,
                       const uint8_t* sr, const uint8_t* w, const uint8_t* sw, int64_t M, int64_t N, int64_t K,
                       void* y, bool y_bf16, int64_t ldy, hipStream_t stream, bool y_trans) {
  GemmParams p;
  p.qx = qx; p.sx = sx; p.qr = qr; p.sr = sr; p.w = w; p.sw = sw;
  p.y = y; p.ldy = ldy;
  p.ldx = 0;
  // four consecutive outputs go out as one 8-byte (bf16) or 16-byte (fp32)
  // store (transposed results go element by element, any alignment)
  const uintptr_t vec_bytes = y_bf16 ? 8 : 16;
  p.vec_out = (y_trans || ((uintptr_t)y % vec_bytes == 0 && ldy % 4 == 0)) ? 1 : 0;
  p.M = (int32_t)M; p.N = (int32_t)N; p.K = (int32_t)K;
  p.rm0 = p.rn0 = 0;
  const bool fast = (K % (kBK * kScaleGroup)) == 0;
  const int cus = cu_count();
  if (qr == nullptr) r_fmt = 0;
  if (x_fmt == 16) {
    // bf16 operands: K counts E2M1-sized elements, 4 per bf16 element, so
    // that bytes per row, stages and 16-byte chunks follow the same rules
    if (y_trans != (r_fmt == 16)) return hipErrorInvalidValue;
    if (r_fmt == 16)
      return y_bf16 ? launch_variant<FmtBf16PairT, true>(p, fast, cus, stream)
                    : launch_variant<FmtBf16PairT, false>(p, fast, cus, stream);
    return y_bf16 ? launch_variant<FmtBf16, true>(p, fast, cus, stream) : launch_variant<FmtBf16, false>(p, fast, cus, stream);
  }
  if (y_trans) return hipErrorInvalidValue;
  switch (x_fmt * 10 + r_fmt) {
    case 40: return y_bf16 ? launch_variant<FmtW4A4, true>(p, fast, cus, stream) : launch_variant<FmtW4A4, false>(p, fast, cus, stream);
    case 44: return y_bf16 ? launch_variant<FmtRfq, true>(p, fast, cus, stream) : launch_variant<FmtRfq, false>(p, fast, cus, stream);
    case 48: return y_bf16 ? launch_variant<FmtRfq8, true>(p, fast, cus, stream) : launch_variant<FmtRfq8, false>(p, fast, cus, stream);
    case 80: return y_bf16 ? launch_variant<FmtW4A8, true>(p, fast, cus, stream) : launch_variant<FmtW4A8, false>(p, fast, cus, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_fused(const uint16_t* x, int64_t ldx, const uint8_t* w, const uint8_t* sw, int64_t M, int64_t N,
                             int64_t K, void* y, bool y_bf16, int64_t ldy, hipStream_t stream) {
  if (K % (kBK * kScaleGroup) != 0) return hipErrorInvalidValue;
  GemmParams p;
  p.qx = reinterpret_cast<const uint8_t*>(x);
  p.sx = p.qr = p.sr = nullptr;
  p.w = w; p.sw = sw;
  p.y = y; p.ldy = ldy;
  p.ldx = ldx;
  const uintptr_t vec_bytes = y_bf16 ? 8 : 16;
  p.vec_out = ((uintptr_t)y % vec_bytes == 0 && ldy % 4 == 0) ? 1 : 0;
  p.M = (int32_t)M; p.N = (int32_t)N; p.K = (int32_t)K;
  p.rm0 = p.rn0 = 0;
  const int cus = cu_count();
  return y_bf16 ? launch_variant<FmtRfqFused, true>(p, true, cus, stream)
                : launch_variant<FmtRfqFused, false>(p, true, cus, stream);
}

}  // namespace rfq
