// MFMA issue ceiling under the power limit: a benchmark-only probe, built
// into its own library (librfqprobe.so) beside bench.py and never linked
// into librfq.so. It runs a loop of the GEMM's scaled MFMA on caller-supplied
// operand bytes, with no memory traffic inside the loop, timed per workgroup
// in shader-clock cycles (s_memtime) and in 100 MHz constant-clock ticks
// (s_memrealtime), so that both the rate and the clock it ran at can be read
// back. Both operand pairs run the 16 x 16 x 128 form the GEMM uses for
// them, 64 instructions per wave per iteration over 32 accumulators: E2M1 x
// E2M1 (RFQ and W4A4) and E2M1 x E4M3 (W4A8), whose instruction takes twice
// the cycles for the same flops.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rfq_probe.h"

namespace {

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;   // two waves per SIMD, like the GEMM's main tile
constexpr int kAcc = 8;         // independent accumulators per wave

// kBFmt: format of the second operand, 4 (E2M1, 16 bytes per lane) or 8
// (E4M3, 32 bytes per lane).
template <int kBFmt>
__global__ __launch_bounds__(kThreads) void mfma_ceiling_kernel(const i32x4_t* a, uint32_t a_n, const i32x4_t* b,
                                                                 uint32_t b_n, int iters, uint64_t* stamps,
                                                                 float* sink) {
  const uint32_t t = threadIdx.x;
  i32x4_t ra[4];
  i32x8_t rb[4];
  for (int i = 0; i < 4; ++i) {
    const uint32_t slot = (blockIdx.x * kThreads + t) * 4 + i;
    ra[i] = a[slot % a_n];
    const i32x4_t lo = b[(2 * slot) % b_n], hi = b[(2 * slot + 1) % b_n];
    rb[i] = kBFmt == 8 ? i32x8_t{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w} : i32x8_t{lo.x, lo.y, lo.z, lo.w, 0, 0, 0, 0};
  }
  float sum = 0.f;
  uint64_t c0, r0, c1, r1;
  {
    constexpr int kAcc16 = 4 * kAcc;   // 32 accumulator tiles of 16 x 16
    f32x4_t acc[kAcc16];
    for (int q = 0; q < kAcc16; ++q)
      for (int e = 0; e < 4; ++e) acc[q][e] = 0.f;
    c0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int q = 0; q < kAcc16; ++q) {
          const i32x4_t x = ra[(q + s) & 3];
          acc[q] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(i32x8_t{x.x, x.y, x.z, x.w, 0, 0, 0, 0},
                                                                    rb[(q / 8 + s) & 3], acc[q], 4, kBFmt == 8 ? 0 : 4,
                                                                    0, 120 + (q & 7), 0, 122);
        }
    }
    c1 = __builtin_amdgcn_s_memtime();
    r1 = __builtin_amdgcn_s_memrealtime();
    for (int q = 0; q < kAcc16; ++q)
      for (int e = 0; e < 4; ++e) sum += acc[q][e];
  }
  sink[blockIdx.x * kThreads + t] = sum;
  if (t == 0) {
    stamps[2 * blockIdx.x] = c1 - c0;
    stamps[2 * blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace

namespace {

int launch_probe(const uint8_t* a, size_t a_bytes, const uint8_t* b, size_t b_bytes, int b_fmt, int workgroups,
                 int iters, uint64_t* stamps, float* sink, hipStream_t stream) {
  if (a == nullptr || b == nullptr || stamps == nullptr || sink == nullptr) return RFQ_PROBE_ERR_ARGUMENT;
  if (reinterpret_cast<uintptr_t>(a) % 16 || reinterpret_cast<uintptr_t>(b) % 16) return RFQ_PROBE_ERR_ARGUMENT;
  const size_t max_bytes = (size_t(1) << 32) * 16 - 16;
  if (a_bytes < 16 || b_bytes < 16 || a_bytes % 16 || b_bytes % 16 || a_bytes > max_bytes || b_bytes > max_bytes)
    return RFQ_PROBE_ERR_ARGUMENT;
  if (workgroups <= 0 || workgroups > 65536 || iters <= 0) return RFQ_PROBE_ERR_ARGUMENT;
  const auto* ap = reinterpret_cast<const i32x4_t*>(a);
  const auto* bp = reinterpret_cast<const i32x4_t*>(b);
  if (b_fmt == 8)
    hipLaunchKernelGGL(mfma_ceiling_kernel<8>, dim3(workgroups), dim3(kThreads), 0, stream, ap, (uint32_t)(a_bytes / 16),
                       bp, (uint32_t)(b_bytes / 16), iters, stamps, sink);
  else
    hipLaunchKernelGGL(mfma_ceiling_kernel<4>, dim3(workgroups), dim3(kThreads), 0, stream, ap, (uint32_t)(a_bytes / 16),
                       bp, (uint32_t)(b_bytes / 16), iters, stamps, sink);
  return hipGetLastError() == hipSuccess ? RFQ_PROBE_OK : RFQ_PROBE_ERR_HIP;
}

}  // namespace

extern "C" {

int rfq_probe_mfma_ceiling(const uint8_t* a_codes, size_t a_bytes, const uint8_t* b_codes, size_t b_bytes,
                           int workgroups, int iters, uint64_t* stamps, float* sink, void* stream) {
  return launch_probe(a_codes, a_bytes, b_codes, b_bytes, 4, workgroups, iters, stamps, sink,
                      static_cast<hipStream_t>(stream));
}

int rfq_probe_mfma_ceiling_e4m3(const uint8_t* a_codes, size_t a_bytes, const uint8_t* b_codes, size_t b_bytes,
                                int workgroups, int iters, uint64_t* stamps, float* sink, void* stream) {
  return launch_probe(a_codes, a_bytes, b_codes, b_bytes, 8, workgroups, iters, stamps, sink,
                      static_cast<hipStream_t>(stream));
}

}  // extern "C"
