/*
 * rfq_probe.h - benchmark-only measurement probe, built into its own
 * library (bench_probe/librfqprobe.so) and loaded only by bench.py; it is not
 * part of librfq.so or of the RFQ layer.
 *
 * The FP4 GEMM on MI355X is limited by the chip's power budget before the
 * MFMA issue rate: with real operand data the shader clock drops well below
 * its 2.4 GHz peak. This probe measures that ceiling directly, as the rate of
 * a loop that does nothing but issue the GEMM's instruction
 * (v_mfma_scale_f32_16x16x128_f8f6f4 with both operands FP4, the form the
 * E2M1 x E2M1 GEMMs use) on operand bytes the caller supplies, with no
 * memory traffic in the loop. The GEMM's throughput is then reported
 * against both the datasheet peak and this ceiling.
 */
#ifndef RFQ_PROBE_H_
#define RFQ_PROBE_H_

#include <stddef.h>
#include <stdint.h>


#ifdef __cplusplus
extern "C" {
#endif

/* Return codes of the probe calls. */
enum { RFQ_PROBE_OK = 0, RFQ_PROBE_ERR_ARGUMENT = 1, RFQ_PROBE_ERR_HIP = 2 };

/*
 * rfq_probe_mfma_ceiling - launch `workgroups` workgroups of 512 threads
 * (two waves per SIMD, as the GEMM runs; launch one per CU), each running
 * `iters` iterations of 64 FP4 scaled 16 x 16 x 128 MFMAs per wave over 32
 * independent accumulators. Each lane loads four 16-byte operands from each buffer once,
 * before the loop, at consecutive 16-byte positions taken modulo the buffer
 * size, so any buffer of at least 16 bytes serves.
 *   a_codes, a_bytes: bytes of the first operand (e.g. Q(X) and Q(R) codes);
 *   b_codes, b_bytes: bytes of the second operand (e.g. W codes); both
 *     device pointers 16-byte aligned, sizes multiples of 16, at least 16;
 *   stamps: device buffer of 2 * workgroups uint64 values (out): per
 *     workgroup the shader-clock cycles and the 100 MHz constant-clock ticks
 *     that its loop took;
 *   sink: device buffer of 512 * workgroups floats (out): accumulator sums,
 *     written so that the loop is not optimised away.
 * Flops per call: 2 * 32 * 32 * 64 * 32 * 8 * iters * workgroups (8 waves of
 * 64 MFMAs of 2 * 16 * 16 * 128 flops per iteration). Asynchronous on
 * `stream` (a hipStream_t; NULL is the null stream). Returns
 * RFQ_PROBE_ERR_ARGUMENT for a NULL or misaligned buffer, a size that is not
 * a multiple of 16 in [16, 2^36), workgroups outside [1, 65536] or iters <= 0
 * (nothing launched), RFQ_PROBE_ERR_HIP if the launch failed.
 */
int rfq_probe_mfma_ceiling(const uint8_t* a_codes, size_t a_bytes, const uint8_t* b_codes, size_t b_bytes,
                           int workgroups, int iters, uint64_t* stamps, float* sink, void* stream);

/*
 * rfq_probe_mfma_ceiling_e4m3 - the same measurement for the instruction of
 * the W4A8 GEMM, v_mfma_scale_f32_16x16x128_f8f6f4 with the MXFP4 weight
 * first and the E4M3 activation second (twice the cycles of the E2M1 x E2M1
 * form for the same flops): 64 MFMAs per wave per iteration over 32
 * accumulators. Each lane loads eight 16-byte pieces of b_codes (two per
 * operand, 32 bytes) at consecutive positions modulo its size; all else as
 * rfq_probe_mfma_ceiling, including the flop count per call.
 */
int rfq_probe_mfma_ceiling_e4m3(const uint8_t* a_codes, size_t a_bytes, const uint8_t* b_codes, size_t b_bytes,
                                int workgroups, int iters, uint64_t* stamps, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RFQ_PROBE_H_ */
