/*
 * rfq.h - C ABI of librfq: Residual Fallback Quantization (RFQ) W4A4 linear
 * layer on AMD Instinct MI355X (gfx950).
 *
 * The method ("Activation Outliers Matter: Robust Recovery for Quantized
 * Multimodal LLMs", arXiv 2608.26581, Abstract and §1): an activation X is
 * quantized to MXFP4; the full quantization error R = X - deq(Q(X)) is
 * quantized to MXFP4 by a second low-bit path; during the GEMM the
 * residual's product with the FP4 weight is accumulated with the primary
 * product:  Y = Q(X) Wq^T + Q(R) Wq^T, both in one fp32 accumulator.
 *
 * Number formats (named on those pages, defined in the OCP Microscaling
 * Formats v1.0 specification, which this library follows):
 *   - a block is 32 consecutive elements of a row along K;
 *   - shared scale: E8M0 code c, value 2^(c-127); c = 255 is NaN;
 *     exponent se = max(floor(log2(amax)) - 2, -127), amax = max |x| of the
 *     block (amax == 0 gives se = -127);
 *   - element: E2M1 code, bit 3 sign, magnitudes {0,.5,1,1.5,2,3,4,6};
 *     x / 2^se is rounded to nearest, ties to even, saturating at +-6; the
 *     sign bit of x is kept (so -0.0 and negatives rounding to zero give 8);
 *   - a block containing NaN or +-Inf gets scale 255 and element codes 0,
 *     and so does its residual block.
 *
 * Data layout (all row-major, all DEVICE memory unless stated):
 *   - X: [rows, K] bfloat16 or float32 (x_dtype), row stride ldx elements
 *     (ldx >= K);
 *   - codes: [rows, K/2] bytes, dense; byte j of a row holds element 2j in
 *     its low nibble and element 2j+1 in its high nibble;
 *   - scales: [rows, K/32] bytes, dense, one E8M0 code per block;
 *   - the weight W [N, K] is quantized along K with rfq_quantize_mxfp4
 *     (codes [N, K/2], scales [N, K/32]);
 *   - Y: [M, N] float32 or bfloat16 (rounded to nearest even), row stride
 *     ldy elements (ldy >= N).
 *
 * Conventions shared by every entry point:
 *   - Ownership: the caller owns and allocates every buffer; the library
 *     allocates no device or pinned memory and keeps no state between calls
 *     besides a thread-local error string.
 *   - Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL is the
 *     null stream) on the current HIP device; buffers must stay alive until
 *     the stream has run it. Calls are thread-safe.
 *   - Errors: arguments are checked on the host before anything is enqueued;
 *     on a non-OK status nothing was launched and no output was written.
 *     rfq_last_error_detail() then names the failing argument. A failed launch
 *     returns RFQ_ERR_HIP with the HIP error text in the detail string.
 *   - Shapes: rows/M, N may be 0 (then nothing is done and RFQ_OK returned);
 *     K must be positive, a multiple of 32 and at most 2^22; rows, M and N
 *     below 2^31; rows * K, M * K and N * K below 2^37; for a GEMM output
 *     Y [M, N], M * N below 2^40.
 *   - Alignment: X and every code pointer 16-byte aligned, and ldx a
 *     multiple of 8 elements for bf16 X or 4 for fp32 X (so every X row
 *     starts 16-byte aligned); Y
 *     aligned to its element size; scale pointers need no alignment; the
 *     workspace 256-byte aligned.
 */
#ifndef RFQ_H_
#define RFQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RFQ_ABI_VERSION 8

typedef enum rfq_status {
  RFQ_OK = 0,
  RFQ_ERR_NULL_POINTER = 1,        /* a required pointer is NULL            */
  RFQ_ERR_INVALID_SHAPE = 2,       /* negative dim, K <= 0, K % 32, too big */
  RFQ_ERR_INVALID_STRIDE = 3,      /* ldx < K, ldx % 8 != 0, ldy < N        */
  RFQ_ERR_MISALIGNED = 4,          /* pointer alignment (see above)         */
  RFQ_ERR_UNSUPPORTED_DTYPE = 5,   /* dtype code not accepted by this call  */
  RFQ_ERR_WORKSPACE_TOO_SMALL = 6, /* workspace_bytes below the size needed */
  RFQ_ERR_HIP = 7                  /* HIP launch or runtime failure         */
} rfq_status_t;

typedef enum rfq_dtype {
  RFQ_DTYPE_BF16 = 0,
  RFQ_DTYPE_FP32 = 1
} rfq_dtype_t;

/* A hipStream_t passed as an opaque pointer; NULL means the null stream. */
typedef void* rfq_stream_t;

/*
 * rfq_quantize_mxfp4 - MXFP4 quantization of a bf16 matrix along K.
 * (The primary low-bit path of the pages' §1; also quantizes the weight.)
 *   x       [rows, K] bf16 or fp32, stride ldx elements. (in, device)
 *   codes   [rows, K/2] bytes, dense.                  (out, device)
 *   scales  [rows, K/32] bytes, dense.                 (out, device)
 *   x_dtype RFQ_DTYPE_BF16 or RFQ_DTYPE_FP32.
 */
rfq_status_t rfq_quantize_mxfp4(const void* x, int x_dtype, int64_t rows, int64_t K, int64_t ldx,
                                uint8_t* codes, uint8_t* scales, rfq_stream_t stream);

/*
 * rfq_residual_quantize - RFQ activation encoding in one pass over X:
 * Q(X), then R = X - deq(Q(X)) exactly in fp32 (never rounded), then Q(R).
 * (The pages' §1: the full quantization error, with no threshold, rebuilt by a
 * second low-bit quantization path.)
 *   x        [M, K] bf16 or fp32, stride ldx.          (in, device)
 *   qx_codes [M, K/2], qx_scales [M, K/32]: Q(X).      (out, device)
 *   qr_codes [M, K/2], qr_scales [M, K/32]: Q(R).      (out, device)
 *   x_dtype RFQ_DTYPE_BF16 or RFQ_DTYPE_FP32.
 * For fp32 X the residual is still exact in fp32: |R| is at most half an
 * E2M1 step of the block scale, so X - deq(Q(X)) drops no bits.
 */
rfq_status_t rfq_residual_quantize(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                                   uint8_t* qx_codes, uint8_t* qx_scales,
                                   uint8_t* qr_codes, uint8_t* qr_scales, rfq_stream_t stream);

/*
 * Block-Hadamard rotation before quantization ("大模型量化中的双线性尾部问题与
 * QuaRot正交旋转解决方案" §3, QuaRot: an orthogonal +-1 matrix applied online
 * to the activation right before it is quantized and folded into the
 * weight, so the layer's product is unchanged). H is the unnormalised
 * 32 x 32 Sylvester Hadamard matrix (H[i][j] = (-1)^popcount(i & j)),
 * applied to every 32-element block along K, i.e. to every MX block; H H^T =
 * 32 I, so with X H on the activation side and W H / 32 on the weight side
 * rfq_gemm_w4a4 returns (X H)(W H / 32)^T = X W^T up to quantization.
 * Each value of X H (of W H / 32) is the exact block sum rounded once to
 * fp32, ties to even, a zero sum being +0; the codes are decided on those
 * fp32 values. The sums are exact when a block's terms lie within 53 bits
 * of each other (nonzero bf16 values within 40 binades, fp32 within 24);
 * in wider blocks an fp64 partial sum can round, and the result can then
 * differ from the exact one (no bound is claimed there).
 *
 * rfq_rotate_residual_quantize - the RFQ encoding of X H: Q(X H), then
 *   R = X H - deq(Q(X H)) (exact in fp32), then Q(R). Arguments, layouts and
 *   errors as rfq_residual_quantize.
 * rfq_rotate_quantize_weight - MXFP4 codes and scales of W H / 32 (the 1/32,
 *   a power of two, is exact). Arguments as rfq_quantize_mxfp4 (w [N, K],
 *   stride ldw).
 */
rfq_status_t rfq_rotate_residual_quantize(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                                          uint8_t* qx_codes, uint8_t* qx_scales,
                                          uint8_t* qr_codes, uint8_t* qr_scales, rfq_stream_t stream);
rfq_status_t rfq_rotate_quantize_weight(const void* w, int w_dtype, int64_t N, int64_t K, int64_t ldw,
                                        uint8_t* codes, uint8_t* scales, rfq_stream_t stream);

/*
 * The same two passes with a 64-point Hadamard H64 (the page's per-head
 * rotation size; Sylvester order, H64[i][j] = (-1)^popcount(i & j)) applied
 * to every 64 elements along K, i.e. to each pair of adjacent MX blocks:
 * X H64 with the residual pass, and W H64 / 64 for the weight (H64 H64^T =
 * 64 I, so rfq_gemm_w4a4 again returns X W^T up to quantization). Each
 * value is the exact 64-term sum (over 64 for the weight) rounded once to
 * fp32, a zero sum being +0; the sums are exact when a block's terms lie
 * within 53 bits of each other (nonzero bf16 values within 39 binades, fp32
 * within 23). K must be a multiple of 64 (RFQ_ERR_INVALID_SHAPE otherwise);
 * arguments, layouts and other errors as the 32-point calls. Quantization
 * blocks stay 32 elements.
 */
rfq_status_t rfq_rotate64_residual_quantize(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                                            uint8_t* qx_codes, uint8_t* qx_scales,
                                            uint8_t* qr_codes, uint8_t* qr_scales, rfq_stream_t stream);
rfq_status_t rfq_rotate64_quantize_weight(const void* w, int w_dtype, int64_t N, int64_t K, int64_t ldw,
                                          uint8_t* codes, uint8_t* scales, rfq_stream_t stream);

/*
 * rfq_gemm_w4a4 - block-scaled FP4 GEMM, K-doubled for RFQ:
 *   Y[m, n] = sum_k deq(QX)[m,k] deq(W)[n,k] + deq(QR)[m,k] deq(W)[n,k]
 * accumulated in one fp32 accumulator per output (the pages' §1
 * contributions: the residual is multiplied during the GEMM and its
 * contribution accumulated). With qr_codes == qr_scales == NULL the residual
 * term is skipped: plain W4A4.
 *   qx_codes/qx_scales [M, K/2]/[M, K/32], qr_* likewise (or both NULL),
 *   w_codes/w_scales [N, K/2]/[N, K/32]                 (in, device)
 *   y [M, N], y_dtype RFQ_DTYPE_FP32 or RFQ_DTYPE_BF16, stride ldy (out, device)
 * Scales of 255 (NaN) give NaN outputs; every other input gives finite
 * outputs except on fp32 overflow.
 */
rfq_status_t rfq_gemm_w4a4(const uint8_t* qx_codes, const uint8_t* qx_scales,
                           const uint8_t* qr_codes, const uint8_t* qr_scales,
                           const uint8_t* w_codes, const uint8_t* w_scales,
                           int64_t M, int64_t N, int64_t K,
                           void* y, int y_dtype, int64_t ldy, rfq_stream_t stream);

/*
 * MXFP8 variants. The pages ("Activation Outliers Matter", Abstract and §1)
 * study MXFP8 beside MXFP4 and find it close to lossless; they name it
 * without defining it. This library follows OCP MX v1.0 MXFP8 with E4M3
 * elements:
 *   - element: E4M3 code, bit 7 sign, 4 exponent bits (bias 7), 3 mantissa
 *     bits, subnormals at exponent 0, S.1111.111 is NaN, no infinities;
 *     largest normal 448;
 *   - shared scale: E8M0 as above with se = max(floor(log2(amax)) - 8, -127);
 *   - x / 2^se is rounded to nearest, ties to even, saturating at +-448; the
 *     sign bit of x is kept; a block holding NaN or +-Inf gets scale 255 and
 *     codes 0;
 *   - layout: codes [rows, K] bytes, dense, byte k = element k; scales
 *     [rows, K/32] as for MXFP4.
 * The weight stays MXFP4 (rfq_quantize_mxfp4) in both GEMM variants.
 *
 * rfq_quantize_mxfp8 - MXFP8 quantization of a bf16 or fp32 matrix along K.
 *   Arguments as rfq_quantize_mxfp4; codes [rows, K] bytes (out, device).
 *
 * rfq_residual_quantize_mxfp8 - RFQ with an MXFP8 second path: Q(X) in
 *   MXFP4, R = X - deq(Q(X)) exactly in fp32, Q(R) in MXFP8.
 *   qx_codes [M, K/2], qx_scales [M, K/32]: Q(X), MXFP4.  (out, device)
 *   qr_codes [M, K],   qr_scales [M, K/32]: Q(R), MXFP8.  (out, device)
 *   Other arguments as rfq_residual_quantize.
 *
 * rfq_gemm_w4a8 - Y = deq(QX8) deq(W)^T for MXFP8 activation codes
 *   qx_codes [M, K] / qx_scales [M, K/32] and the MXFP4 weight; fp32
 *   accumulation. Other arguments and errors as rfq_gemm_w4a4.
 *
 * rfq_gemm_w4a4_mxfp8_residual - the RFQ GEMM with an MXFP8 residual term:
 *   Y = deq(QX) deq(W)^T + deq(QR8) deq(W)^T in one fp32 accumulator, for
 *   QX MXFP4 ([M, K/2] codes) and QR8 MXFP8 ([M, K] codes) as written by
 *   rfq_residual_quantize_mxfp8. Other arguments and errors as rfq_gemm_w4a4
 *   (qr_codes/qr_scales must not be NULL).
 */
rfq_status_t rfq_quantize_mxfp8(const void* x, int x_dtype, int64_t rows, int64_t K, int64_t ldx,
                                uint8_t* codes, uint8_t* scales, rfq_stream_t stream);
rfq_status_t rfq_residual_quantize_mxfp8(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                                         uint8_t* qx_codes, uint8_t* qx_scales,
                                         uint8_t* qr_codes, uint8_t* qr_scales, rfq_stream_t stream);
rfq_status_t rfq_gemm_w4a8(const uint8_t* qx_codes, const uint8_t* qx_scales,
                           const uint8_t* w_codes, const uint8_t* w_scales,
                           int64_t M, int64_t N, int64_t K,
                           void* y, int y_dtype, int64_t ldy, rfq_stream_t stream);
rfq_status_t rfq_gemm_w4a4_mxfp8_residual(const uint8_t* qx_codes, const uint8_t* qx_scales,
                                          const uint8_t* qr_codes, const uint8_t* qr_scales,
                                          const uint8_t* w_codes, const uint8_t* w_scales,
                                          int64_t M, int64_t N, int64_t K,
                                          void* y, int y_dtype, int64_t ldy, rfq_stream_t stream);

/*
 * Straight-through backward pass. The pages ("Activation Outliers Matter",
 * §1) present RFQ as training-aware error modelling for low-bit training
 * but do not write the backward pass out. With Q passing gradients through
 * unchanged, the gradients of the forward product Y = Xh Wd^T
 * (Xh = deq Q(X) + deq Q(R), Wd = deq Q(W)) are
 *   dX = dY Wd                                      (contraction over N)
 *   dW = dY^T Xh = dY^T deq Q(X) + dY^T deq Q(R)     (contraction over M)
 * (the residual adds no gradient path to X: dR/dX = I - I = 0). Both are
 * computed from the decoded operands, exactly, with fp32 accumulation (bf16
 * matrix instructions; every product is exact in fp32).
 *
 * rfq_backward_dx - dX [M, K] from dY [M, N] (bf16, dense: lddy == N, N a
 *   positive multiple of 8 and at most 2^22) and the weight's MXFP4 codes and
 *   scales (as rfq_quantize_mxfp4 wrote them). dx: fp32 or bf16, stride
 *   lddx >= K. workspace: at least rfq_backward_dx_workspace_size(N, K)
 *   bytes, 256-byte aligned, device; on return it holds deq(Wq)^T [K, N]
 *   bf16. M == 0 is a no-op.
 * rfq_backward_dw - dW [N, K] from dY [M, N] (bf16, stride lddy >= N; M
 *   positive and at most 2^22) and the forward's Q(X) and Q(R) codes and
 *   scales (as rfq_residual_quantize wrote them). dw: fp32 or bf16, stride
 *   lddw >= K. workspace: at least rfq_backward_dw_workspace_size(M, N, K)
 *   bytes, 256-byte aligned, device; on return it holds dY^T [N, Mp],
 *   deq Q(X)^T [K, Mp] and deq Q(R)^T [K, Mp] bf16 (Mp = M rounded up to a
 *   multiple of 8, columns past M zero), each region rounded up to 256
 *   bytes. N == 0 is a no-op.
 * Decoded values must lie within bf16's range, which holds for scale codes
 * up to 252 (every quantization of bf16 data). Errors as for the other
 * entry points.
 */
size_t rfq_backward_dx_workspace_size(int64_t N, int64_t K);
size_t rfq_backward_dw_workspace_size(int64_t M, int64_t N, int64_t K);
rfq_status_t rfq_backward_dx(const void* dy, int dy_dtype, int64_t M, int64_t N, int64_t lddy,
                             const uint8_t* w_codes, const uint8_t* w_scales, int64_t K,
                             void* dx, int dx_dtype, int64_t lddx,
                             void* workspace, size_t workspace_bytes, rfq_stream_t stream);
rfq_status_t rfq_backward_dw(const void* dy, int dy_dtype, int64_t M, int64_t N, int64_t lddy,
                             const uint8_t* qx_codes, const uint8_t* qx_scales,
                             const uint8_t* qr_codes, const uint8_t* qr_scales, int64_t K,
                             void* dw, int dw_dtype, int64_t lddw,
                             void* workspace, size_t workspace_bytes, rfq_stream_t stream);

/* Bytes of workspace rfq_linear needs for an [M, K] activation: Q(X) and
 * Q(R) codes and scales, each region rounded up to 256 bytes. Host only;
 * returns 0 for invalid shapes. */
size_t rfq_linear_workspace_size(int64_t M, int64_t K);

/*
 * rfq_linear - the whole RFQ W4A4 linear layer: rfq_residual_quantize into
 * the workspace, then rfq_gemm_w4a4, both on `stream`.
 *   x [M, K] bf16 or fp32 stride ldx; w_codes/w_scales: W quantized by
 *   rfq_quantize_mxfp4; y [M, N] fp32 or bf16 stride ldy;
 *   workspace: at least rfq_linear_workspace_size(M, K) bytes of device
 *   memory, 256-byte aligned, owned by the caller; its contents on return
 *   are Q(X) codes | Q(X) scales | Q(R) codes | Q(R) scales at the offsets
 *   given by the size rule above.
 */
rfq_status_t rfq_linear(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                        const uint8_t* w_codes, const uint8_t* w_scales, int64_t N,
                        void* y, int y_dtype, int64_t ldy,
                        void* workspace, size_t workspace_bytes, rfq_stream_t stream);

/*
 * rfq_linear_fused - the whole layer with the quantization inside the GEMM
 * ("Activation Outliers Matter", §1 contributions: the residual is
 * re-quantized during the GEMM and its contribution accumulated). The GEMM
 * reads bf16 X tiles and, for each K stage of each output tile, forms Q(X),
 * R = X - deq(Q(X)) and Q(R) itself (the same encoding as
 * rfq_residual_quantize) in registers and LDS; Q(X) and Q(R) are never
 * written to memory and no workspace is needed. Y is the same as
 * rfq_linear's, bit for bit: same codes, same accumulation order.
 *   x [M, K] bf16 only (x_dtype RFQ_DTYPE_BF16), row stride ldx elements,
 *     ldx < 2^24;
 *   K a multiple of 512 (whole scale groups of the weight);
 *   other arguments as rfq_linear.
 * Errors as rfq_linear, plus RFQ_ERR_UNSUPPORTED_DTYPE for fp32 X and
 * RFQ_ERR_INVALID_SHAPE for K % 512 != 0, RFQ_ERR_INVALID_STRIDE for
 * ldx >= 2^24.
 */
rfq_status_t rfq_linear_fused(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                              const uint8_t* w_codes, const uint8_t* w_scales, int64_t N,
                              void* y, int y_dtype, int64_t ldy, rfq_stream_t stream);

/*
 * rfq_linear_noalloc - rfq_linear for callers that cannot allocate memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. The same layer, arguments, layout and errors as rfq_linear, but
 * with no workspace argument: Q(X) and Q(R) are staged in a device array that
 * the library owns, rfq_linear_noalloc_max_workspace() bytes (64 MiB) on each
 * GPU it runs on, held until the process ends. The call allocates nothing.
 *   - A shape whose rfq_linear_workspace_size(M, K) exceeds that size is
 *     rejected with RFQ_ERR_WORKSPACE_TOO_SMALL before anything is launched
 *     (K = 5120 allows M up to 12 k rows).
 *   - Every call on one GPU uses the same array, which keeps the last call's
 *     contents (the quantize pass rewrites every byte the GEMM reads, so no
 *     call depends on what an earlier one left). Calls that overlap on one
 *     GPU, on streams not ordered against each other, race on it and give
 *     undefined Y.
 *   - The first call on a device looks up the array's device address there
 *     (with that device current); a failure returns RFQ_ERR_HIP.
 */
rfq_status_t rfq_linear_noalloc(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                                const uint8_t* w_codes, const uint8_t* w_scales, int64_t N,
                                void* y, int y_dtype, int64_t ldy, rfq_stream_t stream);

/* Bytes of the array rfq_linear_noalloc stages in (the largest
 * rfq_linear_workspace_size it accepts). Host only. */
size_t rfq_linear_noalloc_max_workspace(void);

/* Static English text for a status code. Host only. */
const char* rfq_status_string(rfq_status_t status);

/* Thread-local text describing the last non-OK status returned on this
 * thread ("" if none). Host only; valid until the next call on the thread. */
const char* rfq_last_error_detail(void);

/* RFQ_ABI_VERSION of the built library. */
int rfq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RFQ_H_ */
