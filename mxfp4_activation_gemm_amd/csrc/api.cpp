// C ABI of librfq (declared in include/rfq.h): argument validation on the
// host, then stream-ordered launches of the HIP kernels. Nothing here
// allocates memory; every check runs before anything is enqueued.

#include <stdarg.h>
#include <stdio.h>

#include <string>

#include "kernels.h"
#include "rfq.h"

namespace {

thread_local std::string g_detail;

constexpr int64_t kMaxK = int64_t(1) << 22;
constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxElems = int64_t(1) << 37;
constexpr int64_t kMaxOutputs = int64_t(1) << 40;

rfq_status_t fail(rfq_status_t st, const char* fmt, ...) {
  char buf[256];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_detail = buf;
  return st;
}

rfq_status_t ok() {
  g_detail.clear();
  return RFQ_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shape rule shared by every entry point: rows in [0, 2^31), K in (0, 2^22]
// and a multiple of 32, rows * K < 2^37.
rfq_status_t check_rows_k(int64_t rows, int64_t K, const char* rname) {
  if (rows < 0 || rows > kMaxRows) return fail(RFQ_ERR_INVALID_SHAPE, "%s = %lld out of range [0, 2^31)", rname, (long long)rows);
  if (K <= 0 || K % 32 != 0 || K > kMaxK)
    return fail(RFQ_ERR_INVALID_SHAPE, "K = %lld must be positive, a multiple of 32 and at most 2^22", (long long)K);
  if (rows * K >= kMaxElems) return fail(RFQ_ERR_INVALID_SHAPE, "%s * K = %lld exceeds 2^37", rname, (long long)(rows * K));
  return RFQ_OK;
}

// The 64-point rotation spans two MX blocks: K a multiple of 64.
rfq_status_t check_k64(int64_t K) {
  if (K % 64 != 0)
    return fail(RFQ_ERR_INVALID_SHAPE, "K = %lld must be a multiple of 64 for the 64-point rotation", (long long)K);
  return RFQ_OK;
}

// A GEMM output Y [M, N] holds fewer than 2^40 elements (the tile count
// stays in 32-bit arithmetic).
rfq_status_t check_mn(int64_t M, int64_t N) {
  if (M > 0 && N > 0 && M > (kMaxOutputs - 1) / N)
    return fail(RFQ_ERR_INVALID_SHAPE, "M * N = %lld x %lld reaches 2^40", (long long)M, (long long)N);
  return RFQ_OK;
}

rfq_status_t check_dtype(int x_dtype) {
  if (x_dtype != RFQ_DTYPE_BF16 && x_dtype != RFQ_DTYPE_FP32)
    return fail(RFQ_ERR_UNSUPPORTED_DTYPE, "x_dtype %d: must be RFQ_DTYPE_BF16 or RFQ_DTYPE_FP32", x_dtype);
  return RFQ_OK;
}

// X rows must start 16-byte aligned: ldx a multiple of 8 elements (bf16) or 4 (fp32).
rfq_status_t check_x(const void* x, int x_dtype, int64_t K, int64_t ldx) {
  if (rfq_status_t st = check_dtype(x_dtype); st != RFQ_OK) return st;
  const int64_t mult = x_dtype == RFQ_DTYPE_BF16 ? 8 : 4;
  if (ldx < K || ldx % mult != 0)
    return fail(RFQ_ERR_INVALID_STRIDE, "ldx = %lld must be >= K = %lld and a multiple of %lld", (long long)ldx,
                (long long)K, (long long)mult);
  if (x == nullptr) return fail(RFQ_ERR_NULL_POINTER, "x is NULL");
  if (!aligned(x, 16)) return fail(RFQ_ERR_MISALIGNED, "x must be 16-byte aligned");
  return RFQ_OK;
}

rfq_status_t check_codes(const void* codes, const void* scales, const char* name) {
  if (codes == nullptr || scales == nullptr) return fail(RFQ_ERR_NULL_POINTER, "%s codes/scales pointer is NULL", name);
  if (!aligned(codes, 16)) return fail(RFQ_ERR_MISALIGNED, "%s codes must be 16-byte aligned", name);
  return RFQ_OK;
}

rfq_status_t check_y(const void* y, int y_dtype, int64_t N, int64_t ldy) {
  if (y_dtype != RFQ_DTYPE_FP32 && y_dtype != RFQ_DTYPE_BF16)
    return fail(RFQ_ERR_UNSUPPORTED_DTYPE, "y_dtype %d: must be RFQ_DTYPE_FP32 or RFQ_DTYPE_BF16", y_dtype);
  if (ldy < N) return fail(RFQ_ERR_INVALID_STRIDE, "ldy = %lld must be >= N = %lld", (long long)ldy, (long long)N);
  if (y == nullptr) return fail(RFQ_ERR_NULL_POINTER, "y is NULL");
  if (!aligned(y, y_dtype == RFQ_DTYPE_FP32 ? 4 : 2)) return fail(RFQ_ERR_MISALIGNED, "y must be aligned to its element size");
  return RFQ_OK;
}

rfq_status_t launched(hipError_t e) {
  if (e != hipSuccess) return fail(RFQ_ERR_HIP, "HIP: %s", hipGetErrorString(e));
  return ok();
}

size_t round256(size_t b) { return (b + 255) & ~size_t(255); }

#define RFQ_TRY(expr)                     \
  do {                                    \
    rfq_status_t st_ = (expr);            \
    if (st_ != RFQ_OK) return st_;        \
  } while (0)

}  // namespace

namespace {

rfq_status_t quantize_common(const void* x, int x_dtype, int64_t rows, int64_t K, int64_t ldx, uint8_t* codes,
                             uint8_t* scales, int rotate, int fmt, rfq_stream_t stream) {
  RFQ_TRY(check_rows_k(rows, K, "rows"));
  RFQ_TRY(check_dtype(x_dtype));
  if (rows == 0) return ok();
  RFQ_TRY(check_x(x, x_dtype, K, ldx));
  RFQ_TRY(check_codes(codes, scales, "output"));
  return launched(rfq::launch_quantize(x, x_dtype == RFQ_DTYPE_FP32, rotate, fmt, 0, rows, K, ldx, codes, scales,
                                       nullptr, nullptr, static_cast<hipStream_t>(stream)));
}

rfq_status_t residual_common(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, uint8_t* qx_codes,
                             uint8_t* qx_scales, uint8_t* qr_codes, uint8_t* qr_scales, int rotate, int r_fmt,
                             rfq_stream_t stream) {
  RFQ_TRY(check_rows_k(M, K, "M"));
  RFQ_TRY(check_dtype(x_dtype));
  if (M == 0) return ok();
  RFQ_TRY(check_x(x, x_dtype, K, ldx));
  RFQ_TRY(check_codes(qx_codes, qx_scales, "Q(X)"));
  RFQ_TRY(check_codes(qr_codes, qr_scales, "Q(R)"));
  return launched(rfq::launch_quantize(x, x_dtype == RFQ_DTYPE_FP32, rotate, 4, r_fmt, M, K, ldx, qx_codes, qx_scales,
                                       qr_codes, qr_scales, static_cast<hipStream_t>(stream)));
}

// Shared checks and launch of the GEMM entry points: activation formats
// x_fmt / r_fmt (4: MXFP4, 8: MXFP8; r_fmt 0 without a residual term).
rfq_status_t gemm_common(int x_fmt, int r_fmt, const uint8_t* qx_codes, const uint8_t* qx_scales,
                         const uint8_t* qr_codes, const uint8_t* qr_scales, const uint8_t* w_codes,
                         const uint8_t* w_scales, int64_t M, int64_t N, int64_t K, void* y, int y_dtype, int64_t ldy,
                         rfq_stream_t stream) {
  RFQ_TRY(check_rows_k(M, K, "M"));
  RFQ_TRY(check_rows_k(N, K, "N"));
  RFQ_TRY(check_mn(M, N));
  if (y_dtype != RFQ_DTYPE_FP32 && y_dtype != RFQ_DTYPE_BF16)
    return fail(RFQ_ERR_UNSUPPORTED_DTYPE, "y_dtype %d: must be RFQ_DTYPE_FP32 or RFQ_DTYPE_BF16", y_dtype);
  if (M == 0 || N == 0) return ok();
  RFQ_TRY(check_codes(qx_codes, qx_scales, "Q(X)"));
  if (r_fmt != 0) RFQ_TRY(check_codes(qr_codes, qr_scales, "Q(R)"));
  RFQ_TRY(check_codes(w_codes, w_scales, "W"));
  RFQ_TRY(check_y(y, y_dtype, N, ldy));
  return launched(rfq::launch_gemm(x_fmt, r_fmt, qx_codes, qx_scales, r_fmt ? qr_codes : nullptr,
                                   r_fmt ? qr_scales : nullptr, w_codes, w_scales, M, N, K, y,
                                   y_dtype == RFQ_DTYPE_BF16, ldy, static_cast<hipStream_t>(stream)));
}

// Checks shared by the two linear entry points (everything but the workspace).
rfq_status_t check_linear(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, const uint8_t* w_codes,
                          const uint8_t* w_scales, int64_t N, const void* y, int y_dtype, int64_t ldy) {
  RFQ_TRY(check_rows_k(M, K, "M"));
  RFQ_TRY(check_rows_k(N, K, "N"));
  RFQ_TRY(check_mn(M, N));
  RFQ_TRY(check_dtype(x_dtype));
  if (y_dtype != RFQ_DTYPE_FP32 && y_dtype != RFQ_DTYPE_BF16)
    return fail(RFQ_ERR_UNSUPPORTED_DTYPE, "y_dtype %d: must be RFQ_DTYPE_FP32 or RFQ_DTYPE_BF16", y_dtype);
  if (M == 0 || N == 0) return RFQ_OK;
  RFQ_TRY(check_x(x, x_dtype, K, ldx));
  RFQ_TRY(check_codes(w_codes, w_scales, "W"));
  RFQ_TRY(check_y(y, y_dtype, N, ldy));
  return RFQ_OK;
}

// The layer's two launches with Q(X) | SX | Q(R) | SR staged at `ws` (the
// regions of rfq_linear_workspace_size); arguments already checked.
rfq_status_t linear_launch(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, const uint8_t* w_codes,
                           const uint8_t* w_scales, int64_t N, void* y, int y_dtype, int64_t ldy, uint8_t* ws,
                           rfq_stream_t stream) {
  const size_t codes = round256((size_t)(M * (K / 2))), scales = round256((size_t)(M * (K / 32)));
  uint8_t* qx = ws;
  uint8_t* sx = qx + codes;
  uint8_t* qr = sx + scales;
  uint8_t* sr = qr + codes;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = rfq::launch_quantize(x, x_dtype == RFQ_DTYPE_FP32, 0, 4, 4, M, K, ldx, qx, sx, qr, sr, s);
  if (e != hipSuccess) return launched(e);
  return launched(rfq::launch_gemm(4, 4, qx, sx, qr, sr, w_codes, w_scales, M, N, K, y, y_dtype == RFQ_DTYPE_BF16, ldy,
                                   s));
}

}  // namespace

extern "C" {

rfq_status_t rfq_quantize_mxfp4(const void* x, int x_dtype, int64_t rows, int64_t K, int64_t ldx,
                                uint8_t* codes, uint8_t* scales, rfq_stream_t stream) {
  return quantize_common(x, x_dtype, rows, K, ldx, codes, scales, 0, 4, stream);
}

rfq_status_t rfq_quantize_mxfp8(const void* x, int x_dtype, int64_t rows, int64_t K, int64_t ldx,
                                uint8_t* codes, uint8_t* scales, rfq_stream_t stream) {
  return quantize_common(x, x_dtype, rows, K, ldx, codes, scales, 0, 8, stream);
}

rfq_status_t rfq_residual_quantize(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                                   uint8_t* qx_codes, uint8_t* qx_scales,
                                   uint8_t* qr_codes, uint8_t* qr_scales, rfq_stream_t stream) {
  return residual_common(x, x_dtype, M, K, ldx, qx_codes, qx_scales, qr_codes, qr_scales, 0, 4, stream);
}

rfq_status_t rfq_residual_quantize_mxfp8(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                                         uint8_t* qx_codes, uint8_t* qx_scales,
                                         uint8_t* qr_codes, uint8_t* qr_scales, rfq_stream_t stream) {
  return residual_common(x, x_dtype, M, K, ldx, qx_codes, qx_scales, qr_codes, qr_scales, 0, 8, stream);
}

rfq_status_t rfq_rotate_residual_quantize(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                                          uint8_t* qx_codes, uint8_t* qx_scales,
                                          uint8_t* qr_codes, uint8_t* qr_scales, rfq_stream_t stream) {
  return residual_common(x, x_dtype, M, K, ldx, qx_codes, qx_scales, qr_codes, qr_scales, 1, 4, stream);
}

rfq_status_t rfq_rotate_quantize_weight(const void* w, int w_dtype, int64_t N, int64_t K, int64_t ldw,
                                        uint8_t* codes, uint8_t* scales, rfq_stream_t stream) {
  return quantize_common(w, w_dtype, N, K, ldw, codes, scales, 2, 4, stream);
}

rfq_status_t rfq_rotate64_residual_quantize(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                                            uint8_t* qx_codes, uint8_t* qx_scales,
                                            uint8_t* qr_codes, uint8_t* qr_scales, rfq_stream_t stream) {
  RFQ_TRY(check_rows_k(M, K, "M"));
  RFQ_TRY(check_k64(K));
  return residual_common(x, x_dtype, M, K, ldx, qx_codes, qx_scales, qr_codes, qr_scales, 3, 4, stream);
}

rfq_status_t rfq_rotate64_quantize_weight(const void* w, int w_dtype, int64_t N, int64_t K, int64_t ldw,
                                          uint8_t* codes, uint8_t* scales, rfq_stream_t stream) {
  RFQ_TRY(check_rows_k(N, K, "N"));
  RFQ_TRY(check_k64(K));
  return quantize_common(w, w_dtype, N, K, ldw, codes, scales, 4, 4, stream);
}

rfq_status_t rfq_gemm_w4a4(const uint8_t* qx_codes, const uint8_t* qx_scales,
                           const uint8_t* qr_codes, const uint8_t* qr_scales,
                           const uint8_t* w_codes, const uint8_t* w_scales,
                           int64_t M, int64_t N, int64_t K,
                           void* y, int y_dtype, int64_t ldy, rfq_stream_t stream) {
  if ((qr_codes == nullptr) != (qr_scales == nullptr))
    return fail(RFQ_ERR_NULL_POINTER, "Q(R) codes and scales must be both NULL (plain W4A4) or both set");
  return gemm_common(4, qr_codes != nullptr ? 4 : 0, qx_codes, qx_scales, qr_codes, qr_scales, w_codes, w_scales, M,
                     N, K, y, y_dtype, ldy, stream);
}

rfq_status_t rfq_gemm_w4a8(const uint8_t* qx_codes, const uint8_t* qx_scales,
                           const uint8_t* w_codes, const uint8_t* w_scales,
                           int64_t M, int64_t N, int64_t K,
                           void* y, int y_dtype, int64_t ldy, rfq_stream_t stream) {
  return gemm_common(8, 0, qx_codes, qx_scales, nullptr, nullptr, w_codes, w_scales, M, N, K, y, y_dtype, ldy, stream);
}

rfq_status_t rfq_gemm_w4a4_mxfp8_residual(const uint8_t* qx_codes, const uint8_t* qx_scales,
                                          const uint8_t* qr_codes, const uint8_t* qr_scales,
                                          const uint8_t* w_codes, const uint8_t* w_scales,
                                          int64_t M, int64_t N, int64_t K,
                                          void* y, int y_dtype, int64_t ldy, rfq_stream_t stream) {
  return gemm_common(4, 8, qx_codes, qx_scales, qr_codes, qr_scales, w_codes, w_scales, M, N, K, y, y_dtype, ldy,
                     stream);
}

size_t rfq_linear_workspace_size(int64_t M, int64_t K) {
  if (M < 0 || M > kMaxRows || K <= 0 || K % 32 != 0 || K > kMaxK || M * K >= kMaxElems) return 0;
  const size_t codes = round256((size_t)(M * (K / 2))), scales = round256((size_t)(M * (K / 32)));
  return 2 * (codes + scales);
}

rfq_status_t rfq_linear(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                        const uint8_t* w_codes, const uint8_t* w_scales, int64_t N,
                        void* y, int y_dtype, int64_t ldy,
                        void* workspace, size_t workspace_bytes, rfq_stream_t stream) {
  RFQ_TRY(check_linear(x, x_dtype, M, K, ldx, w_codes, w_scales, N, y, y_dtype, ldy));
  if (M == 0 || N == 0) return ok();
  if (workspace == nullptr) return fail(RFQ_ERR_NULL_POINTER, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(RFQ_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  const size_t need = rfq_linear_workspace_size(M, K);
  if (workspace_bytes < need)
    return fail(RFQ_ERR_WORKSPACE_TOO_SMALL, "workspace_bytes = %zu, need %zu", workspace_bytes, need);
  return linear_launch(x, x_dtype, M, K, ldx, w_codes, w_scales, N, y, y_dtype, ldy,
                       static_cast<uint8_t*>(workspace), stream);
}

rfq_status_t rfq_linear_fused(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                              const uint8_t* w_codes, const uint8_t* w_scales, int64_t N,
                              void* y, int y_dtype, int64_t ldy, rfq_stream_t stream) {
  RFQ_TRY(check_linear(x, x_dtype, M, K, ldx, w_codes, w_scales, N, y, y_dtype, ldy));
  if (x_dtype != RFQ_DTYPE_BF16)
    return fail(RFQ_ERR_UNSUPPORTED_DTYPE, "x_dtype %d: the in-GEMM quantization takes bf16 X only", x_dtype);
  if (K % 512 != 0)
    return fail(RFQ_ERR_INVALID_SHAPE, "K = %lld: the in-GEMM quantization needs K a multiple of 512", (long long)K);
  if (ldx >= (int64_t(1) << 24))
    return fail(RFQ_ERR_INVALID_STRIDE, "ldx = %lld: the in-GEMM quantization needs ldx < 2^24", (long long)ldx);
  if (M == 0 || N == 0) return ok();
  return launched(rfq::launch_gemm_fused(static_cast<const uint16_t*>(x), ldx, w_codes, w_scales, M, N, K, y,
                                         y_dtype == RFQ_DTYPE_BF16, ldy, static_cast<hipStream_t>(stream)));
}

size_t rfq_linear_noalloc_max_workspace(void) { return rfq::kNoallocScratchBytes; }

rfq_status_t rfq_linear_noalloc(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                                const uint8_t* w_codes, const uint8_t* w_scales, int64_t N,
                                void* y, int y_dtype, int64_t ldy, rfq_stream_t stream) {
  RFQ_TRY(check_linear(x, x_dtype, M, K, ldx, w_codes, w_scales, N, y, y_dtype, ldy));
  if (M == 0 || N == 0) return ok();
  const size_t need = rfq_linear_workspace_size(M, K);
  if (need > rfq::kNoallocScratchBytes)
    return fail(RFQ_ERR_WORKSPACE_TOO_SMALL,
                "M = %lld, K = %lld need %zu bytes of staging, beyond the %zu bytes of the allocation-free scratch",
                (long long)M, (long long)K, need, rfq::kNoallocScratchBytes);
  uint8_t* scratch = nullptr;
  if (hipError_t e = rfq::noalloc_scratch(&scratch); e != hipSuccess) return launched(e);
  return linear_launch(x, x_dtype, M, K, ldx, w_codes, w_scales, N, y, y_dtype, ldy, scratch, stream);
}

size_t rfq_backward_dx_workspace_size(int64_t N, int64_t K) {
  if (N <= 0 || N % 8 != 0 || N > kMaxK || K <= 0 || K % 32 != 0 || K > kMaxK) return 0;
  return round256((size_t)K * (size_t)N * 2);
}

size_t rfq_backward_dw_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || M > kMaxK || N <= 0 || N > kMaxRows || K <= 0 || K % 32 != 0 || K > kMaxK) return 0;
  const size_t mp = (size_t)((M + 7) / 8 * 8);
  return round256((size_t)N * mp * 2) + 2 * round256((size_t)K * mp * 2);
}

rfq_status_t rfq_backward_dx(const void* dy, int dy_dtype, int64_t M, int64_t N, int64_t lddy,
                             const uint8_t* w_codes, const uint8_t* w_scales, int64_t K,
                             void* dx, int dx_dtype, int64_t lddx,
                             void* workspace, size_t workspace_bytes, rfq_stream_t stream) {
  if (M < 0 || M > kMaxRows) return fail(RFQ_ERR_INVALID_SHAPE, "M = %lld out of range [0, 2^31)", (long long)M);
  if (N <= 0 || N % 8 != 0 || N > kMaxK)
    return fail(RFQ_ERR_INVALID_SHAPE, "N = %lld must be positive, a multiple of 8 and at most 2^22", (long long)N);
  RFQ_TRY(check_rows_k(M, K, "M"));
  RFQ_TRY(check_rows_k(N, K, "N"));
  if (dy_dtype != RFQ_DTYPE_BF16) return fail(RFQ_ERR_UNSUPPORTED_DTYPE, "dy_dtype %d: must be RFQ_DTYPE_BF16", dy_dtype);
  if (dx_dtype != RFQ_DTYPE_FP32 && dx_dtype != RFQ_DTYPE_BF16)
    return fail(RFQ_ERR_UNSUPPORTED_DTYPE, "dx_dtype %d: must be RFQ_DTYPE_FP32 or RFQ_DTYPE_BF16", dx_dtype);
  if (lddy != N) return fail(RFQ_ERR_INVALID_STRIDE, "lddy = %lld: dY must be dense (lddy == N)", (long long)lddy);
  if (M == 0) return ok();
  if (dy == nullptr) return fail(RFQ_ERR_NULL_POINTER, "dy is NULL");
  if (!aligned(dy, 16)) return fail(RFQ_ERR_MISALIGNED, "dy must be 16-byte aligned");
  RFQ_TRY(check_codes(w_codes, w_scales, "W"));
  RFQ_TRY(check_y(dx, dx_dtype, K, lddx));
  if (workspace == nullptr) return fail(RFQ_ERR_NULL_POINTER, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(RFQ_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  const size_t need = rfq_backward_dx_workspace_size(N, K);
  if (workspace_bytes < need)
    return fail(RFQ_ERR_WORKSPACE_TOO_SMALL, "workspace_bytes = %zu, need %zu", workspace_bytes, need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint16_t* wdt = static_cast<uint16_t*>(workspace);                      // deq(Wq)^T [K, N] bf16
  hipError_t e = rfq::launch_decode_transpose(w_codes, w_scales, N, K, wdt, N, s);
  if (e != hipSuccess) return launched(e);
  return launched(rfq::launch_gemm(16, 0, static_cast<const uint8_t*>(dy), nullptr, nullptr, nullptr,
                                   reinterpret_cast<const uint8_t*>(wdt), nullptr, M, K, 4 * N, dx,
                                   dx_dtype == RFQ_DTYPE_BF16, lddx, s));
}

rfq_status_t rfq_backward_dw(const void* dy, int dy_dtype, int64_t M, int64_t N, int64_t lddy,
                             const uint8_t* qx_codes, const uint8_t* qx_scales,
                             const uint8_t* qr_codes, const uint8_t* qr_scales, int64_t K,
                             void* dw, int dw_dtype, int64_t lddw,
                             void* workspace, size_t workspace_bytes, rfq_stream_t stream) {
  if (M <= 0 || M > kMaxK)
    return fail(RFQ_ERR_INVALID_SHAPE, "M = %lld must be positive and at most 2^22", (long long)M);
  if (N < 0 || N > kMaxRows) return fail(RFQ_ERR_INVALID_SHAPE, "N = %lld out of range [0, 2^31)", (long long)N);
  RFQ_TRY(check_rows_k(M, K, "M"));
  RFQ_TRY(check_rows_k(N, K, "N"));
  if (dy_dtype != RFQ_DTYPE_BF16) return fail(RFQ_ERR_UNSUPPORTED_DTYPE, "dy_dtype %d: must be RFQ_DTYPE_BF16", dy_dtype);
  if (dw_dtype != RFQ_DTYPE_FP32 && dw_dtype != RFQ_DTYPE_BF16)
    return fail(RFQ_ERR_UNSUPPORTED_DTYPE, "dw_dtype %d: must be RFQ_DTYPE_FP32 or RFQ_DTYPE_BF16", dw_dtype);
  if (lddy < N) return fail(RFQ_ERR_INVALID_STRIDE, "lddy = %lld must be >= N = %lld", (long long)lddy, (long long)N);
  if (N == 0) return ok();
  if (dy == nullptr) return fail(RFQ_ERR_NULL_POINTER, "dy is NULL");
  if (!aligned(dy, 2)) return fail(RFQ_ERR_MISALIGNED, "dy must be 2-byte aligned");
  RFQ_TRY(check_codes(qx_codes, qx_scales, "Q(X)"));
  RFQ_TRY(check_codes(qr_codes, qr_scales, "Q(R)"));
  RFQ_TRY(check_y(dw, dw_dtype, K, lddw));
  if (workspace == nullptr) return fail(RFQ_ERR_NULL_POINTER, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(RFQ_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  const size_t need = rfq_backward_dw_workspace_size(M, N, K);
  if (workspace_bytes < need)
    return fail(RFQ_ERR_WORKSPACE_TOO_SMALL, "workspace_bytes = %zu, need %zu", workspace_bytes, need);
  const int64_t mp = (M + 7) / 8 * 8;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint16_t* dyt = reinterpret_cast<uint16_t*>(ws);                                          // dY^T [N, Mp]
  uint16_t* xqt = reinterpret_cast<uint16_t*>(ws + round256((size_t)N * mp * 2));            // deq Q(X)^T [K, Mp]
  uint16_t* xrt = reinterpret_cast<uint16_t*>(ws + round256((size_t)N * mp * 2) + round256((size_t)K * mp * 2));
  hipError_t e = rfq::launch_transpose_bf16(static_cast<const uint16_t*>(dy), M, N, lddy, dyt, mp, s);
  if (e == hipSuccess) e = rfq::launch_decode_transpose(qx_codes, qx_scales, M, K, xqt, mp, s);
  if (e == hipSuccess) e = rfq::launch_decode_transpose(qr_codes, qr_scales, M, K, xrt, mp, s);
  if (e != hipSuccess) return launched(e);
  // dW^T [K, N] = Xq^T-rows . dY^T-rows + Xr^T-rows . dY^T-rows over Mp, stored transposed as dW [N, K]
  return launched(rfq::launch_gemm(16, 16, reinterpret_cast<const uint8_t*>(xqt), nullptr,
                                   reinterpret_cast<const uint8_t*>(xrt), nullptr, reinterpret_cast<const uint8_t*>(dyt),
                                   nullptr, K, N, 4 * mp, dw, dw_dtype == RFQ_DTYPE_BF16, lddw, s, true));
}

const char* rfq_status_string(rfq_status_t status) {
  switch (status) {
    case RFQ_OK: return "success";
    case RFQ_ERR_NULL_POINTER: return "a required pointer is NULL";
    case RFQ_ERR_INVALID_SHAPE: return "invalid shape";
    case RFQ_ERR_INVALID_STRIDE: return "invalid row stride";
    case RFQ_ERR_MISALIGNED: return "misaligned pointer";
    case RFQ_ERR_UNSUPPORTED_DTYPE: return "unsupported dtype";
    case RFQ_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case RFQ_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* rfq_last_error_detail(void) { return g_detail.c_str(); }

int rfq_abi_version(void) { return RFQ_ABI_VERSION; }

}  // extern "C"
