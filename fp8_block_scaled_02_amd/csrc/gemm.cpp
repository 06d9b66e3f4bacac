// gemm.cpp -- the large-M route: dequantize the fp8 weight to bf16, then a
// dense bf16 GEMM (rocBLAS, fp32 accumulation).
//
// "feat: add FP8 blockwise weight quantization ..." (Summary) routes M <= 32
// to the fused fp8 GEMV and larger M and prefill to dequantize + a dense
// library GEMM; its Notes for Reviewers keep that fallback selectable for
// every M.  At prefill sizes the GEMM is bound by the matrix cores, and the
// dequantize pass (3 bytes per weight) is small next to it.
//
// One rocBLAS handle per device, created by fp8w_gemm_prepare or by the
// first call on that device, and kept for the life of the process; calls on
// one device are serialized around the handle (the stream is set per call).
// Creating a handle allocates device memory, which a captured stream cannot
// do: a call that would create it while its stream is capturing fails with
// FP8W_ERR_CAPTURE before anything is enqueued.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>
#include <stdint.h>

#include <mutex>

#include "internal.hpp"

namespace fp8w {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_blas_lock;
rocblas_handle g_blas[kMaxDevices] = {};

// This device's handle; created here unless `stream` is capturing.
hipError_t blas_handle(hipStream_t stream, rocblas_handle* out, bool* capture_blocked) {
  *capture_blocked = false;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_blas_lock);
  if (!g_blas[dev]) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(stream, &cap);
    if (e != hipSuccess) return e;
    if (cap != hipStreamCaptureStatusNone) {
      *capture_blocked = true;
      return hipErrorStreamCaptureUnsupported;
    }
    if (rocblas_create_handle(&g_blas[dev]) != rocblas_status_success) {
      g_blas[dev] = nullptr;
      return hipErrorUnknown;
    }
  }
  *out = g_blas[dev];
  return hipSuccess;
}

hipError_t blas_gemm(rocblas_handle h, const uint16_t* x, int m, const uint16_t* w, int n, int k, uint16_t* y,
                     hipStream_t stream) {
  std::lock_guard<std::mutex> lock(g_blas_lock);
  if (rocblas_set_stream(h, stream) != rocblas_status_success) return hipErrorUnknown;
  // Column-major view: y^T [n, m] = W [n, k] . x^T [k, m], where the
  // row-major W [n, k] is the column-major k x n matrix (transposed in) and
  // the row-major x [m, k] is the column-major k x m matrix.
  const float alpha = 1.0f, beta = 0.0f;
  const rocblas_status st = rocblas_gemm_ex(
      h, rocblas_operation_transpose, rocblas_operation_none, n, m, k, &alpha, w,
      rocblas_datatype_bf16_r, k, x, rocblas_datatype_bf16_r, k, &beta, y, rocblas_datatype_bf16_r,
      n, y, rocblas_datatype_bf16_r, n, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
  return st == rocblas_status_success ? hipSuccess : hipErrorUnknown;
}

}  // namespace

hipError_t gemm_prepare() {
  rocblas_handle h = nullptr;
  bool blocked = false;
  return blas_handle(nullptr, &h, &blocked);
}

hipError_t launch_gemm_dequant(const uint16_t* x, int64_t m, const uint8_t* codes,
                               const void* scales, int format, int64_t n, int64_t k, uint16_t* y,
                               uint16_t* w_bf16, hipStream_t stream, bool* capture_blocked) {
  // the handle first: a call that cannot get one enqueues nothing
  rocblas_handle h = nullptr;
  hipError_t e = blas_handle(stream, &h, capture_blocked);
  if (e != hipSuccess) return e;
  e = launch_dequantize_format(codes, scales, format, n, k, w_bf16, stream);
  if (e != hipSuccess) return e;
  return blas_gemm(h, x, (int)m, w_bf16, (int)n, (int)k, y, stream);
}

}  // namespace fp8w
