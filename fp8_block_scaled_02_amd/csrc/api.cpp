// api.cpp -- the extern "C" entry points of libfp8w (declared in fp8w.h).
//
// Every argument is validated on the host before anything is enqueued, so
// an invalid call launches nothing and writes nothing: the shape contract of
// "quantize_fp8_bs.rs" (Atlas weight_map: n > 0 and k > 0 are required) and
// the fail-loudly bounds contract of "feat: add FP8 blockwise weight
// quantization and FP8(E4M3) KV cache support" (Security and Safety).
// The kernel family is chosen from the shape only (never from values), so
// the enqueueing calls can be captured in a HIP graph once their set-up
// calls (GEMM handle, grouped tables) have run outside capture.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "fp8w.h"
#include "internal.hpp"

#define FP8W_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int64_t kMaxDim = 0x7FFFFFFF;   // kernels index rows and columns with int
constexpr int kValuMaxM = 8;
// AUTO route, from the VALU / MFMA crossovers measured on MI355X.
//  - Single calls.  The MFMA kernel's time hardly moves with m: one 16-row
//    MFMA tile serves every m <= 16 (rocprofv3 kernel traces and counters
//    at m = 3, 4, 5: VALU issue 9-11 %, MFMA busy under 2 %).  The VALU
//    kernel's instructions grow with m (VALU issue 18 / 22 / 25 % on
//    [4096x4096] and 29 / 34 / 37 % on [8192x2560] at m = 3 / 4 / 5, both
//    kernels within 1.5 % of the same HBM bytes), so every shape has one
//    crossover, later on shorter weights.  Graph-captured passes over every
//    workload shape (N 2560..151936, K 2048..12288, block and MX scales,
//    m = 2..8; two runs on one box, `route_crossover_single_calls` rows)
//    put it after m = 2 on weights of 32768 rows or more (lm_head at m = 3:
//    MFMA 3-8 % faster with block scales, 9-14 % with MX), after m = 4 on
//    weights up to 8192 rows and K = 4096 (VALU 2-16 % faster at m = 4),
//    and after m = 3 elsewhere ([24576x4096] and [4096x12288] at m = 4:
//    MFMA 0-10 % faster; m = 3 within 3 % either way on those two).  At
//    m = 5 MFMA is as fast or faster on every shape (up to 9 %) but MX
//    [6144x4096], 1 % slower there.  Block and MX scales now share the rule.
//  - Grouped: the streaming VALU kernel at m = 1; VALU tiles at m = 2 for
//    block-scaled formats (+4 % on the projection set, +16 % on dense
//    layers), while MX at m = 2 is 6 % faster on the streaming MFMA kernel.
constexpr int64_t kAutoValuM3MaxN = 32768 - 1;
constexpr int kAutoValuM4MaxN = 8192;
constexpr int kAutoValuM4MaxK = 4096;

bool aligned(const void* p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

struct Span {
  const void* p;
  uint64_t bytes;
};

bool overlap(Span a, Span b) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a.bytes && b.bytes && a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// True if any output span overlaps any other span (inputs or outputs).
bool any_overlap(const Span* outs, int n_out, const Span* ins, int n_in) {
  for (int i = 0; i < n_out; ++i) {
    for (int j = 0; j < n_in; ++j)
      if (overlap(outs[i], ins[j])) return true;
    for (int j = i + 1; j < n_out; ++j)
      if (overlap(outs[i], outs[j])) return true;
  }
  return false;
}

bool dims_ok(int64_t n, int64_t k) { return n >= 1 && k >= 1 && n <= kMaxDim && k <= kMaxDim; }

int64_t block_count(int64_t n, int64_t k) { return ((n + 127) / 128) * ((k + 127) / 128); }
int64_t mx_count(int64_t n, int64_t k) { return n * ((k + 31) / 32); }

bool format_ok(int f) { return f >= FP8W_FORMAT_BLOCK && f <= FP8W_FORMAT_TENSOR; }

// Bytes of the scale buffer of an [n, k] weight in `format`.
uint64_t scale_bytes(int format, int64_t n, int64_t k) {
  switch (format) {
    case FP8W_FORMAT_BLOCK: return (uint64_t)block_count(n, k) * 4;
    case FP8W_FORMAT_MX: return (uint64_t)mx_count(n, k);
    case FP8W_FORMAT_BLOCK_BF16: return (uint64_t)block_count(n, k) * 2;
    case FP8W_FORMAT_ROW: return (uint64_t)n * 4;
    case FP8W_FORMAT_TENSOR: return 4;
  }
  return 0;
}

// Alignment the scale buffer of `format` needs (its element size).
uintptr_t scale_align(int format) {
  return format == FP8W_FORMAT_MX ? 1 : format == FP8W_FORMAT_BLOCK_BF16 ? 2 : 4;
}

fp8w_status from_hip(hipError_t e) { return e == hipSuccess ? FP8W_OK : FP8W_ERR_HIP; }

fp8w_status check_gemv(const uint16_t* x, int64_t m, const uint8_t* codes, const void* scales,
                       int format, int64_t n, int64_t k, uint16_t* y, fp8w_route route) {
  if (!x || !codes || !scales || !y) return FP8W_ERR_NULL;
  if (!format_ok(format)) return FP8W_ERR_UNSUPPORTED;
  if (m < 1 || m > FP8W_MAX_M || !dims_ok(n, k) || k < 16) return FP8W_ERR_SHAPE;
  if (k % 16 != 0 || !aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, scale_align(format)) ||
      !aligned(y, 2))
    return FP8W_ERR_ALIGN;
  if (route != FP8W_ROUTE_AUTO && route != FP8W_ROUTE_VALU && route != FP8W_ROUTE_MFMA)
    return FP8W_ERR_UNSUPPORTED;
  if (route == FP8W_ROUTE_VALU && m > kValuMaxM) return FP8W_ERR_UNSUPPORTED;
  const Span out[1] = {{y, (uint64_t)m * n * 2}};
  const Span in[3] = {{x, (uint64_t)m * k * 2}, {codes, (uint64_t)n * k}, {scales, scale_bytes(format, n, k)}};
  if (any_overlap(out, 1, in, 3)) return FP8W_ERR_OVERLAP;
  return FP8W_OK;
}

fp8w_status gemv_any(const uint16_t* x, int64_t m, const uint8_t* codes, const void* scales, int format,
                     int64_t n, int64_t k, uint16_t* y, fp8w_route route, void* stream);

bool auto_valu_single(int64_t m, int64_t n, int64_t k) {
  switch (m) {
    case 1:
    case 2: return true;
    case 3: return n <= kAutoValuM3MaxN;
    case 4: return n <= kAutoValuM4MaxN && k <= kAutoValuM4MaxK;
    default: return false;
  }
}

bool auto_valu_grouped(int64_t m, bool mx) { return m == 1 || (m == 2 && !mx); }

int resolve_route(fp8w_route route, int64_t m, int64_t n, int64_t k) {
  if (route == FP8W_ROUTE_VALU) return 1;
  if (route == FP8W_ROUTE_MFMA) return 2;
  return auto_valu_single(m, n, k) ? 1 : 2;
}

int resolve_route_grouped(fp8w_route route, int64_t m, bool mx) {
  if (route == FP8W_ROUTE_VALU) return 1;
  if (route == FP8W_ROUTE_MFMA) return 2;
  return auto_valu_grouped(m, mx) ? 1 : 2;
}

}  // namespace

FP8W_API fp8w_route fp8w_gemv_auto_route(fp8w_format format, int64_t m, int64_t n, int64_t k) {
  if (!format_ok(format) || m < 1 || m > FP8W_MAX_M || !dims_ok(n, k)) return FP8W_ROUTE_AUTO;
  return auto_valu_single(m, n, k) ? FP8W_ROUTE_VALU : FP8W_ROUTE_MFMA;
}

FP8W_API int64_t fp8w_scale_bytes(fp8w_format format, int64_t n, int64_t k) {
  return (!format_ok(format) || n < 1 || k < 1) ? 0 : (int64_t)scale_bytes(format, n, k);
}

FP8W_API fp8w_status fp8w_quantize(const uint16_t* w, int64_t n, int64_t k, fp8w_format format,
                                   uint8_t* codes, void* scales, void* workspace,
                                   int64_t workspace_bytes, void* stream) {
  if (!w || !codes || !scales) return FP8W_ERR_NULL;
  if (!format_ok(format)) return FP8W_ERR_UNSUPPORTED;
  if (!dims_ok(n, k)) return FP8W_ERR_SHAPE;
  const bool needs_ws = format == FP8W_FORMAT_TENSOR && n * k > 16384;
  if (needs_ws && !workspace) return FP8W_ERR_NULL;
  if (needs_ws && workspace_bytes < fp8w_quantize_act_workspace_bytes()) return FP8W_ERR_SHAPE;
  if (!aligned(w, 2) || !aligned(scales, scale_align(format)) || (needs_ws && !aligned(workspace, 4)))
    return FP8W_ERR_ALIGN;
  const Span out[3] = {{codes, (uint64_t)n * k}, {scales, scale_bytes(format, n, k)},
                       {workspace, needs_ws ? (uint64_t)fp8w_quantize_act_workspace_bytes() : 0}};
  const Span in[1] = {{w, (uint64_t)n * k * 2}};
  if (any_overlap(out, 3, in, 1)) return FP8W_ERR_OVERLAP;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  switch (format) {
    case FP8W_FORMAT_BLOCK:
      return from_hip(fp8w::launch_quantize_block(w, n, k, codes, static_cast<float*>(scales), s));
    case FP8W_FORMAT_MX:
      return from_hip(fp8w::launch_quantize_mx(w, n, k, codes, static_cast<uint8_t*>(scales), s));
    case FP8W_FORMAT_BLOCK_BF16:
      return from_hip(fp8w::launch_quantize_block_bf16(w, n, k, codes, static_cast<uint16_t*>(scales), s));
    case FP8W_FORMAT_ROW:
      return from_hip(fp8w::launch_quantize_row(w, n, k, codes, static_cast<float*>(scales), s));
    default:
      return from_hip(fp8w::launch_quantize_act(w, n * k, codes, static_cast<float*>(scales),
                                                static_cast<uint32_t*>(workspace), s));
  }
}

FP8W_API fp8w_status fp8w_quantize_block(const uint16_t* w, int64_t n, int64_t k,
                                         uint8_t* codes, float* scales, void* stream) {
  return fp8w_quantize(w, n, k, FP8W_FORMAT_BLOCK, codes, scales, nullptr, 0, stream);
}

FP8W_API fp8w_status fp8w_quantize_mx(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes,
                                      uint8_t* e8m0, void* stream) {
  return fp8w_quantize(w, n, k, FP8W_FORMAT_MX, codes, e8m0, nullptr, 0, stream);
}

namespace {

fp8w_status gemv_any(const uint16_t* x, int64_t m, const uint8_t* codes, const void* scales, int format,
                     int64_t n, int64_t k, uint16_t* y, fp8w_route route, void* stream) {
  const fp8w_status st = check_gemv(x, m, codes, scales, format, n, k, y, route);
  if (st != FP8W_OK) return st;
  const fp8w::GemvJob job{x, codes, scales, y, (int32_t)n, (int32_t)k, 0, format};
  return from_hip(fp8w::launch_gemv(job, (int)m, format == FP8W_FORMAT_MX, resolve_route(route, m, n, k),
                                    static_cast<hipStream_t>(stream)));
}

}  // namespace

FP8W_API fp8w_status fp8w_gemv(const uint16_t* x, int64_t m, const uint8_t* codes, const void* scales,
                               fp8w_format format, int64_t n, int64_t k, uint16_t* y, fp8w_route route,
                               void* stream) {
  return gemv_any(x, m, codes, scales, format, n, k, y, route, stream);
}

FP8W_API fp8w_status fp8w_gemv_block_route(const uint16_t* x, int64_t m, const uint8_t* codes,
                                           const float* scales, int64_t n, int64_t k,
                                           uint16_t* y, fp8w_route route, void* stream) {
  return gemv_any(x, m, codes, scales, FP8W_FORMAT_BLOCK, n, k, y, route, stream);
}

FP8W_API fp8w_status fp8w_gemv_mx_route(const uint16_t* x, int64_t m, const uint8_t* codes,
                                        const uint8_t* e8m0, int64_t n, int64_t k, uint16_t* y,
                                        fp8w_route route, void* stream) {
  return gemv_any(x, m, codes, e8m0, FP8W_FORMAT_MX, n, k, y, route, stream);
}

FP8W_API fp8w_status fp8w_gemv_block(const uint16_t* x, int64_t m, const uint8_t* codes,
                                     const float* scales, int64_t n, int64_t k, uint16_t* y,
                                     void* stream) {
  return gemv_any(x, m, codes, scales, FP8W_FORMAT_BLOCK, n, k, y, FP8W_ROUTE_AUTO, stream);
}

FP8W_API fp8w_status fp8w_gemv_mx(const uint16_t* x, int64_t m, const uint8_t* codes,
                                  const uint8_t* e8m0, int64_t n, int64_t k, uint16_t* y,
                                  void* stream) {
  return gemv_any(x, m, codes, e8m0, FP8W_FORMAT_MX, n, k, y, FP8W_ROUTE_AUTO, stream);
}

// ---------------------------------------------------------- dequantize --

FP8W_API fp8w_status fp8w_dequantize(const uint8_t* codes, const void* scales, fp8w_format format,
                                     int64_t n, int64_t k, uint16_t* w, void* stream) {
  if (!codes || !scales || !w) return FP8W_ERR_NULL;
  if (!format_ok(format)) return FP8W_ERR_UNSUPPORTED;
  if (!dims_ok(n, k)) return FP8W_ERR_SHAPE;
  if (!aligned(scales, scale_align(format)) || !aligned(w, 2)) return FP8W_ERR_ALIGN;
  const Span out[1] = {{w, (uint64_t)n * k * 2}};
  const Span in[2] = {{codes, (uint64_t)n * k}, {scales, scale_bytes(format, n, k)}};
  if (any_overlap(out, 1, in, 2)) return FP8W_ERR_OVERLAP;
  return from_hip(fp8w::launch_dequantize_format(codes, scales, format, n, k, w, static_cast<hipStream_t>(stream)));
}

FP8W_API fp8w_status fp8w_dequantize_block(const uint8_t* codes, const float* scales, int64_t n,
                                           int64_t k, uint16_t* w, void* stream) {
  return fp8w_dequantize(codes, scales, FP8W_FORMAT_BLOCK, n, k, w, stream);
}

FP8W_API fp8w_status fp8w_dequantize_mx(const uint8_t* codes, const uint8_t* e8m0, int64_t n,
                                        int64_t k, uint16_t* w, void* stream) {
  return fp8w_dequantize(codes, e8m0, FP8W_FORMAT_MX, n, k, w, stream);
}

// ---------------------------------------------------------------- GEMM --

FP8W_API int64_t fp8w_gemm_workspace_bytes(int64_t n, int64_t k) {
  return (n < 1 || k < 1) ? 0 : n * k * 2;
}

FP8W_API fp8w_status fp8w_gemm(const uint16_t* x, int64_t m, const uint8_t* codes, const void* scales,
                               fp8w_format format, int64_t n, int64_t k, uint16_t* y, void* workspace,
                               int64_t workspace_bytes, void* stream) {
  if (!x || !codes || !scales || !y || !workspace) return FP8W_ERR_NULL;
  if (!format_ok(format)) return FP8W_ERR_UNSUPPORTED;
  if (m < 1 || m > kMaxDim || !dims_ok(n, k)) return FP8W_ERR_SHAPE;
  if (workspace_bytes < n * k * 2) return FP8W_ERR_SHAPE;
  if (!aligned(x, 2) || !aligned(y, 2) || !aligned(workspace, 16) || !aligned(scales, scale_align(format)))
    return FP8W_ERR_ALIGN;
  const Span out[2] = {{y, (uint64_t)m * n * 2}, {workspace, (uint64_t)n * k * 2}};
  const Span in[3] = {{x, (uint64_t)m * k * 2}, {codes, (uint64_t)n * k}, {scales, scale_bytes(format, n, k)}};
  if (any_overlap(out, 2, in, 3)) return FP8W_ERR_OVERLAP;
  bool capture_blocked = false;
  const hipError_t e = fp8w::launch_gemm_dequant(x, m, codes, scales, format, n, k, y,
                                                 static_cast<uint16_t*>(workspace),
                                                 static_cast<hipStream_t>(stream), &capture_blocked);
  return capture_blocked ? FP8W_ERR_CAPTURE : from_hip(e);
}

FP8W_API fp8w_status fp8w_gemm_prepare(void) { return from_hip(fp8w::gemm_prepare()); }

FP8W_API fp8w_status fp8w_gemm_block(const uint16_t* x, int64_t m, const uint8_t* codes,
                                     const float* scales, int64_t n, int64_t k, uint16_t* y,
                                     void* workspace, int64_t workspace_bytes, void* stream) {
  return fp8w_gemm(x, m, codes, scales, FP8W_FORMAT_BLOCK, n, k, y, workspace, workspace_bytes, stream);
}

FP8W_API fp8w_status fp8w_gemm_mx(const uint16_t* x, int64_t m, const uint8_t* codes,
                                  const uint8_t* e8m0, int64_t n, int64_t k, uint16_t* y,
                                  void* workspace, int64_t workspace_bytes, void* stream) {
  return fp8w_gemm(x, m, codes, e8m0, FP8W_FORMAT_MX, n, k, y, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------- W8A8 --

FP8W_API int64_t fp8w_quantize_act_workspace_bytes(void) {
  return (int64_t)fp8w::act_quant_partials() * 4;
}

FP8W_API fp8w_status fp8w_quantize_act(const uint16_t* x, int64_t m, int64_t k, uint8_t* codes,
                                       float* scale, void* workspace, int64_t workspace_bytes,
                                       void* stream) {
  if (!x || !codes || !scale) return FP8W_ERR_NULL;
  if (m < 1 || k < 1 || m > kMaxDim || k > kMaxDim) return FP8W_ERR_SHAPE;
  const int64_t count = m * k;
  const bool needs_ws = count > 16384;
  if (needs_ws && !workspace) return FP8W_ERR_NULL;
  if (needs_ws && workspace_bytes < fp8w_quantize_act_workspace_bytes()) return FP8W_ERR_SHAPE;
  if (!aligned(x, 2) || !aligned(scale, 4) || (needs_ws && !aligned(workspace, 4))) return FP8W_ERR_ALIGN;
  const Span out[3] = {{codes, (uint64_t)count}, {scale, 4},
                       {workspace, needs_ws ? (uint64_t)fp8w_quantize_act_workspace_bytes() : 0}};
  const Span in[1] = {{x, (uint64_t)count * 2}};
  if (any_overlap(out, 3, in, 1)) return FP8W_ERR_OVERLAP;
  return from_hip(fp8w::launch_quantize_act(x, count, codes, scale, static_cast<uint32_t*>(workspace),
                                            static_cast<hipStream_t>(stream)));
}

FP8W_API fp8w_status fp8w_quantize_act_noalloc(const uint16_t* x, int64_t m, int64_t k, uint8_t* codes,
                                               float* scale, void* stream) {
  if (!x || !codes || !scale) return FP8W_ERR_NULL;
  if (m < 1 || k < 1 || m > kMaxDim || k > kMaxDim) return FP8W_ERR_SHAPE;
  const int64_t count = m * k;
  if (!aligned(x, 2) || !aligned(scale, 4)) return FP8W_ERR_ALIGN;
  const Span out[2] = {{codes, (uint64_t)count}, {scale, 4}};
  const Span in[1] = {{x, (uint64_t)count * 2}};
  if (any_overlap(out, 2, in, 1)) return FP8W_ERR_OVERLAP;
  const hipError_t e = fp8w::launch_quantize_act_noalloc(x, count, codes, scale, static_cast<hipStream_t>(stream));
  return e == hipErrorInvalidValue ? FP8W_ERR_SHAPE : from_hip(e);
}

FP8W_API fp8w_status fp8w_gemv_w8a8(const uint8_t* x_codes, const float* x_scale, int64_t m,
                                    const uint8_t* codes, const void* scales, fp8w_format format,
                                    int64_t n, int64_t k, uint16_t* y, void* stream) {
  if (!x_codes || !x_scale || !codes || !scales || !y) return FP8W_ERR_NULL;
  if (!format_ok(format)) return FP8W_ERR_UNSUPPORTED;
  if (m < 1 || m > FP8W_MAX_M || !dims_ok(n, k) || k < 16) return FP8W_ERR_SHAPE;
  if (k % 16 != 0 || !aligned(x_codes, 16) || !aligned(x_scale, 4) || !aligned(codes, 16) ||
      !aligned(scales, scale_align(format)) || !aligned(y, 2))
    return FP8W_ERR_ALIGN;
  const Span out[1] = {{y, (uint64_t)m * n * 2}};
  const Span in[4] = {{x_codes, (uint64_t)m * k}, {x_scale, 4}, {codes, (uint64_t)n * k},
                      {scales, scale_bytes(format, n, k)}};
  if (any_overlap(out, 1, in, 4)) return FP8W_ERR_OVERLAP;
  const fp8w::GemvJob job{reinterpret_cast<const uint16_t*>(x_codes), codes, scales, y, (int32_t)n,
                          (int32_t)k, 0, format};
  return from_hip(fp8w::launch_gemv_w8a8(job, x_scale, (int)m, format == FP8W_FORMAT_MX,
                                         static_cast<hipStream_t>(stream)));
}

FP8W_API fp8w_status fp8w_gemv_block_w8a8(const uint8_t* x_codes, const float* x_scale, int64_t m,
                                          const uint8_t* codes, const float* scales, int64_t n,
                                          int64_t k, uint16_t* y, void* stream) {
  return fp8w_gemv_w8a8(x_codes, x_scale, m, codes, scales, FP8W_FORMAT_BLOCK, n, k, y, stream);
}

FP8W_API fp8w_status fp8w_gemv_mx_w8a8(const uint8_t* x_codes, const float* x_scale, int64_t m,
                                       const uint8_t* codes, const uint8_t* e8m0, int64_t n, int64_t k,
                                       uint16_t* y, void* stream) {
  return fp8w_gemv_w8a8(x_codes, x_scale, m, codes, e8m0, FP8W_FORMAT_MX, n, k, y, stream);
}

// ------------------------------------------------------------- grouped --

FP8W_API int64_t fp8w_grouped_table_bytes(int64_t count) {
  return count < 1 ? 0 : count * (int64_t)sizeof(fp8w::GemvJob);
}

FP8W_API fp8w_status fp8w_grouped_plan_init(const fp8w_gemv_desc* descs, int64_t count, int64_t m,
                                            fp8w_format format, fp8w_route route,
                                            void* device_table, fp8w_grouped_plan* plan) {
  if (!descs || !device_table || !plan) return FP8W_ERR_NULL;
  if (count < 1 || count > kMaxDim) return FP8W_ERR_SHAPE;
  if (!format_ok(format)) return FP8W_ERR_UNSUPPORTED;
  if (!aligned(device_table, 16)) return FP8W_ERR_ALIGN;
  const bool mx = format == FP8W_FORMAT_MX;
  std::vector<Span> ins, outs;
  ins.reserve(3 * count);
  outs.reserve(count);
  for (int64_t i = 0; i < count; ++i) {
    const fp8w_gemv_desc& d = descs[i];
    const uint64_t sb = scale_bytes(format, d.n, d.k);
    const fp8w_status st = check_gemv(d.x, m, d.codes, d.scales, format, d.n, d.k, d.y, route);
    if (st != FP8W_OK) return st;
    ins.push_back({d.x, (uint64_t)m * d.k * 2});
    ins.push_back({d.codes, (uint64_t)d.n * d.k});
    ins.push_back({d.scales, sb});
    outs.push_back({d.y, (uint64_t)m * d.n * 2});
  }
  const uint64_t table_bytes = (uint64_t)count * sizeof(fp8w::GemvJob);
  ins.push_back({device_table, table_bytes});
  if (any_overlap(outs.data(), (int)outs.size(), ins.data(), (int)ins.size()))
    return FP8W_ERR_OVERLAP;
  const int r = resolve_route_grouped(route, m, mx);
  int64_t max_k = 0;
  for (int64_t i = 0; i < count; ++i) max_k = descs[i].k > max_k ? descs[i].k : max_k;
  // Kernels: VALU at m = 1 with every K in one segment streams (contiguous
  // runs of tiles per workgroup); other VALU plans take one tile per
  // workgroup; MFMA plans always stream, x staged by K segments.
  // (the streaming VALU kernel reads MX exponents as aligned dwords)
  bool mx_dwords = true;
  for (int64_t i = 0; i < count; ++i)
    mx_dwords = mx_dwords && fp8w::mx_rows_stream(descs[i].scales, descs[i].n, descs[i].k);
  const bool valu_stream = r == 1 && m == 1 && max_k <= fp8w::gemv_stream_max_k() && (!mx || mx_dwords);
  const int rows = valu_stream ? fp8w::gemv_stream_rows() : fp8w::gemv_rows_per_block(r, (int)m, true);
  std::vector<fp8w::GemvJob> table((size_t)count);
  int64_t tiles = 0;
  for (int64_t i = 0; i < count; ++i) {
    const fp8w_gemv_desc& d = descs[i];
    table[i] = fp8w::GemvJob{d.x, d.codes, d.scales, d.y, (int32_t)d.n, (int32_t)d.k,
                             (int32_t)tiles, (int32_t)format};
    tiles += (d.n + rows - 1) / rows;
    if (tiles > kMaxDim) return FP8W_ERR_SHAPE;
  }
  int64_t blocks = tiles;
  int32_t per_block = 0, seg_cols = 0;
  if (r == 1 && m == 1 && !valu_stream) {
    // wide tiles at m = 1: 4096-column K segments when, summed over the
    // group's rows, they take fewer segment rounds than 3072-column ones
    int64_t rounds3 = 0, rounds4 = 0;
    for (int64_t i = 0; i < count; ++i) {
      rounds3 += descs[i].n * fp8w::gemv_wide_seg_rounds(descs[i].k, 3072);
      rounds4 += descs[i].n * fp8w::gemv_wide_seg_rounds(descs[i].k, 4096);
    }
    if (rounds4 < rounds3) seg_cols = 4096;
  }
  if (valu_stream || r == 2) {
    int slots = 0;
    int64_t want = 0;
    if (valu_stream) {
      if (fp8w::gemv_stream_slots(mx, &slots) != hipSuccess) return FP8W_ERR_HIP;
      // about sixteen workgroups per resident slot (runs of ~3 tiles on the
      // 48-layer projection set): the hardware dispatcher then balances the
      // runs over the CUs, where long runs left a tail of late workgroups
      // (measured on MI355X: 41-tile runs 6.1 TB/s, 3-tile runs 6.9 TB/s).
      want = (int64_t)16 * slots;
    } else {
      seg_cols = fp8w::gemv_mfma_stream_seg_cols((int)m, max_k);
      if (fp8w::gemv_mfma_stream_slots((int)m, mx, seg_cols, &slots) != hipSuccess)
        return FP8W_ERR_HIP;
      want = (int64_t)8 * slots;
    }
    per_block = (int32_t)((tiles + want - 1) / want);
    blocks = (tiles + per_block - 1) / per_block;
  }
  // MFMA route, MX: one 8-byte exponent load per row and panel when every
  // GEMV's exponent rows start 8-byte aligned
  int32_t mx_packed8 = 0;
  if (r == 2 && mx) {
    mx_packed8 = 1;
    for (int64_t i = 0; i < count; ++i)
      if (!fp8w::mx_rows_packed8(descs[i].scales, descs[i].k)) mx_packed8 = 0;
  }
  if (hipMemcpy(device_table, table.data(), table_bytes, hipMemcpyHostToDevice) != hipSuccess)
    return FP8W_ERR_HIP;
  *plan = fp8w_grouped_plan{device_table, (int32_t)count, (int32_t)m, (int32_t)format,
                            (int32_t)(r == 1 ? FP8W_ROUTE_VALU : FP8W_ROUTE_MFMA), blocks, tiles,
                            per_block, seg_cols, mx_packed8};
  return FP8W_OK;
}

FP8W_API fp8w_status fp8w_gemv_grouped(const fp8w_grouped_plan* plan, void* stream) {
  if (!plan || !plan->table) return FP8W_ERR_NULL;
  const bool route_ok = (plan->route == FP8W_ROUTE_VALU && plan->m <= kValuMaxM) ||
                        plan->route == FP8W_ROUTE_MFMA;
  if (plan->count < 1 || plan->m < 1 || plan->m > FP8W_MAX_M || !route_ok || plan->blocks < 1 ||
      plan->blocks > kMaxDim || plan->tiles < plan->blocks || plan->tiles > kMaxDim ||
      plan->tiles_per_block < 0 ||
      !format_ok(plan->format))
    return FP8W_ERR_SHAPE;
  if (plan->mx_packed8 != 0 &&
      (plan->mx_packed8 != 1 || plan->route != FP8W_ROUTE_MFMA || plan->format != FP8W_FORMAT_MX))
    return FP8W_ERR_SHAPE;
  const bool mx = plan->format == FP8W_FORMAT_MX;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const fp8w::GemvJob* table = static_cast<const fp8w::GemvJob*>(plan->table);
  if (plan->tiles_per_block > 0 && plan->blocks * (int64_t)plan->tiles_per_block < plan->tiles)
    return FP8W_ERR_SHAPE;
  if (plan->route == FP8W_ROUTE_MFMA) {
    const int seg = plan->seg_cols;
    if (plan->tiles_per_block < 1 || !fp8w::gemv_mfma_stream_seg_ok(plan->m, seg)) return FP8W_ERR_SHAPE;
    return from_hip(fp8w::launch_gemv_mfma_stream(table, plan->count, plan->blocks, plan->tiles,
                                                  plan->tiles_per_block, plan->m, seg, plan->format,
                                                  plan->mx_packed8 == 1, s));
  }
  if (plan->seg_cols != 0 && !(plan->seg_cols == 4096 && plan->m == 1 && plan->tiles_per_block == 0))
    return FP8W_ERR_SHAPE;
  if (plan->tiles_per_block > 0) {
    if (plan->m != 1) return FP8W_ERR_SHAPE;
    return from_hip(fp8w::launch_gemv_stream(table, plan->count, plan->blocks, plan->tiles,
                                             plan->tiles_per_block, mx, s));
  }
  if (plan->blocks != plan->tiles) return FP8W_ERR_SHAPE;
  return from_hip(fp8w::launch_gemv_grouped(table, plan->count, plan->blocks, plan->m, mx, plan->seg_cols, s));
}

// ---------------------------------------------------- grouped quantize --

FP8W_API int64_t fp8w_quant_table_bytes(int64_t count) {
  return (count < 1 || count > kMaxDim) ? 0 : count * (int64_t)sizeof(fp8w::QuantJob);
}

namespace {

bool quant_grouped_format(int f) {
  return f == FP8W_FORMAT_BLOCK || f == FP8W_FORMAT_MX || f == FP8W_FORMAT_BLOCK_BF16;
}

}  // namespace

FP8W_API fp8w_status fp8w_quant_plan_init(const fp8w_quant_desc* descs, int64_t count, fp8w_format format,
                                          void* device_table, fp8w_quant_plan* plan) {
  if (!descs || !device_table || !plan) return FP8W_ERR_NULL;
  if (count < 1 || count > kMaxDim) return FP8W_ERR_SHAPE;
  if (!quant_grouped_format(format)) return FP8W_ERR_UNSUPPORTED;
  if (!aligned(device_table, 16)) return FP8W_ERR_ALIGN;
  std::vector<Span> ins, outs;
  ins.reserve(count + 1);
  outs.reserve(2 * count);
  std::vector<fp8w::QuantJob> table((size_t)count);
  int64_t blocks = 0;
  for (int64_t i = 0; i < count; ++i) {
    const fp8w_quant_desc& d = descs[i];
    if (!d.w || !d.codes || !d.scales) return FP8W_ERR_NULL;
    if (!dims_ok(d.n, d.k)) return FP8W_ERR_SHAPE;
    if (!aligned(d.w, 2) || !aligned(d.scales, scale_align(format))) return FP8W_ERR_ALIGN;
    ins.push_back({d.w, (uint64_t)d.n * d.k * 2});
    outs.push_back({d.codes, (uint64_t)d.n * d.k});
    outs.push_back({d.scales, scale_bytes(format, d.n, d.k)});
    const bool vec = fp8w::quant_job_vec(format, d.w, d.k, d.codes);
    table[i] = fp8w::QuantJob{d.w, d.codes, d.scales, (int32_t)d.n, (int32_t)d.k, (int32_t)blocks,
                              vec ? 1 : 0, {0, 0}};
    blocks += fp8w::quant_job_blocks(format, d.n, d.k, vec);
    if (blocks > kMaxDim) return FP8W_ERR_SHAPE;
  }
  const uint64_t table_bytes = (uint64_t)count * sizeof(fp8w::QuantJob);
  ins.push_back({device_table, table_bytes});
  if (any_overlap(outs.data(), (int)outs.size(), ins.data(), (int)ins.size())) return FP8W_ERR_OVERLAP;
  if (hipMemcpy(device_table, table.data(), table_bytes, hipMemcpyHostToDevice) != hipSuccess)
    return FP8W_ERR_HIP;
  *plan = fp8w_quant_plan{device_table, (int32_t)count, (int32_t)format, blocks};
  return FP8W_OK;
}

FP8W_API fp8w_status fp8w_quantize_grouped(const fp8w_quant_plan* plan, void* stream) {
  if (!plan || !plan->table) return FP8W_ERR_NULL;
  if (plan->count < 1 || plan->blocks < plan->count || plan->blocks > kMaxDim ||
      !quant_grouped_format(plan->format) || !aligned(plan->table, 16))
    return FP8W_ERR_SHAPE;
  return from_hip(fp8w::launch_quantize_grouped(static_cast<const fp8w::QuantJob*>(plan->table), plan->count,
                                                plan->blocks, plan->format, static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------------- helpers --

FP8W_API int64_t fp8w_block_scale_count(int64_t n, int64_t k) {
  return (n < 1 || k < 1) ? 0 : block_count(n, k);
}

FP8W_API int64_t fp8w_mx_scale_count(int64_t n, int64_t k) {
  return (n < 1 || k < 1) ? 0 : mx_count(n, k);
}

FP8W_API fp8w_status fp8w_read_ceiling(const void* buf, int64_t bytes, uint32_t* out, int64_t out_words,
                                       void* stream) {
  if (!buf || !out) return FP8W_ERR_NULL;
  if (bytes < 16 || bytes % 16 != 0 || out_words < 1 || out_words > kMaxDim) return FP8W_ERR_SHAPE;
  if (!aligned(buf, 16) || !aligned(out, 4)) return FP8W_ERR_ALIGN;
  const Span o[1] = {{out, (uint64_t)out_words * 4}};
  const Span in[1] = {{buf, (uint64_t)bytes}};
  if (any_overlap(o, 1, in, 1)) return FP8W_ERR_OVERLAP;
  const int64_t blocks = fp8w::read_ceiling_blocks(bytes, out_words);
  return from_hip(fp8w::launch_read_ceiling(buf, bytes, out, blocks, static_cast<hipStream_t>(stream)));
}

FP8W_API const char* fp8w_status_string(fp8w_status status) {
  switch (status) {
    case FP8W_OK: return "FP8W_OK";
    case FP8W_ERR_NULL: return "FP8W_ERR_NULL: a required pointer is NULL";
    case FP8W_ERR_SHAPE: return "FP8W_ERR_SHAPE: n, k or m out of range";
    case FP8W_ERR_ALIGN: return "FP8W_ERR_ALIGN: alignment or k % 16 requirement not met";
    case FP8W_ERR_UNSUPPORTED: return "FP8W_ERR_UNSUPPORTED: route cannot serve this m";
    case FP8W_ERR_OVERLAP: return "FP8W_ERR_OVERLAP: an output overlaps another buffer";
    case FP8W_ERR_HIP: return "FP8W_ERR_HIP: the HIP runtime rejected the launch";
    case FP8W_ERR_CAPTURE:
      return "FP8W_ERR_CAPTURE: first GEMM call on this device made under stream capture "
             "(call fp8w_gemm_prepare first)";
  }
  return "FP8W_ERR_UNKNOWN";
}

FP8W_API int fp8w_version(void) { return 100; }
