// api.cpp -- the extern "C" entry points of libfp8w (declared in fp8w.h).
//
// Every argument is validated on the host before anything is enqueued, so
// an invalid call launches nothing and writes nothing: the shape contract of
// "quantize_fp8_bs.rs" (Atlas weight_map: n > 0 and k > 0 are required) and
// the fail-loudly bounds contract of "feat: add FP8 blockwise weight
// quantization and FP8(E4M3) KV cache support" (Security and Safety).
// The kernel family is chosen from the shape only (never from values), so
// the calls are safe to capture in a HIP graph.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "fp8w.h"
#include "internal.hpp"

#define FP8W_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int64_t kMaxDim = 0x7FFFFFFF;   // kernels index rows and columns with int
constexpr int kValuMaxM = 8;
// AUTO route: VALU up to this m, MFMA above, measured on MI355X over the
// 96-GEMV projection set.  Single calls: VALU is faster at m <= 2.  Grouped:
// the streaming MFMA kernel is faster from m = 2 on (6.4 against 5.5 TB/s).
constexpr int kAutoValuMaxM = 2;
constexpr int kAutoValuMaxMGrouped = 1;

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

fp8w_status from_hip(hipError_t e) { return e == hipSuccess ? FP8W_OK : FP8W_ERR_HIP; }

fp8w_status check_gemv(const uint16_t* x, int64_t m, const uint8_t* codes, const void* scales,
                       uint64_t scale_bytes, int64_t n, int64_t k, uint16_t* y, fp8w_route route,
                       bool block) {
  if (!x || !codes || !scales || !y) return FP8W_ERR_NULL;
  if (m < 1 || m > FP8W_MAX_M || !dims_ok(n, k) || k < 16) return FP8W_ERR_SHAPE;
  if (k % 16 != 0 || !aligned(x, 16) || !aligned(codes, 16) || (block && !aligned(scales, 4)) ||
      !aligned(y, 2))
    return FP8W_ERR_ALIGN;
  if (route != FP8W_ROUTE_AUTO && route != FP8W_ROUTE_VALU && route != FP8W_ROUTE_MFMA)
    return FP8W_ERR_UNSUPPORTED;
  if (route == FP8W_ROUTE_VALU && m > kValuMaxM) return FP8W_ERR_UNSUPPORTED;
  const Span out[1] = {{y, (uint64_t)m * n * 2}};
  const Span in[3] = {{x, (uint64_t)m * k * 2}, {codes, (uint64_t)n * k}, {scales, scale_bytes}};
  if (any_overlap(out, 1, in, 3)) return FP8W_ERR_OVERLAP;
  return FP8W_OK;
}

int resolve_route(fp8w_route route, int64_t m, bool grouped) {
  if (route == FP8W_ROUTE_VALU) return 1;
  if (route == FP8W_ROUTE_MFMA) return 2;
  return m <= (grouped ? kAutoValuMaxMGrouped : kAutoValuMaxM) ? 1 : 2;
}

}  // namespace

FP8W_API fp8w_status fp8w_quantize_block(const uint16_t* w, int64_t n, int64_t k,
                                         uint8_t* codes, float* scales, void* stream) {
  if (!w || !codes || !scales) return FP8W_ERR_NULL;
  if (!dims_ok(n, k)) return FP8W_ERR_SHAPE;
  if (!aligned(w, 2) || !aligned(scales, 4)) return FP8W_ERR_ALIGN;
  const Span out[2] = {{codes, (uint64_t)n * k}, {scales, (uint64_t)block_count(n, k) * 4}};
  const Span in[1] = {{w, (uint64_t)n * k * 2}};
  if (any_overlap(out, 2, in, 1)) return FP8W_ERR_OVERLAP;
  return from_hip(fp8w::launch_quantize_block(w, n, k, codes, scales,
                                              static_cast<hipStream_t>(stream)));
}

FP8W_API fp8w_status fp8w_quantize_mx(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes,
                                      uint8_t* e8m0, void* stream) {
  if (!w || !codes || !e8m0) return FP8W_ERR_NULL;
  if (!dims_ok(n, k)) return FP8W_ERR_SHAPE;
  if (!aligned(w, 2)) return FP8W_ERR_ALIGN;
  const Span out[2] = {{codes, (uint64_t)n * k}, {e8m0, (uint64_t)mx_count(n, k)}};
  const Span in[1] = {{w, (uint64_t)n * k * 2}};
  if (any_overlap(out, 2, in, 1)) return FP8W_ERR_OVERLAP;
  return from_hip(
      fp8w::launch_quantize_mx(w, n, k, codes, e8m0, static_cast<hipStream_t>(stream)));
}

FP8W_API fp8w_status fp8w_gemv_block_route(const uint16_t* x, int64_t m, const uint8_t* codes,
                                           const float* scales, int64_t n, int64_t k,
                                           uint16_t* y, fp8w_route route, void* stream) {
  const fp8w_status st =
      check_gemv(x, m, codes, scales, (uint64_t)block_count(n, k) * 4, n, k, y, route, true);
  if (st != FP8W_OK) return st;
  const fp8w::GemvJob job{x, codes, scales, y, (int32_t)n, (int32_t)k, 0, 0};
  return from_hip(fp8w::launch_gemv(job, (int)m, false, resolve_route(route, m, false),
                                    static_cast<hipStream_t>(stream)));
}

FP8W_API fp8w_status fp8w_gemv_mx_route(const uint16_t* x, int64_t m, const uint8_t* codes,
                                        const uint8_t* e8m0, int64_t n, int64_t k, uint16_t* y,
                                        fp8w_route route, void* stream) {
  const fp8w_status st =
      check_gemv(x, m, codes, e8m0, (uint64_t)mx_count(n, k), n, k, y, route, false);
  if (st != FP8W_OK) return st;
  const fp8w::GemvJob job{x, codes, e8m0, y, (int32_t)n, (int32_t)k, 0, 0};
  return from_hip(fp8w::launch_gemv(job, (int)m, true, resolve_route(route, m, false),
                                    static_cast<hipStream_t>(stream)));
}

FP8W_API fp8w_status fp8w_gemv_block(const uint16_t* x, int64_t m, const uint8_t* codes,
                                     const float* scales, int64_t n, int64_t k, uint16_t* y,
                                     void* stream) {
  return fp8w_gemv_block_route(x, m, codes, scales, n, k, y, FP8W_ROUTE_AUTO, stream);
}

FP8W_API fp8w_status fp8w_gemv_mx(const uint16_t* x, int64_t m, const uint8_t* codes,
                                  const uint8_t* e8m0, int64_t n, int64_t k, uint16_t* y,
                                  void* stream) {
  return fp8w_gemv_mx_route(x, m, codes, e8m0, n, k, y, FP8W_ROUTE_AUTO, stream);
}

// ---------------------------------------------------------- dequantize --

namespace {

fp8w_status check_dequant(const uint8_t* codes, const void* scales, uint64_t scale_bytes,
                          int64_t n, int64_t k, const uint16_t* w, bool block) {
  if (!codes || !scales || !w) return FP8W_ERR_NULL;
  if (!dims_ok(n, k)) return FP8W_ERR_SHAPE;
  if ((block && !aligned(scales, 4)) || !aligned(w, 2)) return FP8W_ERR_ALIGN;
  const Span out[1] = {{w, (uint64_t)n * k * 2}};
  const Span in[2] = {{codes, (uint64_t)n * k}, {scales, scale_bytes}};
  if (any_overlap(out, 1, in, 2)) return FP8W_ERR_OVERLAP;
  return FP8W_OK;
}

}  // namespace

FP8W_API fp8w_status fp8w_dequantize_block(const uint8_t* codes, const float* scales, int64_t n,
                                           int64_t k, uint16_t* w, void* stream) {
  const fp8w_status st = check_dequant(codes, scales, (uint64_t)block_count(n, k) * 4, n, k, w, true);
  if (st != FP8W_OK) return st;
  return from_hip(fp8w::launch_dequantize_block(codes, scales, n, k, w, static_cast<hipStream_t>(stream)));
}

FP8W_API fp8w_status fp8w_dequantize_mx(const uint8_t* codes, const uint8_t* e8m0, int64_t n,
                                        int64_t k, uint16_t* w, void* stream) {
  const fp8w_status st = check_dequant(codes, e8m0, (uint64_t)mx_count(n, k), n, k, w, false);
  if (st != FP8W_OK) return st;
  return from_hip(fp8w::launch_dequantize_mx(codes, e8m0, n, k, w, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------- GEMM --

namespace {

fp8w_status check_gemm(const uint16_t* x, int64_t m, const uint8_t* codes, const void* scales,
                       uint64_t scale_bytes, int64_t n, int64_t k, const uint16_t* y,
                       const void* workspace, int64_t workspace_bytes, bool block) {
  if (!x || !codes || !scales || !y || !workspace) return FP8W_ERR_NULL;
  if (m < 1 || m > kMaxDim || !dims_ok(n, k)) return FP8W_ERR_SHAPE;
  if (workspace_bytes < n * k * 2) return FP8W_ERR_SHAPE;
  if (!aligned(x, 2) || !aligned(y, 2) || !aligned(workspace, 16) || (block && !aligned(scales, 4)))
    return FP8W_ERR_ALIGN;
  const Span out[2] = {{y, (uint64_t)m * n * 2}, {workspace, (uint64_t)n * k * 2}};
  const Span in[3] = {{x, (uint64_t)m * k * 2}, {codes, (uint64_t)n * k}, {scales, scale_bytes}};
  if (any_overlap(out, 2, in, 3)) return FP8W_ERR_OVERLAP;
  return FP8W_OK;
}

}  // namespace

FP8W_API int64_t fp8w_gemm_workspace_bytes(int64_t n, int64_t k) {
  return (n < 1 || k < 1) ? 0 : n * k * 2;
}

FP8W_API fp8w_status fp8w_gemm_block(const uint16_t* x, int64_t m, const uint8_t* codes,
                                     const float* scales, int64_t n, int64_t k, uint16_t* y,
                                     void* workspace, int64_t workspace_bytes, void* stream) {
  const fp8w_status st = check_gemm(x, m, codes, scales, (uint64_t)block_count(n, k) * 4, n, k, y,
                                    workspace, workspace_bytes, true);
  if (st != FP8W_OK) return st;
  return from_hip(fp8w::launch_gemm_dequant(x, m, codes, scales, false, n, k, y,
                                            static_cast<uint16_t*>(workspace),
                                            static_cast<hipStream_t>(stream)));
}

FP8W_API fp8w_status fp8w_gemm_mx(const uint16_t* x, int64_t m, const uint8_t* codes,
                                  const uint8_t* e8m0, int64_t n, int64_t k, uint16_t* y,
                                  void* workspace, int64_t workspace_bytes, void* stream) {
  const fp8w_status st = check_gemm(x, m, codes, e8m0, (uint64_t)mx_count(n, k), n, k, y, workspace,
                                    workspace_bytes, false);
  if (st != FP8W_OK) return st;
  return from_hip(fp8w::launch_gemm_dequant(x, m, codes, e8m0, true, n, k, y,
                                            static_cast<uint16_t*>(workspace),
                                            static_cast<hipStream_t>(stream)));
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

namespace {

fp8w_status check_w8a8(const uint8_t* xc, const float* xs, int64_t m, const uint8_t* codes,
                       const void* scales, uint64_t scale_bytes, int64_t n, int64_t k,
                       const uint16_t* y, bool block) {
  if (!xc || !xs || !codes || !scales || !y) return FP8W_ERR_NULL;
  if (m < 1 || m > FP8W_MAX_M || !dims_ok(n, k) || k < 16) return FP8W_ERR_SHAPE;
  if (k % 16 != 0 || !aligned(xc, 16) || !aligned(xs, 4) || !aligned(codes, 16) ||
      (block && !aligned(scales, 4)) || !aligned(y, 2))
    return FP8W_ERR_ALIGN;
  const Span out[1] = {{y, (uint64_t)m * n * 2}};
  const Span in[4] = {{xc, (uint64_t)m * k}, {xs, 4}, {codes, (uint64_t)n * k}, {scales, scale_bytes}};
  if (any_overlap(out, 1, in, 4)) return FP8W_ERR_OVERLAP;
  return FP8W_OK;
}

}  // namespace

FP8W_API fp8w_status fp8w_gemv_block_w8a8(const uint8_t* x_codes, const float* x_scale, int64_t m,
                                          const uint8_t* codes, const float* scales, int64_t n,
                                          int64_t k, uint16_t* y, void* stream) {
  const fp8w_status st = check_w8a8(x_codes, x_scale, m, codes, scales, (uint64_t)block_count(n, k) * 4,
                                    n, k, y, true);
  if (st != FP8W_OK) return st;
  const fp8w::GemvJob job{reinterpret_cast<const uint16_t*>(x_codes), codes, scales, y, (int32_t)n,
                          (int32_t)k, 0, 0};
  return from_hip(fp8w::launch_gemv_w8a8(job, x_scale, (int)m, false, static_cast<hipStream_t>(stream)));
}

FP8W_API fp8w_status fp8w_gemv_mx_w8a8(const uint8_t* x_codes, const float* x_scale, int64_t m,
                                       const uint8_t* codes, const uint8_t* e8m0, int64_t n, int64_t k,
                                       uint16_t* y, void* stream) {
  const fp8w_status st = check_w8a8(x_codes, x_scale, m, codes, e8m0, (uint64_t)mx_count(n, k), n, k, y,
                                    false);
  if (st != FP8W_OK) return st;
  const fp8w::GemvJob job{reinterpret_cast<const uint16_t*>(x_codes), codes, e8m0, y, (int32_t)n,
                          (int32_t)k, 0, 0};
  return from_hip(fp8w::launch_gemv_w8a8(job, x_scale, (int)m, true, static_cast<hipStream_t>(stream)));
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
  if (format != FP8W_FORMAT_BLOCK && format != FP8W_FORMAT_MX) return FP8W_ERR_UNSUPPORTED;
  if (!aligned(device_table, 16)) return FP8W_ERR_ALIGN;
  const bool block = format == FP8W_FORMAT_BLOCK;
  std::vector<Span> ins, outs;
  ins.reserve(3 * count);
  outs.reserve(count);
  for (int64_t i = 0; i < count; ++i) {
    const fp8w_gemv_desc& d = descs[i];
    const uint64_t sb = block ? (uint64_t)block_count(d.n, d.k) * 4 : (uint64_t)mx_count(d.n, d.k);
    const fp8w_status st = check_gemv(d.x, m, d.codes, d.scales, sb, d.n, d.k, d.y, route, block);
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
  const int r = resolve_route(route, m, true);
  int64_t max_k = 0;
  for (int64_t i = 0; i < count; ++i) max_k = descs[i].k > max_k ? descs[i].k : max_k;
  // Kernels: VALU at m = 1 with every K in one segment streams (contiguous
  // runs of tiles per workgroup); other VALU plans take one tile per
  // workgroup; MFMA plans always stream, x staged by K segments.
  const bool valu_stream = r == 1 && m == 1 && max_k <= fp8w::gemv_stream_max_k();
  const int rows = valu_stream ? fp8w::gemv_stream_rows() : fp8w::gemv_rows_per_block(r, (int)m, true);
  std::vector<fp8w::GemvJob> table((size_t)count);
  int64_t tiles = 0;
  for (int64_t i = 0; i < count; ++i) {
    const fp8w_gemv_desc& d = descs[i];
    table[i] = fp8w::GemvJob{d.x, d.codes, d.scales, d.y, (int32_t)d.n, (int32_t)d.k,
                             (int32_t)tiles, 0};
    tiles += (d.n + rows - 1) / rows;
    if (tiles > kMaxDim) return FP8W_ERR_SHAPE;
  }
  int64_t blocks = tiles;
  int32_t per_block = 0, seg_cols = 0;
  if (valu_stream || r == 2) {
    int slots = 0;
    int64_t want = 0;
    if (valu_stream) {
      if (fp8w::gemv_stream_slots(!block, &slots) != hipSuccess) return FP8W_ERR_HIP;
      // about sixteen workgroups per resident slot (runs of ~3 tiles on the
      // 48-layer projection set): the hardware dispatcher then balances the
      // runs over the CUs, where long runs left a tail of late workgroups
      // (measured on MI355X: 41-tile runs 6.1 TB/s, 3-tile runs 6.9 TB/s).
      want = (int64_t)16 * slots;
    } else {
      seg_cols = fp8w::gemv_mfma_stream_seg_cols((int)m, max_k);
      if (fp8w::gemv_mfma_stream_slots((int)m, !block, seg_cols, &slots) != hipSuccess)
        return FP8W_ERR_HIP;
      want = (int64_t)8 * slots;
    }
    per_block = (int32_t)((tiles + want - 1) / want);
    blocks = (tiles + per_block - 1) / per_block;
  }
  if (hipMemcpy(device_table, table.data(), table_bytes, hipMemcpyHostToDevice) != hipSuccess)
    return FP8W_ERR_HIP;
  *plan = fp8w_grouped_plan{device_table, (int32_t)count, (int32_t)m, (int32_t)format,
                            (int32_t)(r == 1 ? FP8W_ROUTE_VALU : FP8W_ROUTE_MFMA), blocks, tiles,
                            per_block, seg_cols};
  return FP8W_OK;
}

FP8W_API fp8w_status fp8w_gemv_grouped(const fp8w_grouped_plan* plan, void* stream) {
  if (!plan || !plan->table) return FP8W_ERR_NULL;
  const bool route_ok = (plan->route == FP8W_ROUTE_VALU && plan->m <= kValuMaxM) ||
                        plan->route == FP8W_ROUTE_MFMA;
  if (plan->count < 1 || plan->m < 1 || plan->m > FP8W_MAX_M || !route_ok || plan->blocks < 1 ||
      plan->blocks > kMaxDim || plan->tiles < plan->blocks || plan->tiles > kMaxDim ||
      plan->tiles_per_block < 0 ||
      (plan->format != FP8W_FORMAT_BLOCK && plan->format != FP8W_FORMAT_MX))
    return FP8W_ERR_SHAPE;
  const bool mx = plan->format == FP8W_FORMAT_MX;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const fp8w::GemvJob* table = static_cast<const fp8w::GemvJob*>(plan->table);
  if (plan->tiles_per_block > 0 && plan->blocks * (int64_t)plan->tiles_per_block < plan->tiles)
    return FP8W_ERR_SHAPE;
  if (plan->route == FP8W_ROUTE_MFMA) {
    const int seg = plan->seg_cols;
    if (plan->tiles_per_block < 1 || seg < 256 || seg % 256 != 0 ||
        fp8w::gemv_mfma_stream_lds(plan->m, seg) > fp8w::gemv_mfma_stream_lds_limit())
      return FP8W_ERR_SHAPE;
    return from_hip(fp8w::launch_gemv_mfma_stream(table, plan->count, plan->blocks, plan->tiles,
                                                  plan->tiles_per_block, plan->m, seg, mx, s));
  }
  if (plan->seg_cols != 0) return FP8W_ERR_SHAPE;
  if (plan->tiles_per_block > 0) {
    if (plan->m != 1) return FP8W_ERR_SHAPE;
    return from_hip(fp8w::launch_gemv_stream(table, plan->count, plan->blocks, plan->tiles,
                                             plan->tiles_per_block, mx, s));
  }
  if (plan->blocks != plan->tiles) return FP8W_ERR_SHAPE;
  return from_hip(fp8w::launch_gemv_grouped(table, plan->count, plan->blocks, plan->m, mx, s));
}

// ------------------------------------------------------------- helpers --

FP8W_API int64_t fp8w_block_scale_count(int64_t n, int64_t k) {
  return (n < 1 || k < 1) ? 0 : block_count(n, k);
}

FP8W_API int64_t fp8w_mx_scale_count(int64_t n, int64_t k) {
  return (n < 1 || k < 1) ? 0 : mx_count(n, k);
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
  }
  return "FP8W_ERR_UNKNOWN";
}

FP8W_API int fp8w_version(void) { return 100; }
