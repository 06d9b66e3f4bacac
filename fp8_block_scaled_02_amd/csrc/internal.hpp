// internal.hpp -- launchers behind the C ABI (not exported).
//
// Each launcher assumes its arguments were validated by the caller (api.cpp)
// and returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8w {

// Weight scale formats (the values of fp8w_format).
constexpr int kFmtBlock = 0;       // fp32 per 128x128 tile
constexpr int kFmtMx = 1;          // e8m0 per row and 32 columns
constexpr int kFmtBlockBf16 = 2;   // bf16 per 128x128 tile
constexpr int kFmtRow = 3;         // fp32 per row
constexpr int kFmtTensor = 4;      // one fp32 for the whole weight

// One GEMV y[m, n] = x[m, k] . deq(codes)^T.  The same layout is the row of
// a grouped launch's device table (fp8w_grouped_plan_init writes it).
struct GemvJob {
  const uint16_t* x;        // bf16 [m, k] (W8A8: e4m3 codes [m, k])
  const uint8_t* codes;     // e4m3fn [n, k]
  const void* scales;       // in `format`: block grid, e8m0 grid, bf16 grid, [n] or [1]
  uint16_t* y;              // bf16 [m, n]
  int32_t n, k;             // validated to fit int32 on the host
  int32_t item0;            // first workgroup of this job in a grouped launch
  int32_t format;           // kFmt*; kFmtMx jobs run the MX kernel variants
};
static_assert(sizeof(GemvJob) == 48, "device table row");

// One weight of a grouped quantize launch (device table row).
struct QuantJob {
  const uint16_t* w;        // bf16 [n, k]
  uint8_t* codes;           // e4m3fn [n, k]
  void* scales;             // the launch's format: f32 / bf16 block grid or e8m0 [n, ceil(k/32)]
  int32_t n, k;             // validated to fit int32 on the host
  int32_t item0;            // first workgroup of this weight in the launch
  int32_t vec;              // 1: the 16-byte path (quant_job_vec)
  int32_t pad[2];
};
static_assert(sizeof(QuantJob) == 48, "device table row");

// Workgroups of one weight in a grouped quantize launch, and whether its
// shape and alignment take the 16-byte path (format: kFmtBlock,
// kFmtBlockBf16 or kFmtMx).
int64_t quant_job_blocks(int format, int64_t n, int64_t k, bool vec);
bool quant_job_vec(int format, const void* w, int64_t k, const void* codes);
hipError_t launch_quantize_grouped(const QuantJob* device_table, int njobs, int64_t blocks, int format,
                                   hipStream_t stream);

hipError_t launch_quantize_block(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes,
                                 float* scales, hipStream_t stream);
hipError_t launch_quantize_mx(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes,
                              uint8_t* e8m0, hipStream_t stream);

hipError_t launch_quantize_block_bf16(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes,
                                      uint16_t* scales, hipStream_t stream);
hipError_t launch_quantize_row(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes, float* scales,
                               hipStream_t stream);
hipError_t launch_dequantize_format(const uint8_t* codes, const void* scales, int format, int64_t n,
                                    int64_t k, uint16_t* out, hipStream_t stream);
hipError_t launch_dequantize_block(const uint8_t* codes, const float* scales, int64_t n, int64_t k,
                                   uint16_t* out, hipStream_t stream);
hipError_t launch_dequantize_mx(const uint8_t* codes, const uint8_t* e8m0, int64_t n, int64_t k,
                                uint16_t* out, hipStream_t stream);
// Dequantize into w_bf16 [n, k], then y = x . w^T with rocBLAS.  When the
// device has no rocBLAS handle yet and `stream` is capturing, nothing is
// enqueued and *capture_blocked is set.
hipError_t launch_gemm_dequant(const uint16_t* x, int64_t m, const uint8_t* codes,
                               const void* scales, int format, int64_t n, int64_t k, uint16_t* y,
                               uint16_t* w_bf16, hipStream_t stream, bool* capture_blocked);
// Create the current device's rocBLAS handle now (outside capture).
hipError_t gemm_prepare();

// W8A8 GEMV: job.x points at e4m3 activation codes [m, k]; x_scale is a
// device pointer to the activation's fp32 scale.
hipError_t launch_gemv_w8a8(const GemvJob& job, const float* x_scale, int m, bool mx,
                            hipStream_t stream);
// Per-tensor activation quantization; workspace holds act_quant_partials()
// uint32 partial maxima.
int act_quant_partials();
hipError_t launch_quantize_act(const uint16_t* x, int64_t count, uint8_t* codes, float* scale,
                               uint32_t* workspace, hipStream_t stream);
// The same with the partial maxima in a file-scope device array of
// act_quant_partials() words (one per device, shared by every call on it).
hipError_t launch_quantize_act_noalloc(const uint16_t* x, int64_t count, uint8_t* codes, float* scale,
                                       hipStream_t stream);

// route: 1 = VALU (m <= 8), 2 = MFMA (m <= 32).
int gemv_rows_per_block(int route, int m, bool grouped);
hipError_t launch_gemv(const GemvJob& job, int m, bool mx, int route, hipStream_t stream);
// Grouped VALU launch, one tile of gemv_rows_per_block(1, m, true) rows per
// workgroup.  At m = 1 the tiles walk K in segments of seg_cols columns:
// 3072 (seg_cols 0 or 3072) or 4096.
hipError_t launch_gemv_grouped(const GemvJob* device_table, int njobs, int64_t blocks, int m,
                               bool mx, int seg_cols, hipStream_t stream);
// Wide VALU tiles at m = 1 (single calls on many rows, grouped launches
// with a K above the streaming limit): K segments of 3072 columns, or 4096
// where those need fewer segments per tile (4096 holds more registers per
// wave: fewer waves per SIMD).  gemv_wide_seg_rounds = segments per tile.
int gemv_wide_seg_rounds(int64_t k, int seg_cols);
int gemv_wide_seg_cols(int64_t k);

// Streaming grouped VALU kernel (m = 1, every K <= gemv_stream_max_k(), MX
// exponent arrays as mx_rows_stream requires):
// tiles of gemv_stream_rows() rows, a contiguous run of tiles per workgroup.
int gemv_stream_max_k();
int gemv_stream_rows();
hipError_t gemv_stream_slots(bool mx, int* slots);   // resident workgroups on the device
hipError_t launch_gemv_stream(const GemvJob* device_table, int njobs, int64_t blocks,
                              int64_t tiles, int tiles_per_block, bool mx, hipStream_t stream);

// Streaming grouped MFMA kernel (any m <= 32, any K): tiles of
// gemv_rows_per_block(2, m, true) rows, x staged in LDS by K segments of
// seg_cols columns (a multiple of 256 chosen by gemv_mfma_stream_seg_cols).
int gemv_mfma_stream_seg_cols(int m, int64_t max_k);
int gemv_mfma_stream_lds(int m, int seg_cols);      // LDS bytes per workgroup
bool gemv_mfma_stream_seg_ok(int m, int seg_cols);  // a segment the kernel can stage
hipError_t gemv_mfma_stream_slots(int m, bool mx, int seg_cols, int* slots);
// MX weights whose exponent rows all start 8-byte aligned (ceil(k/32) % 8
// == 0 and an 8-byte aligned array): the MFMA kernels then read each row's
// exponents for a 256-column panel with one 8-byte load.
bool mx_rows_packed8(const void* e8m0, int64_t k);
// MX weights the streaming VALU kernel reads exponents of as dwords: a
// 4-byte aligned array of a whole number of dwords (n * ceil(k/32) % 4 == 0).
bool mx_rows_stream(const void* e8m0, int64_t n, int64_t k);
// `format` is the format every job of the table shares.
hipError_t launch_gemv_mfma_stream(const GemvJob* device_table, int njobs, int64_t blocks,
                                   int64_t tiles, int tiles_per_block, int m, int seg_cols,
                                   int format, bool mx_packed8, hipStream_t stream);

// Read-only pass over `bytes` (a multiple of 16) of device memory, one
// 32-bit XOR per workgroup into out[0 .. blocks).
int64_t read_ceiling_blocks(int64_t bytes, int64_t max_blocks);
hipError_t launch_read_ceiling(const void* buf, int64_t bytes, uint32_t* out, int64_t blocks,
                               hipStream_t stream);

}  // namespace fp8w
