// dequant.hip -- e4m3fn codes + scales -> bf16 weights, for gfx950.
//
// The inverse of the quantizers, and the first half of the large-M route
// (dequantize to bf16, then a dense GEMM: "feat: add FP8 blockwise weight
// quantization ...", Summary).  Each weight is the decoded code (exact in
// fp32) times its scale in one fp32 multiply, rounded to nearest even bf16.
// For MX the scale 2^(E-127) is a power of two and the product is exact.
// HBM-bound: 1 byte in, 2 bytes out per weight (plus the scales).
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "internal.hpp"

namespace fp8w {
namespace {

constexpr int kThreads = 256;
constexpr int kUnitsPerThread = 8;   // 8-code units in flight per thread

__device__ __forceinline__ float pow2_e8m0(uint8_t e) {
  return __uint_as_float(e ? (uint32_t)e << 23 : 0x00400000u);   // 2^(e-127), exact
}

// Scale of weight (row, col) for the formats other than MX: an fp32 or
// bf16 128x128 grid (scale_cols tiles per row), one fp32 per row, or one for
// the whole weight.  The format is uniform over the launch.
__device__ __forceinline__ float weight_scale(const void* scales, int format, int64_t row, int col,
                                              int scale_cols) {
  const size_t tile = (size_t)(row / kTile) * scale_cols + col / kTile;
  if (format == kFmtBlock) return ld_global<float>(scales, tile * 4);
  if (format == kFmtBlockBf16) return bf16_lo(ld_global<uint16_t>(scales, tile * 2));
  if (format == kFmtRow) return ld_global<float>(scales, (size_t)row * 4);
  return ld_global<float>(scales, 0);
}

// The stored scale of weight (row, col) as loaded, in any format (an e8m0
// byte, bf16 bits or fp32 bits), and its value.  The vector kernel loads
// every unit's raw scale before it converts any: a conversion right after
// its load would wait for that load before the next unit's loads issue.
__device__ __forceinline__ uint32_t raw_scale(const void* scales, int format, int64_t row, int col,
                                              int scale_cols) {
  if (format == kFmtMx) return ld_global<uint8_t>(scales, (size_t)row * scale_cols + col / kGroup);
  const size_t tile = (size_t)(row / kTile) * scale_cols + col / kTile;
  if (format == kFmtBlock) return ld_global<uint32_t>(scales, tile * 4);
  if (format == kFmtBlockBf16) return ld_global<uint16_t>(scales, tile * 2);
  return ld_global<uint32_t>(scales, (size_t)row * 4);   // kFmtRow (kFmtTensor: loaded once per thread)
}

__device__ __forceinline__ float scale_value(uint32_t raw, int format) {
  if (format == kFmtMx) return pow2_e8m0((uint8_t)raw);
  if (format == kFmtBlockBf16) return __uint_as_float(raw << 16);
  return __uint_as_float(raw);
}

// Eight codes (two dwords) times s -> eight bf16, rounded to nearest even
// by the hardware conversion (v_cvt_pk_bf16_f32).
__device__ __forceinline__ u32x4 dequant8(u32x2 d, float s) {
  u32x4 o;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(d[h], false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(d[h], true);
    const bf16x2 a = {(__bf16)(lo.x * s), (__bf16)(lo.y * s)};
    const bf16x2 b = {(__bf16)(hi.x * s), (__bf16)(hi.y * s)};
    o[2 * h] = __builtin_bit_cast(uint32_t, a);
    o[2 * h + 1] = __builtin_bit_cast(uint32_t, b);
  }
  return o;
}

// Vector path (k % 8 == 0, codes 8-byte and out 16-byte aligned): unit u is
// codes[8u .. 8u+7] of the flat [n, k] array, written as one 16-byte store
// at out + 16u, so both the loads and the stores of a wave are contiguous.
// A unit never straddles a row, a 128-column block or a 32-column MX group.
// Thread t of workgroup b takes units (b*8 + i)*256 + t, i = 0..7: all
// loads first, then the stores.  IDX is the index type of the row division
// (32-bit when every unit index fits).
template <bool MX, typename IDX>
__global__ __launch_bounds__(kThreads) void k_dequant_vec(const uint8_t* __restrict__ codes,
                                                          const void* __restrict__ scales,
                                                          uint16_t* __restrict__ out, int64_t units,
                                                          int units_per_row, int scale_cols, int format) {
  const int fmt = MX ? kFmtMx : format;
  const uint32_t whole = fmt == kFmtTensor ? ld_global<uint32_t>(scales, 0) : 0u;
  u32x2 c[kUnitsPerThread];
  uint32_t raw[kUnitsPerThread];
#pragma unroll
  for (int i = 0; i < kUnitsPerThread; ++i) {
    const int64_t u = ((int64_t)blockIdx.x * kUnitsPerThread + i) * kThreads + threadIdx.x;
    c[i] = u32x2{0u, 0u};
    raw[i] = 0u;
    if (u < units) {
      c[i] = __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x2*)(codes + (size_t)u * 8));
      const IDX row = (IDX)u / (IDX)units_per_row;
      const int col = (int)((IDX)u - row * (IDX)units_per_row) * 8;
      raw[i] = fmt == kFmtTensor ? whole : raw_scale(scales, fmt, (int64_t)row, col, scale_cols);
    }
  }
#pragma unroll
  for (int i = 0; i < kUnitsPerThread; ++i) {
    const int64_t u = ((int64_t)blockIdx.x * kUnitsPerThread + i) * kThreads + threadIdx.x;
    if (u < units) st_global<u32x4>(out, (size_t)u * 16, dequant8(c[i], scale_value(raw[i], fmt)));
  }
}

// Any k and alignment: one weight per thread.
template <bool MX>
__global__ __launch_bounds__(kThreads) void k_dequant_any(const uint8_t* __restrict__ codes,
                                                          const void* __restrict__ scales,
                                                          uint16_t* __restrict__ out, int64_t total,
                                                          int k, int scale_cols, int format) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= total) return;
  const int64_t row = i / k;
  const int col = (int)(i - row * k);
  const float s = MX ? pow2_e8m0(ld_global<uint8_t>(scales, (size_t)row * scale_cols + col / kGroup))
                     : weight_scale(scales, format, row, col, scale_cols);
  const f32x2 v = __builtin_amdgcn_cvt_pk_f32_fp8((uint32_t)codes[i], false);
  out[i] = __builtin_bit_cast(uint16_t, (__bf16)(v.x * s));
}

inline bool aligned_to(const void* p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

template <bool MX>
hipError_t launch_dequant(const uint8_t* codes, const void* scales, int format, int64_t n, int64_t k,
                          uint16_t* out, hipStream_t stream) {
  const int scale_cols = (int)(MX ? (k + kGroup - 1) / kGroup : (k + kTile - 1) / kTile);
  if (k % 8 == 0 && aligned_to(codes, 8) && aligned_to(out, 16)) {
    const int64_t units = n * (k / 8);
    const int64_t per_block = (int64_t)kThreads * kUnitsPerThread;
    const dim3 grid((unsigned)((units + per_block - 1) / per_block));
    // 32-bit row division when every unit index of the grid fits
    if ((int64_t)grid.x * per_block <= 0xFFFFFFFFLL)
      hipLaunchKernelGGL((k_dequant_vec<MX, uint32_t>), grid, dim3(kThreads), 0, stream, codes, scales, out,
                         units, (int)(k / 8), scale_cols, format);
    else
      hipLaunchKernelGGL((k_dequant_vec<MX, int64_t>), grid, dim3(kThreads), 0, stream, codes, scales, out,
                         units, (int)(k / 8), scale_cols, format);
  } else {
    const int64_t total = n * k;
    const dim3 grid((unsigned)((total + kThreads - 1) / kThreads));
    hipLaunchKernelGGL((k_dequant_any<MX>), grid, dim3(kThreads), 0, stream, codes, scales, out, total,
                       (int)k, scale_cols, format);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dequantize_format(const uint8_t* codes, const void* scales, int format, int64_t n,
                                    int64_t k, uint16_t* out, hipStream_t stream) {
  return format == kFmtMx ? launch_dequant<true>(codes, scales, format, n, k, out, stream)
                          : launch_dequant<false>(codes, scales, format, n, k, out, stream);
}

hipError_t launch_dequantize_block(const uint8_t* codes, const float* scales, int64_t n, int64_t k,
                                   uint16_t* out, hipStream_t stream) {
  return launch_dequant<false>(codes, scales, kFmtBlock, n, k, out, stream);
}

hipError_t launch_dequantize_mx(const uint8_t* codes, const uint8_t* e8m0, int64_t n, int64_t k,
                                uint16_t* out, hipStream_t stream) {
  return launch_dequant<true>(codes, e8m0, kFmtMx, n, k, out, stream);
}

}  // namespace fp8w
