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
constexpr int kChunksPerThread = 4;   // 16-code chunks in flight per thread

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

// Four codes of d times s -> four bf16 (two packed dwords).
__device__ __forceinline__ uint2 dequant4(uint32_t d, float s) {
  const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(d, false);
  const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(d, true);
  return make_uint2(f32_to_bf16_rne(lo.x * s) | (f32_to_bf16_rne(lo.y * s) << 16),
                    f32_to_bf16_rne(hi.x * s) | (f32_to_bf16_rne(hi.y * s) << 16));
}

// Vector path (k % 16 == 0, codes 16-B and out 16-B aligned): chunk c is
// codes[c*16 .. c*16+15] of the flat [n, k] array; a chunk never straddles a
// row, a 128-column block or a 32-column MX group.  Thread t of workgroup b
// takes chunks (b*4 + u)*256 + t, u = 0..3: all loads first, then the
// stores.
template <bool MX>
__global__ __launch_bounds__(kThreads) void k_dequant_vec(const uint8_t* __restrict__ codes,
                                                          const void* __restrict__ scales,
                                                          uint16_t* __restrict__ out, int64_t chunks,
                                                          int chunks_per_row, int scale_cols, int format) {
  uint4 c[kChunksPerThread];
  float s[kChunksPerThread];
#pragma unroll
  for (int u = 0; u < kChunksPerThread; ++u) {
    const int64_t ch = ((int64_t)blockIdx.x * kChunksPerThread + u) * kThreads + threadIdx.x;
    c[u] = make_uint4(0, 0, 0, 0);
    s[u] = 0.0f;
    if (ch < chunks) {
      c[u] = ld_stream_u4(codes, (size_t)ch * 16);
      const int64_t row = ch / chunks_per_row;
      const int col = (int)(ch - row * chunks_per_row) * 16;
      if (MX)
        s[u] = pow2_e8m0(ld_global<uint8_t>(scales, (size_t)row * scale_cols + col / kGroup));
      else
        s[u] = weight_scale(scales, format, row, col, scale_cols);
    }
  }
#pragma unroll
  for (int u = 0; u < kChunksPerThread; ++u) {
    const int64_t ch = ((int64_t)blockIdx.x * kChunksPerThread + u) * kThreads + threadIdx.x;
    if (ch < chunks) {
      const uint2 a = dequant4(c[u].x, s[u]), b = dequant4(c[u].y, s[u]);
      const uint2 d = dequant4(c[u].z, s[u]), e = dequant4(c[u].w, s[u]);
      st_global<u32x4>(out, (size_t)ch * 32, u32x4{a.x, a.y, b.x, b.y});
      st_global<u32x4>(out, (size_t)ch * 32 + 16, u32x4{d.x, d.y, e.x, e.y});
    }
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
  out[i] = (uint16_t)f32_to_bf16_rne(v.x * s);
}

inline bool aligned_to(const void* p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

template <bool MX>
hipError_t launch_dequant(const uint8_t* codes, const void* scales, int format, int64_t n, int64_t k,
                          uint16_t* out, hipStream_t stream) {
  const int scale_cols = (int)(MX ? (k + kGroup - 1) / kGroup : (k + kTile - 1) / kTile);
  if (k % 16 == 0 && aligned_to(codes, 16) && aligned_to(out, 16)) {
    const int64_t chunks = n * (k / 16);
    const int64_t per_block = (int64_t)kThreads * kChunksPerThread;
    const dim3 grid((unsigned)((chunks + per_block - 1) / per_block));
    hipLaunchKernelGGL((k_dequant_vec<MX>), grid, dim3(kThreads), 0, stream, codes, scales, out, chunks,
                       (int)(k / 16), scale_cols, format);
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
