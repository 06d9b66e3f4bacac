// device.hpp -- device helpers shared by the libfp8w kernels (gfx950 only).
//
// bf16 <-> fp32 bit helpers, the e4m3fn encoder, the e8m0 exponent rule and
// wavefront reductions.  Nothing here is shared with the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8w {

constexpr int kWave = 64;       // CDNA wavefront width
constexpr int kTile = 128;      // block-scale tile edge, both axes
constexpr int kGroup = 32;      // elements per e8m0 scale, along K
constexpr uint32_t kF32Bits448 = 0x43E00000u;   // 448.0f
constexpr uint32_t kF32BitsMinNormalE4M3 = 0x3C800000u;   // 2^-6

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Loads and stores through the global address space.  Pointers read from a
// job table are generic; generic (flat) accesses also count against the LDS
// counter, so a wait for an LDS write would wait for the weight stream too.
// Scalar types only (the global address space does not bind to class types).
template <typename T>
__device__ __forceinline__ T ld_global(const void* p, size_t byte_offset = 0) {
  return *(const __attribute__((address_space(1))) T*)((const char*)p + byte_offset);
}
template <typename T>
__device__ __forceinline__ void st_global(void* p, size_t byte_offset, T v) {
  *(__attribute__((address_space(1))) T*)((char*)p + byte_offset) = v;
}
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_global_u4(const void* p, size_t byte_offset) {
  const u32x4 v = ld_global<u32x4>(p, byte_offset);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// Non-temporal 16-byte load, for data read exactly once (the weight stream):
// on MI355X it lifts a pure streaming read from about 6.3 to 6.8 TB/s.
__device__ __forceinline__ uint4 ld_stream_u4(const void* p, size_t byte_offset) {
  const u32x4 v = __builtin_nontemporal_load(
      (const __attribute__((address_space(1))) u32x4*)((const char*)p + byte_offset));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Non-temporal 8-byte store, for outputs written once (quantized codes).
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void st_stream_u2(void* p, size_t byte_offset, uint2 v) {
  __builtin_nontemporal_store(u32x2{v.x, v.y},
                              (__attribute__((address_space(1))) u32x2*)((char*)p + byte_offset));
}

// s_waitcnt vmcnt(0), leaving the LDS/scalar and export counters alone
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
__device__ __forceinline__ void vm_wait_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// bf16 halves of a packed dword, widened exactly to fp32.
__device__ __forceinline__ float bf16_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// e4m3fn codes by the hardware conversion (v_cvt_pk_fp8_f32: round to
// nearest even, OCP e4m3fn on gfx950, sign kept, -0 -> 0x80) after clamping
// to [-448, 448], which is the saturation.  Measured on MI355X over every
// non-NaN fp32 bit pattern, in both byte positions of the packed result: the
// byte equals an integer RNE encoder of the bit pattern (top three mantissa
// bits kept, 20 dropped bits rounded to nearest even, exponent rebiased; the
// uniform 2^-9 grid below 2^-6) in every case.  Inputs must not be NaN.
__device__ __forceinline__ float clamp448(float q) { return __builtin_fminf(__builtin_fmaxf(q, -448.0f), 448.0f); }

// Four codes packed little-endian: a in bits 0-7, ..., d in bits 24-31.
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(clamp448(c), clamp448(d), lo, true);
}

__device__ __forceinline__ uint32_t e4m3_code(float q) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(clamp448(q), 0.0f, 0, false) & 0xFFu;
}

// MX exponent of a group from its amax (the fp32 bit pattern of a
// non-negative value): the smallest e with amax <= 448 * 2^e, clamped to
// [-127, 127].  With amax = 2^x * 1.f and 448 = 2^8 * 1.75, e = x - 8 when
// 1.f <= 1.75 and x - 7 otherwise.  fp32 subnormals and zero land below
// -127 and clamp there; no finite amax reaches 127.
__device__ __forceinline__ int e8m0_exponent(uint32_t amax_bits) {
  const int field = (int)(amax_bits >> 23);
  if (field == 0) return -127;
  const int e = field - 127 - 8 + ((amax_bits & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return e < -127 ? -127 : e;
}

// Sum over aligned groups of `width` consecutive lanes (width a power of two
// <= 64).  Every lane of the group ends with the group's sum.
template <int width>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = width / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, width);
  return v;
}

template <int width>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
#pragma unroll
  for (int off = width / 2; off > 0; off >>= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)v, off, width);
    v = o > v ? o : v;
  }
  return v;
}

}  // namespace fp8w
