// quantize.hip -- load-time bf16 -> e4m3fn quantizers for gfx950.
//
// Block format: one fp32 scale per 128x128 tile, scale = amax/448 and
// code = enc(w/scale) with both divisions correctly rounded in fp32
// ("quantize_fp8_bs.rs", Atlas weight_map: one byte per weight, one f32 per
// [128,128] tile, a ceil(k/128) x ceil(n/128) grid of 256-thread blocks).
// MX format: one e8m0 exponent per 32 elements along K, e = ceil(log2(
// amax/448)), code = enc(w * 2^-e) ("Load-time MXFP8 requantization ..."
// issue, Proposed solution).  The issue's 32 MB row-chunked fp32 transient
// bounds host memory in a torch implementation; the result is the same for
// any chunking, so the kernel streams rows with no transient.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <stddef.h>

#include "device.hpp"
#include "internal.hpp"

namespace fp8w {
namespace {

constexpr int kThreads = 256;

// Largest |bf16| of a packed pair, compared as bit patterns: for
// non-negative finite values the bit order is the value order.
__device__ __forceinline__ uint32_t abs_max_pair(uint32_t d, uint32_t acc) {
  const uint32_t lo = d & 0x7FFFu, hi = (d >> 16) & 0x7FFFu;
  acc = lo > acc ? lo : acc;
  return hi > acc ? hi : acc;
}

// Four codes of four packed bf16 (two dwords) divided by `scale`.
__device__ __forceinline__ uint32_t encode4_div(uint32_t d0, uint32_t d1, float scale) {
  return e4m3_pack4(bf16_lo(d0) / scale, bf16_hi(d0) / scale, bf16_lo(d1) / scale, bf16_hi(d1) / scale);
}

// Four codes of four packed bf16 multiplied by a power of two.
__device__ __forceinline__ uint32_t encode4_mul(uint32_t d0, uint32_t d1, float mul) {
  return e4m3_pack4(bf16_lo(d0) * mul, bf16_hi(d0) * mul, bf16_lo(d1) * mul, bf16_hi(d1) * mul);
}

// Block-wide max of a per-thread value (256 threads = 4 waves).
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v) {
  __shared__ uint32_t partial[kThreads / kWave];
  v = group_max_u32<kWave>(v);
  if ((threadIdx.x & (kWave - 1)) == 0) partial[threadIdx.x / kWave] = v;
  __syncthreads();
  uint32_t r = partial[0];
#pragma unroll
  for (int i = 1; i < kThreads / kWave; ++i) r = partial[i] > r ? partial[i] : r;
  return r;
}

// The tile's scale amax/448 (1.0 for an all-zero tile), stored by thread 0
// as fp32, or rounded to the nearest bf16 (at least the smallest positive
// bf16, 2^-133) and stored as bf16 -- then the codes divide by that rounded
// scale ("feat(quant): opt-in fp8-block QAT for the lm_head", How it works:
// a bf16 128-block scale).
template <bool BF16S>
__device__ __forceinline__ float tile_scale(float amax_f, void* scales, size_t at) {
  float scale = amax_f > 0.0f ? amax_f / 448.0f : 1.0f;
  if (BF16S) {
    uint32_t bits = f32_to_bf16_rne(scale);
    if (bits == 0) bits = 1;
    scale = bf16_lo(bits);
    if (threadIdx.x == 0) st_global<uint16_t>(scales, at * 2, (uint16_t)bits);
  } else if (threadIdx.x == 0) {
    st_global<float>(scales, at * 4, scale);
  }
  return scale;
}

// One 256-thread block per 128x128 tile (ti, tj), whose scale is element
// ti * tiles_k + tj of the grid.  Vector path: k % 8 == 0, w 16-B aligned
// and codes 8-B aligned.  Thread t owns columns 8*(t%16) .. +7 of rows
// t/16 + 16*i (i = 0..7): each row of the tile is read as 16 x 16 B and
// written as 16 x 8 B, and the tile stays in registers between the amax and
// the encode pass (the bf16 source is read from HBM once).
template <bool BF16S>
__device__ __forceinline__ void block_tile_vec(const uint16_t* __restrict__ w, uint8_t* __restrict__ codes,
                                               void* __restrict__ scales, int n, int k, int ti, int tj,
                                               size_t at) {
  const int col = tj * kTile + (threadIdx.x & 15) * 8;
  const int row0 = ti * kTile + (threadIdx.x >> 4);
  const bool col_ok = col < k;
  uint4 v[8];
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = row0 + 16 * i;
    v[i] = make_uint4(0, 0, 0, 0);
    if (col_ok && row < n) v[i] = ld_stream_u4(w, ((size_t)row * k + col) * 2);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    amax = abs_max_pair(v[i].x, amax);
    amax = abs_max_pair(v[i].y, amax);
    amax = abs_max_pair(v[i].z, amax);
    amax = abs_max_pair(v[i].w, amax);
  }
  amax = block_max_u32(amax);
  const float amax_f = __uint_as_float(amax << 16);
  const float scale = tile_scale<BF16S>(amax_f, scales, at);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = row0 + 16 * i;
    if (col_ok && row < n) {
      uint2 out;
      out.x = encode4_div(v[i].x, v[i].y, scale);
      out.y = encode4_div(v[i].z, v[i].w, scale);
      st_stream_u2(codes, (size_t)row * k + col, out);
    }
  }
}

// Any shape and alignment: element e = t + 256*j (j = 0..63) of the tile,
// row e/128, column e%128, 2-byte loads and 1-byte stores.  The tile is
// read twice (amax, then encode; the second read hits L2) so that the
// grouped kernel, which also runs the 16-byte body, keeps its registers.
template <bool BF16S>
__device__ __forceinline__ void block_tile_any(const uint16_t* __restrict__ w, uint8_t* __restrict__ codes,
                                               void* __restrict__ scales, int n, int k, int ti, int tj,
                                               size_t at) {
  uint32_t amax = 0;
  for (int j = 0; j < 64; ++j) {
    const int e = threadIdx.x + kThreads * j;
    const int row = ti * kTile + (e >> 7), col = tj * kTile + (e & 127);
    if (row < n && col < k) {
      const uint32_t a = w[(size_t)row * k + col] & 0x7FFFu;
      amax = a > amax ? a : amax;
    }
  }
  amax = block_max_u32(amax);
  const float amax_f = __uint_as_float(amax << 16);
  const float scale = tile_scale<BF16S>(amax_f, scales, at);
  for (int j = 0; j < 64; ++j) {
    const int e = threadIdx.x + kThreads * j;
    const int row = ti * kTile + (e >> 7), col = tj * kTile + (e & 127);
    if (row < n && col < k) {
      const size_t i = (size_t)row * k + col;
      codes[i] = (uint8_t)e4m3_code(__uint_as_float((uint32_t)w[i] << 16) / scale);
    }
  }
}

// Single weight: flat block index b -> tile (b / tiles_k, b % tiles_k).
template <bool BF16S>
__global__ __launch_bounds__(kThreads) void k_quant_block_vec(const uint16_t* __restrict__ w,
                                                              uint8_t* __restrict__ codes,
                                                              void* __restrict__ scales, int n,
                                                              int k, int tiles_k) {
  const int ti = blockIdx.x / tiles_k, tj = blockIdx.x % tiles_k;
  block_tile_vec<BF16S>(w, codes, scales, n, k, ti, tj, blockIdx.x);
}

template <bool BF16S>
__global__ __launch_bounds__(kThreads) void k_quant_block_any(const uint16_t* __restrict__ w,
                                                              uint8_t* __restrict__ codes,
                                                              void* __restrict__ scales, int n,
                                                              int k, int tiles_k) {
  const int ti = blockIdx.x / tiles_k, tj = blockIdx.x % tiles_k;
  block_tile_any<BF16S>(w, codes, scales, n, k, ti, tj, blockIdx.x);
}

// 2^-e as an fp32 (e in [-127, 120], so the result is a normal number).
__device__ __forceinline__ float pow2_neg(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }

// MX vector path: k % 32 == 0, w 16-B aligned, codes 8-B aligned.  With k a
// multiple of 32 the groups tile the flat [n*k] array of 8-element units;
// a workgroup takes kMxUnits * 256 consecutive units, thread t units t,
// t + 256, ... (every load instruction reads 4 KB contiguous), and the four
// lanes 4g .. 4g+3 of a pass form one group.  All of a thread's loads are
// issued before any encode, so each wave keeps kMxUnits * 1 KB in flight.
// Two units per thread, graph-captured single calls on MI355X (µs per call,
// 1 / 2 / 3 / 4 / 5 units): [8192x2560] 13.47 / 12.09 / 12.44 / 12.72 /
// 12.97, [2560x3072] 6.48 / 5.91 / 6.07 / 6.17 / 5.97, [6656x2560] 11.37 /
// 10.25 / 10.75 / 10.92 / 11.14; grouped launches +1-2 % over four.
constexpr int kMxUnits = 2;

// Units t0, t0 + 256, ..., t0 + 256 * (kMxUnits - 1) of the flat unit array
// (threads_total units).
__device__ __forceinline__ void mx_units_vec(const uint16_t* __restrict__ w, uint8_t* __restrict__ codes,
                                             uint8_t* __restrict__ e8m0, size_t t0, size_t threads_total) {
  uint4 v[kMxUnits];
#pragma unroll
  for (int u = 0; u < kMxUnits; ++u) {
    const size_t t = t0 + (size_t)u * kThreads;
    v[u] = make_uint4(0, 0, 0, 0);
    if (t < threads_total) v[u] = ld_stream_u4(w, 16 * t);
  }
#pragma unroll
  for (int u = 0; u < kMxUnits; ++u) {
    const size_t t = t0 + (size_t)u * kThreads;
    uint32_t amax = abs_max_pair(v[u].x, 0);
    amax = abs_max_pair(v[u].y, amax);
    amax = abs_max_pair(v[u].z, amax);
    amax = abs_max_pair(v[u].w, amax);
    amax = group_max_u32<4>(amax);
    const int e = e8m0_exponent(amax << 16);
    if (t < threads_total) {
      if ((t & 3) == 0) e8m0[t >> 2] = (uint8_t)(e + 127);
      const float mul = pow2_neg(e);
      uint2 out;
      out.x = encode4_mul(v[u].x, v[u].y, mul);
      out.y = encode4_mul(v[u].z, v[u].w, mul);
      st_stream_u2(codes, 8 * t, out);
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_quant_mx_vec(const uint16_t* __restrict__ w,
                                                           uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ e8m0,
                                                           size_t threads_total) {
  mx_units_vec(w, codes, e8m0, (size_t)blockIdx.x * (kThreads * kMxUnits) + threadIdx.x, threads_total);
}

// MX, any shape: one thread per (row, group), 2-byte loads; t is the flat
// (row, group) index.
__device__ __forceinline__ void mx_group_any(const uint16_t* __restrict__ w, uint8_t* __restrict__ codes,
                                             uint8_t* __restrict__ e8m0, int n, int k, int groups, size_t t) {
  if (t >= (size_t)n * groups) return;
  const size_t row = t / groups;
  const int c0 = (int)(t % groups) * kGroup;
  const int c1 = c0 + kGroup < k ? c0 + kGroup : k;
  const uint16_t* src = w + row * k;
  uint32_t amax = 0;
  for (int c = c0; c < c1; ++c) {
    const uint32_t a = src[c] & 0x7FFFu;
    amax = a > amax ? a : amax;
  }
  const int e = e8m0_exponent(amax << 16);
  e8m0[t] = (uint8_t)(e + 127);
  const float mul = pow2_neg(e);
  for (int c = c0; c < c1; ++c)
    codes[row * k + c] = (uint8_t)e4m3_code(__uint_as_float((uint32_t)src[c] << 16) * mul);
}

__global__ __launch_bounds__(kThreads) void k_quant_mx_any(const uint16_t* __restrict__ w,
                                                           uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ e8m0, int n,
                                                           int k, int groups) {
  mx_group_any(w, codes, e8m0, n, k, groups, (size_t)blockIdx.x * kThreads + threadIdx.x);
}

// ------------------------------------------------------------- grouped --
//
// Many weights in one launch, for load time: the launch's fixed cost (about
// 1.7 us of a graph-captured launch on MI355X) is paid once, and the chip
// streams the whole set as it does one large weight.  Workgroups are dealt
// to the weights in table order (job j owns workgroups [item0_j,
// item0_{j+1})); each workgroup finds its weight by a binary search of the
// table and runs the single-weight body on its tile (block formats) or
// chunk (MX).
__device__ __forceinline__ void find_quant_job(const QuantJob* __restrict__ jobs, int njobs, QuantJob& job,
                                               int& item) {
  const int b = blockIdx.x;
  int lo = 0, hi = njobs - 1;   // last job whose first workgroup is <= b
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (ld_global<int32_t>(jobs, (size_t)mid * sizeof(QuantJob) + offsetof(QuantJob, item0)) <= b)
      lo = mid;
    else
      hi = mid - 1;
  }
  const size_t row = (size_t)lo * sizeof(QuantJob);
  job.w = (const uint16_t*)ld_global<uint64_t>(jobs, row + offsetof(QuantJob, w));
  job.codes = (uint8_t*)ld_global<uint64_t>(jobs, row + offsetof(QuantJob, codes));
  job.scales = (void*)ld_global<uint64_t>(jobs, row + offsetof(QuantJob, scales));
  job.n = ld_global<int32_t>(jobs, row + offsetof(QuantJob, n));
  job.k = ld_global<int32_t>(jobs, row + offsetof(QuantJob, k));
  job.item0 = ld_global<int32_t>(jobs, row + offsetof(QuantJob, item0));
  job.vec = ld_global<int32_t>(jobs, row + offsetof(QuantJob, vec));
  item = b - job.item0;
}

template <bool BF16S>
__global__ __launch_bounds__(kThreads) void k_quant_block_grouped(const QuantJob* __restrict__ jobs, int njobs) {
  QuantJob j;
  int t;
  find_quant_job(jobs, njobs, j, t);
  const int tiles_k = (j.k + kTile - 1) / kTile;
  const int ti = t / tiles_k, tj = t - ti * tiles_k;
  if (j.vec)
    block_tile_vec<BF16S>(j.w, j.codes, j.scales, j.n, j.k, ti, tj, (size_t)t);
  else
    block_tile_any<BF16S>(j.w, j.codes, j.scales, j.n, j.k, ti, tj, (size_t)t);
}

__global__ __launch_bounds__(kThreads) void k_quant_mx_grouped(const QuantJob* __restrict__ jobs, int njobs) {
  QuantJob j;
  int t;
  find_quant_job(jobs, njobs, j, t);
  uint8_t* e8m0 = static_cast<uint8_t*>(j.scales);
  if (j.vec)
    mx_units_vec(j.w, j.codes, e8m0, (size_t)t * (kThreads * kMxUnits) + threadIdx.x, (size_t)j.n * j.k / 8);
  else
    mx_group_any(j.w, j.codes, e8m0, j.n, j.k, (j.k + kGroup - 1) / kGroup, (size_t)t * kThreads + threadIdx.x);
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// ------------------------------------------------------------ per row --
//
// One wave per row, 4 rows per workgroup: scale[r] = amax(row r)/448 (1.0
// for an all-zero row), codes enc(w/scale[r]).  The row is read twice (amax,
// then encode); the second read mostly hits L2.  Vector path when k % 8 == 0
// and w / codes are 16- / 8-byte aligned.
__global__ __launch_bounds__(kThreads) void k_quant_row(const uint16_t* __restrict__ w,
                                                        uint8_t* __restrict__ codes,
                                                        float* __restrict__ scales, int n, int k,
                                                        bool vec) {
  const int lane = threadIdx.x & (kWave - 1);
  const int row = blockIdx.x * (kThreads / kWave) + (int)(threadIdx.x / kWave);
  if (row >= n) return;   // a whole wave; this kernel has no workgroup barrier
  const size_t base = (size_t)row * k;
  uint32_t amax = 0;
  if (vec) {
    for (int c = lane * 8; c < k; c += kWave * 8) {
      const uint4 v = ld_global_u4(w, (base + c) * 2);
      amax = abs_max_pair(v.x, amax);
      amax = abs_max_pair(v.y, amax);
      amax = abs_max_pair(v.z, amax);
      amax = abs_max_pair(v.w, amax);
    }
  } else {
    for (int c = lane; c < k; c += kWave) {
      const uint32_t a = ld_global<uint16_t>(w, (base + c) * 2) & 0x7FFFu;
      amax = a > amax ? a : amax;
    }
  }
  amax = group_max_u32<kWave>(amax);
  const float amax_f = __uint_as_float(amax << 16);
  const float scale = amax_f > 0.0f ? amax_f / 448.0f : 1.0f;
  if (lane == 0) scales[row] = scale;
  if (vec) {
    for (int c = lane * 8; c < k; c += kWave * 8) {
      const uint4 v = ld_global_u4(w, (base + c) * 2);
      st_global<u32x2>(codes, base + c, u32x2{encode4_div(v.x, v.y, scale), encode4_div(v.z, v.w, scale)});
    }
  } else {
    for (int c = lane; c < k; c += kWave)
      codes[base + c] = (uint8_t)e4m3_code(bf16_lo(ld_global<uint16_t>(w, (base + c) * 2)) / scale);
  }
}

// ------------------------------------------------ activation (per tensor) --
//
// Dynamic per-tensor quantization of an activation x [m, k] ("feat(qwen4_exp):
// load-time per-tensor FP8 dense projections", What this adds and its
// perf(fp8) follow-up): one scale fl32(amax/448) for the whole tensor (1.0
// when amax == 0) and codes enc(fl32(x/scale)).  Up to kActSmall elements
// one workgroup does the amax pass and the cast in one launch; above that a
// grid-strided pass writes one partial amax per workgroup (about one 16-byte
// vector per thread, at most kActPartials workgroups, their count a runtime
// argument) and the cast pass reduces the partials in every workgroup.  The maximum is exact in any order, so
// both paths give the same bits.
constexpr int64_t kActSmall = 16384;
constexpr int kActPartials = 256;
constexpr int kActVec = 8;   // elements per 16-byte load

// |x| maximum (as bf16 magnitude bits) over elements [i0 + stride*j ...) of
// this thread, vectorized when `vec`.
__device__ __forceinline__ uint32_t act_amax_range(const uint16_t* __restrict__ x, int64_t count,
                                                   bool vec, int64_t first, int64_t stride) {
  uint32_t amax = 0;
  if (vec) {
    for (int64_t i = first * kActVec; i < count; i += stride * kActVec) {
      const uint4 v = ld_global_u4(x, (size_t)i * 2);
      amax = abs_max_pair(v.x, amax);
      amax = abs_max_pair(v.y, amax);
      amax = abs_max_pair(v.z, amax);
      amax = abs_max_pair(v.w, amax);
    }
  } else {
    for (int64_t i = first; i < count; i += stride) {
      const uint32_t a = ld_global<uint16_t>(x, (size_t)i * 2) & 0x7FFFu;
      amax = a > amax ? a : amax;
    }
  }
  return amax;
}

__device__ __forceinline__ void act_cast_range(const uint16_t* __restrict__ x, int64_t count, bool vec,
                                               int64_t first, int64_t stride, float scale,
                                               uint8_t* __restrict__ codes) {
  if (vec) {
    for (int64_t i = first * kActVec; i < count; i += stride * kActVec) {
      const uint4 v = ld_global_u4(x, (size_t)i * 2);
      st_global<u32x2>(codes, (size_t)i, u32x2{encode4_div(v.x, v.y, scale), encode4_div(v.z, v.w, scale)});
    }
  } else {
    for (int64_t i = first; i < count; i += stride) {
      const uint32_t b = ld_global<uint16_t>(x, (size_t)i * 2);
      codes[i] = (uint8_t)e4m3_code(bf16_lo(b) / scale);
    }
  }
}

__device__ __forceinline__ float act_scale(uint32_t amax_bits) {
  const float amax = bf16_lo(amax_bits);
  return amax > 0.0f ? amax / 448.0f : 1.0f;
}

// One workgroup, count <= kActSmall.  Vector path: thread t holds vectors
// t + 256*j (j < 8) in registers between the amax and the cast, so x is read
// once; the scalar path (odd count or alignment) reads it twice.
__global__ __launch_bounds__(kThreads) void k_act_quant_small(const uint16_t* __restrict__ x, int64_t count,
                                                              bool vec, uint8_t* __restrict__ codes,
                                                              float* __restrict__ scale_out) {
  constexpr int kPer = (int)(kActSmall / kActVec / kThreads);   // 8 vectors per thread
  if (vec) {
    uint4 v[kPer];
    uint32_t amax = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int64_t e = ((int64_t)j * kThreads + threadIdx.x) * kActVec;
      v[j] = e < count ? ld_global_u4(x, (size_t)e * 2) : make_uint4(0, 0, 0, 0);
      amax = abs_max_pair(v[j].x, amax);
      amax = abs_max_pair(v[j].y, amax);
      amax = abs_max_pair(v[j].z, amax);
      amax = abs_max_pair(v[j].w, amax);
    }
    const float scale = act_scale(block_max_u32(amax));
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int64_t e = ((int64_t)j * kThreads + threadIdx.x) * kActVec;
      if (e < count)
        st_global<u32x2>(codes, (size_t)e, u32x2{encode4_div(v[j].x, v[j].y, scale), encode4_div(v[j].z, v[j].w, scale)});
    }
    if (threadIdx.x == 0) *scale_out = scale;
    return;
  }
  const uint32_t amax = block_max_u32(act_amax_range(x, count, false, threadIdx.x, kThreads));
  const float scale = act_scale(amax);
  act_cast_range(x, count, false, threadIdx.x, kThreads, scale, codes);
  if (threadIdx.x == 0) *scale_out = scale;
}

__global__ __launch_bounds__(kThreads) void k_act_amax_partial(const uint16_t* __restrict__ x, int64_t count,
                                                               bool vec, uint32_t* __restrict__ partial) {
  const uint32_t amax = block_max_u32(act_amax_range(
      x, count, vec, (int64_t)blockIdx.x * kThreads + threadIdx.x, (int64_t)gridDim.x * kThreads));
  if (threadIdx.x == 0) st_global<uint32_t>(partial, (size_t)blockIdx.x * 4, amax);
}

__global__ __launch_bounds__(kThreads) void k_act_quant_cast(const uint16_t* __restrict__ x, int64_t count,
                                                             bool vec, const uint32_t* __restrict__ partial,
                                                             int partials, uint8_t* __restrict__ codes,
                                                             float* __restrict__ scale_out) {
  const uint32_t p = (int)threadIdx.x < partials ? ld_global<uint32_t>(partial, (size_t)threadIdx.x * 4) : 0u;
  const float scale = act_scale(block_max_u32(p));
  act_cast_range(x, count, vec, (int64_t)blockIdx.x * kThreads + threadIdx.x, (int64_t)gridDim.x * kThreads,
                 scale, codes);
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale_out = scale;
}

// Partial maxima of fp8w_quantize_act_noalloc, for callers that cannot
// allocate: a file-scope array, one copy per device for the life of the
// process.  Host code never passes the name itself to a kernel (on the host
// it is a stand-in, not a device address): act_scratch() resolves the
// device's own address once and every launch takes that pointer.
static __device__ __align__(256) uint32_t scratch[kActPartials];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
std::atomic<uint32_t*> g_scratch[kMaxDevices];

// This device's address of `scratch`, resolved on the first call with the
// device current (hipGetSymbolAddress) and kept per device.
hipError_t act_scratch(uint32_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  uint32_t* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* addr = nullptr;
      e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!addr) return hipErrorInvalidSymbol;
      p = static_cast<uint32_t*>(addr);
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

// Workgroups of the amax pass (= partial maxima written) for `count` elements.
int act_partials_for(int64_t count) {
  const int64_t want = (count + kThreads * kActVec - 1) / (kThreads * kActVec);
  return (int)(want < kActPartials ? want : kActPartials);
}

}  // namespace

int act_quant_partials() { return kActPartials; }

hipError_t launch_quantize_act_noalloc(const uint16_t* x, int64_t count, uint8_t* codes, float* scale,
                                       hipStream_t stream) {
  uint32_t* ws = nullptr;
  const hipError_t e = act_scratch(&ws);
  if (e != hipSuccess) return e;
  // every size fits: the amax pass never uses more partials than the array holds
  if (count > kActSmall && act_partials_for(count) > kActPartials) return hipErrorInvalidValue;
  return launch_quantize_act(x, count, codes, scale, ws, stream);
}

hipError_t launch_quantize_act(const uint16_t* x, int64_t count, uint8_t* codes, float* scale,
                               uint32_t* workspace, hipStream_t stream) {
  const bool vec = count % kActVec == 0 && aligned(x, 16) && aligned(codes, 8);
  if (count <= kActSmall) {
    hipLaunchKernelGGL(k_act_quant_small, dim3(1), dim3(kThreads), 0, stream, x, count, vec, codes, scale);
    return hipGetLastError();
  }
  // about one 16-byte vector per thread per pass: the passes are latency-bound
  const int partials = act_partials_for(count);
  hipLaunchKernelGGL(k_act_amax_partial, dim3(partials), dim3(kThreads), 0, stream, x, count, vec, workspace);
  const int64_t per_block = (int64_t)kThreads * kActVec;
  const int64_t cast_blocks = (count + per_block - 1) / per_block;
  hipLaunchKernelGGL(k_act_quant_cast, dim3((unsigned)(cast_blocks < 65535 ? cast_blocks : 65535)),
                     dim3(kThreads), 0, stream, x, count, vec, workspace, partials, codes, scale);
  return hipGetLastError();
}

template <bool BF16S>
hipError_t quantize_block_tiles(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes, void* scales,
                                hipStream_t stream) {
  const int64_t tiles_n = (n + kTile - 1) / kTile, tiles_k = (k + kTile - 1) / kTile;
  const dim3 grid((unsigned)(tiles_n * tiles_k)), block(kThreads);
  if (k % 8 == 0 && aligned(w, 16) && aligned(codes, 8))
    hipLaunchKernelGGL((k_quant_block_vec<BF16S>), grid, block, 0, stream, w, codes, scales, (int)n, (int)k,
                       (int)tiles_k);
  else
    hipLaunchKernelGGL((k_quant_block_any<BF16S>), grid, block, 0, stream, w, codes, scales, (int)n, (int)k,
                       (int)tiles_k);
  return hipGetLastError();
}

hipError_t launch_quantize_block(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes,
                                 float* scales, hipStream_t stream) {
  return quantize_block_tiles<false>(w, n, k, codes, scales, stream);
}

hipError_t launch_quantize_block_bf16(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes,
                                      uint16_t* scales, hipStream_t stream) {
  return quantize_block_tiles<true>(w, n, k, codes, scales, stream);
}

hipError_t launch_quantize_row(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes, float* scales,
                               hipStream_t stream) {
  const bool vec = k % 8 == 0 && aligned(w, 16) && aligned(codes, 8);
  const int rows_per_block = kThreads / kWave;
  hipLaunchKernelGGL(k_quant_row, dim3((unsigned)((n + rows_per_block - 1) / rows_per_block)), dim3(kThreads),
                     0, stream, w, codes, scales, (int)n, (int)k, vec);
  return hipGetLastError();
}

hipError_t launch_quantize_mx(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes,
                              uint8_t* e8m0, hipStream_t stream) {
  const int64_t groups = (k + kGroup - 1) / kGroup;
  if (k % kGroup == 0 && aligned(w, 16) && aligned(codes, 8)) {
    const size_t threads_total = (size_t)n * k / 8;
    const dim3 grid((unsigned)((threads_total + kThreads * kMxUnits - 1) / (kThreads * kMxUnits)));
    hipLaunchKernelGGL(k_quant_mx_vec, grid, dim3(kThreads), 0, stream, w, codes, e8m0,
                       threads_total);
  } else {
    const size_t total = (size_t)n * groups;
    const dim3 grid((unsigned)((total + kThreads - 1) / kThreads));
    hipLaunchKernelGGL(k_quant_mx_any, grid, dim3(kThreads), 0, stream, w, codes, e8m0, (int)n,
                       (int)k, (int)groups);
  }
  return hipGetLastError();
}

int64_t quant_job_blocks(int format, int64_t n, int64_t k, bool vec) {
  if (format == kFmtMx) {
    if (vec) return (n * k / 8 + kThreads * kMxUnits - 1) / (kThreads * kMxUnits);
    return (n * ((k + kGroup - 1) / kGroup) + kThreads - 1) / kThreads;
  }
  return ((n + kTile - 1) / kTile) * ((k + kTile - 1) / kTile);
}

bool quant_job_vec(int format, const void* w, int64_t k, const void* codes) {
  if (format == kFmtMx) return k % kGroup == 0 && aligned(w, 16) && aligned(codes, 8);
  return k % 8 == 0 && aligned(w, 16) && aligned(codes, 8);
}

hipError_t launch_quantize_grouped(const QuantJob* table, int njobs, int64_t blocks, int format,
                                   hipStream_t stream) {
  const dim3 grid((unsigned)blocks), block(kThreads);
  switch (format) {
    case kFmtBlock:
      hipLaunchKernelGGL(k_quant_block_grouped<false>, grid, block, 0, stream, table, njobs);
      break;
    case kFmtBlockBf16:
      hipLaunchKernelGGL(k_quant_block_grouped<true>, grid, block, 0, stream, table, njobs);
      break;
    case kFmtMx:
      hipLaunchKernelGGL(k_quant_mx_grouped, grid, block, 0, stream, table, njobs);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fp8w
