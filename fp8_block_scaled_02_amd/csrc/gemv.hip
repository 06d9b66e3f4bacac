// gemv.hip -- W8A16 (and W8A8) decode GEMV / skinny GEMM for gfx950.
//
// y[m][n] = bf16( sum_k x[m][k] * dec(code[n][k]) * scale(n, k) ), fp32
// accumulation, for 1 <= M <= 32.  The fp8 weight stream dominates the
// traffic, so every kernel reads each code byte once with 16-byte loads and
// converts e4m3 -> bf16 in registers (exact: 4 significant bits); x (at most
// 32 rows) is re-read from LDS or from L2.  Two kernel families, split on M
// as the fused W8A16 GEMM of "feat: add FP8 blockwise weight quantization
// and FP8(E4M3) KV cache support" (Summary; Notes for Reviewers) splits its
// SIMT and tensor-core routes:
//
//  * VALU (M <= 8): v_dot2c_f32_bf16 products; the 64 lanes of a wave walk
//    rows along K, and the wave's partial sums are folded four at a time
//    with lane-swap and DPP row operations (no LDS round trips).
//    k_gemv_valu: one tile of rows per workgroup, K in segments staged
//    with x in LDS.  k_gemv_valu_stream (M = 1, K <= 3072): a contiguous
//    run of 16-row tiles per workgroup, the next tile's codes requested
//    before the current one is computed.  k_gemv_valu_rows (single calls,
//    M <= 4, fewer than 16384 rows): one wave per workgroup, a few rows per
//    wave, x held in registers.
//  * MFMA (M <= 32): v_mfma_f32_16x16x32_bf16 on 16-row tiles of W against
//    x^T padded to 16 or 32 columns.  Codes reach the A layout through a
//    per-wave LDS transpose of 16-row x 256-byte panels.  k_gemv_mfma_direct
//    (single calls): one 16-row tile per workgroup (two above M = 8,
//    sharing each x^T fragment), its 4 or 8 waves splitting the panels, x
//    fragments from L2.
//    k_gemv_mfma_stream16 / k_gemv_mfma_stream32 (up to 16 / 17..32 rows):
//    runs of 128-row tiles, one 16-row tile per wave, x staged in LDS by K
//    segments (one buffer / two, the next segment prefetched).
//    k_gemv_mfma_xreg (single calls, 17..32 rows, K of eight panels): runs
//    of 16-row tiles, wave w taking panel w of each, its x^T fragments held
//    in registers for the whole run, partial sums met in LDS per tile.
//  * W8A8: fp8 x fp8 v_mfma_scale_f32_16x16x128_f8f6f4 (k_gemv_w8a8_direct,
//    and k_gemv_w8a8_tiles on weights with many rows), and k_gemv_valu with
//    the activation codes widened to bf16 at M <= 2.
//
// Each call is a few microseconds of HBM traffic, so latency decides the
// time: every kernel keeps its weight loads (non-temporal: each code byte
// is read once) in flight while x is staged.  Vector-memory waits count in
// issue order, so what must be ready first is requested first: the
// per-tile VALU kernel requests x and the scales just before the codes,
// and scale bytes are kept as loaded and converted where they are used.
//
// A launch covers either one GEMV (the job travels as a kernel argument) or
// a group of independent GEMVs (a job table in device memory; a workgroup
// finds its job by binary search on the jobs' first tile index), which
// removes the fixed per-launch cost from a sequence of small GEMVs.  Single
// calls on weights with many rows run the streaming kernels with their one
// job passed by value.
//
// Block scales: one fp32 per 128x128 tile.  A 16-byte code chunk never
// straddles a 128-column block and a workgroup's rows never straddle a
// 128-row block, so the scale multiplies a chunk's (VALU) or a 128-column
// block's (MFMA) partial sum.  MX scales: 2^(E-127) per row and 32 columns.
// A 16-byte chunk lies in one group, so the VALU route scales the chunk's
// fp32 partial sum by the exactly built fp32 2^(E-127); the MFMA route
// multiplies the decoded codes by it in fp32 (exact) and rounds to bf16 for
// the A operand (exact while the product is a normal bf16).  Dequantized
// weights must be finite in fp32 (|deq| < 2^128): only e8m0 bytes >= 247,
// i.e. weights within 0.4 % of the bf16 maximum, can break that.  Row and
// tensor scales multiply each output.
#include <hip/hip_runtime.h>

#include <atomic>
#include <stddef.h>
#include <type_traits>

#include "device.hpp"
#include "internal.hpp"

namespace fp8w {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

// The lane index, recomputed at every call (an opaque v_mbcnt pair): kernels
// at the register limit otherwise keep lane-derived row indices live from the
// start, and spill them.
__device__ __forceinline__ int lane_fresh() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// 2^(e - 127) as an exact fp32: a normal number for e >= 1, the subnormal
// 2^-127 for e == 0.
__device__ __forceinline__ float mx_scale(uint8_t e) {
  return __uint_as_float(e ? (uint32_t)e << 23 : 0x00400000u);
}

// Two e4m3 codes (bytes 0,1 or 2,3 of d) -> two bf16 (exact).
__device__ __forceinline__ bf16x2 cvt_lo(uint32_t d) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d, 1.0f, false);
}
__device__ __forceinline__ bf16x2 cvt_hi(uint32_t d) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d, 1.0f, true);
}

// Two e4m3 codes times the MX scale s = 2^(E-127), rounded to bf16, in one
// instruction.  Measured on MI355X over every code and every e8m0 byte
// 0..254: bit-identical to rounding fp32(code) * s (exact in fp32) to bf16;
// byte 255, E8M0's NaN, gives NaN where that product would be infinite (a
// non-finite weight, outside the contract either way).
template <bool HI>
__device__ __forceinline__ bf16x2 cvt_scaled(uint32_t d, float s) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d, s, HI);
}

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t d) { return __builtin_bit_cast(bf16x2, d); }

// Non-MX scale formats.  The scale of 128-column block kb for the 128-row
// block holding row0 (fp32 or bf16 grid), or 1 when the format scales whole
// rows or the whole weight -- those multiply each output once, at the end.
// The format is uniform across a launch, so the branches cost nothing.
__device__ __forceinline__ float block_scale(const GemvJob& j, int row0, int kb, int nkb) {
  const size_t at = (size_t)(row0 / kTile) * nkb + kb;
  if (j.format == kFmtBlock) return ld_global<float>(j.scales, at * 4);
  if (j.format == kFmtBlockBf16) return bf16_lo(ld_global<uint16_t>(j.scales, at * 2));
  return 1.0f;
}
__device__ __forceinline__ float output_scale(const GemvJob& j, int row) {
  if (j.format == kFmtRow) return ld_global<float>(j.scales, (size_t)row * 4);
  if (j.format == kFmtTensor) return ld_global<float>(j.scales, 0);
  return 1.0f;
}

// Index into the block-scale grid of 128-column block kb for the 128-row
// block holding row0, both clamped into the grid: kernels that request the
// scale ahead of its use load it unconditionally from here (a load behind a
// branch, or joined with a default, gets a copy after the join, and the copy
// waits for the load -- and, since vector-memory waits count in issue order,
// for every load the wave issued before it).
__device__ __forceinline__ size_t block_scale_at(const GemvJob& j, int row0, int kb, int nkb) {
  return (size_t)(min(row0, j.n - 1) / kTile) * nkb + min(kb, nkb - 1);
}

// sum_j x[j] * dec(code[j]) over one 16-byte chunk (16 codes, 16 bf16 x).
__device__ __forceinline__ float dot16(const bf16x2 (&w)[8], uint4 x0, uint4 x1) {
  float p = 0.0f;
  p = __builtin_amdgcn_fdot2_f32_bf16(w[0], as_bf16x2(x0.x), p, false);
  p = __builtin_amdgcn_fdot2_f32_bf16(w[1], as_bf16x2(x0.y), p, false);
  p = __builtin_amdgcn_fdot2_f32_bf16(w[2], as_bf16x2(x0.z), p, false);
  p = __builtin_amdgcn_fdot2_f32_bf16(w[3], as_bf16x2(x0.w), p, false);
  p = __builtin_amdgcn_fdot2_f32_bf16(w[4], as_bf16x2(x1.x), p, false);
  p = __builtin_amdgcn_fdot2_f32_bf16(w[5], as_bf16x2(x1.y), p, false);
  p = __builtin_amdgcn_fdot2_f32_bf16(w[6], as_bf16x2(x1.z), p, false);
  p = __builtin_amdgcn_fdot2_f32_bf16(w[7], as_bf16x2(x1.w), p, false);
  return p;
}

// Four wave-wide sums at once: returns, in every lane of 16-lane row q, the
// sum over the 64 lanes of the q-th argument.  v_permlane32_swap folds the
// upper half-wave onto the lower one for two values per instruction pair
// (after it, lanes 0-31 carry a0 + ... and lanes 32-63 carry a2 + ...);
// v_permlane16_swap then does the same between the 16-lane rows, leaving
// value q in row q, summed over the four lanes {j, j+16, j+32, j+48}; four DPP
// steps inside each row (quad_perm [1,0,3,2] and [2,3,0,1], row half mirror,
// row mirror) finish the sums.  10 instructions for 4 values, against 7 per
// value for a separate butterfly and readlane.
#define FP8W_DPP_ADD(v, ctrl)                                                                   \
  (v) += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, (v)), \
                                                               (ctrl), 0xF, 0xF, false))
__device__ __forceinline__ float fold_halves(float a, float b, bool rows16) {
  const auto r = rows16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false)
                        : __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float wave_sum4(float a0, float a1, float a2, float a3) {
  const float t02 = fold_halves(a0, a2, false);   // lanes 0-31: a0, lanes 32-63: a2
  const float t13 = fold_halves(a1, a3, false);   // lanes 0-31: a1, lanes 32-63: a3
  float v = fold_halves(t02, t13, true);          // row q: a_q
  FP8W_DPP_ADD(v, 0xB1);    // quad_perm [1,0,3,2]
  FP8W_DPP_ADD(v, 0x4E);    // quad_perm [2,3,0,1]
  FP8W_DPP_ADD(v, 0x141);   // row_half_mirror
  FP8W_DPP_ADD(v, 0x140);   // row_mirror
  return v;
}
#undef FP8W_DPP_ADD

// Wave sums of V values v[0..V) (any V): value f ends in every lane of row
// f % 4 of the returned group f / 4.
template <int V>
struct WaveSums {
  static constexpr int kGroups = (V + 3) / 4;
  float g[kGroups];
  __device__ __forceinline__ explicit WaveSums(const float (&v)[V]) {
#pragma unroll
    for (int q = 0; q < kGroups; ++q) {
      const float a0 = v[4 * q];
      const float a1 = 4 * q + 1 < V ? v[(4 * q + 1) % V] : 0.0f;
      const float a2 = 4 * q + 2 < V ? v[(4 * q + 2) % V] : 0.0f;
      const float a3 = 4 * q + 3 < V ? v[(4 * q + 3) % V] : 0.0f;
      g[q] = wave_sum4(a0, a1, a2, a3);
    }
  }
};

// The job of this workgroup and the index of its tile within the job.
template <bool GROUPED>
__device__ __forceinline__ void find_job(const GemvJob& arg, const GemvJob* __restrict__ jobs,
                                         int njobs, GemvJob& job, int& tile) {
  if (!GROUPED) {
    job = arg;
    tile = blockIdx.x;
    return;
  }
  const int b = blockIdx.x;
  int lo = 0, hi = njobs - 1;   // last job whose first workgroup is <= b
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (ld_global<int32_t>(jobs, (size_t)mid * sizeof(GemvJob) + offsetof(GemvJob, item0)) <= b)
      lo = mid;
    else
      hi = mid - 1;
  }
  const size_t row = (size_t)lo * sizeof(GemvJob);
  job.x = (const uint16_t*)ld_global<uint64_t>(jobs, row + offsetof(GemvJob, x));
  job.codes = (const uint8_t*)ld_global<uint64_t>(jobs, row + offsetof(GemvJob, codes));
  job.scales = (const void*)ld_global<uint64_t>(jobs, row + offsetof(GemvJob, scales));
  job.y = (uint16_t*)ld_global<uint64_t>(jobs, row + offsetof(GemvJob, y));
  job.n = ld_global<int32_t>(jobs, row + offsetof(GemvJob, n));
  job.k = ld_global<int32_t>(jobs, row + offsetof(GemvJob, k));
  job.item0 = ld_global<int32_t>(jobs, row + offsetof(GemvJob, item0));
  job.format = ld_global<int32_t>(jobs, row + offsetof(GemvJob, format));
  tile = b - job.item0;
}

// A workgroup-wide copy of `total` units into LDS: unit u is fetched by
// load(u) and written by store(u, v).  Each thread issues the loads of up to
// kBatch units before the first of their stores, so a staging pass waits on
// memory once per batch rather than once per unit.  (Vector-memory waits
// count in issue order, so a wait for one unit also waits for every weight
// load a wave issued before it: a pass of one-unit round trips would drain
// the weight stream once per unit.)
template <int kBatch, int kStride, typename T, typename Load, typename Store>
__device__ __forceinline__ void copy_batched(int total, Load load, Store store) {
  for (int base = threadIdx.x; base < total; base += kBatch * kStride) {
    T v[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q)
      if (base + q * kStride < total) v[q] = load(base + q * kStride);
#pragma unroll
    for (int q = 0; q < kBatch; ++q)
      if (base + q * kStride < total) store(base + q * kStride, v[q]);
  }
}

// Units of the staging copies in flight per thread.
constexpr int kStageBatch = 4;

// x[0, 0:k] (one activation row, k a multiple of 8) into LDS.
__device__ __forceinline__ void stage_row(const uint16_t* __restrict__ x, int k, uint16_t* xs) {
  copy_batched<kStageBatch, kThreads, uint4>(
      k / 8, [&](int u) { return ld_global_u4(x, (size_t)u * 16); },
      [&](int u, uint4 v) { *reinterpret_cast<uint4*>(xs + u * 8) = v; });
}

// ------------------------------------------------------------------ VALU --
//
// Workgroup = 4 waves x R rows.  Wave w owns rows row0 + r (r < R); lane l
// takes the 16-byte chunks l, l + 64, ..., of each K segment (C chunks per
// lane, so a segment is 1024*C columns).  Per segment: x and the block
// scales (or MX exponents) are requested, then the codes of all R rows;
// the staged values reach LDS while the codes are in flight, and the
// segment is accumulated chunk by chunk as its codes arrive.
template <int M, int R, int C>
struct ValuShape {
  static constexpr int kRows = kWaves * R;
  static constexpr int kSeg = 1024 * C;
  static constexpr int kSegGroups = kSeg / kGroup;   // MX exponents per row and segment
  static constexpr int kLdsX = M * kSeg * 2;
  static constexpr int kLdsScales = (kSeg / kTile) * 4;
  static constexpr int kLdsBytes = kLdsX + (kLdsScales > kRows * kSegGroups ? kLdsScales : kRows * kSegGroups);
  // staging loads per thread and segment: 8-element x units (at most 8 in
  // registers; a larger M stages the rest after the codes) and MX exponents
  static constexpr int kXUnits = (M * kSeg / 8 + kThreads - 1) / kThreads;
  static constexpr int kXPre = kXUnits < 8 ? kXUnits : 8;
  static constexpr int kExpPre = (kRows * kSegGroups + kThreads - 1) / kThreads;
  static_assert(kTile % kRows == 0, "a workgroup must stay inside one 128-row block");
  static_assert(kLdsBytes <= 64 * 1024, "LDS budget");
};

// The segment's codes, every load unconditional: rows past n read row n-1
// and chunks past nch read chunk nch-1; the accumulation skips those chunks
// and the store skips those rows.  (A conditional load is one the compiler
// cannot count, and it then waits for every load before the staged x can
// be written to LDS; unconditional loads let it wait for exactly the ones
// it needs.)
// rows[r]: the codes of row min(row0 + r, n - 1), computed once per tile.
template <int R, int C>
__device__ __forceinline__ void valu_load(const uint8_t* const (&rows)[R], int seg0, int nch, uint4 (&wv)[R][C]) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int off = seg0 + 16 * min(lane + kWave * c, nch - 1);
#pragma unroll
    for (int r = 0; r < R; ++r) wv[r][c] = ld_stream_u4(rows[r], off);
  }
}

// u / d for a d that is the compile-time D on every full segment (only the
// last segment of a row has another length): the constant divides with a
// multiply, and the runtime divide runs once per launch at most.
template <int D>
__device__ __forceinline__ int div_seg(int u, int d) {
  return d == D ? u / D : u / d;
}

// What one K segment stages in LDS besides the codes: x (bf16, or e4m3
// codes widened to bf16 for X8) and the block scales or MX exponents.  The
// loads are issued before the segment's codes (load) and written to LDS
// after them (commit): vector-memory waits count in issue order, so staging
// loads issued after the codes could only be written once every code had
// arrived; issued first, x and the scales reach LDS while the codes are
// still in flight.  Loads are unconditional, from indices clamped into
// their arrays; commit writes only the valid ones.
template <int M, int R, int C, bool MX, bool X8>
struct SegStage {
  using S = ValuShape<M, R, C>;
  using XU = typename std::conditional<X8, u32x2, uint4>::type;   // 8 elements of x
  XU x[S::kXPre];
  uint32_t e[MX ? S::kExpPre : 1];      // MX: exponent bytes
  uint16_t lo, hi;                      // block grids: the scale's 16-bit halves

  // unit u of the segment's [M][len / 8] grid of 8-element x units
  static __device__ __forceinline__ void unit_rc(int u, int units, int& r, int& c) {
    if constexpr (M == 1) {
      r = 0;
      c = u * 8;
    } else {
      r = div_seg<S::kSeg / 8>(u, units);
      c = (u - r * units) * 8;
    }
  }

  __device__ __forceinline__ void load(const GemvJob& j, int tile, int seg0, int len, int tiles_k, int groups) {
    const int units = len / 8, total = M * units;
#pragma unroll
    for (int q = 0; q < S::kXPre; ++q) {
      const int u = min((int)threadIdx.x + q * kThreads, total - 1);
      int r, c;
      unit_rc(u, units, r, c);
      if constexpr (X8) x[q] = ld_x8(j, (size_t)r * j.k + seg0 + c);
      else x[q] = ld_x16(j, ((size_t)r * j.k + seg0 + c) * 2);
    }
    if (MX) {
      const int ng = (len + kGroup - 1) / kGroup, gs = seg0 / kGroup;
#pragma unroll
      for (int q = 0; q < S::kExpPre; ++q) {
        const int u = min((int)threadIdx.x + q * kThreads, S::kRows * ng - 1);
        const int r = div_seg<S::kSegGroups>(u, ng), g = u - r * ng;
        const int row = min(tile * S::kRows + r, j.n - 1);
        e[q] = ld_global<uint8_t>(j.scales, (size_t)row * groups + gs + g);
      }
    } else {
      // fp32 grid: both halves of the scale; bf16 grid: its bits are the
      // high half; row and tensor scales (applied at the store) read the
      // array's first word and stage 1
      const int nkb = (len + kTile - 1) / kTile;
      const size_t at = (size_t)((tile * S::kRows) / kTile) * tiles_k + seg0 / kTile +
                        min((int)threadIdx.x, nkb - 1);
      const bool f32 = j.format == kFmtBlock, b16 = j.format == kFmtBlockBf16;
      lo = ld_global<uint16_t>(j.scales, f32 ? at * 4 : 0);
      hi = ld_global<uint16_t>(j.scales, f32 ? at * 4 + 2 : (b16 ? at * 2 : 0));
    }
  }

  __device__ __forceinline__ void commit(const GemvJob& j, int tile, int seg0, int len, int groups,
                                         uint16_t* xs, float* ss, unsigned char* ex) const {
    const int units = len / 8, total = M * units;
#pragma unroll
    for (int q = 0; q < S::kXPre; ++q) {
      const int u = (int)threadIdx.x + q * kThreads;
      int r, c;
      unit_rc(u, units, r, c);
      if (u < total) *reinterpret_cast<uint4*>(xs + r * S::kSeg + c) = widen(x[q]);
    }
    for (int u = (int)threadIdx.x + S::kXPre * kThreads; u < total; u += kThreads) {   // M beyond the registers
      int r, c;
      unit_rc(u, units, r, c);
      if constexpr (X8) *reinterpret_cast<uint4*>(xs + r * S::kSeg + c) = widen(ld_x8(j, (size_t)r * j.k + seg0 + c));
      else *reinterpret_cast<uint4*>(xs + r * S::kSeg + c) = ld_x16(j, ((size_t)r * j.k + seg0 + c) * 2);
    }
    if (MX) {
      const int ng = (len + kGroup - 1) / kGroup;
#pragma unroll
      for (int q = 0; q < S::kExpPre; ++q) {
        const int u = (int)threadIdx.x + q * kThreads;
        const int r = div_seg<S::kSegGroups>(u, ng), g = u - r * ng;
        if (u < S::kRows * ng) ex[r * S::kSegGroups + g] = (unsigned char)e[q];
      }
    } else {
      const int nkb = (len + kTile - 1) / kTile;
      if ((int)threadIdx.x < nkb)
        ss[threadIdx.x] = j.format == kFmtBlock       ? __uint_as_float((uint32_t)hi << 16 | lo)
                          : j.format == kFmtBlockBf16 ? __uint_as_float((uint32_t)hi << 16)
                                                      : 1.0f;
    }
    (void)tile;
    (void)groups;
  }

 private:
  static __device__ __forceinline__ u32x2 ld_x8(const GemvJob& j, size_t off) { return ld_global<u32x2>(j.x, off); }
  static __device__ __forceinline__ uint4 ld_x16(const GemvJob& j, size_t off) { return ld_global_u4(j.x, off); }
  // x as staged: bf16 passes through; e4m3 codes widen to bf16 (exact)
  static __device__ __forceinline__ uint4 widen(uint4 v) { return v; }
  static __device__ __forceinline__ uint4 widen(u32x2 v) {
    const bf16x2 a = cvt_lo(v.x), b = cvt_hi(v.x), d = cvt_lo(v.y), f = cvt_hi(v.y);
    return make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                      __builtin_bit_cast(uint32_t, d), __builtin_bit_cast(uint32_t, f));
  }
};

// X8: the activation is e4m3 codes (j.x points at bytes) with the fp32
// tensor scale at *xscale (the W8A8 path at small m): the codes are widened
// to bf16 while x is staged and the outputs are multiplied by the scale.
template <int M, int R, int C, bool MX, bool GROUPED, bool X8 = false>
__global__ __launch_bounds__(kThreads) void k_gemv_valu(GemvJob arg, const GemvJob* __restrict__ jobs,
                                                        int njobs, const float* __restrict__ xscale = nullptr) {
  using S = ValuShape<M, R, C>;
  __shared__ __align__(16) unsigned char smem[S::kLdsBytes];
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  float* ss = reinterpret_cast<float*>(smem + S::kLdsX);            // block: the segment's block scales
  unsigned char* ex = smem + S::kLdsX;                               // MX: [kRows][kSegGroups] exponents

  GemvJob j;
  int tile;
  find_job<GROUPED>(arg, jobs, njobs, j, tile);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int row0 = tile * S::kRows + wave * R;
  const int tiles_k = (j.k + kTile - 1) / kTile;
  const int groups = (j.k + kGroup - 1) / kGroup;

  float acc[R][M];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;
  const uint8_t* rows[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rows[r] = j.codes + (size_t)min(row0 + r, j.n - 1) * j.k;

  for (int seg0 = 0; seg0 < j.k; seg0 += S::kSeg) {
    const int len = min(S::kSeg, j.k - seg0);
    const int nch = len / 16;
    SegStage<M, R, C, MX, X8> st;
    st.load(j, tile, seg0, len, tiles_k, groups);
    uint4 cw[R][C];
    valu_load<R, C>(rows, seg0, nch, cw);
    if (seg0 > 0) __syncthreads();   // the previous segment's LDS reads are done
    st.commit(j, tile, seg0, len, groups, xs, ss, ex);
    __syncthreads();

    for (int c = 0; c < C; ++c) {
      const int ch = lane + kWave * c;
      if (ch < nch) {
        uint4 x0[M], x1[M];
#pragma unroll
        for (int m = 0; m < M; ++m) {
          x0[m] = *reinterpret_cast<const uint4*>(xs + m * S::kSeg + ch * 16);
          x1[m] = *reinterpret_cast<const uint4*>(xs + m * S::kSeg + ch * 16 + 8);
        }
        const float bs = MX ? 0.0f : ss[ch >> 3];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint4 d = cw[r][c];
          const bf16x2 w[8] = {cvt_lo(d.x), cvt_hi(d.x), cvt_lo(d.y), cvt_hi(d.y),
                               cvt_lo(d.z), cvt_hi(d.z), cvt_lo(d.w), cvt_hi(d.w)};
          const float s = MX ? mx_scale(ex[(wave * R + r) * S::kSegGroups + ch / 2]) : bs;
#pragma unroll
          for (int m = 0; m < M; ++m) acc[r][m] = __builtin_fmaf(s, dot16(w, x0[m], x1[m]), acc[r][m]);
        }
      }
    }
  }

  float flat[R * M];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) flat[r * M + m] = acc[r][m];
  const WaveSums<R * M> sums(flat);
  const float xf = X8 ? ld_global<float>(xscale, 0) : 1.0f;
  if ((lane & 15) == 0) {
#pragma unroll
    for (int q = 0; q < WaveSums<R * M>::kGroups; ++q) {
      const int f = 4 * q + (lane >> 4);   // value index r * M + m held by this row
      const int r = f / M, m = f % M;
      if (f < R * M && row0 + r < j.n) {
        const float v = sums.g[q] * output_scale(j, row0 + r);
        st_global<uint16_t>(j.y, ((size_t)m * j.n + row0 + r) * 2, (uint16_t)f32_to_bf16_rne(X8 ? v * xf : v));
      }
    }
  }
}

// ------------------------------------------------- VALU, rows per wave --
//
// Single calls at M <= 4 on weights with fewer rows than the streaming
// threshold and K <= 4096 (K <= 3072 at M > 1): one wave per workgroup, R
// rows per wave, and each lane's x chunks (32 bytes per 16-code chunk and
// activation row) loaded straight into registers, shared by the wave's R
// rows.  No LDS and no barrier: on
// MI355X, staging x through LDS with a workgroup barrier cost about 0.8 us
// of a 4.6 us call over a bare read of the same codes (graph-captured
// projection-set calls), and loading x per wave costs about half of that
// once R >= 2 rows share it.  x is requested before the codes.
template <int R, int C, bool MX, int M>
__global__ __launch_bounds__(kWave) void k_gemv_valu_rows(GemvJob j) {
  static_assert(kTile % R == 0, "a wave's rows stay inside one 128-row block");
  const int lane = threadIdx.x & (kWave - 1);
  const int row0 = blockIdx.x * R;
  const int nch = j.k / 16;
  const int nkb = (j.k + kTile - 1) / kTile, groups = (j.k + kGroup - 1) / kGroup;
  int ch[C];
#pragma unroll
  for (int c = 0; c < C; ++c) ch[c] = min(lane + kWave * c, nch - 1);
  uint4 x0[M][C], x1[M][C];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const size_t off = ((size_t)m * j.k + 16 * (size_t)ch[c]) * 2;
      x0[m][c] = ld_global_u4(j.x, off);
      x1[m][c] = ld_global_u4(j.x, off + 16);
    }
  const uint8_t* rows[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rows[r] = j.codes + (size_t)min(row0 + r, j.n - 1) * j.k;
  uint4 w[R][C];
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int r = 0; r < R; ++r) w[r][c] = ld_stream_u4(rows[r], 16 * ch[c]);
  float sc[MX ? 1 : C];
  uint32_t e[MX ? R : 1][MX ? C : 1];
  if (MX) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int c = 0; c < C; ++c)
        e[r][c] = ld_global<uint8_t>(j.scales, (size_t)min(row0 + r, j.n - 1) * groups + ch[c] / 2);
  } else {
#pragma unroll
    for (int c = 0; c < C; ++c) sc[c] = block_scale(j, min(row0, j.n - 1), ch[c] >> 3, nkb);
  }
  float acc[R * M];   // row r, activation row m at r * M + m
#pragma unroll
  for (int f = 0; f < R * M; ++f) acc[f] = 0.0f;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    if (lane + kWave * c < nch) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint4 d = w[r][c];
        const bf16x2 wv[8] = {cvt_lo(d.x), cvt_hi(d.x), cvt_lo(d.y), cvt_hi(d.y),
                              cvt_lo(d.z), cvt_hi(d.z), cvt_lo(d.w), cvt_hi(d.w)};
        const float s = MX ? mx_scale((uint8_t)e[MX ? r : 0][MX ? c : 0]) : sc[MX ? 0 : c];
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r * M + m] = __builtin_fmaf(s, dot16(wv, x0[m][c], x1[m][c]), acc[r * M + m]);
      }
    }
  }
  const WaveSums<R * M> sums(acc);
  if ((lane & 15) == 0) {
#pragma unroll
    for (int q = 0; q < WaveSums<R * M>::kGroups; ++q) {
      const int f = 4 * q + (lane >> 4), r = f / M, m = f % M;
      if (f < R * M && row0 + r < j.n)
        st_global<uint16_t>(j.y, ((size_t)m * j.n + row0 + r) * 2,
                            (uint16_t)f32_to_bf16_rne(sums.g[q] * output_scale(j, row0 + r)));
    }
  }
}

// ------------------------------------------------------- VALU streaming --
//
// Grouped launches at M = 1 whose GEMVs all have K <= 1024*C: each
// workgroup owns a contiguous run of row tiles (across job boundaries) and
// requests tile t+1's codes and scales before computing tile t, so the weight
// stream never waits for a workgroup to start, look up its job or stage x.
// x is restaged in LDS only when the run crosses into the next job.
// Single calls at M = 1 on many rows use the same kernel with the job passed
// by value and one tile per workgroup.
template <int R, int C, bool MX>
struct TileRegs {
  uint4 w[R][C];
  float s[C];         // block: the scale of each chunk's 128-column block
  uint32_t e[2];      // MX: the wave's R rows of exponent bytes, 4 per lane (two halves)
};

// MX exponents of a wave's R rows: rows row0..row0+R-1 are contiguous in the
// [n, groups] array, R * groups <= 512 bytes, read as dwords (lane l: bytes
// 4l and 256 + 4l of the span) instead of one byte load per row and chunk.
// row0 is a multiple of R = 4, so with a 4-byte aligned base every dword is
// aligned, and the host streams MX weights only when the whole array is a
// whole number of dwords (n * groups % 4 == 0, mx_rows_stream): each dword
// lies inside the array or wholly past its end.  Those past the end load the
// array's last dword instead (rows >= n, whose sums are never stored), so
// the loads are unconditional and the compiler can count them.
__device__ __forceinline__ void mx_span_issue(const GemvJob& j, int row0, int rows, int groups,
                                              uint32_t (&e)[2]) {
  (void)rows;
  const int lane = threadIdx.x & (kWave - 1);
  const size_t total = (size_t)j.n * groups;
  const size_t base = (size_t)row0 * groups;
#pragma unroll
  for (int h = 0; h < 2; ++h) e[h] = ld_global<uint32_t>(j.scales, min(base + 4 * (lane + kWave * h), total - 4));
}

__device__ __forceinline__ void load_job_row(const GemvJob* __restrict__ jobs, int jn, GemvJob& job) {
  const size_t row = (size_t)jn * sizeof(GemvJob);
  job.x = (const uint16_t*)ld_global<uint64_t>(jobs, row + offsetof(GemvJob, x));
  job.codes = (const uint8_t*)ld_global<uint64_t>(jobs, row + offsetof(GemvJob, codes));
  job.scales = (const void*)ld_global<uint64_t>(jobs, row + offsetof(GemvJob, scales));
  job.y = (uint16_t*)ld_global<uint64_t>(jobs, row + offsetof(GemvJob, y));
  job.n = ld_global<int32_t>(jobs, row + offsetof(GemvJob, n));
  job.k = ld_global<int32_t>(jobs, row + offsetof(GemvJob, k));
  job.item0 = ld_global<int32_t>(jobs, row + offsetof(GemvJob, item0));
  job.format = ld_global<int32_t>(jobs, row + offsetof(GemvJob, format));
}

__device__ __forceinline__ int next_item0(const GemvJob* __restrict__ jobs, int jn, int njobs) {
  return jn + 1 < njobs
             ? ld_global<int32_t>(jobs, (size_t)(jn + 1) * sizeof(GemvJob) + offsetof(GemvJob, item0))
             : 0x7FFFFFFF;
}

// Where a streaming kernel finds its GEMVs: the device table `jobs` of
// `njobs` jobs (grouped launches, ONE = false), or the single job `one`
// passed by value with item0 = 0 (single calls, ONE = true: no table, no
// search).  The table stays a __restrict__ kernel parameter, so its rows
// are read with scalar loads that no pending weight load has to wait for.
struct JobList {
  const GemvJob* __restrict__ table;
  int count;
  const GemvJob& one;
};

// Index of the job that holds tile t (the last one whose first tile is <= t).
template <bool ONE>
__device__ __forceinline__ int job_of_tile(const JobList& l, int t) {
  if (ONE) return 0;
  int lo = 0, hi = l.count - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (ld_global<int32_t>(l.table, (size_t)mid * sizeof(GemvJob) + offsetof(GemvJob, item0)) <= t)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

template <bool ONE>
__device__ __forceinline__ void load_job(const JobList& l, int jn, GemvJob& j) {
  if (ONE) j = l.one;
  else load_job_row(l.table, jn, j);
}

// First tile after job jn.
template <bool ONE>
__device__ __forceinline__ int job_end(const JobList& l, int jn) {
  return ONE ? 0x7FFFFFFF : next_item0(l.table, jn, l.count);
}

template <int R, int C, bool MX>
__device__ __forceinline__ void stream_issue(const GemvJob& j, int tile, TileRegs<R, C, MX>& t) {
  constexpr int kRows = kWaves * R;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int row0 = tile * kRows + wave * R;
  const int nch = j.k / 16;
  const int tiles_k = (j.k + kTile - 1) / kTile;
  const int groups = (j.k + kGroup - 1) / kGroup;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = row0 + r;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int ch = lane + kWave * c;
      t.w[r][c] = make_uint4(0, 0, 0, 0);
      if (ch < nch && row < j.n) t.w[r][c] = ld_stream_u4(j.codes, (size_t)row * j.k + ch * 16);
    }
  }
  if (MX) {
    mx_span_issue(j, row0, R, groups, t.e);
  } else {
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int ch = lane + kWave * c;
      t.s[c] = ch < nch ? block_scale(j, tile * kRows, ch >> 3, tiles_k) : 0.0f;
    }
  }
}

template <int R, int C, bool MX, bool ONE>
__global__ __launch_bounds__(kThreads) void k_gemv_valu_stream(const GemvJob* __restrict__ table,
                                                               int njobs, GemvJob one, int total_tiles,
                                                               int tiles_per_block) {
  const JobList jobs{table, njobs, one};
  constexpr int kRows = kWaves * R, kSeg = 1024 * C;
  static_assert(kTile % kRows == 0, "a tile must stay inside one 128-row block");
  static_assert(!MX || (R == 4 && kSeg / kGroup * R <= 2 * 4 * kWave), "MX exponent span: two dwords per lane");
  __shared__ __align__(16) uint16_t xs[kSeg];
  __shared__ __align__(16) uint32_t ex[MX ? kWaves * 2 * kWave : 1];   // each wave's exponent span
  const int t_begin = blockIdx.x * tiles_per_block;
  const int t_end = min(total_tiles, t_begin + tiles_per_block);
  if (t_begin >= t_end) return;   // whole workgroup: no barrier is skipped by part of it
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;

  int jn = job_of_tile<ONE>(jobs, t_begin);
  GemvJob j;
  load_job<ONE>(jobs, jn, j);
  int boundary = job_end<ONE>(jobs, jn);

  TileRegs<R, C, MX> cur, nxt;
  stream_issue<R, C, MX>(j, t_begin - j.item0, cur);
  stage_row(j.x, min(j.k, kSeg), xs);   // the host streams only K <= kSeg
  __syncthreads();

  for (int t = t_begin; t < t_end; ++t) {
    // A single call (ONE) takes one tile per workgroup: no next tile is
    // requested, and the kernel holds no registers for one (78 VGPRs
    // against 133, so twice the waves per SIMD).
    const bool more = !ONE && t + 1 < t_end;
    GemvJob jnext = j;
    int jn_next = jn, boundary_next = boundary;
    if (more) {
      if (t + 1 >= boundary) {   // the run crosses into the next job
        jn_next = jn + 1;
        load_job<ONE>(jobs, jn_next, jnext);
        boundary_next = job_end<ONE>(jobs, jn_next);
      }
      stream_issue<R, C, MX>(jnext, t + 1 - jnext.item0, nxt);
    }

    const int row0 = (t - j.item0) * kRows + wave * R;
    const int nch = j.k / 16;
    const int groups = (j.k + kGroup - 1) / kGroup;
    // MX: this wave's exponent span through its own LDS slice (one wave's
    // LDS operations complete in order, so no barrier)
    uint32_t* exw = ex + (MX ? wave * 2 * kWave : 0);
    if (MX) {
      exw[lane] = cur.e[0];
      exw[kWave + lane] = cur.e[1];
    }
    const uint8_t* exb = reinterpret_cast<const uint8_t*>(exw);
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int ch = lane + kWave * c;
      if (ch < nch) {
        const uint4 x0 = *reinterpret_cast<const uint4*>(xs + ch * 16);
        const uint4 x1 = *reinterpret_cast<const uint4*>(xs + ch * 16 + 8);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint4 d = cur.w[r][c];
          const bf16x2 w[8] = {cvt_lo(d.x), cvt_hi(d.x), cvt_lo(d.y), cvt_hi(d.y),
                               cvt_lo(d.z), cvt_hi(d.z), cvt_lo(d.w), cvt_hi(d.w)};
          const float sc = MX ? mx_scale(exb[r * groups + ch / 2]) : cur.s[c];
          acc[r] = __builtin_fmaf(sc, dot16(w, x0, x1), acc[r]);
        }
      }
    }
    const WaveSums<R> sums(acc);
    if ((lane & 15) == 0) {
#pragma unroll
      for (int q = 0; q < WaveSums<R>::kGroups; ++q) {
        const int r = 4 * q + (lane >> 4);
        if (r < R && row0 + r < j.n)
          st_global<uint16_t>(j.y, (size_t)(row0 + r) * 2,
                              (uint16_t)f32_to_bf16_rne(sums.g[q] * output_scale(j, row0 + r)));
      }
    }
    if (!more) break;
    if (jn_next != jn) {   // restage x for the next job
      __syncthreads();
      stage_row(jnext.x, min(jnext.k, kSeg), xs);
      __syncthreads();
    }
    j = jnext;
    jn = jn_next;
    boundary = boundary_next;
    cur = nxt;
  }
}

// ------------------------------------------------------------------ MFMA --
//
// bf16 v_mfma_f32_16x16x32_bf16 on 16-row tiles of W.  Lane l holds A row
// i = l%16 and K-quarter g = l/16; the B operand (x^T) takes the same K
// positions, and D[4*(l/16) + j][l%16] (j = 0..3) is y^T of the tile.
//
// Codes reach the A layout through a panel: a wave loads 16 rows x 256
// bytes of its tile with four 16-byte loads per lane, each covering 4 rows x
// 256 contiguous bytes (lane l: row 4q + l/16, bytes 16*(l%16)), writes the
// panel to its own 4 KB of LDS and reads it back as A operands.  The A layout
// loaded straight from memory would read 64 bytes from each of 16 rows per
// instruction, which caps a pure read of the weight stream at about 5 TB/s
// on MI355X against 6.9 TB/s for 256-byte row pieces.  Only the owning wave
// touches its panel buffer, so no barrier is needed: one wave's LDS
// operations complete in order.  The buffer is XOR-swizzled in 16-byte units
// (unit c of panel row r at r*256 + 16*(c ^ r)), which keeps both the writes
// and the A reads free of bank conflicts without padding.
constexpr int kPanelCols = 256;                 // columns of a panel (two 128-column blocks)
constexpr int kPanelBytes = 16 * kPanelCols;    // LDS bytes of one wave's panel buffer

template <bool MX>
struct Panel {
  uint4 v[4];                // lane l: row 4q + l/16 of the tile, bytes 16*(l%16)
  // the scales as loaded (panel_scales converts them where the MFMA step
  // uses them): MX: the exponent byte of each (block, chunk) of the A layout;
  // otherwise the scale of each 128-column block, fp32 (f) or bf16 bits (h)
  uint32_t s[4];
  float f[2];
  uint16_t h[2];
  u32x2 e8;                  // MX, packed rows: the row's 8 exponent bytes of the panel
};

// The scale format of a panel request.  kSfAny: any non-MX format, chosen at
// run time, each block scale loaded only where it exists (kernels that
// request every panel of a call up front).  kFmtBlock, kFmtBlockBf16: that
// block grid, loaded unconditionally from a clamped index (kernels that
// pipeline panels in a loop).  kFmtRow: no block scale (row and tensor
// scales multiply the outputs).
constexpr int kSfAny = -1;

// The panel's scales as the MFMA step uses them: block: per 128-column
// block; MX: 2^(E-127) per (block, chunk) of the A layout (lane l reads the
// exponents of groups 8p + 2c + (l/16)/2, c = 0..3, of row l%16).
template <bool MX, bool PK = false, int SF = kSfAny>
__device__ __forceinline__ void panel_scales(const Panel<MX>& r, float (&sc)[MX ? 4 : 2]) {
  if (MX) {
    if (PK) {
      const int sh = 8 * (((threadIdx.x & (kWave - 1)) >> 5) & 1);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        sc[c] = mx_scale((uint8_t)(((c < 2 ? r.e8.x : r.e8.y) >> (16 * (c & 1) + sh)) & 0xFF));
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) sc[c] = mx_scale((uint8_t)r.s[c]);
    }
    // The scales are built here, not where the MFMA step uses them: left to
    // the compiler, the conversion moves after the slot's next request, the
    // exponent registers stay live across it, the request loads elsewhere,
    // and the copy back at the loop's end waits for it.
#pragma unroll
    for (int c = 0; c < 4; ++c) asm volatile("" : "+v"(sc[c]));
  } else {
    // A block scale is the same in every lane (one 16-row tile, one
    // block): taken into a scalar register here, its vector register is free
    // before the slot's next request, which can then load into it (a request
    // into another register would need a copy back at the loop's end, and
    // the copy would wait for it).
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const float v = SF == kFmtBlockBf16 ? __uint_as_float((uint32_t)r.h[b] << 16) : r.f[b];
      sc[b] = SF == kFmtRow ? 1.0f : __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
    }
  }
}

// Panel registers -> LDS -> A operands: a[b][c] = row l%16, bytes
// 128b + 64c + 16*(l/16) of the panel.
__device__ __forceinline__ void panel_to_a(const uint4 (&v)[4], unsigned char* buf, uint4 (&a)[2][2]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int i = lane & 15, g = lane >> 4;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 4 * q + g;
    *reinterpret_cast<uint4*>(buf + r * kPanelCols + 16 * (i ^ r)) = v[q];
  }
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int c = 0; c < 2; ++c)
      a[b][c] = *reinterpret_cast<const uint4*>(buf + i * kPanelCols + 16 * ((8 * b + 4 * c + g) ^ i));
}

// 16 e4m3 codes -> the two bf16x8 A operands of one 64-column chunk (first
// and last 8 K positions of each lane's 16), scaled by s for MX.
template <bool MX>
__device__ __forceinline__ void a_operands(uint4 d, float s, bf16x8& A0, bf16x8& A1) {
  bf16x2 a0, a1, a2, a3, b0, b1, b2, b3;
  if (MX) {
    a0 = cvt_scaled<false>(d.x, s), a1 = cvt_scaled<true>(d.x, s);
    a2 = cvt_scaled<false>(d.y, s), a3 = cvt_scaled<true>(d.y, s);
    b0 = cvt_scaled<false>(d.z, s), b1 = cvt_scaled<true>(d.z, s);
    b2 = cvt_scaled<false>(d.w, s), b3 = cvt_scaled<true>(d.w, s);
  } else {
    a0 = cvt_lo(d.x), a1 = cvt_hi(d.x), a2 = cvt_lo(d.y), a3 = cvt_hi(d.y);
    b0 = cvt_lo(d.z), b1 = cvt_hi(d.z), b2 = cvt_lo(d.w), b3 = cvt_hi(d.w);
  }
  A0 = bf16x8{a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
  A1 = bf16x8{b0[0], b0[1], b1[0], b1[1], b2[0], b2[1], b3[0], b3[1]};
}

// acc += the panel's products.  get_b(t, b, c, B0, B1) supplies the x^T
// operands of m-tile t for block b, chunk c.  Block scales multiply each
// 128-column block's partial sum; MX scales are already in the A operands.
template <int MT, bool MX, typename GetB>
__device__ __forceinline__ void panel_mfma(const uint4 (&a)[2][2], const float* s, GetB get_b,
                                           f32x4 (&acc)[MT]) {
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    f32x4 part[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) part[t] = MX ? acc[t] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      bf16x8 A0, A1;
      a_operands<MX>(a[b][c], MX ? s[2 * b + c] : 0.0f, A0, A1);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        uint4 B0, B1;
        get_b(t, b, c, B0, B1);
        part[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, __builtin_bit_cast(bf16x8, B0), part[t], 0, 0, 0);
        part[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, __builtin_bit_cast(bf16x8, B1), part[t], 0, 0, 0);
      }
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      if (MX) {
        acc[t] = part[t];
      } else {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[t][jj] = __builtin_fmaf(s[b], part[t][jj], acc[t][jj]);
      }
    }
  }
}

// The panel half of panel_to_a: registers -> the wave's panel buffer.
__device__ __forceinline__ void panel_write(const uint4 (&v)[4], unsigned char* buf) {
  const int lane = threadIdx.x & (kWave - 1);
  const int i = lane & 15, g = lane >> 4;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 4 * q + g;
    *reinterpret_cast<uint4*>(buf + r * kPanelCols + 16 * (i ^ r)) = v[q];
  }
}

// panel_mfma reading each A operand from the panel buffer where it is used,
// with the scheduler fenced between the two 128-column blocks: the A
// operands then hold 4 registers at a time instead of 16 (for kernels at the
// register limit).
template <int MT, bool MX, typename GetB>
__device__ __forceinline__ void panel_mfma_lds(const unsigned char* buf, const float* s, GetB get_b,
                                               f32x4 (&acc)[MT]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int i = lane & 15, g = lane >> 4;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    f32x4 part[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) part[t] = MX ? acc[t] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint4 a = *reinterpret_cast<const uint4*>(buf + i * kPanelCols + 16 * ((8 * b + 4 * c + g) ^ i));
      bf16x8 A0, A1;
      a_operands<MX>(a, MX ? s[2 * b + c] : 0.0f, A0, A1);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        uint4 B0, B1;
        get_b(t, b, c, B0, B1);
        part[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, __builtin_bit_cast(bf16x8, B0), part[t], 0, 0, 0);
        part[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, __builtin_bit_cast(bf16x8, B1), part[t], 0, 0, 0);
      }
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      if (MX) {
        acc[t] = part[t];
      } else {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[t][jj] = __builtin_fmaf(s[b], part[t][jj], acc[t][jj]);
      }
    }
    if (b == 0) __builtin_amdgcn_sched_barrier(0);
  }
}

// y^T of a 16-row tile from the D layout; columns (activation rows) >= m_rows
// and rows >= n are not written.  OS: the format may scale rows or the whole
// weight (kFmtRow, kFmtTensor), whose scales are loaded here and used under
// the bounds branches; the explicit wait at the end (where those formats have
// just waited for their scale loads anyway) keeps the compiler from treating
// a load on a path that skipped its use as still pending, which would make
// it wait for all vector memory at the top of a caller's panel loop.  Kernels
// that pipeline panels across tiles take OS = false for the other formats.
// FRESH: the lane index comes from lane_fresh, so the output offsets are
// recomputed at each store (a kernel at the register limit otherwise keeps
// them from the start, and spills).
template <int MT, bool OS = true, bool FRESH = false>
__device__ __forceinline__ void store_tile(const GemvJob& j, int row0, int m_rows, const f32x4 (&acc)[MT],
                                           float factor = 1.0f) {
  const int lane = FRESH ? lane_fresh() : (int)(threadIdx.x & (kWave - 1));
  const int i = lane & 15, g = lane >> 4;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int r = row0 + 4 * g + jj;
    if (r >= j.n) continue;
    const float os = OS ? factor * output_scale(j, r) : factor;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int mcol = 16 * t + i;
      if (mcol < m_rows)
        st_global<uint16_t>(j.y, ((size_t)mcol * j.n + r) * 2, (uint16_t)f32_to_bf16_rne(acc[t][jj] * os));
    }
  }
  if (OS) vm_wait_all();
}

// ------------------------------------------------------- MFMA streaming --
//
// Grouped launches.  A tile is 16*NW rows, one 16-row MFMA tile per wave;
// each workgroup owns a contiguous run of tiles across job boundaries (as the
// VALU streaming kernel) and walks them panel by panel, the panel D ahead
// already requested.  x is staged in LDS by K segments of seg_cols columns
// (a multiple of 256).  Segments of at most kStreamXElems elements use two
// buffers: while the workgroup works on one segment, the next one (of this
// tile, the next tile or the next job) goes into the other buffer.  Larger
// ones (chosen on the host only when every job's x fits one segment) use one
// buffer, restaged at job changes behind a barrier.
// Where a wave's panel loads point inside one 16-row tile: base is the
// tile's first row (uniform), off[q] the lane's byte offset of row 4q + l/16
// plus its 16-byte column (rows past the weight's last row are clamped to
// it: their sums are never stored).  Computed once per tile, so a panel
// load costs one 64-bit add instead of a row multiply and bounds checks.
struct TileLoads {
  const uint8_t* base;
  uint64_t off[4];
};

__device__ __forceinline__ void tile_loads(const GemvJob& j, int row0, TileLoads& t) {
  const int lane = threadIdx.x & (kWave - 1);
  t.base = j.codes + (size_t)row0 * j.k;
  const int last = j.n - 1 - row0;   // >= 0 for a live tile
#pragma unroll
  for (int q = 0; q < 4; ++q)
    t.off[q] = (uint64_t)min(4 * q + (lane >> 4), last) * (uint64_t)j.k + 16 * (lane & 15);
}

// The 17..32-row streaming kernel's view of a 16-row tile: the address of the row each
// of the lane's four loads reads (rows past the weight's last row clamped to
// it: their sums are never stored).  Computed once per tile.
struct TileRows {
  const uint8_t* row[4];
};

__device__ __forceinline__ void tile_rows(const GemvJob& j, int row0, TileRows& t) {
  const int lane = lane_fresh();
  const int last = j.n - 1 - row0;   // >= 0 for a live tile
#pragma unroll
  for (int q = 0; q < 4; ++q)
    t.row[q] = j.codes + (size_t)(row0 + min(4 * q + (lane >> 4), last)) * (size_t)j.k;
}

// The 17..32-row streaming kernel's request of panel p: every lane loads, with no
// branch.  A branch between full panels and a partial last one makes the
// compiler count a path with fewer requests, and every wait it then sizes for
// an earlier request also waits for requests issued after it.  Columns are
// clamped to the row's last 16 bytes (a no-op on full panels; on a partial
// last panel the clamped codes meet the zeros that pad x past k in LDS).
// Scales as panel_issue_tile.
// A dead request (live false: past the run) reads column 0 of the rows `t`
// holds, which the caller points at one row: one cache line, not a panel.
template <bool MX, bool PK, int SF>
__device__ __forceinline__ void panel_issue_rows(const GemvJob& j, const TileRows& t, int row0, int p, bool live,
                                                 int nkb, int groups, Panel<MX>& r) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t col = live ? (uint32_t)min(p * kPanelCols + 16 * (lane & 15), j.k - 16) : 0u;
#pragma unroll
  for (int q = 0; q < 4; ++q) r.v[q] = ld_stream_u4(t.row[q], col);
  if (MX) {
    // the tile's exponent rows from a uniform base: a 32-bit lane offset
    // (16 rows of at most 2^26 bytes), so no 64-bit address stays live.
    // row0 may lie past the last row (a wave's slice of a job's last tile, a
    // dead request past the run): the base row is clamped, so every lane
    // reads an existing row (n - 1 past the end; those sums are not stored).
    const int r0 = min(row0, j.n - 1);
    const uint8_t* __restrict__ e8 = static_cast<const uint8_t*>(j.scales) + (size_t)r0 * groups;
    const uint32_t rofs = (uint32_t)min(lane & 15, j.n - 1 - r0) * (uint32_t)groups;
    if (PK) {
      const int pc = min(p, (j.k - 1) / kPanelCols);
      r.e8 = ld_global<u32x2>(e8, rofs + 8 * pc);
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int kx = min(p * kPanelCols + 64 * c + 16 * (lane >> 4), j.k - 1);
        r.s[c] = ld_global<uint8_t>(e8, rofs + (uint32_t)(kx / kGroup));
      }
    }
  } else if (SF == kFmtBlock) {
#pragma unroll
    for (int b = 0; b < 2; ++b) r.f[b] = ld_global<float>(j.scales, block_scale_at(j, row0, 2 * p + b, nkb) * 4);
  } else if (SF == kFmtBlockBf16) {
#pragma unroll
    for (int b = 0; b < 2; ++b)
      r.h[b] = ld_global<uint16_t>(j.scales, block_scale_at(j, row0, 2 * p + b, nkb) * 2);
  }
}

// Request panel p (columns [256p, 256p + 256)) of the 16-row tile at row0,
// with its scales, through the row offsets of `t`.  Every load is in bounds.
// A partial last panel either clamps its columns to the row's last 16 bytes,
// whose codes then meet the zeros that pad x past k in LDS (ZT = false: the
// streaming kernel), or loads zeros past k (ZT = true: kernels whose x
// operands are not zero there).  PK (MX only): every exponent row starts
// 8-byte aligned (groups % 8 == 0 and an aligned array; the host checks,
// mx_rows_packed8), so one 8-byte load per row brings the panel's exponents.
// It is a template choice, not a branch: with both loads behind a runtime
// branch the compiler joins their results with copies, and a copy waits for
// its load, and so for every weight load the wave issued before it.  A dead
// panel (live false) gets zero codes where its products reach a stored sum
// (DZ); with DZ false its registers keep the codes they held (finite).
template <bool MX, bool PK, bool ZT = false, int SF = kSfAny, bool DZ = true>
__device__ __forceinline__ void panel_issue_tile(const GemvJob& j, const TileLoads& t, int row0, int p, bool live,
                                                 int nkb, int groups, Panel<MX>& r) {
  const int lane = threadIdx.x & (kWave - 1);
  if (live) {
    const uint8_t* pb = t.base + (size_t)p * kPanelCols;
    if ((p + 1) * kPanelCols <= j.k) {
#pragma unroll
      for (int q = 0; q < 4; ++q) r.v[q] = ld_stream_u4(pb, t.off[q]);
    } else if (ZT) {
      const bool in = p * kPanelCols + 16 * (lane & 15) < j.k;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        r.v[q] = make_uint4(0, 0, 0, 0);
        if (in) r.v[q] = ld_stream_u4(pb, t.off[q]);
      }
    } else {
      const int over = max(0, p * kPanelCols + 16 * (lane & 15) + 16 - j.k);   // bytes past the row's end
#pragma unroll
      for (int q = 0; q < 4; ++q) r.v[q] = ld_stream_u4(pb, t.off[q] - (uint64_t)over);
    }
  } else if (DZ) {
#pragma unroll
    for (int q = 0; q < 4; ++q) r.v[q] = make_uint4(0, 0, 0, 0);
  }
  if (MX) {
    const int row = min(row0 + (lane & 15), j.n - 1);
    const uint8_t* __restrict__ e8 = static_cast<const uint8_t*>(j.scales);
    if (PK) {
      const int pc = min(p, (j.k - 1) / kPanelCols);
      r.e8 = ld_global<u32x2>(e8, (size_t)row * groups + 8 * pc);
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int kx = min(p * kPanelCols + 64 * c + 16 * (lane >> 4), j.k - 1);
        r.s[c] = ld_global<uint8_t>(e8, (size_t)row * groups + kx / kGroup);
      }
    }
  } else if (SF == kFmtBlock) {
    // a block past k (clamped to the last one) multiplies zero products,
    // and the scale of a tile past the last row is never stored
#pragma unroll
    for (int b = 0; b < 2; ++b) r.f[b] = ld_global<float>(j.scales, block_scale_at(j, row0, 2 * p + b, nkb) * 4);
  } else if (SF == kFmtBlockBf16) {
#pragma unroll
    for (int b = 0; b < 2; ++b)
      r.h[b] = ld_global<uint16_t>(j.scales, block_scale_at(j, row0, 2 * p + b, nkb) * 2);
  } else if (SF == kSfAny) {
    r.f[0] = r.f[1] = 0.0f;
    if (live && row0 < j.n) {
      r.f[0] = block_scale(j, row0, 2 * p, nkb);
      if (2 * p + 1 < nkb) r.f[1] = block_scale(j, row0, 2 * p + 1, nkb);
    }
  }
}

// The order a wave walks a tile's panels in.  The tile's K splits into
// segments of sp panels (the x segments staged in LDS; one segment when x
// fits whole).  In plain order every wave walks them from the first panel.
// Rotated, the workgroup visits them starting at segment s0 and wrapping,
// and inside a segment of len panels each wave starts at its own offset,
// wave * len / NW, and wraps, so at any moment the workgroups of the chip,
// and the waves of a workgroup, read different column ranges.  With all of
// them at the same columns, weights whose row stride is a multiple of 4 KB
// read slowly: a read-only pass with this kernel's access pattern over
// [8192 x K] weights on MI355X moves 5.7 / 5.5 / 6.4 TB/s at K = 4096 / 8192
// / 12288 in plain order and 6.6 / 6.5 / 6.8 rotated (K = 2048..3072 and
// 4608 / 6144 within 2 % either way).  In the GEMV the rotation gained 3-4 %
// on the dense layer's K = 4096 / 12288 weights and 1-3 % on lm_head
// (K = 2048) at M = 4..16, but lost 4 % on lm_head at M = 32, whose
// segments are two panels long, and 1-2 % on K = 2560 / 3072; so only jobs
// with K a multiple of 2048 and segments of at least four panels (or one
// segment) are rotated.  Every field is uniform across the wave; stepping
// needs no division.
struct PanelWalk {
  int sp, nseg, np;   // segment length, segments and panels of the job
  int seg, len;       // current segment and its panel count
  int off, pos, cnt;  // the wave's start in the segment, its current panel there, panels done there
  int segs_done;      // segments of the tile done
  bool rot;           // rotated order

  __device__ __forceinline__ void start_segment(int wave, int nw) {
    len = min(sp, np - seg * sp);
    off = rot ? (wave * len) / nw : 0;
    pos = off;
    cnt = 0;
  }
  // A new job's first tile: s0 = the workgroup's starting segment if rotated.
  __device__ __forceinline__ void start_job(int k, int seg_panels, int s0, int wave, int nw) {
    np = (k + kPanelCols - 1) / kPanelCols;
    sp = seg_panels;
    nseg = (np + sp - 1) / sp;
    rot = k % 2048 == 0 && (sp >= 4 || nseg == 1);
    seg = rot ? s0 % nseg : 0;
    segs_done = 0;
    start_segment(wave, nw);
  }
  __device__ __forceinline__ int panel() const { return seg * sp + pos; }
  __device__ __forceinline__ int seg_col0() const { return seg * sp * kPanelCols; }
  // One panel on; returns 0 (same segment), 1 (next segment of the tile) or
  // 2 (tile done: the walk restarts at the tile's first segment).
  __device__ __forceinline__ int step(int wave, int nw) {
    ++cnt;
    if (++pos == len) pos = 0;
    if (cnt < len) return 0;
    if (++seg == nseg) seg = 0;
    const int r = ++segs_done == nseg ? 2 : 1;
    if (r == 2) segs_done = 0;
    start_segment(wave, nw);
    return r;
  }
};

// x elements a double-buffered segment of the streaming MFMA kernel holds:
// two 16-byte units per thread of its 512, so that a whole segment is in
// flight in eight registers per thread.
constexpr int kStreamXUnits = 2;
constexpr int kStreamXElems = kStreamXUnits * 512 * 8;
static_assert(32 * kPanelCols <= kStreamXElems, "a one-panel segment of 32 rows must fit the staging units");

// Up to 16 activation rows: x^T is one 16-row m-tile, x is staged in one
// buffer by segments as large as the workgroup's LDS share allows (x whole
// for most shapes), restaged behind barriers.  Four waves per SIMD (at most
// 128 VGPRs): two 8-wave workgroups per CU, so one workgroup's staging
// barriers are covered by the other's loads.
template <int NW, int D, bool MX, bool ONE, bool PK, int SF>
__global__ __launch_bounds__(NW * kWave, 4) void k_gemv_mfma_stream16(const GemvJob* __restrict__ table,
                                                                   int njobs, GemvJob one, int total_tiles,
                                                                   int tiles_per_block, int m_rows,
                                                                   int seg_cols) {
  constexpr int MT = 1;
  const JobList jobs{table, njobs, one};
  constexpr int kRows = 16 * NW;
  extern __shared__ __align__(16) unsigned char smem[];
  const int t_begin = blockIdx.x * tiles_per_block;
  const int t_end = min(total_tiles, t_begin + tiles_per_block);
  if (t_begin >= t_end) return;   // whole workgroup: no barrier is skipped by part of it
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int i = lane & 15, g = lane >> 4;
  unsigned char* pbuf = smem + wave * kPanelBytes;
  // x rows of seg_cols bf16, the 16-byte units of row r XOR-swizzled by
  // r % 16 inside each group of 16 units: the 16 rows a B read spans then
  // hit 16 different bank groups, with no padding (so more columns fit)
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem + NW * kPanelBytes);
  const int seg_panels = seg_cols / kPanelCols;
  // B operands: lane (i, g) reads x row 16t + i (rows past m_rows read row
  // m_rows - 1: their products land in output columns that are not stored),
  // units 32 * panel + 16b + 8c + 2g + h, swizzled: the panel's units keep
  // their group of 32, 16b is an offset, and (8c + 2g + h) ^ i for c, h in
  // {0, 1} is one of four per-lane unit offsets
  int brow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) brow[t] = min(16 * t + i, m_rows - 1) * seg_cols;
  int bunit[2][2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int h = 0; h < 2; ++h) bunit[c][h] = 8 * ((8 * c + 2 * g + h) ^ (min(i, m_rows - 1) & 15));
  // staging: this thread's first unit of the [m_rows][seg_cols / 8] grid of
  // 8-element units, and the stride in rows and units between its units
  const int units_row = seg_cols / 8;
  const int st_r0 = threadIdx.x / units_row, st_c0 = threadIdx.x % units_row;
  const int st_dr = (NW * kWave) / units_row, st_dc = (NW * kWave) % units_row;

  // the workgroup's first segment in every tile
  const int s0 = blockIdx.x;
  int jn = job_of_tile<ONE>(jobs, t_begin);
  // compute cursor: tile ct of job cj, the walk cw through its panels
  GemvJob cj;
  load_job<ONE>(jobs, jn, cj);
  int c_bound = job_end<ONE>(jobs, jn);
  PanelWalk cw;
  cw.start_job(cj.k, seg_panels, s0, wave, NW);
  int ct = t_begin;
  // issue cursor: tile it of job ij, the walk iw, D panels ahead
  GemvJob ij = cj;
  int ijn = jn, i_bound = c_bound, it = t_begin;
  PanelWalk iw = cw;
  TileLoads tl;
  tile_loads(ij, (it - ij.item0) * kRows + 16 * wave, tl);

  auto issue = [&](Panel<MX>& r) {
    const bool live = it < t_end;
    panel_issue_tile<MX, PK, false, SF, false>(ij, tl, (it - ij.item0) * kRows + 16 * wave, iw.panel(), live,
                                        (ij.k + kTile - 1) / kTile, (ij.k + kGroup - 1) / kGroup, r);
    if (!live) return;
    if (iw.step(wave, NW) == 2 && ++it < t_end) {
      if (it >= i_bound) {
        load_job<ONE>(jobs, ++ijn, ij);
        i_bound = job_end<ONE>(jobs, ijn);
        iw.start_job(ij.k, seg_panels, s0, wave, NW);
      }
      tile_loads(ij, (it - ij.item0) * kRows + 16 * wave, tl);
    }
  };
  // x[:, seg0 : seg0 + seg_cols) of job j into LDS, zeros past k (the codes
  // of a clamped last panel meet zeros there)
  auto stage = [&](const GemvJob& j, int seg0) {
    const int valid = min(seg_cols, j.k - seg0) / 8;
    int r = st_r0, c = st_c0;
    while (r < m_rows) {
      uint4 v[kStageBatch];
      int dst[kStageBatch];
#pragma unroll
      for (int q = 0; q < kStageBatch; ++q) {
        dst[q] = r < m_rows ? r * seg_cols + 8 * (c ^ (r & 15)) : -1;
        v[q] = make_uint4(0, 0, 0, 0);
        if (r < m_rows && c < valid) v[q] = ld_global_u4(j.x, ((size_t)r * j.k + seg0 + 8 * c) * 2);
        c += st_dc;
        r += st_dr;
        if (c >= units_row) {
          c -= units_row;
          ++r;
        }
      }
#pragma unroll
      for (int q = 0; q < kStageBatch; ++q)
        if (dst[q] >= 0) *reinterpret_cast<uint4*>(xs + dst[q]) = v[q];
    }
    // Every staged load has been waited for by its store, but the stores
    // are conditional and the compiler cannot pair them with the loads: it
    // would wait for all vector memory at the top of the panel loop, on
    // every pass.  An explicit wait here (where staging has already drained
    // the weight loads requested before it) tells it nothing is pending.
    vm_wait_all();
  };

  // Panel steps are fenced off from the scheduler (sched_barrier): left
  // free, it gathers the requests of several slots in one place, so a wait
  // for one slot would also wait for the next.
  Panel<MX> slot[D];
#pragma unroll
  for (int s = 0; s < D; ++s) {
    issue(slot[s]);
    __builtin_amdgcn_sched_barrier(0);
  }
  stage(cj, cw.seg_col0());
  __syncthreads();

  f32x4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // One exit, after every D panel steps: an exit between steps becomes a
  // branch to a block shared with the loop's head, reached there with the
  // slots' requests in another order, and the compiler, merging the two
  // orders, would wait at the head for every request in flight.  So the last
  // pass may consume up to D - 1 panels past the run: they were requested as
  // dead (not loaded: the slot keeps the codes it held, finite values), and
  // a tile past the run is neither stored nor staged.
  for (;;) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      uint4 a[2][2];
      panel_to_a(slot[s].v, pbuf, a);
      float sc[MX ? 4 : 2];
      panel_scales<MX, PK, SF>(slot[s], sc);
      issue(slot[s]);
      const int kseg = cw.pos * kPanelCols;   // panel start within the staged segment
      panel_mfma<MT, MX>(a, sc, [&](int t, int b, int c, uint4& B0, uint4& B1) {
        const uint16_t* bp = xs + brow[t] + kseg + 128 * b;
        B0 = *reinterpret_cast<const uint4*>(bp + bunit[c][0]);
        B1 = *reinterpret_cast<const uint4*>(bp + bunit[c][1]);
      }, acc);
      const int moved = cw.step(wave, NW);
      if (moved == 2) {   // tile done
        if (ct < t_end) store_tile<MT, SF == kFmtRow>(cj, (ct - cj.item0) * kRows + 16 * wave, m_rows, acc);
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if (++ct < t_end) {
          if (ct >= c_bound) {   // the run enters the next job
            load_job<ONE>(jobs, ++jn, cj);
            c_bound = job_end<ONE>(jobs, jn);
            cw.start_job(cj.k, seg_panels, s0, wave, NW);
            __syncthreads();
            stage(cj, cw.seg_col0());
            __syncthreads();
          } else if (cw.nseg > 1) {   // next tile of a multi-segment job
            __syncthreads();
            stage(cj, cw.seg_col0());
            __syncthreads();
          }
        }
      } else if (moved == 1 && ct < t_end) {   // next segment of this tile
        __syncthreads();
        stage(cj, cw.seg_col0());
        __syncthreads();
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (ct >= t_end) return;
  }
}


// 17..32 activation rows: x^T is two 16-row m-tiles, an x segment is one
// panel (256 columns: m_rows * 256 <= kStreamXElems), double-buffered.  Four
// waves per SIMD (at most 128 VGPRs): two 8-wave workgroups per CU, so one
// workgroup's barriers are covered by the other's loads.
//
// Staging without a drain: vector memory requests complete in issue order,
// so a wait for x loads issued after the weight requests in flight would wait
// for those too, and stall the pipeline at every segment.  The next
// segment's x is therefore requested at the start of the step that begins a
// segment, before that step's weight request, and written into the other
// buffer at the end of the step: its wait covers only the panel the next
// step consumes anyway.  The buffers switch behind one barrier, which also
// tells every wave that the buffer written next is no longer read.
template <int NW, int D, bool MX, bool ONE, bool PK, int SF>
__global__ __launch_bounds__(NW * kWave, 4) void k_gemv_mfma_stream32(const GemvJob* __restrict__ table,
                                                                   int njobs, GemvJob one, int total_tiles,
                                                                   int tiles_per_block, int m_rows, int) {
  static_assert(NW * kWave == 512, "staging geometry assumes 512 threads");
  constexpr int MT = 2;
  constexpr int seg_cols = kPanelCols;   // one-panel segments (checked on the host)
  const JobList jobs{table, njobs, one};
  constexpr int kRows = 16 * NW;
  extern __shared__ __align__(16) unsigned char smem[];
  const int t_begin = blockIdx.x * tiles_per_block;
  const int t_end = min(total_tiles, t_begin + tiles_per_block);
  if (t_begin >= t_end) return;   // whole workgroup: no barrier is skipped by part of it
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int i = lane & 15, g = lane >> 4;
  unsigned char* pbuf = smem + wave * kPanelBytes;
  // two x buffers of m_rows rows of seg_cols bf16, the 16-byte units of row
  // r XOR-swizzled by r % 16 inside each group of 16 units: the 16 rows a B
  // read spans then hit 16 different bank groups, with no padding
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem + NW * kPanelBytes);
  const int xbuf = m_rows * seg_cols;   // elements of one buffer
  int xcur = 0;                         // the buffer in use: 0 or xbuf
  const int seg_panels = seg_cols / kPanelCols;
  // B operands: lane (i, g) reads x row 16t + i (rows past m_rows read row
  // m_rows - 1: their products land in output columns that are not stored),
  // units 32 * panel + 16b + 8c + 2g + h, swizzled: the panel's units keep
  // their group of 32, 16b is an offset, and (8c + 2g + h) ^ i for c, h in
  // {0, 1} is one of four per-lane unit offsets
  int brow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) brow[t] = min(16 * t + i, m_rows - 1) * seg_cols;
  int bunit[2][2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int h = 0; h < 2; ++h) bunit[c][h] = 8 * ((8 * c + 2 * g + h) ^ (min(i, m_rows - 1) & 15));
  // staging: this thread's units u = tid + 512q of the [m_rows][32] grid of
  // 8-element units (one-panel segments): row r, unit c, LDS element offset
  // dst (valid for r < m_rows); shifts of the thread index
  auto x_unit = [&](int q, int& r, int& c, int& dst) {
    r = (int)(threadIdx.x >> 5) + 16 * q;
    c = threadIdx.x & 31;
    dst = r * kPanelCols + 8 * (c ^ (r & 15));
  };
  // x[:, seg0 : seg0 + seg_cols) of a job (pointer, k) into registers.  The
  // loads are unconditional (rows clamped to m_rows - 1, columns to k - 8):
  // a load behind a branch would be joined by copies, and a copy waits for
  // its load.  Units past k are zeroed where they are written (the codes of
  // a clamped last panel meet zeros there).
  auto x_request = [&](const uint16_t* x, int k, int seg0, uint4 (&v)[kStreamXUnits]) {
#pragma unroll
    for (int q = 0; q < kStreamXUnits; ++q) {
      int r, c, dst;
      x_unit(q, r, c, dst);
      v[q] = ld_global_u4(x, ((size_t)min(r, m_rows - 1) * k + min(seg0 + 8 * c, k - 8)) * 2);
    }
  };
  // to buffer `buf` (live), else, and for rows past m_rows, to the wave's
  // panel buffer `spare`.  Every lane stores: a store under a lane mask gets
  // its wait inside the masked block, and the compiler then takes the loads
  // as still pending on the path that skips it.
  // Units past k are zeroed only on a segment that reaches past k (a job's
  // last one); both paths have waited for the loads where they join.
  auto x_write = [&](uint4 (&v)[kStreamXUnits], int k, int seg0, bool live, int buf, unsigned char* spare) {
    if (seg0 + seg_cols > k) {
#pragma unroll
      for (int q = 0; q < kStreamXUnits; ++q) {
        int r, c, dst;
        x_unit(q, r, c, dst);
        if (seg0 + 8 * c + 8 > k) v[q] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int q = 0; q < kStreamXUnits; ++q) {
      int r, c, dst;
      x_unit(q, r, c, dst);
      uint4* to = live && r < m_rows
                      ? reinterpret_cast<uint4*>(xs + buf + dst)
                      : reinterpret_cast<uint4*>(spare + 16 * (threadIdx.x & (kWave - 1)) + 1024 * q);
      *to = v[q];
    }
  };

  // the workgroup's first segment in every tile
  const int s0 = blockIdx.x;
  int jn = job_of_tile<ONE>(jobs, t_begin);
  // compute cursor: tile ct of job cj, the walk cw through its panels
  GemvJob cj;
  load_job<ONE>(jobs, jn, cj);
  int c_bound = job_end<ONE>(jobs, jn);
  PanelWalk cw;
  cw.start_job(cj.k, seg_panels, s0, wave, NW);
  int ct = t_begin;
  // issue cursor: tile it of job ij, the walk iw, D panels ahead
  GemvJob ij = cj;
  int ijn = jn, i_bound = c_bound, it = t_begin;
  PanelWalk iw = cw;
  TileRows tl;
  tile_rows(ij, (it - ij.item0) * kRows + 16 * wave, tl);

  // Requests past the run (dead: their sums are never stored) are loaded
  // like live ones, all from the job's first 16 code bytes (one cache line).
  auto issue = [&](Panel<MX>& r) {
    const bool live = it < t_end;
    panel_issue_rows<MX, PK, SF>(ij, tl, (it - ij.item0) * kRows + 16 * wave, iw.panel(), live,
                                 (ij.k + kTile - 1) / kTile, (ij.k + kGroup - 1) / kGroup, r);
    if (!live) return;
    if (iw.step(wave, NW) == 2) {
      if (++it < t_end) {
        if (it >= i_bound) {
          load_job<ONE>(jobs, ++ijn, ij);
          i_bound = job_end<ONE>(jobs, ijn);
          iw.start_job(ij.k, seg_panels, s0, wave, NW);
        }
        tile_rows(ij, (it - ij.item0) * kRows + 16 * wave, tl);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) tl.row[q] = ij.codes;
      }
    }
  };

  // Panel steps are fenced off from the scheduler (sched_barrier): left
  // free, it gathers the requests of several slots in one place, so a wait
  // for one slot would also wait for the next.
  Panel<MX> slot[D];
#pragma unroll
  for (int s = 0; s < D; ++s) {
    issue(slot[s]);
    __builtin_amdgcn_sched_barrier(0);
  }
  {
    uint4 v[kStreamXUnits];
    x_request(cj.x, cj.k, cw.seg_col0(), v);
    x_write(v, cj.k, cw.seg_col0(), true, 0, pbuf);
  }
  __syncthreads();

  f32x4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  bool staged = false;   // the next segment's x is in the other buffer
  // One exit, after every D panel steps: an exit between steps becomes a
  // branch to a block shared with the loop's head, reached there with the
  // slots' requests in another order, and the compiler, merging the two
  // orders, would wait at the head for every request in flight.  So the last
  // pass may consume up to D - 1 panels past the run: they were requested as
  // dead (loaded again from the run's last tile: finite codes), and a tile
  // past the run is neither stored nor staged.
  for (;;) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      // The step that begins a segment requests the segment after it: the
      // next one of this tile, else the first one of the next tile (the same
      // segment, and nothing to stage, when the job's x fits one segment),
      // else that of the next job.  Uniform across the workgroup.
      // The branches choose the segment (scalars only); one request follows.
      uint4 xv[kStreamXUnits];
      bool pre = false;
      const uint16_t* xp = cj.x;
      int xk = 0, xseg0 = 0;
      if (cw.cnt == 0 && ct < t_end) {
        const bool tile_end = cw.segs_done + 1 == cw.nseg;
        if (!tile_end || (ct + 1 < t_end && (ONE || ct + 1 < c_bound))) {
          if (cw.nseg > 1) {
            pre = true;
            xk = cj.k;
            xseg0 = (cw.seg + 1 == cw.nseg ? 0 : cw.seg + 1) * seg_cols;
          }
        } else if (!ONE && ct + 1 < t_end) {
          GemvJob nj;
          load_job<ONE>(jobs, jn + 1, nj);
          PanelWalk nw;
          nw.start_job(nj.k, seg_panels, s0, wave, NW);
          pre = true;
          xp = nj.x;
          xk = nj.k;
          xseg0 = nw.seg_col0();
        }
      }
      if (pre) x_request(xp, xk, xseg0, xv);
      // the A operands are read from the panel buffer where the MFMAs use
      // them (register limit)
      panel_write(slot[s].v, pbuf);
      float sc[MX ? 4 : 2];
      panel_scales<MX, PK, SF>(slot[s], sc);
      issue(slot[s]);
      const uint16_t* xb = xs + xcur + cw.pos * kPanelCols;   // panel start within the staged segment
      auto get_b = [&](int t, int b, int c, uint4& B0, uint4& B1) {
        const uint16_t* bp = xb + brow[t] + 128 * b;
        B0 = *reinterpret_cast<const uint4*>(bp + bunit[c][0]);
        B1 = *reinterpret_cast<const uint4*>(bp + bunit[c][1]);
      };
      panel_mfma_lds<MT, MX>(pbuf, sc, get_b, acc);
      // The write is unconditional: without a request it stores whatever the
      // registers hold into the wave's own panel buffer (free until the next
      // step).  Behind a branch of its own the compiler could not pair it
      // with the request's branch, would take the loads as possibly pending
      // after the step, and wait at the next request for them and for every
      // weight request older than them.  Here its wait, at the end of a step
      // without a request, covers only the panel the next step consumes.
      x_write(xv, xk, xseg0, pre, xbuf - xcur, pbuf);
      staged = staged || pre;
      const int moved = cw.step(wave, NW);
      if (moved == 2) {   // tile done
        if (ct < t_end)
          store_tile<MT, SF == kFmtRow, true>(cj, (ct - cj.item0) * kRows + 16 * wave, m_rows, acc);
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if (++ct < t_end && !ONE && ct >= c_bound) {   // the run enters the next job
          load_job<ONE>(jobs, ++jn, cj);
          c_bound = job_end<ONE>(jobs, jn);
          cw.start_job(cj.k, seg_panels, s0, wave, NW);
        }
      }
      if (moved != 0 && staged) {   // switch to the segment staged meanwhile
        __syncthreads();
        xcur = xbuf - xcur;
        staged = false;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (ct >= t_end) return;
  }
}

// ----------------------------------------------------- MFMA, single call --
//
// One 16-row tile per workgroup; its NW waves split the tile's panels (wave
// w takes panels w, w + NW, ...) with a register pipeline two panels deep,
// and read their x^T fragments straight from global memory (x is small and
// stays in L2), so no barrier waits for a staging pass.  The waves' partial
// sums meet in LDS at the end.  A call is latency-bound when its grid is
// small: with one workgroup or less per CU (N <= 4096 on MI355X), 8 waves
// per tile halve the panels each wave waits for in turn.
template <int MT, bool MX, int T>
struct DirectSlot {
  Panel<MX> p[T];          // the panel of each of the workgroup's T 16-row tiles
  uint4 xb[MT][2][2][2];   // [m tile][block][chunk][first / last 8 K positions], shared by the T tiles
};

// T 16-row tiles per workgroup (T = 2: 32 rows) share each x^T fragment a
// wave loads, so x costs 1/T of the fragment reads per weight byte.
template <int MT, int D, bool MX, int NW, bool PK, int T, int SF>
__global__ __launch_bounds__(NW * kWave) void k_gemv_mfma_direct(GemvJob j, int m_rows) {
  __shared__ __align__(16) unsigned char pb[NW * kPanelBytes];
  __shared__ float red[NW * T * MT * 4 * kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int i = lane & 15, g = lane >> 4;
  const int np = (j.k + kPanelCols - 1) / kPanelCols;
  const int nkb = (j.k + kTile - 1) / kTile;
  const int groups = (j.k + kGroup - 1) / kGroup;
  const int nq = (np - wave + NW - 1) / NW;   // this wave's panels
  const int rot = j.k % 2048 == 0 ? blockIdx.x % np : 0;

  // each tile's row offsets (tiles past the last row load nothing), and
  // each lane's x rows (rows past m_rows read row m_rows - 1: their
  // products land in output columns not stored)
  int row0[T];
  bool tlive[T];
  TileLoads tl[T];
#pragma unroll
  for (int u = 0; u < T; ++u) {
    row0[u] = (blockIdx.x * T + u) * 16;
    tlive[u] = row0[u] < j.n;
    if (tlive[u]) tile_loads(j, row0[u], tl[u]);
  }
  const uint8_t* xrow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t)
    xrow[t] = reinterpret_cast<const uint8_t*>(j.x) + ((size_t)min(16 * t + i, m_rows - 1) * j.k + 16 * g) * 2;

  auto issue = [&](int q, DirectSlot<MT, MX, T>& r) {
    // panels rotated by the workgroup's index when K is a multiple of 2048
    // (PanelWalk: weights whose row stride is a multiple of 4 KB read slowly
    // when every workgroup starts at the same columns; single calls on the
    // dense layer's K = 4096 weights gained 1-6 %, K = 2560 / 3072 lost 1 %);
    // wave + NW * q < np, so one subtraction wraps it
    int p = wave + NW * q + rot;
    if (p >= np) p -= np;
    const bool live = q < nq;
#pragma unroll
    for (int u = 0; u < T; ++u)
      panel_issue_tile<MX, PK, true, SF>(j, tl[u], row0[u], p, live && tlive[u], nkb, groups, r.p[u]);
    if (live && (p + 1) * kPanelCols <= j.k) {   // a whole panel: every x load in bounds
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            const size_t off = (size_t)(p * kPanelCols + 128 * b + 64 * c) * 2;
            r.xb[t][b][c][0] = ld_global_u4(xrow[t], off);
            r.xb[t][b][c][1] = ld_global_u4(xrow[t], off + 16);
          }
    } else {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int kx = p * kPanelCols + 128 * b + 64 * c + 16 * g;
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            const int m = 16 * t + i;
            r.xb[t][b][c][0] = r.xb[t][b][c][1] = make_uint4(0, 0, 0, 0);
            if (live && m < m_rows && kx < j.k) {
              r.xb[t][b][c][0] = ld_global_u4(j.x, ((size_t)m * j.k + kx) * 2);
              r.xb[t][b][c][1] = ld_global_u4(j.x, ((size_t)m * j.k + kx + 8) * 2);
            }
          }
        }
    }
  };

  f32x4 acc[T][MT];
#pragma unroll
  for (int u = 0; u < T; ++u)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[u][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  DirectSlot<MT, MX, T> slot[D];
#pragma unroll
  for (int s = 0; s < D; ++s) issue(s, slot[s]);
  for (int q0 = 0; q0 < nq; q0 += D) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      if (q0 + s < nq) {
#pragma unroll
        for (int u = 0; u < T; ++u) {
          if (!tlive[u]) continue;
          uint4 a[2][2];
          panel_to_a(slot[s].p[u].v, pb + wave * kPanelBytes, a);
          float sc[MX ? 4 : 2];
          panel_scales<MX, PK, SF>(slot[s].p[u], sc);
          panel_mfma<MT, MX>(a, sc, [&](int t, int b, int c, uint4& B0, uint4& B1) {
            B0 = slot[s].xb[t][b][c][0];
            B1 = slot[s].xb[t][b][c][1];
          }, acc[u]);
        }
      }
      issue(q0 + s + D, slot[s]);
    }
  }

#pragma unroll
  for (int u = 0; u < T; ++u)
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) red[(((wave * T + u) * MT + t) * 4 + jj) * kWave + lane] = acc[u][t][jj];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int u = 0; u < T; ++u) {
      if (!tlive[u]) continue;
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int w = 1; w < NW; ++w) acc[u][t][jj] += red[(((w * T + u) * MT + t) * 4 + jj) * kWave + lane];
      store_tile<MT, SF == kFmtRow>(j, row0[u], m_rows, acc[u]);
    }
  }
}

// ------------------------------------------- MFMA, x in registers --
//
// Single calls on many rows whose K spans at most NW panels: wave w owns
// panel w of every tile, so its x^T fragments are the same for the whole
// run and are loaded once, into registers; the workgroup walks a
// contiguous run of 16-row tiles (16 rows x K contiguous bytes each), the
// panel of the tile D ahead in flight, and the waves' partial sums meet in
// LDS once per tile (two buffers, one barrier per tile).
template <int MT, int D, bool MX, int NW, bool PK, int SF>
__global__ __launch_bounds__(NW * kWave, MT == 1 ? 4 : 2) void k_gemv_mfma_xreg(GemvJob j, int m_rows, int tiles_per_block) {
  __shared__ __align__(16) unsigned char pb[NW * kPanelBytes];
  __shared__ float red[2][NW * MT * 4 * kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int i = lane & 15, g = lane >> 4;
  const int np = (j.k + kPanelCols - 1) / kPanelCols;
  const int nkb = (j.k + kTile - 1) / kTile;
  const int groups = (j.k + kGroup - 1) / kGroup;
  const int ntiles = (j.n + 15) / 16;
  const int t_begin = blockIdx.x * tiles_per_block;
  const int t_end = min(ntiles, t_begin + tiles_per_block);
  const bool pl = wave < np;          // waves past the last panel add zeros
  const int p = min(wave, np - 1);    // every request in bounds

  uint4 xb[MT][2][2][2];
  if (pl && (p + 1) * kPanelCols <= j.k) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const uint8_t* xr =
          reinterpret_cast<const uint8_t*>(j.x) + ((size_t)min(16 * t + i, m_rows - 1) * j.k + 16 * g) * 2;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const size_t off = (size_t)(p * kPanelCols + 128 * b + 64 * c) * 2;
          xb[t][b][c][0] = ld_global_u4(xr, off);
          xb[t][b][c][1] = ld_global_u4(xr, off + 16);
        }
    }
  } else {
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int kx = p * kPanelCols + 128 * b + 64 * c + 16 * g;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const int m = 16 * t + i;
          xb[t][b][c][0] = xb[t][b][c][1] = make_uint4(0, 0, 0, 0);
          if (pl && m < m_rows && kx < j.k) {
            xb[t][b][c][0] = ld_global_u4(j.x, ((size_t)m * j.k + kx) * 2);
            xb[t][b][c][1] = ld_global_u4(j.x, ((size_t)m * j.k + kx + 8) * 2);
          }
        }
      }
  }

  auto issue = [&](int t, Panel<MX>& r) {
    const int row0 = min(t, ntiles - 1) * 16;
    TileLoads tl;
    tile_loads(j, row0, tl);
    panel_issue_tile<MX, PK, true, SF>(j, tl, row0, p, pl && t < t_end, nkb, groups, r);
  };
  Panel<MX> slot[D];
#pragma unroll
  for (int s = 0; s < D; ++s) issue(t_begin + s, slot[s]);
  int buf = 0;
  for (int t0 = t_begin; t0 < t_end; t0 += D) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      const int t = t0 + s;
      if (t >= t_end) break;
      f32x4 acc[MT];
#pragma unroll
      for (int u = 0; u < MT; ++u) acc[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      uint4 a[2][2];
      panel_to_a(slot[s].v, pb + wave * kPanelBytes, a);
      float sc[MX ? 4 : 2];
      panel_scales<MX, PK, SF>(slot[s], sc);
      panel_mfma<MT, MX>(a, sc, [&](int u, int b, int c, uint4& B0, uint4& B1) {
        B0 = xb[u][b][c][0];
        B1 = xb[u][b][c][1];
      }, acc);
      issue(t + D, slot[s]);
#pragma unroll
      for (int u = 0; u < MT; ++u)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) red[buf][((wave * MT + u) * 4 + jj) * kWave + lane] = acc[u][jj];
      __syncthreads();
      // thread (mcol, row): 16 consecutive threads store 16 consecutive rows
      for (int v = threadIdx.x; v < MT * 16 * 16; v += NW * kWave) {
        const int row = v & 15, mcol = v >> 4;
        const int src = (((mcol >> 4) * 4 + (row & 3)) * kWave) + 16 * (row >> 2) + (mcol & 15);
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) sum += red[buf][w * MT * 4 * kWave + src];
        const int r = t * 16 + row;
        if (r < j.n && mcol < m_rows) {
          const float os = SF == kFmtRow ? output_scale(j, r) : 1.0f;
          st_global<uint16_t>(j.y, ((size_t)mcol * j.n + r) * 2, (uint16_t)f32_to_bf16_rne(sum * os));
        }
      }
      buf ^= 1;
    }
  }
}

// ------------------------------------------------------------------ W8A8 --
//
// The activation arrives quantized: e4m3fn codes xc[m, k] with one fp32
// scale xs for the whole tensor (per-tensor dynamic activation quantization,
// "feat(qwen4_exp): load-time per-tensor FP8 dense projections", What this
// adds), and y = xs * sum_kb scale_w(kb) * sum_{k in kb} dec(xc) dec(code).
// fp8 x fp8 products go straight to v_mfma_scale_f32_16x16x128_f8f6f4: one
// instruction per 16-row tile and 128-column block, no decode.  Its K layout
// (measured on MI355X): byte p of lane (i, g) is K position 16g + p for
// p < 16 and 64 + 16g + (p - 16) for p >= 16, so a lane's operand is the two
// 16-byte pieces at 16g and 64 + 16g -- exactly a[b][0] and a[b][1] of the
// panel transpose.  The instruction's per-lane e8m0 scale applies to row i
// and the 32-column group 4b + g of that block -- the MX layout -- so MX weights
// pass their scale bytes to the instruction; block weights pass 2^0 and
// scale each block's partial sum.  Its products are exact; its internal
// accumulation is a little coarser than fp32 (about 2^-14 of sum |p|
// measured), far inside the GEMV bound.
typedef int i32x8 __attribute__((ext_vector_type(8)));
constexpr int kE8m0One = 127;

template <bool MX>
struct Panel8 {
  uint4 v[4];     // as Panel: lane l holds row 4q + l/16, bytes 16*(l%16)
  float s[2];     // block: scale of each 128-column block (fp32 grid, or any format chosen at run time)
  uint16_t h[2];  // bf16 block grid: the scale bits as loaded
  int e[2];       // MX: e8m0 byte of row l%16, group 4*(block) + l/16
};

// SF as for panel_issue_tile: kSfAny picks the format at run time and loads
// each block scale only where it exists; kFmtBlock / kFmtBlockBf16 load it
// unconditionally from a clamped index; kFmtRow loads none.
template <bool MX, int SF = kSfAny>
__device__ __forceinline__ void panel8_issue(const GemvJob& j, int row0, int p, bool live, int nkb,
                                             int groups, Panel8<MX>& r) {
  const int lane = threadIdx.x & (kWave - 1);
  const int col = p * kPanelCols + 16 * (lane & 15);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = row0 + 4 * q + (lane >> 4);
    r.v[q] = make_uint4(0, 0, 0, 0);
    if (live && row < j.n && col < j.k) r.v[q] = ld_stream_u4(j.codes, (size_t)row * j.k + col);
  }
  r.s[0] = r.s[1] = 0.0f;
  if (MX) {
    // Unconditional loads from a row and group clamped into the weight (as
    // panel_issue): rows and columns outside it have zero codes.  A default
    // joined with a conditional load would make the wave wait for the load.
    const int row = min(row0 + (lane & 15), j.n - 1);
    const uint8_t* __restrict__ e8 = static_cast<const uint8_t*>(j.scales);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int grp = min(4 * (2 * p + b) + (lane >> 4), groups - 1);
      r.e[b] = ld_global<uint8_t>(e8, (size_t)row * groups + grp);
    }
  } else {
    r.e[0] = r.e[1] = kE8m0One;
  }
  if (!MX && SF == kFmtBlock) {
#pragma unroll
    for (int b = 0; b < 2; ++b) r.s[b] = ld_global<float>(j.scales, block_scale_at(j, row0, 2 * p + b, nkb) * 4);
  } else if (!MX && SF == kFmtBlockBf16) {
#pragma unroll
    for (int b = 0; b < 2; ++b)
      r.h[b] = ld_global<uint16_t>(j.scales, block_scale_at(j, row0, 2 * p + b, nkb) * 2);
  } else if (!MX && SF == kSfAny && live && row0 < j.n) {
    r.s[0] = block_scale(j, row0, 2 * p, nkb);
    if (2 * p + 1 < nkb) r.s[1] = block_scale(j, row0, 2 * p + 1, nkb);
  } else if (!MX && SF == kFmtRow) {
    r.s[0] = r.s[1] = 1.0f;
  }
}

// A panel's block scales as the MFMA step uses them: the same in every lane
// (one 16-row tile, one block), so taken into scalar registers where the
// panel is consumed (panel_scales has the reason).
template <bool MX, int SF>
__device__ __forceinline__ void panel8_scales(Panel8<MX>& r) {
  if (MX) return;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const float v = SF == kFmtBlockBf16 ? __uint_as_float((uint32_t)r.h[b] << 16) : r.s[b];
    r.s[b] = SF == kFmtRow ? 1.0f : __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
  }
}

__device__ __forceinline__ i32x8 join8(uint4 lo, uint4 hi) {
  return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// acc += the panel's products; get_b(t, b, B_lo, B_hi) supplies the x codes
// of m-tile t for block b (the pieces at 16g and 64 + 16g).
template <int MT, bool MX, typename GetB>
__device__ __forceinline__ void panel8_mfma(const uint4 (&a)[2][2], const Panel8<MX>& p, GetB get_b,
                                            f32x4 (&acc)[MT]) {
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const i32x8 A = join8(a[b][0], a[b][1]);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      uint4 lo, hi;
      get_b(t, b, lo, hi);
      const i32x8 B = join8(lo, hi);
      if (MX) {
        acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc[t], 0, 0, 0, p.e[b], 0, kE8m0One);
      } else {
        const f32x4 part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            A, B, f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0, kE8m0One, 0, kE8m0One);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[t][jj] = __builtin_fmaf(p.s[b], part[jj], acc[t][jj]);
      }
    }
  }
}

// Single call: one 16-row tile per workgroup, the 4 waves split its panels
// (as k_gemv_mfma_direct); x codes from global memory.  xc is [m, k] e4m3,
// xs a device pointer to the activation scale.
template <int MT, bool MX>
struct Direct8Slot {
  Panel8<MX> p;
  uint4 xb[MT][2][2];   // [m tile][block][piece at 16g / at 64 + 16g]
};

template <int MT, int D, bool MX, int NW, int SF>
__global__ __launch_bounds__(NW * kWave) void k_gemv_w8a8_direct(GemvJob j, const float* __restrict__ xs,
                                                                 int m_rows) {
  __shared__ __align__(16) unsigned char pb[NW * kPanelBytes];
  __shared__ float red[NW * MT * 4 * kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int i = lane & 15, g = lane >> 4;
  const int row0 = blockIdx.x * 16;
  const int np = (j.k + kPanelCols - 1) / kPanelCols;
  const int nkb = (j.k + kTile - 1) / kTile;
  const int groups = (j.k + kGroup - 1) / kGroup;
  const int nq = (np - wave + NW - 1) / NW;
  const int rot = j.k % 2048 == 0 ? blockIdx.x % np : 0;   // as k_gemv_mfma_direct
  const uint8_t* __restrict__ xc = reinterpret_cast<const uint8_t*>(j.x);

  auto issue = [&](int q, Direct8Slot<MT, MX>& r) {
    int p = wave + NW * q + rot;
    if (p >= np) p -= np;
    const bool live = q < nq;
    panel8_issue<MX, SF>(j, row0, p, live, nkb, groups, r.p);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kx = p * kPanelCols + 128 * b + 64 * h + 16 * g;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const int m = 16 * t + i;
          r.xb[t][b][h] = make_uint4(0, 0, 0, 0);
          if (live && m < m_rows && kx < j.k) r.xb[t][b][h] = ld_global_u4(xc, (size_t)m * j.k + kx);
        }
      }
  };

  f32x4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  Direct8Slot<MT, MX> slot[D];
#pragma unroll
  for (int s = 0; s < D; ++s) issue(s, slot[s]);
  for (int q0 = 0; q0 < nq; q0 += D) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      if (q0 + s < nq) {
        uint4 a[2][2];
        panel_to_a(slot[s].p.v, pb + wave * kPanelBytes, a);
        panel8_scales<MX, SF>(slot[s].p);
        panel8_mfma<MT, MX>(a, slot[s].p, [&](int t, int b, uint4& lo, uint4& hi) {
          lo = slot[s].xb[t][b][0];
          hi = slot[s].xb[t][b][1];
        }, acc);
      }
      issue(q0 + s + D, slot[s]);
    }
  }

#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) red[((wave * MT + t) * 4 + jj) * kWave + lane] = acc[t][jj];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int w = 1; w < NW; ++w) acc[t][jj] += red[((w * MT + t) * 4 + jj) * kWave + lane];
    store_tile<MT, SF == kFmtRow>(j, row0, m_rows, acc, ld_global<float>(xs, 0));
  }
}

// Single calls on weights with many rows: one 128-row tile per workgroup, a
// 16-row tile per wave over the whole K, the x codes staged once per tile in
// LDS by K segments of seg_cols columns (rows of seg_cols + 16 bytes), so x
// is read from L2 once per 128 rows instead of once per 16.
template <int MT, bool MX>
__global__ __launch_bounds__(8 * kWave) void k_gemv_w8a8_tiles(GemvJob j, const float* __restrict__ xs_scale,
                                                               int m_rows, int seg_cols) {
  constexpr int NW = 8, D = 2;
  extern __shared__ __align__(16) unsigned char smem[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int i = lane & 15, g = lane >> 4;
  unsigned char* pbuf = smem + wave * kPanelBytes;
  unsigned char* xs = smem + NW * kPanelBytes;
  const int ldx = seg_cols + 16;
  const int seg_panels = seg_cols / kPanelCols;
  const int row0 = blockIdx.x * (16 * NW) + 16 * wave;
  const int np = (j.k + kPanelCols - 1) / kPanelCols;
  const int nkb = (j.k + kTile - 1) / kTile;
  const int groups = (j.k + kGroup - 1) / kGroup;
  const uint8_t* __restrict__ xc = reinterpret_cast<const uint8_t*>(j.x);
  // x codes [0, m_rows) x [seg0, seg0 + seg_cols) into LDS (columns < k only:
  // the B reads never look past k)
  auto stage = [&](int seg0) {
    const int units = min(seg_cols, j.k - seg0) / 16;
    copy_batched<kStageBatch, NW * kWave, uint4>(
        m_rows * units,
        [&](int u) {
          const int r = u / units, c = (u - r * units) * 16;
          return ld_global_u4(xc, (size_t)r * j.k + seg0 + c);
        },
        [&](int u, uint4 v) {
          const int r = u / units, c = (u - r * units) * 16;
          *reinterpret_cast<uint4*>(xs + r * ldx + c) = v;
        });
  };

  Panel8<MX> slot[D];
#pragma unroll
  for (int s = 0; s < D; ++s) panel8_issue<MX>(j, row0, s, s < np, nkb, groups, slot[s]);
  stage(0);
  __syncthreads();
  f32x4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int p0 = 0; p0 < np; p0 += D) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      const int p = p0 + s;
      if (p < np) {   // uniform over the workgroup
        if (p > 0 && p % seg_panels == 0) {   // next K segment of x
          __syncthreads();
          stage(p * kPanelCols);
          __syncthreads();
        }
        uint4 a[2][2];
        panel_to_a(slot[s].v, pbuf, a);
        Panel8<MX> cur;
        cur.s[0] = slot[s].s[0], cur.s[1] = slot[s].s[1];
        cur.e[0] = slot[s].e[0], cur.e[1] = slot[s].e[1];
        panel8_issue<MX>(j, row0, p + D, p + D < np, nkb, groups, slot[s]);
        const int kseg = (p % seg_panels) * kPanelCols, kp = p * kPanelCols;
        panel8_mfma<MT, MX>(a, cur, [&](int t, int b, uint4& lo, uint4& hi) {
          const int m = 16 * t + i;
          const int kx = 128 * b + 16 * g;
          lo = hi = make_uint4(0, 0, 0, 0);
          if (m < m_rows && kp + kx < j.k) lo = *reinterpret_cast<const uint4*>(xs + m * ldx + kseg + kx);
          if (m < m_rows && kp + kx + 64 < j.k) hi = *reinterpret_cast<const uint4*>(xs + m * ldx + kseg + kx + 64);
        }, acc);
      }
    }
  }
  store_tile<MT>(j, row0, m_rows, acc, ld_global<float>(xs_scale, 0));
}

// ------------------------------------------------------------ dispatch --
//
// One compiled variant per (route, M, single/grouped), any N and K:
//   VALU single call: R = 1 row per wave (4 rows per workgroup: the most
//     workgroups for small N); grouped: more rows per wave (fewer, larger
//     workgroups once many GEMVs share the launch).
//   MFMA single call: k_gemv_mfma_direct, one 16-row tile per workgroup
//     (4 waves; 8 on at most kDirect8MaxRows rows).
//   MFMA grouped: k_gemv_mfma_stream16 / 32, 8 waves, 128-row tiles.

template <int M, int R, int C, bool MX, bool G>
hipError_t run_valu(const GemvJob& job, const GemvJob* table, int njobs, int64_t blocks,
                    hipStream_t stream) {
  hipLaunchKernelGGL((k_gemv_valu<M, R, C, MX, G>), dim3((unsigned)blocks), dim3(kThreads), 0,
                     stream, job, table, njobs);
  return hipGetLastError();
}

// (rows per wave R, 16-byte chunks per lane per segment C) of the VALU
// route.  WIDE (grouped launches, and single calls with many rows): 4 rows
// per wave, fewer and larger workgroups; otherwise 1 or 2 rows per wave, the
// most workgroups for small N.
template <bool MX, bool G>
hipError_t dispatch_valu(int m, bool wide, bool seg4096, const GemvJob& job, const GemvJob* table, int njobs,
                         int64_t blocks, hipStream_t s) {
  if (wide) {
    switch (m) {
      case 1:
        return seg4096 ? run_valu<1, 4, 4, MX, G>(job, table, njobs, blocks, s)
                       : run_valu<1, 4, 3, MX, G>(job, table, njobs, blocks, s);
      case 2: return run_valu<2, 4, 2, MX, G>(job, table, njobs, blocks, s);
      case 3: return run_valu<3, 4, 2, MX, G>(job, table, njobs, blocks, s);
      case 4: return run_valu<4, 4, 2, MX, G>(job, table, njobs, blocks, s);
      case 5: return run_valu<5, 4, 2, MX, G>(job, table, njobs, blocks, s);
      case 6: return run_valu<6, 4, 2, MX, G>(job, table, njobs, blocks, s);
      case 7: return run_valu<7, 4, 2, MX, G>(job, table, njobs, blocks, s);
      case 8: return run_valu<8, 4, 2, MX, G>(job, table, njobs, blocks, s);
    }
  } else {
    switch (m) {
      case 1: return run_valu<1, 1, 4, MX, G>(job, table, njobs, blocks, s);
      case 2: return run_valu<2, 2, 4, MX, G>(job, table, njobs, blocks, s);
      case 3: return run_valu<3, 2, 4, MX, G>(job, table, njobs, blocks, s);
      case 4: return run_valu<4, 2, 4, MX, G>(job, table, njobs, blocks, s);
      case 5: return run_valu<5, 2, 2, MX, G>(job, table, njobs, blocks, s);
      case 6: return run_valu<6, 2, 2, MX, G>(job, table, njobs, blocks, s);
      case 7: return run_valu<7, 2, 2, MX, G>(job, table, njobs, blocks, s);
      case 8: return run_valu<8, 2, 2, MX, G>(job, table, njobs, blocks, s);
    }
  }
  return hipErrorInvalidValue;
}

// MFMA streaming kernel: waves per workgroup (panel pipeline two deep) and
// the LDS each workgroup may take (two workgroups per CU).  Measured on the
// projection set: a deeper pipeline or 16-wave workgroups with twice the LDS
// are no faster, and cost occupancy.
constexpr int kMfmaStreamWaves = 8;
constexpr int kMfmaStreamLds = 80 * 1024;

// Streaming kernel of M = 1 VALU launches: (R, C) and its K limit.
constexpr int kStreamR = 4, kStreamC = 3;

// Single MFMA calls on at most this many rows (one 16-row workgroup or less
// per CU) split each tile's panels over 8 waves instead of 4.
constexpr int64_t kDirect8MaxRows = 4096;
// Two-tile single MFMA calls at 9 <= M <= 16 on at most this many rows
// split each workgroup's panels over 8 waves, on more rows over 4.
constexpr int64_t kDirectT2Wave8MaxRows = 8192;

// MT = 1: up to 16 rows (k_gemv_mfma_stream16); MT = 2: 17..32 rows
// (k_gemv_mfma_stream32).  Both take the same arguments.
template <int MT, bool MX, bool ONE, bool PK, int SF>
constexpr auto mfma_stream_kernel() {
  if constexpr (MT == 1) return &k_gemv_mfma_stream16<kMfmaStreamWaves, 2, MX, ONE, PK, SF>;
  else return &k_gemv_mfma_stream32<kMfmaStreamWaves, 2, MX, ONE, PK, SF>;
}

// The kernel needs more than the default 64 KB of dynamic LDS: raise the
// limit once per device and variant.  Host threads may race here; setting
// the attribute twice is harmless, so a relaxed flag suffices.
template <int MT, bool MX, bool ONE, bool PK, int SF>
hipError_t allow_mfma_stream_lds() {
  static std::atomic<bool> done[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!done[dev].load(std::memory_order_relaxed)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(mfma_stream_kernel<MT, MX, ONE, PK, SF>()),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kMfmaStreamLds);
    if (e != hipSuccess) return e;
    done[dev].store(true, std::memory_order_relaxed);
  }
  return hipSuccess;
}

// Launch arguments of a streaming kernel: a job table, or one job.
struct StreamJobs {
  const GemvJob* table;
  int count;
  GemvJob one;
};

template <bool MX, bool ONE>
hipError_t run_valu_stream(const StreamJobs& l, int64_t blocks, int64_t tiles, int tiles_per_block,
                           hipStream_t stream) {
  if (ONE && (tiles_per_block != 1 || blocks != tiles)) return hipErrorInvalidValue;   // one tile each
  hipLaunchKernelGGL((k_gemv_valu_stream<kStreamR, kStreamC, MX, ONE>), dim3((unsigned)blocks),
                     dim3(kThreads), 0, stream, l.table, l.count, l.one, (int)tiles, tiles_per_block);
  return hipGetLastError();
}

int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int c = cache[dev].load();
  if (c == 0) {
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
    cache[dev].store(c);
  }
  return c;
}

// Waves per workgroup (one panel each) and panels in flight per wave of the
// x-in-registers kernel: at 17..32 rows its x fragments take 64 VGPRs, so one
// 8-wave workgroup runs per CU, and four panels in flight per wave keep HBM
// busy (single calls on MI355X, [151936x2048] M = 32, % of 8 TB/s with two /
// three / four: 57.5 / 59.3 / 59.8).
constexpr int kXregWaves = 8;
constexpr int kXregDepth = 4;

template <int MT>
hipError_t launch_mfma_xreg(const GemvJob& job, int m, bool mx, bool pk, hipStream_t stream) {
  constexpr int D = kXregDepth, NW = kXregWaves;
  const int64_t ntiles = (job.n + 15) / 16;
  const int64_t slots = (MT == 1 ? 2 : 1) * (int64_t)device_cus();   // workgroups resident per CU
  const int tpb = (int)((ntiles + slots - 1) / slots);
  const dim3 grid((unsigned)((ntiles + tpb - 1) / tpb)), block(NW * kWave);
  if (mx && pk)
    hipLaunchKernelGGL((k_gemv_mfma_xreg<MT, D, true, NW, true, kFmtMx>), grid, block, 0, stream, job, m, tpb);
  else if (mx)
    hipLaunchKernelGGL((k_gemv_mfma_xreg<MT, D, true, NW, false, kFmtMx>), grid, block, 0, stream, job, m, tpb);
  else if (job.format == kFmtBlock)
    hipLaunchKernelGGL((k_gemv_mfma_xreg<MT, D, false, NW, false, kFmtBlock>), grid, block, 0, stream, job, m, tpb);
  else if (job.format == kFmtBlockBf16)
    hipLaunchKernelGGL((k_gemv_mfma_xreg<MT, D, false, NW, false, kFmtBlockBf16>), grid, block, 0, stream, job, m,
                       tpb);
  else
    hipLaunchKernelGGL((k_gemv_mfma_xreg<MT, D, false, NW, false, kFmtRow>), grid, block, 0, stream, job, m, tpb);
  return hipGetLastError();
}

template <int MT, bool MX, bool ONE, bool PK, int SF>
hipError_t run_mfma_stream(const StreamJobs& l, int64_t blocks, int64_t tiles, int tiles_per_block, int m,
                           int seg_cols, hipStream_t stream);

// The scale format every job of the launch shares selects the variant.
template <int MT, bool ONE>
hipError_t dispatch_mfma_stream_mt(const StreamJobs& l, int64_t blocks, int64_t tiles, int tiles_per_block,
                                   int m, int seg_cols, int format, bool pk, hipStream_t s) {
  switch (format) {
    case kFmtMx:
      return pk ? run_mfma_stream<MT, true, ONE, true, kFmtMx>(l, blocks, tiles, tiles_per_block, m, seg_cols, s)
                : run_mfma_stream<MT, true, ONE, false, kFmtMx>(l, blocks, tiles, tiles_per_block, m, seg_cols, s);
    case kFmtBlock:
      return run_mfma_stream<MT, false, ONE, false, kFmtBlock>(l, blocks, tiles, tiles_per_block, m, seg_cols, s);
    case kFmtBlockBf16:
      return run_mfma_stream<MT, false, ONE, false, kFmtBlockBf16>(l, blocks, tiles, tiles_per_block, m,
                                                                   seg_cols, s);
    default:   // kFmtRow, kFmtTensor
      return run_mfma_stream<MT, false, ONE, false, kFmtRow>(l, blocks, tiles, tiles_per_block, m, seg_cols, s);
  }
}

template <bool ONE>
hipError_t dispatch_mfma_stream(const StreamJobs& l, int64_t blocks, int64_t tiles, int tiles_per_block,
                                int m, int seg_cols, int format, bool pk, hipStream_t s) {
  return m <= 16 ? dispatch_mfma_stream_mt<1, ONE>(l, blocks, tiles, tiles_per_block, m, seg_cols, format, pk, s)
                 : dispatch_mfma_stream_mt<2, ONE>(l, blocks, tiles, tiles_per_block, m, seg_cols, format, pk, s);
}

// Single calls with many rows take the wide VALU tiles (the streaming
// kernel at m = 1, K <= 3072) and the streaming MFMA kernel (one job passed
// by value, one 128-row tile per workgroup, x staged once per tile in LDS):
// their larger tiles keep more weight bytes in flight per wave, and once
// the launch has enough tiles to fill the chip that wins.  Crossovers
// measured on MI355X over N = 4096..65536, K = 2048..4096: VALU from N =
// 16384 (1.05-1.2x at K <= 3072, even at K = 4096); MFMA from N = 32768
// (1.1-2.5x, the gain growing with m), and from N = 16384 when m > 16.
constexpr int64_t kSingleWideMinRowsValu = 16384;

// Single calls below that many rows with M <= kRowsMaxM run the one-wave
// kernel up to K = 1024 * kRowsMaxC (M = 1) or 1024 * kRowsMultiMaxC (M > 1).
constexpr int kRowsMaxC = 4;
constexpr int kRowsMaxM = 4;
constexpr int kRowsMultiMaxC = 3;
// Rows per wave at M = 1: one up to 4096 rows, where the call has too few
// rows to keep every SIMD busy with two (graph-captured single calls on
// MI355X: [2560x3072] 1.4 % faster with block scales and 2.5 % with MX; two
// rows per wave stay faster on [6656x2560] and [8192x2560], by 7-8 %).
constexpr int64_t kRowsOneMaxN = 4096;

template <int R, int C, bool MX, int M>
hipError_t run_valu_rows(const GemvJob& job, hipStream_t stream) {
  hipLaunchKernelGGL((k_gemv_valu_rows<R, C, MX, M>), dim3((unsigned)((job.n + R - 1) / R)),
                     dim3(kWave), 0, stream, job);
  return hipGetLastError();
}

template <int R, bool MX, int M>
hipError_t dispatch_valu_rows_r(const GemvJob& job, hipStream_t stream) {
  switch ((job.k + 1023) / 1024) {
    case 1: return run_valu_rows<R, 1, MX, M>(job, stream);
    case 2: return run_valu_rows<R, 2, MX, M>(job, stream);
    case 3: return run_valu_rows<R, 3, MX, M>(job, stream);
    case 4:
      if constexpr (M == 1) return run_valu_rows<R, 4, MX, M>(job, stream);
      break;
  }
  return hipErrorInvalidValue;
}

// One wave reads R rows against M activation rows held in registers.  Each
// wave loads all of x from L2, so more rows per wave pay off as M grows.
// Graph-captured single calls on MI355X, M = 2..4, block / MX scales,
// against the LDS-staging kernel: [2560x3072] with 2 rows per wave +7..+9 /
// +17..+21 %; [6656x2560] with 4 rows +0.5..+6.5 / +7..+12 %; [8192x2560]
// -4.6 (block, M = 3)..+3 / -2..+8 %.  One row per wave loses 10-40 %.  At
// K = 4096 the registers for x cut occupancy and the LDS-staging kernel
// stays 10-25 % ahead, hence M > 1 stops at K = 3072.
template <bool MX, int M>
hipError_t dispatch_valu_rows_m(const GemvJob& job, hipStream_t stream) {
  if constexpr (M == 1) {
    return job.n <= kRowsOneMaxN ? dispatch_valu_rows_r<1, MX, M>(job, stream)
                                 : dispatch_valu_rows_r<2, MX, M>(job, stream);
  } else {
    return job.n <= kRowsOneMaxN ? dispatch_valu_rows_r<2, MX, M>(job, stream)
                                 : dispatch_valu_rows_r<4, MX, M>(job, stream);
  }
}

template <bool MX>
hipError_t dispatch_valu_rows(const GemvJob& job, int m, hipStream_t stream) {
  switch (m) {
    case 1: return dispatch_valu_rows_m<MX, 1>(job, stream);
    case 2: return dispatch_valu_rows_m<MX, 2>(job, stream);
    case 3: return dispatch_valu_rows_m<MX, 3>(job, stream);
    case 4: return dispatch_valu_rows_m<MX, 4>(job, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_valu_rows(const GemvJob& job, int m, bool mx, hipStream_t stream) {
  return mx ? dispatch_valu_rows<true>(job, m, stream) : dispatch_valu_rows<false>(job, m, stream);
}

bool single_call_streams_mfma(int64_t n, int m) { return n >= 32768 || (n >= 16384 && m > 16); }

}  // namespace

int gemv_rows_per_block(int route, int m, bool grouped) {
  if (route == 1) {
    if (grouped) return kWaves * 4;
    return kWaves * (m == 1 ? 1 : 2);
  }
  return grouped ? 16 * kMfmaStreamWaves : 16;
}

int gemv_stream_max_k() { return 1024 * kStreamC; }

int gemv_wide_seg_rounds(int64_t k, int seg_cols) { return (int)((k + seg_cols - 1) / seg_cols); }

int gemv_wide_seg_cols(int64_t k) {
  return gemv_wide_seg_rounds(k, 4096) < gemv_wide_seg_rounds(k, 3072) ? 4096 : 3072;
}
int gemv_stream_rows() { return kWaves * kStreamR; }

// Up to 16 rows: LDS bytes x may take, 1 KB under the per-workgroup share
// (at exactly half of the CU's LDS the measured rates fall as if only one
// workgroup fitted per CU).
constexpr int kStream16XBytes = kMfmaStreamLds - kMfmaStreamWaves * kPanelBytes - 1024;

int gemv_mfma_stream_seg_cols(int m, int64_t max_k) {
  if (m > 16) return kPanelCols;   // k_gemv_mfma_stream32: one-panel segments
  const int cap = kStream16XBytes / (2 * m) / kPanelCols * kPanelCols;
  const int64_t kmax = (max_k + kPanelCols - 1) / kPanelCols * kPanelCols;
  if (kmax <= cap) return (int)kmax;
  const int64_t nseg = (kmax + cap - 1) / cap;
  const int64_t per = (kmax + nseg - 1) / nseg;
  return (int)((per + kPanelCols - 1) / kPanelCols * kPanelCols);
}

int gemv_mfma_stream_lds(int m, int seg_cols) {
  // up to 16 rows one x buffer, above two
  return kMfmaStreamWaves * kPanelBytes + (m <= 16 ? 1 : 2) * m * seg_cols * 2;
}

bool gemv_mfma_stream_seg_ok(int m, int seg_cols) {
  if (m < 1 || m > 32) return false;
  if (m > 16) return seg_cols == kPanelCols;
  return seg_cols >= kPanelCols && seg_cols % kPanelCols == 0 &&
         (int64_t)m * seg_cols * 2 <= kStream16XBytes + 1024;
}


namespace {

// The job's scale format selects the variant (each loads its own scales
// unconditionally, so no join waits for them).
template <int MT, int NW, int T>
hipError_t launch_mfma_direct(const GemvJob& job, int m, bool mx, bool pk, hipStream_t stream) {
  const dim3 grid((unsigned)((job.n + 16 * T - 1) / (16 * T))), block(NW * kWave);
  if (mx && pk)
    hipLaunchKernelGGL((k_gemv_mfma_direct<MT, 2, true, NW, true, T, kFmtMx>), grid, block, 0, stream, job, m);
  else if (mx)
    hipLaunchKernelGGL((k_gemv_mfma_direct<MT, 2, true, NW, false, T, kFmtMx>), grid, block, 0, stream, job, m);
  else if (job.format == kFmtBlock)
    hipLaunchKernelGGL((k_gemv_mfma_direct<MT, 2, false, NW, false, T, kFmtBlock>), grid, block, 0, stream, job, m);
  else if (job.format == kFmtBlockBf16)
    hipLaunchKernelGGL((k_gemv_mfma_direct<MT, 2, false, NW, false, T, kFmtBlockBf16>), grid, block, 0, stream, job,
                       m);
  else
    hipLaunchKernelGGL((k_gemv_mfma_direct<MT, 2, false, NW, false, T, kFmtRow>), grid, block, 0, stream, job, m);
  return hipGetLastError();
}

template <int MT, bool MX, bool ONE, bool PK, int SF>
hipError_t run_mfma_stream(const StreamJobs& l, int64_t blocks, int64_t tiles, int tiles_per_block, int m,
                           int seg_cols, hipStream_t stream) {
  const hipError_t e = allow_mfma_stream_lds<MT, MX, ONE, PK, SF>();
  if (e != hipSuccess) return e;
  const size_t lds = (size_t)gemv_mfma_stream_lds(m, seg_cols);
  if constexpr (MT == 1)
    hipLaunchKernelGGL((k_gemv_mfma_stream16<kMfmaStreamWaves, 2, MX, ONE, PK, SF>), dim3((unsigned)blocks),
                       dim3(kMfmaStreamWaves * kWave), lds, stream, l.table, l.count, l.one, (int)tiles,
                       tiles_per_block, m, seg_cols);
  else
    hipLaunchKernelGGL((k_gemv_mfma_stream32<kMfmaStreamWaves, 2, MX, ONE, PK, SF>), dim3((unsigned)blocks),
                       dim3(kMfmaStreamWaves * kWave), lds, stream, l.table, l.count, l.one, (int)tiles,
                       tiles_per_block, m, seg_cols);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(const GemvJob& job, int m, bool mx, int route, hipStream_t stream) {
  if (route == 1) {
    const bool wide = job.n >= kSingleWideMinRowsValu;
    if (wide && m == 1 && job.k <= gemv_stream_max_k() && (!mx || mx_rows_stream(job.scales, job.n, job.k))) {
      StreamJobs l{nullptr, 1, job};
      l.one.item0 = 0;
      const int64_t tiles = (job.n + gemv_stream_rows() - 1) / gemv_stream_rows();
      return mx ? run_valu_stream<true, true>(l, tiles, tiles, 1, stream)
                : run_valu_stream<false, true>(l, tiles, tiles, 1, stream);
    }
    if (!wide && m <= kRowsMaxM && job.k <= 1024 * (m == 1 ? kRowsMaxC : kRowsMultiMaxC))
      return launch_valu_rows(job, m, mx, stream);
    const int rows = wide ? gemv_rows_per_block(route, m, true) : gemv_rows_per_block(route, m, false);
    const int64_t blocks = (job.n + rows - 1) / rows;
    const bool seg4096 = wide && m == 1 && gemv_wide_seg_cols(job.k) == 4096;
    return mx ? dispatch_valu<true, false>(m, wide, seg4096, job, nullptr, 1, blocks, stream)
              : dispatch_valu<false, false>(m, wide, seg4096, job, nullptr, 1, blocks, stream);
  }
  // Above 16 rows, on K of eight panels (1793..2048), each wave keeps its x^T
  // fragments in registers for a whole run of tiles instead of staging x in
  // LDS per tile (single calls on MI355X, [151936x2048] M = 32: 57.6 -> 59.8 %
  // of 8 TB/s; at M = 4 / 16, two workgroups per CU, it lost 1-2 % to the
  // streaming kernel).
  if (m > 16 && single_call_streams_mfma(job.n, m) && (job.k + kPanelCols - 1) / kPanelCols == kXregWaves)
    return launch_mfma_xreg<2>(job, m, mx, mx && mx_rows_packed8(job.scales, job.k), stream);
  if (single_call_streams_mfma(job.n, m)) {
    StreamJobs l{nullptr, 1, job};
    l.one.item0 = 0;
    const int rows = gemv_rows_per_block(route, m, true);
    const int64_t tiles = (job.n + rows - 1) / rows;
    return dispatch_mfma_stream<true>(l, tiles, tiles, 1, m, gemv_mfma_stream_seg_cols(m, job.k), job.format,
                                      mx && mx_rows_packed8(job.scales, job.k), stream);
  }
  const bool pk = mx && mx_rows_packed8(job.scales, job.k);
  if (job.n <= kDirect8MaxRows) {
    return m <= 16 ? launch_mfma_direct<1, 8, 1>(job, m, mx, pk, stream)
                   : launch_mfma_direct<2, 8, 1>(job, m, mx, pk, stream);
  }
  // Above M = 8 two 16-row tiles per workgroup share each x^T fragment
  // (graph-captured single calls on MI355X, block / MX: M = 16 on
  // [8192x2560] +6 / +6 % with 8 waves, [6144x4096] +15 / +12 %,
  // [24576x4096] +4 / +7 % with 4 waves; M = 32 +6..+21 / +4..+28 % with 4
  // waves).  At M <= 8 the fragments are half duplicates (rows past M) and
  // the shared tiles lose 3-9 %.
  if (m <= 8) return launch_mfma_direct<1, kWaves, 1>(job, m, mx, pk, stream);
  if (m <= 16) {
    return job.n <= kDirectT2Wave8MaxRows ? launch_mfma_direct<1, 8, 2>(job, m, mx, pk, stream)
                                          : launch_mfma_direct<1, kWaves, 2>(job, m, mx, pk, stream);
  }
  return launch_mfma_direct<2, kWaves, 2>(job, m, mx, pk, stream);
}

bool mx_rows_stream(const void* e8m0, int64_t n, int64_t k) {
  return reinterpret_cast<uintptr_t>(e8m0) % 4 == 0 && (n * ((k + kGroup - 1) / kGroup)) % 4 == 0;
}

bool mx_rows_packed8(const void* e8m0, int64_t k) {
  return ((k + kGroup - 1) / kGroup) % 8 == 0 && reinterpret_cast<uintptr_t>(e8m0) % 8 == 0;
}

hipError_t gemv_stream_slots(bool mx, int* slots) {
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = mx ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                 &per_cu, k_gemv_valu_stream<kStreamR, kStreamC, true, false>, kThreads, 0)
           : hipOccupancyMaxActiveBlocksPerMultiprocessor(
                 &per_cu, k_gemv_valu_stream<kStreamR, kStreamC, false, false>, kThreads, 0);
  *slots = cus * (per_cu > 0 ? per_cu : 1);
  return e;
}

hipError_t launch_gemv_stream(const GemvJob* table, int njobs, int64_t blocks, int64_t tiles,
                              int tiles_per_block, bool mx, hipStream_t stream) {
  const StreamJobs l{table, njobs, GemvJob{}};
  return mx ? run_valu_stream<true, false>(l, blocks, tiles, tiles_per_block, stream)
            : run_valu_stream<false, false>(l, blocks, tiles, tiles_per_block, stream);
}

hipError_t launch_gemv_grouped(const GemvJob* table, int njobs, int64_t blocks, int m, bool mx, int seg_cols,
                               hipStream_t stream) {
  const GemvJob none{};
  const bool seg4096 = m == 1 && seg_cols == 4096;
  return mx ? dispatch_valu<true, true>(m, true, seg4096, none, table, njobs, blocks, stream)
            : dispatch_valu<false, true>(m, true, seg4096, none, table, njobs, blocks, stream);
}

namespace {

// Resident workgroups per CU of a streaming MFMA variant at `lds` bytes.
template <int MT, bool MX>
hipError_t stream_occupancy(int threads, size_t lds, int* per_cu) {
  constexpr int SF = MX ? kFmtMx : kFmtBlock;
  hipError_t e = allow_mfma_stream_lds<MT, MX, false, false, SF>();
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, mfma_stream_kernel<MT, MX, false, false, SF>(),
                                                     threads, lds);
  return e;
}

}  // namespace

hipError_t gemv_mfma_stream_slots(int m, bool mx, int seg_cols, int* slots) {
  const size_t lds = (size_t)gemv_mfma_stream_lds(m, seg_cols);
  const int threads = kMfmaStreamWaves * kWave;
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) {
    if (m > 16)
      e = mx ? stream_occupancy<2, true>(threads, lds, &per_cu) : stream_occupancy<2, false>(threads, lds, &per_cu);
    else
      e = mx ? stream_occupancy<1, true>(threads, lds, &per_cu) : stream_occupancy<1, false>(threads, lds, &per_cu);
  }
  *slots = cus * (per_cu > 0 ? per_cu : 1);
  return e;
}

namespace {

template <int M, int R, int C, bool MX>
hipError_t run_valu_x8(const GemvJob& job, const float* x_scale, hipStream_t stream) {
  const int rows = kWaves * R;
  hipLaunchKernelGGL((k_gemv_valu<M, R, C, MX, false, true>), dim3((unsigned)((job.n + rows - 1) / rows)),
                     dim3(kThreads), 0, stream, job, nullptr, 1, x_scale);
  return hipGetLastError();
}

template <bool MX>
hipError_t dispatch_valu_x8(const GemvJob& job, const float* x_scale, int m, hipStream_t s) {
  const bool wide = job.n >= kSingleWideMinRowsValu;
  if (m == 1) return wide ? run_valu_x8<1, 4, 3, MX>(job, x_scale, s) : run_valu_x8<1, 1, 4, MX>(job, x_scale, s);
  return wide ? run_valu_x8<2, 4, 2, MX>(job, x_scale, s) : run_valu_x8<2, 2, 4, MX>(job, x_scale, s);
}

// The 128-row W8A8 kernel's LDS: eight 4 KB panel buffers and the staged x
// codes, within the same per-workgroup budget as the streaming MFMA kernel.
int w8a8_tiles_seg_cols(int m, int64_t k) {
  const int x_budget = kMfmaStreamLds - 8 * kPanelBytes;
  const int cap = (x_budget / m - 16) / kPanelCols * kPanelCols;
  const int64_t kmax = (k + kPanelCols - 1) / kPanelCols * kPanelCols;
  if (kmax <= cap) return (int)kmax;
  const int64_t nseg = (kmax + cap - 1) / cap;
  const int64_t per = (kmax + nseg - 1) / nseg;
  return (int)((per + kPanelCols - 1) / kPanelCols * kPanelCols);
}

template <int MT, bool MX>
hipError_t run_w8a8_tiles(const GemvJob& job, const float* x_scale, int m, hipStream_t stream) {
  static std::atomic<bool> done[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!done[dev].load(std::memory_order_relaxed)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemv_w8a8_tiles<MT, MX>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kMfmaStreamLds);
    if (e != hipSuccess) return e;
    done[dev].store(true, std::memory_order_relaxed);
  }
  const int seg = w8a8_tiles_seg_cols(m, job.k);
  const size_t lds = (size_t)8 * kPanelBytes + (size_t)m * (seg + 16);
  hipLaunchKernelGGL((k_gemv_w8a8_tiles<MT, MX>), dim3((unsigned)((job.n + 127) / 128)), dim3(8 * kWave), lds,
                     stream, job, x_scale, m, seg);
  return hipGetLastError();
}

// The non-MX W8A8 direct kernel for the job's scale format.
template <int MT, int NW>
void launch_w8a8_direct_fmt(dim3 grid, dim3 block, const GemvJob& job, const float* x_scale, int m,
                            hipStream_t stream) {
  if (job.format == kFmtBlock)
    hipLaunchKernelGGL((k_gemv_w8a8_direct<MT, 2, false, NW, kFmtBlock>), grid, block, 0, stream, job, x_scale, m);
  else if (job.format == kFmtBlockBf16)
    hipLaunchKernelGGL((k_gemv_w8a8_direct<MT, 2, false, NW, kFmtBlockBf16>), grid, block, 0, stream, job, x_scale,
                       m);
  else
    hipLaunchKernelGGL((k_gemv_w8a8_direct<MT, 2, false, NW, kFmtRow>), grid, block, 0, stream, job, x_scale, m);
}

}  // namespace

// W8A8: m <= 2 on the VALU kernel with the codes widened while x is staged
// (as the W8A16 route, which is faster than the MFMA kernel at these m);
// larger m on the fp8 x fp8 MFMA.  Above m = 8 on weights with many rows
// (the W8A16 MFMA route's size rule), 128-row tiles with x staged in LDS:
// lm_head [151936x2048] at m = 16 / 32 5.3 / 4.8 TB/s against 4.5 / 2.9 with
// 16-row tiles; at m = 4 the 16-row tiles are ahead (6.1 against 5.8).
hipError_t launch_gemv_w8a8(const GemvJob& job, const float* x_scale, int m, bool mx,
                            hipStream_t stream) {
  if (m <= 2) return mx ? dispatch_valu_x8<true>(job, x_scale, m, stream) : dispatch_valu_x8<false>(job, x_scale, m, stream);
  if (m > 8 && single_call_streams_mfma(job.n, m)) {
    if (m <= 16) return mx ? run_w8a8_tiles<1, true>(job, x_scale, m, stream) : run_w8a8_tiles<1, false>(job, x_scale, m, stream);
    return mx ? run_w8a8_tiles<2, true>(job, x_scale, m, stream) : run_w8a8_tiles<2, false>(job, x_scale, m, stream);
  }
  const dim3 grid((unsigned)((job.n + 15) / 16));
  if (job.n <= kDirect8MaxRows) {   // as the bf16 single call: 8 waves per tile on few rows
    const dim3 block(8 * kWave);
    if (m <= 16) {
      if (mx) hipLaunchKernelGGL((k_gemv_w8a8_direct<1, 2, true, 8, kFmtMx>), grid, block, 0, stream, job, x_scale, m);
      else launch_w8a8_direct_fmt<1, 8>(grid, block, job, x_scale, m, stream);
    } else {
      if (mx) hipLaunchKernelGGL((k_gemv_w8a8_direct<2, 2, true, 8, kFmtMx>), grid, block, 0, stream, job, x_scale, m);
      else launch_w8a8_direct_fmt<2, 8>(grid, block, job, x_scale, m, stream);
    }
    return hipGetLastError();
  }
  const dim3 block(kThreads);
  if (m <= 16) {
    if (mx) hipLaunchKernelGGL((k_gemv_w8a8_direct<1, 2, true, kWaves, kFmtMx>), grid, block, 0, stream, job, x_scale, m);
    else launch_w8a8_direct_fmt<1, kWaves>(grid, block, job, x_scale, m, stream);
  } else {
    if (mx) hipLaunchKernelGGL((k_gemv_w8a8_direct<2, 2, true, kWaves, kFmtMx>), grid, block, 0, stream, job, x_scale, m);
    else launch_w8a8_direct_fmt<2, kWaves>(grid, block, job, x_scale, m, stream);
  }
  return hipGetLastError();
}

hipError_t launch_gemv_mfma_stream(const GemvJob* table, int njobs, int64_t blocks, int64_t tiles,
                                   int tiles_per_block, int m, int seg_cols, int format, bool mx_packed8,
                                   hipStream_t stream) {
  const StreamJobs l{table, njobs, GemvJob{}};
  return dispatch_mfma_stream<false>(l, blocks, tiles, tiles_per_block, m, seg_cols, format,
                                     format == kFmtMx && mx_packed8, stream);
}

}  // namespace fp8w
