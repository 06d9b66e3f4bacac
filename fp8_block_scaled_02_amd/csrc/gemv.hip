// gemv.hip -- W8A16 decode GEMV / skinny GEMM for gfx950.
//
// y[m][n] = bf16( sum_k x[m][k] * dec(code[n][k]) * scale(n, k) ), fp32
// accumulation, for 1 <= M <= 32.  The fp8 weight stream dominates the
// traffic, so every kernel reads each code byte once with 16-byte loads and
// converts e4m3 -> bf16 in registers (exact: 4 significant bits); x (at most
// 32 rows) is re-read from LDS or from L2.  Two kernel families, split on M
// as the fused W8A16 GEMM of "feat:
// add FP8 blockwise weight quantization and FP8(E4M3) KV cache support"
// (Summary; Notes for Reviewers) splits its SIMT and tensor-core routes:
//
//  * VALU (M <= 8): v_dot2c_f32_bf16 products; the 64 lanes of a wave walk
//    one row along K, and the wave's partial sums are folded four at a time
//    with lane-swap and DPP row operations (no LDS round trips).
//  * MFMA (M <= 32): v_mfma_f32_16x16x32_bf16 on 16-row tiles of W against
//    x^T padded to 16 or 32 columns.
//
// Each call is a few microseconds of HBM traffic, so latency decides the
// time: every kernel issues its weight loads first (non-temporal: each code
// byte is read once).  The VALU kernels and the grouped MFMA kernel then
// stage a K segment of x (and the block-scale row) in LDS while those loads
// are in flight; segments are sized so that the common K (up to a few
// thousand) is one segment.  The single-call MFMA kernel keeps no x in LDS:
// each wave walks its 128-column blocks with a register pipeline two blocks
// deep, loading codes, x fragments and the scale of block q+2 before the
// MFMAs of block q, so no barrier ever waits for a staging pass.
//
// A launch covers either one GEMV (the job travels as a kernel argument) or
// a group of independent GEMVs (a job table in device memory; workgroup b
// finds its job by binary search on the jobs' first workgroup index), which
// removes the fixed per-launch cost from a sequence of small GEMVs.
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
// i.e. weights within 0.4 % of the bf16 maximum, can break that.
#include <hip/hip_runtime.h>
#include <stddef.h>

#include "device.hpp"
#include "internal.hpp"

namespace fp8w {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

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

// Two e4m3 codes -> fp32 (exact), times the MX scale (exact in fp32),
// rounded to bf16.
template <bool HI>
__device__ __forceinline__ bf16x2 cvt_scaled(uint32_t d, float s) {
  const f32x2 v = __builtin_amdgcn_cvt_pk_f32_fp8(d, HI);
  return bf16x2{(__bf16)(v.x * s), (__bf16)(v.y * s)};
}

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t d) { return __builtin_bit_cast(bf16x2, d); }

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
  tile = b - job.item0;
}

// Copy x[0:rows, seg0 : seg0+len] (len a multiple of 16) into LDS rows of
// stride `ld` elements, covering columns [0, len_pad); columns >= len and
// rows rows..rows_pad-1 are zero-filled, so padded products are exact zeros.
__device__ __forceinline__ void stage_x(const uint16_t* __restrict__ x, int rows, int rows_pad,
                                        int k, int seg0, int len, int len_pad, uint16_t* xs,
                                        int ld) {
  const int units = len_pad / 8;   // 16-byte units per row
  for (int u = threadIdx.x; u < rows_pad * units; u += kThreads) {
    const int r = u / units, c = (u % units) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < rows && c < len) v = ld_global_u4(x, ((size_t)r * k + seg0 + c) * 2);
    *reinterpret_cast<uint4*>(xs + r * ld + c) = v;
  }
}

// ------------------------------------------------------------------ VALU --
//
// Workgroup = 4 waves x R rows.  Wave w owns rows row0 + r (r < R); lane l
// takes the 16-byte chunks l, l + 64, ..., of each K segment (C chunks per
// lane, so a segment is 1024*C columns).  Per segment: the codes (and MX
// scale bytes) of all R rows are requested, x and the block-scale row are
// staged in LDS while they arrive, then the segment is accumulated.
template <int M, int R, int C>
struct ValuShape {
  static constexpr int kRows = kWaves * R;
  static constexpr int kSeg = 1024 * C;
  static constexpr int kLdsX = M * kSeg * 2;
  static constexpr int kLdsBytes = kLdsX + (kSeg / kTile) * 4;
  static_assert(kTile % kRows == 0, "a workgroup must stay inside one 128-row block");
  static_assert(kLdsBytes <= 64 * 1024, "LDS budget");
};

template <int R, int C, bool MX>
__device__ __forceinline__ void valu_load(const GemvJob& j, int row0, int seg0, int nch, int groups,
                                          uint4 (&wv)[R][C], float (&ws)[R][C]) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint8_t* __restrict__ e8 = static_cast<const uint8_t*>(j.scales);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = row0 + r;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int ch = lane + kWave * c;
      wv[r][c] = make_uint4(0, 0, 0, 0);
      ws[r][c] = 0.0f;
      if (ch < nch && row < j.n) {
        wv[r][c] = ld_stream_u4(j.codes, (size_t)row * j.k + seg0 + ch * 16);
        if (MX) ws[r][c] = mx_scale(ld_global<uint8_t>(e8, (size_t)row * groups + (seg0 + ch * 16) / kGroup));
      }
    }
  }
}

template <int M, int R, int C, bool MX, bool GROUPED>
__global__ __launch_bounds__(kThreads) void k_gemv_valu(GemvJob arg, const GemvJob* __restrict__ jobs,
                                                        int njobs) {
  using S = ValuShape<M, R, C>;
  __shared__ __align__(16) unsigned char smem[S::kLdsBytes];
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  float* ss = reinterpret_cast<float*>(smem + S::kLdsX);

  GemvJob j;
  int tile;
  find_job<GROUPED>(arg, jobs, njobs, j, tile);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int row0 = tile * S::kRows + wave * R;
  const int tiles_k = (j.k + kTile - 1) / kTile;
  const int groups = (j.k + kGroup - 1) / kGroup;
  const float* __restrict__ srow =
      MX ? nullptr
         : static_cast<const float*>(j.scales) + (size_t)(tile * S::kRows / kTile) * tiles_k;

  float acc[R][M];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

  for (int seg0 = 0; seg0 < j.k; seg0 += S::kSeg) {
    const int len = min(S::kSeg, j.k - seg0);
    const int nch = len / 16;
    uint4 cw[R][C];
    float cs[R][C];
    valu_load<R, C, MX>(j, row0, seg0, nch, groups, cw, cs);
    if (seg0 > 0) __syncthreads();   // the previous segment's LDS reads are done
    stage_x(j.x, M, M, j.k, seg0, len, len, xs, S::kSeg);
    if (!MX) {
      const int nkb = (len + kTile - 1) / kTile;
      if ((int)threadIdx.x < nkb) ss[threadIdx.x] = ld_global<float>(srow, (size_t)(seg0 / kTile + threadIdx.x) * 4);
    }
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
          const float s = MX ? cs[r][c] : bs;
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
  if ((lane & 15) == 0) {
#pragma unroll
    for (int q = 0; q < WaveSums<R * M>::kGroups; ++q) {
      const int f = 4 * q + (lane >> 4);   // value index r * M + m held by this row
      const int r = f / M, m = f % M;
      if (f < R * M && row0 + r < j.n)
        st_global<uint16_t>(j.y, ((size_t)m * j.n + row0 + r) * 2, (uint16_t)f32_to_bf16_rne(sums.g[q]));
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
template <int R, int C, bool MX>
struct TileRegs {
  uint4 w[R][C];
  float s[R][C];   // MX: per row and chunk; block: row 0 holds the chunk scales
};

__device__ __forceinline__ void load_job_row(const GemvJob* __restrict__ jobs, int jn, GemvJob& job) {
  const size_t row = (size_t)jn * sizeof(GemvJob);
  job.x = (const uint16_t*)ld_global<uint64_t>(jobs, row + offsetof(GemvJob, x));
  job.codes = (const uint8_t*)ld_global<uint64_t>(jobs, row + offsetof(GemvJob, codes));
  job.scales = (const void*)ld_global<uint64_t>(jobs, row + offsetof(GemvJob, scales));
  job.y = (uint16_t*)ld_global<uint64_t>(jobs, row + offsetof(GemvJob, y));
  job.n = ld_global<int32_t>(jobs, row + offsetof(GemvJob, n));
  job.k = ld_global<int32_t>(jobs, row + offsetof(GemvJob, k));
  job.item0 = ld_global<int32_t>(jobs, row + offsetof(GemvJob, item0));
}

__device__ __forceinline__ int next_item0(const GemvJob* __restrict__ jobs, int jn, int njobs) {
  return jn + 1 < njobs
             ? ld_global<int32_t>(jobs, (size_t)(jn + 1) * sizeof(GemvJob) + offsetof(GemvJob, item0))
             : 0x7FFFFFFF;
}

template <int R, int C, bool MX>
__device__ __forceinline__ void stream_issue(const GemvJob& j, int tile, TileRegs<R, C, MX>& t) {
  constexpr int kRows = kWaves * R;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int row0 = tile * kRows + wave * R;
  const int nch = j.k / 16;
  const int tiles_k = (j.k + kTile - 1) / kTile;
  const int groups = (j.k + kGroup - 1) / kGroup;
  const float* __restrict__ srow =
      MX ? nullptr : static_cast<const float*>(j.scales) + (size_t)(tile * kRows / kTile) * tiles_k;
  const uint8_t* __restrict__ e8 = static_cast<const uint8_t*>(j.scales);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = row0 + r;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int ch = lane + kWave * c;
      t.w[r][c] = make_uint4(0, 0, 0, 0);
      t.s[r][c] = 0.0f;
      if (ch < nch && row < j.n) {
        t.w[r][c] = ld_stream_u4(j.codes, (size_t)row * j.k + ch * 16);
        if (MX) t.s[r][c] = mx_scale(ld_global<uint8_t>(e8, (size_t)row * groups + ch / 2));
      }
    }
  }
  if (!MX) {
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int ch = lane + kWave * c;
      t.s[0][c] = ch < nch ? ld_global<float>(srow, (size_t)(ch >> 3) * 4) : 0.0f;
    }
  }
}

template <int R, int C, bool MX>
__global__ __launch_bounds__(kThreads) void k_gemv_valu_stream(const GemvJob* __restrict__ jobs,
                                                               int njobs, int total_tiles,
                                                               int tiles_per_block) {
  constexpr int kRows = kWaves * R, kSeg = 1024 * C;
  static_assert(kTile % kRows == 0, "a tile must stay inside one 128-row block");
  __shared__ __align__(16) uint16_t xs[kSeg];
  const int t_begin = blockIdx.x * tiles_per_block;
  const int t_end = min(total_tiles, t_begin + tiles_per_block);
  if (t_begin >= t_end) return;   // whole workgroup: no barrier is skipped by part of it
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;

  int jn = 0;
  {
    int lo = 0, hi = njobs - 1;   // last job whose first tile is <= t_begin
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (ld_global<int32_t>(jobs, (size_t)mid * sizeof(GemvJob) + offsetof(GemvJob, item0)) <= t_begin)
        lo = mid;
      else
        hi = mid - 1;
    }
    jn = lo;
  }
  GemvJob j;
  load_job_row(jobs, jn, j);
  int boundary = next_item0(jobs, jn, njobs);

  TileRegs<R, C, MX> cur, nxt;
  stream_issue<R, C, MX>(j, t_begin - j.item0, cur);
  for (int u = threadIdx.x; u < j.k / 8; u += kThreads)
    *reinterpret_cast<uint4*>(xs + u * 8) = ld_global_u4(j.x, (size_t)u * 16);
  __syncthreads();

  for (int t = t_begin; t < t_end; ++t) {
    const bool more = t + 1 < t_end;
    GemvJob jnext = j;
    int jn_next = jn, boundary_next = boundary;
    if (more) {
      if (t + 1 >= boundary) {   // the run crosses into the next job
        jn_next = jn + 1;
        load_job_row(jobs, jn_next, jnext);
        boundary_next = next_item0(jobs, jn_next, njobs);
      }
      stream_issue<R, C, MX>(jnext, t + 1 - jnext.item0, nxt);
    }

    const int row0 = (t - j.item0) * kRows + wave * R;
    const int nch = j.k / 16;
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
          const float sc = MX ? cur.s[r][c] : cur.s[0][c];
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
          st_global<uint16_t>(j.y, (size_t)(row0 + r) * 2, (uint16_t)f32_to_bf16_rne(sums.g[q]));
      }
    }
    if (!more) break;
    if (jn_next != jn) {   // restage x for the next job
      __syncthreads();
      for (int u = threadIdx.x; u < jnext.k / 8; u += kThreads)
        *reinterpret_cast<uint4*>(xs + u * 8) = ld_global_u4(jnext.x, (size_t)u * 16);
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
// Workgroup = 4 waves on 4/KW tiles of 16 rows; KW waves split K by 128-
// column blocks.  Lane l holds row i = l%16 of the tile and K-quarter
// g = l/16: per 64-column chunk it loads codes [16g, 16g+16), whose first 8
// feed one MFMA and last 8 a second one; the B operand (x^T) uses the same
// K positions, so the two MFMAs sum exactly the chunk.  The D layout of the
// 16x16 tile is D[4*(l/16) + j][l%16], j = 0..3.  A K segment holds CKB
// column blocks per wave (KW*CKB*128 columns).
template <int MT, int KW, int CKB>
struct MfmaShape {
  static constexpr int kTiles = kWaves / KW;
  static constexpr int kRows = 16 * kTiles;
  static constexpr int kMPad = 16 * MT;
  static constexpr int kSeg = KW * CKB * kTile;
  static constexpr int kLd = kSeg + 8;   // +16 B per row spreads B-operand reads over the banks
  static constexpr int kLdsX = kMPad * kLd * 2;
  static constexpr int kLdsRed = KW > 1 ? kWaves * MT * 4 * kWave * 4 : 0;
  static constexpr int kLdsBytes = kLdsX > kLdsRed ? kLdsX : kLdsRed;
  static_assert(kTile % kRows == 0 || kRows % kTile == 0, "tiles align with 128-row blocks");
  static_assert(kLdsBytes <= 64 * 1024, "LDS budget");
};

// Codes (and MX scale factors) of the wave's column blocks kb = kw + KW*q of
// the K segment starting at seg0.
template <int KW, int CKB, bool MX>
__device__ __forceinline__ void mfma_load(const GemvJob& j, int row, bool row_ok, int seg0, int kw,
                                          int groups, uint4 (&wv)[CKB][2], float (&ws)[CKB][2]) {
  constexpr int kSeg = KW * CKB * kTile;
  const int g = (threadIdx.x & (kWave - 1)) >> 4;
  const int len = min(kSeg, j.k - seg0);
  const uint8_t* __restrict__ e8 = static_cast<const uint8_t*>(j.scales);
#pragma unroll
  for (int q = 0; q < CKB; ++q) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int koff = (kw + KW * q) * kTile + h * 64 + 16 * g;
      wv[q][h] = make_uint4(0, 0, 0, 0);
      ws[q][h] = 0.0f;
      if (row_ok && koff < len) {
        wv[q][h] = ld_stream_u4(j.codes, (size_t)row * j.k + seg0 + koff);
        if (MX) ws[q][h] = mx_scale(ld_global<uint8_t>(e8, (size_t)row * groups + (seg0 + koff) / kGroup));
      }
    }
  }
}

template <int MT, int KW, int CKB, bool MX, bool GROUPED>
__global__ __launch_bounds__(kThreads) void k_gemv_mfma(GemvJob arg, const GemvJob* __restrict__ jobs,
                                                        int njobs, int m_rows) {
  using S = MfmaShape<MT, KW, CKB>;
  __shared__ __align__(16) unsigned char smem[S::kLdsBytes];
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);

  GemvJob j;
  int tile_group;
  find_job<GROUPED>(arg, jobs, njobs, j, tile_group);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int kw = wave % KW, tile = wave / KW;
  const int i = lane & 15, g = lane >> 4;
  const int row0 = (tile_group * S::kTiles + tile) * 16;
  const int row = row0 + i;
  const bool row_ok = row < j.n;
  const bool tile_live = row0 < j.n;   // a tile past the last row only joins the barriers
  const int tiles_k = (j.k + kTile - 1) / kTile;
  const int groups = (j.k + kGroup - 1) / kGroup;
  const float* __restrict__ srow =
      MX ? nullptr
         : static_cast<const float*>(j.scales) + (size_t)(min(row0, j.n - 1) / kTile) * tiles_k;

  f32x4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  for (int seg0 = 0; seg0 < j.k; seg0 += S::kSeg) {
    const int len = min(S::kSeg, j.k - seg0);
    const int nkb = (len + kTile - 1) / kTile;
    uint4 cw[CKB][2];
    float cs[CKB][2];
    mfma_load<KW, CKB, MX>(j, row, row_ok, seg0, kw, groups, cw, cs);
    if (seg0 > 0) __syncthreads();
    stage_x(j.x, m_rows, S::kMPad, j.k, seg0, len, nkb * kTile, xs, S::kLd);
    __syncthreads();

#pragma unroll
    for (int q = 0; q < CKB; ++q) {
      const int kb = kw + KW * q;
      if (!tile_live || kb >= nkb) break;
      f32x4 part[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) part[t] = MX ? acc[t] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint4 d = cw[q][h];
        const float s = cs[q][h];
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
        const bf16x8 A0 = {a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
        const bf16x8 A1 = {b0[0], b0[1], b1[0], b1[1], b2[0], b2[1], b3[0], b3[1]};
        const int kx = kb * kTile + h * 64 + 16 * g;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const uint16_t* xr = xs + (16 * t + i) * S::kLd + kx;
          const bf16x8 B0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(xr));
          const bf16x8 B1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(xr + 8));
          part[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, B0, part[t], 0, 0, 0);
          part[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, B1, part[t], 0, 0, 0);
        }
      }
      if (MX) {
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[t] = part[t];
      } else {
        const float bs = ld_global<float>(srow, (size_t)((seg0 + kb * kTile) / kTile) * 4);
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) acc[t][jj] = __builtin_fmaf(bs, part[t][jj], acc[t][jj]);
      }
    }
  }

  if (KW > 1) {
    __syncthreads();   // the x staging area is reused for the partial sums
    float* red = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) red[((wave * MT + t) * 4 + jj) * kWave + lane] = acc[t][jj];
    __syncthreads();
    if (kw == 0) {
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          float s = acc[t][jj];
          for (int w2 = 1; w2 < KW; ++w2) s += red[(((wave + w2) * MT + t) * 4 + jj) * kWave + lane];
          acc[t][jj] = s;
        }
    }
  }
  if (kw == 0) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int mcol = 16 * t + i;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = row0 + 4 * g + jj;
        if (r < j.n && mcol < m_rows)
          st_global<uint16_t>(j.y, ((size_t)mcol * j.n + r) * 2, (uint16_t)f32_to_bf16_rne(acc[t][jj]));
      }
    }
  }
}

// ------------------------------------------------------ MFMA, direct x --
//
// Single calls.  Same tile, lane and D layouts as above; the 4 waves of a
// workgroup are 4/KW tiles of 16 rows, KW waves splitting K by 128-column
// blocks (wave kw takes blocks kw, kw + KW, ...).  Each block's registers --
// two 16-byte code chunks per lane, the x^T fragments of the same K
// positions read from global memory (x is small and stays in L2), and the
// block scale or the chunks' MX scales -- are requested D blocks ahead.
template <int MT, bool MX>
struct DirectRegs {
  uint4 w[2];
  uint4 xb[MT][2][2];   // [m tile][chunk][first / last 8 K positions]
  float s[2];           // block: s[0] is the block scale; MX: one per chunk
};

template <int MT, int KW, int D, bool MX>
__global__ __launch_bounds__(kThreads) void k_gemv_mfma_direct(GemvJob j, int m_rows) {
  constexpr int kTiles = kWaves / KW;
  __shared__ float red[KW > 1 ? kWaves * MT * 4 * kWave : 1];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int kw = wave % KW, tile = wave / KW;
  const int i = lane & 15, g = lane >> 4;
  const int row0 = (blockIdx.x * kTiles + tile) * 16;
  const int row = row0 + i;
  const bool row_ok = row < j.n;
  const int nkb = (j.k + kTile - 1) / kTile;
  const int groups = (j.k + kGroup - 1) / kGroup;
  const int nq = row0 < j.n ? (nkb - kw + KW - 1) / KW : 0;   // this wave's column blocks
  const float* __restrict__ srow =
      MX ? nullptr
         : static_cast<const float*>(j.scales) + (size_t)(min(row0, j.n - 1) / kTile) * nkb;
  const uint8_t* __restrict__ e8 = static_cast<const uint8_t*>(j.scales);

  auto issue = [&](int q, DirectRegs<MT, MX>& r) {
    const int kb = kw + KW * q;
    const bool live = q < nq;
    r.s[0] = r.s[1] = 0.0f;
    if (!MX && live) r.s[0] = ld_global<float>(srow, (size_t)kb * 4);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kx = kb * kTile + h * 64 + 16 * g;
      const bool in = live && kx < j.k;
      r.w[h] = make_uint4(0, 0, 0, 0);
      if (in && row_ok) {
        r.w[h] = ld_stream_u4(j.codes, (size_t)row * j.k + kx);
        if (MX) r.s[h] = mx_scale(ld_global<uint8_t>(e8, (size_t)row * groups + kx / kGroup));
      }
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int m = 16 * t + i;
        r.xb[t][h][0] = r.xb[t][h][1] = make_uint4(0, 0, 0, 0);
        if (in && m < m_rows) {
          r.xb[t][h][0] = ld_global_u4(j.x, ((size_t)m * j.k + kx) * 2);
          r.xb[t][h][1] = ld_global_u4(j.x, ((size_t)m * j.k + kx + 8) * 2);
        }
      }
    }
  };

  f32x4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  DirectRegs<MT, MX> slot[D];
#pragma unroll
  for (int s = 0; s < D; ++s) issue(s, slot[s]);
  for (int q0 = 0; q0 < nq; q0 += D) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      if (q0 + s < nq) {
        f32x4 part[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) part[t] = MX ? acc[t] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint4 d = slot[s].w[h];
          bf16x2 a0, a1, a2, a3, b0, b1, b2, b3;
          if (MX) {
            const float sc = slot[s].s[h];
            a0 = cvt_scaled<false>(d.x, sc), a1 = cvt_scaled<true>(d.x, sc);
            a2 = cvt_scaled<false>(d.y, sc), a3 = cvt_scaled<true>(d.y, sc);
            b0 = cvt_scaled<false>(d.z, sc), b1 = cvt_scaled<true>(d.z, sc);
            b2 = cvt_scaled<false>(d.w, sc), b3 = cvt_scaled<true>(d.w, sc);
          } else {
            a0 = cvt_lo(d.x), a1 = cvt_hi(d.x), a2 = cvt_lo(d.y), a3 = cvt_hi(d.y);
            b0 = cvt_lo(d.z), b1 = cvt_hi(d.z), b2 = cvt_lo(d.w), b3 = cvt_hi(d.w);
          }
          const bf16x8 A0 = {a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
          const bf16x8 A1 = {b0[0], b0[1], b1[0], b1[1], b2[0], b2[1], b3[0], b3[1]};
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            part[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                A0, __builtin_bit_cast(bf16x8, slot[s].xb[t][h][0]), part[t], 0, 0, 0);
            part[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                A1, __builtin_bit_cast(bf16x8, slot[s].xb[t][h][1]), part[t], 0, 0, 0);
          }
        }
        if (MX) {
#pragma unroll
          for (int t = 0; t < MT; ++t) acc[t] = part[t];
        } else {
          const float bs = slot[s].s[0];
#pragma unroll
          for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) acc[t][jj] = __builtin_fmaf(bs, part[t][jj], acc[t][jj]);
        }
      }
      issue(q0 + s + D, slot[s]);
    }
  }

  if (KW > 1) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) red[((wave * MT + t) * 4 + jj) * kWave + lane] = acc[t][jj];
    __syncthreads();
    if (kw == 0) {
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          float v = acc[t][jj];
          for (int w2 = 1; w2 < KW; ++w2) v += red[(((wave + w2) * MT + t) * 4 + jj) * kWave + lane];
          acc[t][jj] = v;
        }
    }
  }
  if (kw == 0) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int mcol = 16 * t + i;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = row0 + 4 * g + jj;
        if (r < j.n && mcol < m_rows)
          st_global<uint16_t>(j.y, ((size_t)mcol * j.n + r) * 2, (uint16_t)f32_to_bf16_rne(acc[t][jj]));
      }
    }
  }
}

// ------------------------------------------------------------ dispatch --
//
// One compiled variant per (route, M, single/grouped), any N and K:
//   VALU single call: R = 1 row per wave (4 rows per workgroup: the most
//     workgroups for small N); grouped: more rows per wave (fewer, larger
//     workgroups once many GEMVs share the launch).
//   MFMA single call: direct-x kernel, the 4 waves of a 16-row tile split
//     K; grouped: LDS-staged kernel, each wave owns a 16-row tile.

template <int M, int R, int C, bool MX, bool G>
hipError_t run_valu(const GemvJob& job, const GemvJob* table, int njobs, int64_t blocks,
                    hipStream_t stream) {
  hipLaunchKernelGGL((k_gemv_valu<M, R, C, MX, G>), dim3((unsigned)blocks), dim3(kThreads), 0,
                     stream, job, table, njobs);
  return hipGetLastError();
}

template <int MT, int KW, int CKB, bool MX, bool G>
hipError_t run_mfma(const GemvJob& job, const GemvJob* table, int njobs, int64_t blocks, int m,
                    hipStream_t stream) {
  hipLaunchKernelGGL((k_gemv_mfma<MT, KW, CKB, MX, G>), dim3((unsigned)blocks), dim3(kThreads), 0,
                     stream, job, table, njobs, m);
  return hipGetLastError();
}

// (rows per wave R, 16-byte chunks per lane per segment C) of the VALU route
template <bool MX, bool G>
hipError_t dispatch_valu(int m, const GemvJob& job, const GemvJob* table, int njobs, int64_t blocks,
                         hipStream_t s) {
  if (G) {
    switch (m) {
      case 1: return run_valu<1, 4, 3, MX, G>(job, table, njobs, blocks, s);
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

template <bool MX, bool G>
hipError_t dispatch_mfma(int m, const GemvJob& job, const GemvJob* table, int njobs, int64_t blocks,
                         hipStream_t s) {
  if (G) {
    if (m <= 16) return run_mfma<1, 1, 4, MX, G>(job, table, njobs, blocks, m, s);
    return run_mfma<2, 1, 2, MX, G>(job, table, njobs, blocks, m, s);
  }
  if (m <= 16)
    hipLaunchKernelGGL((k_gemv_mfma_direct<1, 4, 2, MX>), dim3((unsigned)blocks), dim3(kThreads), 0, s, job, m);
  else
    hipLaunchKernelGGL((k_gemv_mfma_direct<2, 4, 2, MX>), dim3((unsigned)blocks), dim3(kThreads), 0, s, job, m);
  return hipGetLastError();
}

}  // namespace

int gemv_rows_per_block(int route, int m, bool grouped) {
  if (route == 1) {
    if (grouped) return kWaves * 4;
    return kWaves * (m == 1 ? 1 : 2);
  }
  return grouped ? 64 : 16;
}

hipError_t launch_gemv(const GemvJob& job, int m, bool mx, int route, hipStream_t stream) {
  const int rows = gemv_rows_per_block(route, m, false);
  const int64_t blocks = (job.n + rows - 1) / rows;
  if (route == 1)
    return mx ? dispatch_valu<true, false>(m, job, nullptr, 1, blocks, stream)
              : dispatch_valu<false, false>(m, job, nullptr, 1, blocks, stream);
  return mx ? dispatch_mfma<true, false>(m, job, nullptr, 1, blocks, stream)
            : dispatch_mfma<false, false>(m, job, nullptr, 1, blocks, stream);
}

// Streaming kernel of grouped M = 1 VALU plans: (R, C) and its K limit.
constexpr int kStreamR = 4, kStreamC = 3;

int gemv_stream_max_k() { return 1024 * kStreamC; }
int gemv_stream_rows() { return kWaves * kStreamR; }

hipError_t gemv_stream_slots(bool mx, int* slots) {
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = mx ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                 &per_cu, k_gemv_valu_stream<kStreamR, kStreamC, true>, kThreads, 0)
           : hipOccupancyMaxActiveBlocksPerMultiprocessor(
                 &per_cu, k_gemv_valu_stream<kStreamR, kStreamC, false>, kThreads, 0);
  *slots = cus * (per_cu > 0 ? per_cu : 1);
  return e;
}

hipError_t launch_gemv_stream(const GemvJob* table, int njobs, int64_t blocks, int64_t tiles,
                              int tiles_per_block, bool mx, hipStream_t stream) {
  if (mx)
    hipLaunchKernelGGL((k_gemv_valu_stream<kStreamR, kStreamC, true>), dim3((unsigned)blocks),
                       dim3(kThreads), 0, stream, table, njobs, (int)tiles, tiles_per_block);
  else
    hipLaunchKernelGGL((k_gemv_valu_stream<kStreamR, kStreamC, false>), dim3((unsigned)blocks),
                       dim3(kThreads), 0, stream, table, njobs, (int)tiles, tiles_per_block);
  return hipGetLastError();
}

hipError_t launch_gemv_grouped(const GemvJob* table, int njobs, int64_t blocks, int m, bool mx,
                               int route, hipStream_t stream) {
  const GemvJob none{};
  if (route == 1)
    return mx ? dispatch_valu<true, true>(m, none, table, njobs, blocks, stream)
              : dispatch_valu<false, true>(m, none, table, njobs, blocks, stream);
  return mx ? dispatch_mfma<true, true>(m, none, table, njobs, blocks, stream)
            : dispatch_mfma<false, true>(m, none, table, njobs, blocks, stream);
}

}  // namespace fp8w
