/*
 * fp8w_oracle.c -- plain, slow, obviously-correct CPU oracle for the FP8
 * weight path (bf16 -> e4m3fn quantization with 128x128 fp32 block scales or
 * 32-element e8m0 scales, and the W8A16 GEMV computed in fp64).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this file; only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load it.  It shares no code, header, table or
 * constant generator with the HIP path.
 *
 * Sources of each definition (the pages are cited by title and section):
 *  - e4m3 "fn" bit layout and decode: OCP 8-bit Floating Point Specification
 *    (OFP8), E4M3 encoding (bias 7, no infinities, NaN = S.1111.111, largest
 *    finite magnitude 448).  The pages use the same 448 ceiling ("Load-time
 *    MXFP8 requantization ..." issue, Proposed solution: exponent from
 *    amax/448) and call the format FP8 E4M3 ("feat: add FP8 blockwise weight
 *    quantization ...", Summary).
 *  - encode: round to nearest, ties to the even code, saturating at +-448,
 *    sign kept (so negative values that round to zero give 0x80).
 *  - block quantize: one fp32 scale per 128x128 tile, scale = amax/448,
 *    codes = enc(w/scale).  "quantize_fp8_bs.rs" (Atlas weight_map): one byte
 *    per weight, one f32 per [128,128] tile, grid of ceil(n/128) x
 *    ceil(k/128) tiles, n > 0 and k > 0 required; "feat(quant): opt-in
 *    fp8-block QAT for the lm_head", Changes (per-block quantizer that is the
 *    inverse of the block dequantizer).
 *  - MX quantize: e4m3 codes with one e8m0 scale per 32 elements along K,
 *    exponent = ceil(log2(amax/448)), computed row-chunked so that the fp32
 *    transient stays near 32 MB ("Load-time MXFP8 requantization ..." issue,
 *    Proposed solution).
 *  - dequantize to bf16: fp32 product of the decoded value and the scale,
 *    rounded to bf16 (the dense-GEMM fallback of "feat: add FP8 blockwise
 *    weight quantization ...", Summary, consumes bf16 weights).
 *  - GEMV reference: y = x . deq(W)^T with x bf16 [M,K] and W [N,K]; each
 *    product is exact in fp64 and the sum is taken in fp64 ("feat: add FP8
 *    blockwise weight quantization ...", Summary: fused W8A16 GEMM for
 *    M <= 32; "feat(qwen4_exp): load-time per-tensor FP8 ...", Testing: the
 *    op checked against a linear on the dequantized weight).
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  - the scale and the quotient are fp32 IEEE divisions (correctly rounded),
 *    so codes are enc(fl32(w / fl32(amax / 448)));
 *  - an all-zero tile gets scale 1.0; an all-zero MX group gets exponent -127;
 *  - the MX exponent is clamped to [-127, 127] and stored with bias 127;
 *  - tiles and groups at the right/bottom edge are partial: amax is taken
 *    over the valid elements only (equal to zero padding since |0| <= amax);
 *  - non-finite inputs are out of contract and rejected.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -fPIC -shared.
 * No fast-math: every fp32 operation must be the IEEE one.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_NONFINITE 2
#define ORACLE_ERR_NOMEM 3

#define TILE 128        /* block-scale tile edge, both axes */
#define MX_GROUP 32     /* elements per e8m0 scale, along K */
#define E4M3_MAX 448.0  /* largest finite e4m3fn magnitude (code 0x7E) */

/* ---------------------------------------------------------------- bf16 -- */

/* A bf16 value is the top half of an fp32 bit pattern: widening is exact. */
static float bf16_to_float(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

float oracle_bf16_to_float(uint16_t b) { return bf16_to_float(b); }

/* ---------------------------------------------------------------- e4m3 -- */

/* OFP8 E4M3: sign (1 bit), exponent E (4 bits, bias 7), mantissa m (3 bits).
 *   E == 0           : subnormal, value = m * 2^-9
 *   E == 15, m == 7  : NaN (the format has no infinities)
 *   otherwise        : value = (1 + m/8) * 2^(E-7)                        */
double oracle_e4m3_decode(uint8_t code) {
  int sign = code >> 7;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double mag;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    mag = ldexp((double)m, -9);
  else
    mag = ldexp(1.0 + m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* Magnitudes of the 127 finite non-negative codes 0x00..0x7E, ascending. */
static double g_mag[127];

__attribute__((constructor)) static void build_magnitude_table(void) {
  for (int c = 0; c < 127; ++c) g_mag[c] = oracle_e4m3_decode((uint8_t)c);
}

/* Round a finite fp32 to the nearest e4m3fn code, ties to the even code,
 * saturating at +-448.  Search the table of magnitudes for the largest code
 * not above |q|, then compare |q| with the (exactly representable) midpoint
 * to its upper neighbour.                                                  */
uint8_t oracle_e4m3_encode(float q) {
  uint8_t sign = signbit(q) ? 0x80 : 0x00;
  double a = fabs((double)q);
  int c;
  if (a >= E4M3_MAX) {
    c = 126; /* saturate: the nearest finite magnitude is 448 */
  } else {
    int lo = 0, hi = 126; /* invariant: g_mag[lo] <= a < g_mag[hi + 1] */
    while (lo < hi) {
      int mid = (lo + hi + 1) / 2;
      if (g_mag[mid] <= a)
        lo = mid;
      else
        hi = mid - 1;
    }
    c = lo; /* a < 448 so c <= 125 and c + 1 is a finite code */
    if (g_mag[c] != a) {
      double midpoint = 0.5 * (g_mag[c] + g_mag[c + 1]); /* exact in fp64 */
      if (a > midpoint || (a == midpoint && (c & 1))) c = c + 1;
    }
  }
  return (uint8_t)(sign | c);
}

void oracle_e4m3_encode_array(const float* q, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(q[i]);
}

void oracle_e4m3_decode_array(const uint8_t* c, int64_t n, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_decode(c[i]);
}

/* ------------------------------------------------------------- helpers -- */

static int all_finite(const uint16_t* w, int64_t count) {
  int ok = 1;
#pragma omp parallel for reduction(& : ok) schedule(static)
  for (int64_t i = 0; i < count; ++i)
    if ((w[i] & 0x7F80) == 0x7F80) ok = 0; /* exponent all ones: inf/NaN */
  return ok;
}

void oracle_set_threads(int threads) {
#ifdef _OPENMP
  if (threads > 0) omp_set_num_threads(threads);
#else
  (void)threads;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

int64_t oracle_block_scale_count(int64_t n, int64_t k) {
  return ((n + TILE - 1) / TILE) * ((k + TILE - 1) / TILE);
}

int64_t oracle_mx_scale_count(int64_t n, int64_t k) {
  return n * ((k + MX_GROUP - 1) / MX_GROUP);
}

/* ---------------------------------------------------- block quantize -- */

/* Per 128x128 tile (partial at the edges):
 *   amax  = max |w| over the tile's valid elements (exact in fp32)
 *   scale = amax / 448   (fp32 division), or 1.0 when amax == 0
 *   code  = enc(w / scale)   (fp32 division), for every valid element
 * codes is [n, k] row-major; scales is [ceil(n/128), ceil(k/128)] row-major. */
int oracle_quantize_block(const uint16_t* w, int64_t n, int64_t k,
                          uint8_t* codes, float* scales) {
  if (!w || !codes || !scales || n < 1 || k < 1) return ORACLE_ERR_ARG;
  if (!all_finite(w, n * k)) return ORACLE_ERR_NONFINITE;
  const int64_t tiles_n = (n + TILE - 1) / TILE;
  const int64_t tiles_k = (k + TILE - 1) / TILE;
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
  for (int64_t ti = 0; ti < tiles_n; ++ti) {
    for (int64_t tj = 0; tj < tiles_k; ++tj) {
      const int64_t r0 = ti * TILE, r1 = (r0 + TILE < n) ? r0 + TILE : n;
      const int64_t c0 = tj * TILE, c1 = (c0 + TILE < k) ? c0 + TILE : k;
      float amax = 0.0f;
      for (int64_t r = r0; r < r1; ++r)
        for (int64_t c = c0; c < c1; ++c) {
          float a = fabsf(bf16_to_float(w[r * k + c]));
          if (a > amax) amax = a;
        }
      const float scale = (amax > 0.0f) ? amax / 448.0f : 1.0f;
      scales[ti * tiles_k + tj] = scale;
      for (int64_t r = r0; r < r1; ++r)
        for (int64_t c = c0; c < c1; ++c) {
          float q = bf16_to_float(w[r * k + c]) / scale;
          codes[r * k + c] = oracle_e4m3_encode(q);
        }
    }
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------- MX quantize -- */

/* ceil(log2(amax / 448)) as an exact integer: the smallest e with
 * amax <= 448 * 2^e.  The fp64 log2 gives the starting guess; the two loops
 * make the result exact whatever the rounding of log2 was.  Clamped to
 * [-127, 127]; an all-zero group gets -127.                              */
int oracle_e8m0_exponent(float amax) {
  if (!(amax > 0.0f)) return -127;
  const double a = (double)amax;
  int e = (int)ceil(log2(a / E4M3_MAX));
  while (ldexp(E4M3_MAX, e) < a) ++e;
  while (ldexp(E4M3_MAX, e - 1) >= a) --e;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return e;
}

void oracle_e8m0_exponent_array(const float* amax, int64_t n, int32_t* e) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) e[i] = oracle_e8m0_exponent(amax[i]);
}

/* Default rows per chunk: as many rows as fit an fp32 transient of 32 MiB. */
int64_t oracle_mx_default_chunk_rows(int64_t k) {
  int64_t rows = ((int64_t)1 << 25) / (4 * k);
  return rows > 0 ? rows : 1;
}

/* Row-chunked: each chunk of rows is widened to an fp32 transient buffer,
 * then for every row and every 32-element group along K (the last group of a
 * row may be partial):
 *   amax = max |v|;  e = oracle_e8m0_exponent(amax);  E = e + 127
 *   code = enc(v * 2^-e)   (power-of-two scaling, exact unless it underflows)
 * codes is [n, k] row-major, e8m0 is [n, ceil(k/32)] row-major.
 * chunk_rows <= 0 selects the 32 MiB default.                             */
int oracle_quantize_mx(const uint16_t* w, int64_t n, int64_t k,
                       uint8_t* codes, uint8_t* e8m0, int64_t chunk_rows) {
  if (!w || !codes || !e8m0 || n < 1 || k < 1) return ORACLE_ERR_ARG;
  if (!all_finite(w, n * k)) return ORACLE_ERR_NONFINITE;
  if (chunk_rows <= 0) chunk_rows = oracle_mx_default_chunk_rows(k);
  if (chunk_rows > n) chunk_rows = n;
  const int64_t groups = (k + MX_GROUP - 1) / MX_GROUP;
  float* transient = (float*)malloc((size_t)(chunk_rows * k) * sizeof(float));
  if (!transient) return ORACLE_ERR_NOMEM;
  for (int64_t row0 = 0; row0 < n; row0 += chunk_rows) {
    const int64_t rows = (row0 + chunk_rows < n) ? chunk_rows : n - row0;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows * k; ++i)
      transient[i] = bf16_to_float(w[row0 * k + i]);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
      const float* v = transient + r * k;
      for (int64_t g = 0; g < groups; ++g) {
        const int64_t c0 = g * MX_GROUP;
        const int64_t c1 = (c0 + MX_GROUP < k) ? c0 + MX_GROUP : k;
        float amax = 0.0f;
        for (int64_t c = c0; c < c1; ++c)
          if (fabsf(v[c]) > amax) amax = fabsf(v[c]);
        const int e = oracle_e8m0_exponent(amax);
        e8m0[(row0 + r) * groups + g] = (uint8_t)(e + 127);
        for (int64_t c = c0; c < c1; ++c)
          codes[(row0 + r) * k + c] = oracle_e4m3_encode(ldexpf(v[c], -e));
      }
    }
  }
  free(transient);
  return ORACLE_OK;
}

/* ------------------------------------------------ other scale formats -- */

/* Scale formats, numbered as the library's fp8w_format. */
#define FMT_BLOCK 0      /* fp32 per 128x128 tile                 */
#define FMT_MX 1         /* e8m0 per row and 32 columns           */
#define FMT_BLOCK_BF16 2 /* bf16 per 128x128 tile                 */
#define FMT_ROW 3        /* fp32 per row                          */
#define FMT_TENSOR 4     /* one fp32 for the whole tensor         */

uint16_t oracle_round_bf16(double v);

/* Block quantization with a bf16 scale per 128x128 tile ("feat(quant):
 * opt-in fp8-block QAT for the lm_head", How it works: fp8 plus a bf16
 * 128-block scale).  The fp32 scale amax/448 is rounded to the nearest bf16
 * (ties to even; 1.0 for an all-zero tile) and the codes divide by that
 * stored scale, so that dequantizing with it inverts them; a scale rounded
 * down can put amax/scale just above 448, which saturates.  A scale that
 * would round to zero (amax below 448 * 2^-134) is the smallest positive
 * bf16, 2^-133, instead. */
int oracle_quantize_block_bf16(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes,
                               uint16_t* scales) {
  if (!w || !codes || !scales || n < 1 || k < 1) return ORACLE_ERR_ARG;
  if (!all_finite(w, n * k)) return ORACLE_ERR_NONFINITE;
  const int64_t tiles_n = (n + TILE - 1) / TILE;
  const int64_t tiles_k = (k + TILE - 1) / TILE;
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
  for (int64_t ti = 0; ti < tiles_n; ++ti) {
    for (int64_t tj = 0; tj < tiles_k; ++tj) {
      const int64_t r0 = ti * TILE, r1 = (r0 + TILE < n) ? r0 + TILE : n;
      const int64_t c0 = tj * TILE, c1 = (c0 + TILE < k) ? c0 + TILE : k;
      float amax = 0.0f;
      for (int64_t r = r0; r < r1; ++r)
        for (int64_t c = c0; c < c1; ++c) {
          const float a = fabsf(bf16_to_float(w[r * k + c]));
          if (a > amax) amax = a;
        }
      uint16_t sb = amax > 0.0f ? oracle_round_bf16((double)(amax / 448.0f)) : 0x3F80;
      if (sb == 0) sb = 1;   /* amax/448 below half the smallest bf16: keep the scale positive */
      const float scale = bf16_to_float(sb);
      scales[ti * tiles_k + tj] = sb;
      for (int64_t r = r0; r < r1; ++r)
        for (int64_t c = c0; c < c1; ++c)
          codes[r * k + c] = oracle_e4m3_encode(bf16_to_float(w[r * k + c]) / scale);
    }
  }
  return ORACLE_OK;
}

/* Per-row quantization ("quantize_fp8_bs.rs", Atlas weight_map: the per-ROW
 * BF16 -> FP8 quantizer of the DFlash head; "feat(qwen4_exp): load-time
 * per-tensor FP8 dense projections", Why: the per-row W8A16 route): the
 * block rule with a 1 x k tile -- scale[r] = amax(row r)/448 in fp32 (1.0
 * for an all-zero row), code = enc(w/scale[r]). */
int oracle_quantize_row(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes, float* scales) {
  if (!w || !codes || !scales || n < 1 || k < 1) return ORACLE_ERR_ARG;
  if (!all_finite(w, n * k)) return ORACLE_ERR_NONFINITE;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r) {
    float amax = 0.0f;
    for (int64_t c = 0; c < k; ++c) {
      const float a = fabsf(bf16_to_float(w[r * k + c]));
      if (a > amax) amax = a;
    }
    const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
    scales[r] = scale;
    for (int64_t c = 0; c < k; ++c) codes[r * k + c] = oracle_e4m3_encode(bf16_to_float(w[r * k + c]) / scale);
  }
  return ORACLE_OK;
}

/* The scale that multiplies dec(code[r][c]) in each format. */
static double format_scale(int format, const void* scales, int64_t k, int64_t r, int64_t c) {
  switch (format) {
    case FMT_BLOCK:
      return (double)((const float*)scales)[(r / TILE) * ((k + TILE - 1) / TILE) + c / TILE];
    case FMT_MX:
      return ldexp(1.0, (int)((const uint8_t*)scales)[r * ((k + MX_GROUP - 1) / MX_GROUP) + c / MX_GROUP] - 127);
    case FMT_BLOCK_BF16:
      return (double)bf16_to_float(((const uint16_t*)scales)[(r / TILE) * ((k + TILE - 1) / TILE) + c / TILE]);
    case FMT_ROW:
      return (double)((const float*)scales)[r];
    case FMT_TENSOR:
      return (double)((const float*)scales)[0];
  }
  return NAN;
}

static int format_ok(int format) { return format >= FMT_BLOCK && format <= FMT_TENSOR; }

/* Dequantize to bf16 in any format: bf16_rne(fl32(dec(code) * scale)). */
int oracle_dequant_format_bf16(const uint8_t* codes, const void* scales, int format, int64_t n,
                               int64_t k, uint16_t* out) {
  if (!codes || !scales || !out || n < 1 || k < 1 || !format_ok(format)) return ORACLE_ERR_ARG;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r)
    for (int64_t c = 0; c < k; ++c) {
      const float p = (float)(oracle_e4m3_decode(codes[r * k + c]) * format_scale(format, scales, k, r, c));
      out[r * k + c] = oracle_round_bf16((double)p);
    }
  return ORACLE_OK;
}

/* GEMV reference in any format, fp64: y[i][j] = sum_k x[i][k] * deq[r][k]
 * with deq = dec(code) * scale (the scale as format_scale gives it). */
int oracle_gemv_format_f64(const uint16_t* x, int64_t m, const uint8_t* codes, const void* scales,
                           int format, int64_t n, int64_t k, const int64_t* rows, int64_t nrows,
                           double* y, double* bound) {
  if (!x || !codes || !scales || !y || m < 1 || n < 1 || k < 1 || !format_ok(format))
    return ORACLE_ERR_ARG;
  if (!rows) nrows = n;
  for (int64_t j = 0; rows && j < nrows; ++j)
    if (rows[j] < 0 || rows[j] >= n) return ORACLE_ERR_ARG;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t j = 0; j < nrows; ++j) {
    const int64_t r = rows ? rows[j] : j;
    for (int64_t i = 0; i < m; ++i) {
      double acc = 0.0, mag = 0.0;
      for (int64_t c = 0; c < k; ++c) {
        const double d = oracle_e4m3_decode(codes[r * k + c]) * format_scale(format, scales, k, r, c);
        const double xv = (double)bf16_to_float(x[i * k + c]);
        acc += xv * d;
        mag += fabs(xv) * fabs(d);
      }
      y[i * nrows + j] = acc;
      if (bound) bound[i * nrows + j] = mag;
    }
  }
  return ORACLE_OK;
}

/* -------------------------------------------------------- dequantize -- */

/* deq[n][k] = dec(code) * scale[n/128][k/128], exact in fp64 (4 + 24 bits). */
int oracle_dequant_block(const uint8_t* codes, const float* scales, int64_t n,
                         int64_t k, double* out) {
  if (!codes || !scales || !out || n < 1 || k < 1) return ORACLE_ERR_ARG;
  const int64_t tiles_k = (k + TILE - 1) / TILE;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r)
    for (int64_t c = 0; c < k; ++c)
      out[r * k + c] = oracle_e4m3_decode(codes[r * k + c]) *
                       (double)scales[(r / TILE) * tiles_k + c / TILE];
  return ORACLE_OK;
}

/* deq[n][k] = dec(code) * 2^(E[n][k/32] - 127), exact in fp64. */
int oracle_dequant_mx(const uint8_t* codes, const uint8_t* e8m0, int64_t n,
                      int64_t k, double* out) {
  if (!codes || !e8m0 || !out || n < 1 || k < 1) return ORACLE_ERR_ARG;
  const int64_t groups = (k + MX_GROUP - 1) / MX_GROUP;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r)
    for (int64_t c = 0; c < k; ++c)
      out[r * k + c] = ldexp(oracle_e4m3_decode(codes[r * k + c]),
                             (int)e8m0[r * groups + c / MX_GROUP] - 127);
  return ORACLE_OK;
}

/* ------------------------------------------------ dequantize to bf16 -- */

/* bf16 nearest to v, ties to the even bit pattern; magnitudes at or above
 * the midpoint between the largest finite bf16 and 2^128 become infinity
 * (IEEE overflow under round-to-nearest).  A binary search over the 32,640
 * non-negative finite bf16 patterns, which are ordered like their values;
 * the two neighbours are compared in fp64, where every bf16 value and every
 * fp32 input is exact. */
uint16_t oracle_round_bf16(double v) {
  if (isnan(v)) return 0x7FC0;
  const uint16_t sign = signbit(v) ? 0x8000 : 0;
  const double a = fabs(v);
  const uint16_t kMaxFinite = 0x7F7F;
  if (a >= (double)bf16_to_float(kMaxFinite)) {
    const double top = ldexp(1.0, 128);   /* the value the next pattern would have */
    const double lo = (double)bf16_to_float(kMaxFinite);
    if (a - lo < top - a) return sign | kMaxFinite;
    return sign | 0x7F80;                 /* at or past the midpoint: infinity */
  }
  uint16_t lo = 0, hi = kMaxFinite;       /* largest pattern with value <= a */
  while (lo < hi) {
    const uint16_t mid = (uint16_t)((lo + hi + 1) / 2);
    if ((double)bf16_to_float(mid) <= a) lo = mid;
    else hi = (uint16_t)(mid - 1);
  }
  const double below = (double)bf16_to_float(lo);
  if (below == a) return sign | lo;
  const double above = (double)bf16_to_float((uint16_t)(lo + 1));
  const double d_lo = a - below, d_hi = above - a;
  uint16_t pick;
  if (d_lo < d_hi) pick = lo;
  else if (d_hi < d_lo) pick = (uint16_t)(lo + 1);
  else pick = (lo % 2 == 0) ? lo : (uint16_t)(lo + 1);
  return sign | pick;
}

void oracle_round_bf16_array(const double* v, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_round_bf16(v[i]);
}

/* Dequantize to bf16 as a dequantize-then-dense-GEMM path consumes it: the
 * decoded value times the scale, rounded to fp32 (one IEEE multiply; the
 * fp64 product is exact, so converting it to float is that multiply), then
 * rounded to bf16 ("feat: add FP8 blockwise weight quantization ...",
 * Summary: larger M and prefill dequantize to bf16 for a dense GEMM; the
 * round-trip check of "feat(quant): opt-in fp8-block QAT for the lm_head",
 * Validation, pairs the quantizer with this dequantizer).  MX scales are
 * powers of two, so there the fp32 product is exact and only the bf16
 * rounding remains. */
int oracle_dequant_block_bf16(const uint8_t* codes, const float* scales, int64_t n,
                              int64_t k, uint16_t* out) {
  if (!codes || !scales || !out || n < 1 || k < 1) return ORACLE_ERR_ARG;
  const int64_t tiles_k = (k + TILE - 1) / TILE;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r)
    for (int64_t c = 0; c < k; ++c) {
      const double exact = oracle_e4m3_decode(codes[r * k + c]) *
                           (double)scales[(r / TILE) * tiles_k + c / TILE];
      const float p = (float)exact;
      out[r * k + c] = oracle_round_bf16((double)p);
    }
  return ORACLE_OK;
}

int oracle_dequant_mx_bf16(const uint8_t* codes, const uint8_t* e8m0, int64_t n,
                           int64_t k, uint16_t* out) {
  if (!codes || !e8m0 || !out || n < 1 || k < 1) return ORACLE_ERR_ARG;
  const int64_t groups = (k + MX_GROUP - 1) / MX_GROUP;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r)
    for (int64_t c = 0; c < k; ++c) {
      const double exact = ldexp(oracle_e4m3_decode(codes[r * k + c]),
                                 (int)e8m0[r * groups + c / MX_GROUP] - 127);
      const float p = (float)exact;
      out[r * k + c] = oracle_round_bf16((double)p);
    }
  return ORACLE_OK;
}

/* ------------------------------------------- activation quantization -- */

/* Dynamic per-tensor activation quantization ("feat(qwen4_exp): load-time
 * per-tensor FP8 dense projections", What this adds: a per-tensor
 * activation scale from an amax pass, then the cast; its perf(fp8)
 * follow-up computes the same amax block-parallel, bit for bit): one scale
 * for the whole x [m, k], by the rule of the block quantizer applied to a
 * single tile -- amax over every element, scale = fl32(amax / 448) (1.0 when
 * amax == 0), code = enc(fl32(x / scale)). */
int oracle_quantize_act_tensor(const uint16_t* x, int64_t m, int64_t k, uint8_t* codes,
                               float* scale) {
  if (!x || !codes || !scale || m < 1 || k < 1) return ORACLE_ERR_ARG;
  const int64_t count = m * k;
  if (!all_finite(x, count)) return ORACLE_ERR_NONFINITE;
  float amax = 0.0f;
  for (int64_t i = 0; i < count; ++i) {
    const float a = fabsf(bf16_to_float(x[i]));
    if (a > amax) amax = a;
  }
  const float s = amax > 0.0f ? (float)(amax / (float)E4M3_MAX) : 1.0f;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) codes[i] = oracle_e4m3_encode(bf16_to_float(x[i]) / s);
  *scale = s;
  return ORACLE_OK;
}

/* W8A8 GEMV reference on a quantized activation: y[i][j] = sum_k
 * (dec(xc[i][k]) * xs) * deq[j][k] and bound[i][j] = sum_k |.| |.|, in fp64,
 * for the requested weight rows (all when rows is NULL); deq as above. */
static int gemv_xq_f64(const uint8_t* xc, float xs, int64_t m, const uint8_t* codes,
                       const float* block_scales, const uint8_t* e8m0, int64_t n, int64_t k,
                       const int64_t* rows, int64_t nrows, double* y, double* bound) {
  if (!xc || !codes || !y || m < 1 || n < 1 || k < 1) return ORACLE_ERR_ARG;
  if (!rows) nrows = n;
  for (int64_t j = 0; rows && j < nrows; ++j)
    if (rows[j] < 0 || rows[j] >= n) return ORACLE_ERR_ARG;
  const int64_t tiles_k = (k + TILE - 1) / TILE;
  const int64_t groups = (k + MX_GROUP - 1) / MX_GROUP;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t j = 0; j < nrows; ++j) {
    const int64_t r = rows ? rows[j] : j;
    for (int64_t i = 0; i < m; ++i) {
      double acc = 0.0, mag = 0.0;
      for (int64_t c = 0; c < k; ++c) {
        double d = oracle_e4m3_decode(codes[r * k + c]);
        if (block_scales)
          d *= (double)block_scales[(r / TILE) * tiles_k + c / TILE];
        else
          d = ldexp(d, (int)e8m0[r * groups + c / MX_GROUP] - 127);
        const double xv = oracle_e4m3_decode(xc[i * k + c]) * (double)xs;
        acc += xv * d;
        mag += fabs(xv) * fabs(d);
      }
      y[i * nrows + j] = acc;
      if (bound) bound[i * nrows + j] = mag;
    }
  }
  return ORACLE_OK;
}

int oracle_gemv_w8a8_block_f64(const uint8_t* xc, float xs, int64_t m, const uint8_t* codes,
                               const float* scales, int64_t n, int64_t k, const int64_t* rows,
                               int64_t nrows, double* y, double* bound) {
  if (!scales) return ORACLE_ERR_ARG;
  return gemv_xq_f64(xc, xs, m, codes, scales, NULL, n, k, rows, nrows, y, bound);
}

int oracle_gemv_w8a8_mx_f64(const uint8_t* xc, float xs, int64_t m, const uint8_t* codes,
                            const uint8_t* e8m0, int64_t n, int64_t k, const int64_t* rows,
                            int64_t nrows, double* y, double* bound) {
  if (!e8m0) return ORACLE_ERR_ARG;
  return gemv_xq_f64(xc, xs, m, codes, NULL, e8m0, n, k, rows, nrows, y, bound);
}

/* -------------------------------------------------------------- GEMV -- */

/* For each requested weight row n (rows[j], or every row when rows is NULL)
 * and each activation row i:
 *   y[i][j]     = sum_k x[i][k] * deq[n][k]       (fp64)
 *   bound[i][j] = sum_k |x[i][k]| * |deq[n][k]|   (fp64)
 * deq is rebuilt per element from the codes and scales, exactly as in the
 * dequantizers above.  y and bound are [m, nrows] row-major.              */
static int gemv_f64(const uint16_t* x, int64_t m, const uint8_t* codes,
                    const float* block_scales, const uint8_t* e8m0, int64_t n,
                    int64_t k, const int64_t* rows, int64_t nrows, double* y,
                    double* bound) {
  if (!x || !codes || !y || m < 1 || n < 1 || k < 1) return ORACLE_ERR_ARG;
  if (!rows) nrows = n;
  for (int64_t j = 0; rows && j < nrows; ++j)
    if (rows[j] < 0 || rows[j] >= n) return ORACLE_ERR_ARG;
  const int64_t tiles_k = (k + TILE - 1) / TILE;
  const int64_t groups = (k + MX_GROUP - 1) / MX_GROUP;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t j = 0; j < nrows; ++j) {
    const int64_t r = rows ? rows[j] : j;
    for (int64_t i = 0; i < m; ++i) {
      double acc = 0.0, mag = 0.0;
      for (int64_t c = 0; c < k; ++c) {
        double d = oracle_e4m3_decode(codes[r * k + c]);
        if (block_scales)
          d *= (double)block_scales[(r / TILE) * tiles_k + c / TILE];
        else
          d = ldexp(d, (int)e8m0[r * groups + c / MX_GROUP] - 127);
        const double xv = (double)bf16_to_float(x[i * k + c]);
        acc += xv * d;
        mag += fabs(xv) * fabs(d);
      }
      y[i * nrows + j] = acc;
      if (bound) bound[i * nrows + j] = mag;
    }
  }
  return ORACLE_OK;
}

int oracle_gemv_block_f64(const uint16_t* x, int64_t m, const uint8_t* codes,
                          const float* scales, int64_t n, int64_t k,
                          const int64_t* rows, int64_t nrows, double* y,
                          double* bound) {
  if (!scales) return ORACLE_ERR_ARG;
  return gemv_f64(x, m, codes, scales, NULL, n, k, rows, nrows, y, bound);
}

int oracle_gemv_mx_f64(const uint16_t* x, int64_t m, const uint8_t* codes,
                       const uint8_t* e8m0, int64_t n, int64_t k,
                       const int64_t* rows, int64_t nrows, double* y,
                       double* bound) {
  if (!e8m0) return ORACLE_ERR_ARG;
  return gemv_f64(x, m, codes, NULL, e8m0, n, k, rows, nrows, y, bound);
}
