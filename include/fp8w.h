/*
 * fp8w.h -- C ABI of libfp8w: FP8 (OCP e4m3fn) weights for the decode path
 * on AMD Instinct MI355X (gfx950).
 *
 * Operations (each in every scale format below):
 *
 *   quantize    bf16 W[n,k]  ->  e4m3fn codes[n,k] + a scale grid
 *   GEMV        y[m,n] = x[m,k] . deq(W)^T, bf16 in, bf16 out, fp32
 *               accumulate, m <= 32 (single calls or grouped)
 *   dequantize  codes + scales -> bf16 W[n,k]
 *   W8A8        per-tensor activation quantization, and the GEMV on fp8
 *               activations (fp8 x fp8 matrix-core products)
 *   GEMM        the same product for any m, through dequantize + a dense
 *               bf16 GEMM (the large-M / prefill route)
 * and a measurement aid: a read-only pass over device memory with the
 * GEMV's loads (fp8w_read_ceiling).
 *
 * Scale formats:
 *   block : one fp32 scale per 128x128 tile, grid [ceil(n/128), ceil(k/128)]
 *           row-major; scale = amax/448 (1.0 for an all-zero tile) and
 *           deq = dec(code) * scale.  Format of "quantize_fp8_bs.rs" (Atlas
 *           spark_model/weight_map: one byte per weight, one f32 per
 *           [128,128] tile) and of the 128x128 block checkpoints of "feat: add
 *           FP8 blockwise weight quantization and FP8(E4M3) KV cache support"
 *           (Summary); the per-block quantizer of "feat(quant): opt-in
 *           fp8-block QAT for the lm_head" (Changes).
 *   mx    : one e8m0 byte per 32 elements along K, grid [n, ceil(k/32)]
 *           row-major; exponent e = ceil(log2(amax/448)) clamped to
 *           [-127, 127], byte = e + 127 (an all-zero group stores 0), and
 *           deq = dec(code) * 2^(byte - 127).  "Load-time MXFP8
 *           requantization of bf16 dense, hyper-connection and lm_head
 *           weights" (Proposed solution).
 *
 * Encoding (both formats): the quotient w/scale (fp32, correctly rounded),
 * or w * 2^-e, is rounded to the nearest e4m3fn value with ties to the even
 * code, saturating at +-448; the sign is kept (negative values that round to
 * zero give 0x80).  NaN codes (0x7F, 0xFF) are never produced.
 *
 * Data types: bf16 tensors are passed as their raw 16-bit patterns
 * (uint16_t), since C has no bf16 type.  All matrices are dense row-major.
 *
 * Memory and ownership: every tensor pointer is a DEVICE pointer on the
 * current HIP device.  The caller allocates and frees every buffer; the
 * library keeps no pointer after a call returns and never allocates (the
 * GEMM calls alone create one rocBLAS handle per device, in
 * fp8w_gemm_prepare or on their first use).
 *
 * Execution: every call only enqueues work on `stream` (a hipStream_t;
 * NULL means the default stream) and returns without synchronizing.  Calls
 * never read tensor values on the host, and the kernel chosen depends on the
 * shape only, so the calls may be captured in a HIP graph, with two
 * exceptions that need a set-up call outside capture first: the GEMM calls
 * (fp8w_gemm_prepare, or one GEMM call, on the device) and the grouped
 * calls (fp8w_grouped_plan_init, fp8w_quant_plan_init).
 * fp8w_quantize_act_noalloc resolves its device array on its first call on
 * a device; make that call outside capture too.  Results are bitwise
 * reproducible run to run (no atomics, fixed reduction order).
 *
 * Errors: arguments are checked on the host before anything is enqueued; on
 * any error nothing is launched and no output byte is written.  A fault
 * during execution surfaces at the caller's next synchronization of
 * `stream`.  Non-finite inputs are outside the contract: the calls do not
 * fault on them but their outputs are unspecified.  Mis-shaped calls fail
 * loudly instead of miscomputing, as the bounds contract of "feat: add FP8
 * blockwise weight quantization ..." (Security and Safety) asks.
 */
#ifndef FP8W_H_
#define FP8W_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fp8w_status {
  FP8W_OK = 0,
  FP8W_ERR_NULL = 1,        /* a required pointer is NULL                      */
  FP8W_ERR_SHAPE = 2,       /* n, k or m out of range (n, k >= 1; m in 1..32)   */
  FP8W_ERR_ALIGN = 3,       /* GEMV: k % 16 != 0 or x / codes not 16-B aligned, */
                            /* or a scale pointer not 4-B aligned               */
  FP8W_ERR_UNSUPPORTED = 4, /* the requested route cannot serve this m          */
  FP8W_ERR_OVERLAP = 5,     /* an output byte range overlaps another buffer     */
  FP8W_ERR_HIP = 6,         /* the HIP runtime rejected the launch              */
  FP8W_ERR_CAPTURE = 7      /* GEMM: the device's rocBLAS handle would have to  */
                            /* be created under stream capture                  */
} fp8w_status;

/* GEMV kernel family.  The two routes follow the fused W8A16 GEMM of "feat:
 * add FP8 blockwise weight quantization ..." (Summary; Notes for Reviewers:
 * SIMT for M <= 8, tensor-core mma for 9 <= M <= 32): VALU serves
 * 1 <= m <= 8 only; MFMA serves 1 <= m <= 32.  AUTO follows the crossovers
 * measured on MI355X: single calls take VALU for m <= 2, for m = 3 on
 * weights of fewer than 32768 rows, and for m = 4 on weights of at most
 * 8192 rows and K <= 4096, in every scale format (fp8w_gemv_auto_route
 * gives the choice); grouped launches take VALU for m = 1, and for m = 2 on
 * every format but MX; MFMA otherwise.  Within a route the
 * kernel also depends on n and k (weights with many rows take the streaming
 * kernels; K above 3072 is walked in 3072- or 4096-column segments) and, for
 * MX, on how the exponent array is laid out (4-byte aligned with n *
 * ceil(k/32) % 4 == 0: the M = 1 streaming kernel; 8-byte aligned with
 * ceil(k/32) % 8 == 0: one 8-byte exponent load per row and panel in the
 * MFMA kernels) -- never on values.  Every route meets the same error
 * bound. */
typedef enum fp8w_route {
  FP8W_ROUTE_AUTO = 0,
  FP8W_ROUTE_VALU = 1,
  FP8W_ROUTE_MFMA = 2
} fp8w_route;

/* Scale formats.  The calls named _block / _mx fix BLOCK / MX; the generic
 * calls (fp8w_quantize, fp8w_dequantize, fp8w_gemv, fp8w_gemm,
 * fp8w_gemv_w8a8, grouped plans) take any of them.  The other three are
 * degenerate tilings of the same rule -- scale = amax/448 over the tile, 1.0
 * for an all-zero tile, code = enc(w/scale):
 *   BLOCK_BF16 : the 128x128 tile, scale stored as the nearest bf16 (at
 *                least 2^-133) and the codes divided by that stored value
 *                ("feat(quant): opt-in fp8-block QAT for the lm_head", How it
 *                works: a bf16 128-block scale)
 *   ROW        : a 1 x k tile, f32 [n] ("quantize_fp8_bs.rs", Atlas
 *                weight_map: the per-ROW quantizer of the DFlash head; the
 *                per-row W8A16 route of "feat(qwen4_exp): load-time
 *                per-tensor FP8 dense projections", Why)
 *   TENSOR     : one tile covering the weight, f32 [1] (the per-tensor
 *                weights of the same page, What this adds)
 * A scale buffer of the wrong format cannot be detected by a kernel
 * ("quantize_fp8_bs.rs", module notes), so the format is always explicit. */
typedef enum fp8w_format {
  FP8W_FORMAT_BLOCK = 0,      /* f32 [ceil(n/128), ceil(k/128)]  */
  FP8W_FORMAT_MX = 1,         /* u8 e8m0 [n, ceil(k/32)]          */
  FP8W_FORMAT_BLOCK_BF16 = 2, /* bf16 [ceil(n/128), ceil(k/128)] */
  FP8W_FORMAT_ROW = 3,        /* f32 [n]                          */
  FP8W_FORMAT_TENSOR = 4      /* f32 [1]                          */
} fp8w_format;

/* Bytes of the scale buffer of an [n, k] weight in `format` (0 if the
 * format or the shape is invalid).  Scale buffers are aligned to their
 * element size (4, 1, 2, 4, 4 bytes). */
int64_t fp8w_scale_bytes(fp8w_format format, int64_t n, int64_t k);

/* Largest m (activation rows) served by the GEMV calls.  Larger batches are
 * prefill work, served elsewhere ("feat: add FP8 blockwise weight
 * quantization ...", Summary: M > 32 uses dequantize + dense GEMM). */
#define FP8W_MAX_M 32

/* ------------------------------------------------------------ quantize -- */

/* Block quantization, load time.
 *   w      : bf16 [n, k] (2-byte aligned)                          input
 *   codes  : u8   [n, k]                                           output
 *   scales : f32  [ceil(n/128), ceil(k/128)] (4-byte aligned)      output
 * Per tile: amax = max |w| over the tile's valid elements; scale =
 * amax/448 in fp32 (1.0 if amax == 0); code = enc(w/scale) in fp32.
 * Tiles at the bottom/right edges are partial.  Any n, k >= 1.
 * Errors: NULL, SHAPE (n < 1, k < 1, n or k > 2^31 - 1), ALIGN, OVERLAP, HIP. */
fp8w_status fp8w_quantize_block(const uint16_t* w, int64_t n, int64_t k,
                                uint8_t* codes, float* scales, void* stream);

/* MX quantization, load time.
 *   w     : bf16 [n, k]                        input
 *   codes : u8   [n, k]                        output
 *   e8m0  : u8   [n, ceil(k/32)]               output
 * Per row and 32-element group along K (the last group may be partial):
 * e = smallest integer with amax <= 448 * 2^e, clamped to [-127, 127]
 * (-127 if amax == 0); byte = e + 127; code = enc(w * 2^-e).  The result
 * does not depend on how rows are chunked, so no transient is needed.
 * Errors: NULL, SHAPE, OVERLAP, HIP. */
fp8w_status fp8w_quantize_mx(const uint16_t* w, int64_t n, int64_t k,
                             uint8_t* codes, uint8_t* e8m0, void* stream);

/* Quantization in any format, load time: codes [n, k] and the format's
 * scale buffer.  TENSOR needs `workspace` (>= fp8w_quantize_act_workspace_bytes()
 * bytes, 4-byte aligned) when n * k > 16384, as fp8w_quantize_act; the other
 * formats ignore it (may be NULL).  Any n, k >= 1.
 * Errors: NULL, SHAPE, ALIGN, UNSUPPORTED (format), OVERLAP, HIP. */
fp8w_status fp8w_quantize(const uint16_t* w, int64_t n, int64_t k, fp8w_format format,
                          uint8_t* codes, void* scales, void* workspace,
                          int64_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- GEMV -- */

/* Block-scaled W8A16 GEMV / skinny GEMM.
 *   x      : bf16 [m, k], 16-byte aligned                   input
 *   codes  : u8   [n, k], 16-byte aligned                   input
 *   scales : f32  [ceil(n/128), ceil(k/128)], 4-B aligned    input
 *   y      : bf16 [m, n]                                    output
 * y[i][j] = bf16_rne( sum_k x[i][k] * dec(codes[j][k]) * scale[j/128][k/128] )
 * accumulated in fp32.  Bound met for every output, with y_ref in fp64:
 * |y - y_ref| <= 2^-7 * sum_k |x[i][k]| |deq[j][k]| + 1e-6.
 * Requires 1 <= m <= 32, n >= 1, k >= 16 and k % 16 == 0.
 * Errors: NULL, SHAPE, ALIGN, UNSUPPORTED, OVERLAP, HIP. */
fp8w_status fp8w_gemv_block(const uint16_t* x, int64_t m, const uint8_t* codes,
                            const float* scales, int64_t n, int64_t k,
                            uint16_t* y, void* stream);

/* MX-scaled W8A16 GEMV: as fp8w_gemv_block with
 * deq[j][k] = dec(codes[j][k]) * 2^(e8m0[j][k/32] - 127).
 *   e8m0 : u8 [n, ceil(k/32)]   input (no alignment requirement) */
fp8w_status fp8w_gemv_mx(const uint16_t* x, int64_t m, const uint8_t* codes,
                         const uint8_t* e8m0, int64_t n, int64_t k,
                         uint16_t* y, void* stream);

/* The route AUTO takes for a single-call GEMV of m activation rows on an
 * [n, k] weight with scales of the given format: FP8W_ROUTE_VALU or
 * FP8W_ROUTE_MFMA, or FP8W_ROUTE_AUTO when the format is unknown or m, n or
 * k is out of range (m outside 1..32, n or k outside 1..2^31-1).  Pure host
 * function; touches no device state. */
fp8w_route fp8w_gemv_auto_route(fp8w_format format, int64_t m, int64_t n, int64_t k);

/* The same two GEMVs with an explicit kernel family, for A/B measurement
 * and for testing every route at every m.  FP8W_ROUTE_AUTO is identical to
 * the calls above. */
fp8w_status fp8w_gemv_block_route(const uint16_t* x, int64_t m,
                                  const uint8_t* codes, const float* scales,
                                  int64_t n, int64_t k, uint16_t* y,
                                  fp8w_route route, void* stream);
fp8w_status fp8w_gemv_mx_route(const uint16_t* x, int64_t m,
                               const uint8_t* codes, const uint8_t* e8m0,
                               int64_t n, int64_t k, uint16_t* y,
                               fp8w_route route, void* stream);

/* ---------------------------------------------------------- dequantize -- */

/* Block dequantization: the inverse of fp8w_quantize_block.
 *   codes  : u8   [n, k]                                      input
 *   scales : f32  [ceil(n/128), ceil(k/128)] (4-byte aligned)  input
 *   w      : bf16 [n, k]                                      output
 * w[r][c] = bf16_rne( fl32( dec(codes[r][c]) * scales[r/128][c/128] ) ): one
 * fp32 multiply, then rounding to nearest even bf16 (overflow gives inf).
 * The dequantizer the lm_head QAT page pairs with its block quantizer ("feat
 * (quant): opt-in fp8-block QAT for the lm_head", Changes), feeding the
 * dense-GEMM route of "feat: add FP8 blockwise weight quantization ..."
 * (Summary).  Any n, k >= 1; a 16-byte path when k % 16 == 0 and codes and w
 * are 16-byte aligned.  NaN codes give NaN.
 * Errors: NULL, SHAPE, ALIGN, OVERLAP, HIP. */
fp8w_status fp8w_dequantize_block(const uint8_t* codes, const float* scales,
                                  int64_t n, int64_t k, uint16_t* w, void* stream);

/* MX dequantization: w[r][c] = bf16_rne( dec(codes[r][c]) *
 * 2^(e8m0[r][c/32] - 127) ), the product exact in fp32 (a decoded code has
 * 4 significant bits), so the result is the exact value wherever it is a
 * normal bf16.
 * Errors: NULL, SHAPE, OVERLAP, HIP. */
fp8w_status fp8w_dequantize_mx(const uint8_t* codes, const uint8_t* e8m0,
                               int64_t n, int64_t k, uint16_t* w, void* stream);

/* ---------------------------------------------------------------- GEMM -- */

/* The large-M route: y[m, n] = x[m, k] . deq(W)^T for any m >= 1, as
 * "feat: add FP8 blockwise weight quantization ..." routes M > 32 and
 * prefill (Summary): dequantize W into `workspace` (bf16 [n, k], as
 * fp8w_dequantize_block / _mx write it), then one dense bf16 GEMM with fp32
 * accumulation and a bf16 result (rocBLAS gemm_ex).
 *   x         : bf16 [m, k]            input
 *   y         : bf16 [m, n]            output
 *   workspace : >= fp8w_gemm_workspace_bytes(n, k) bytes of device memory,
 *               16-byte aligned; overwritten (holds deq(W) afterwards)
 * Bound, with y_ref in fp64 from the exact dequantized weight:
 * |y - y_ref| <= 2^-7 * sum_k |x[i][k]| |deq[j][k]| + 1e-6 (the bf16 weight
 * adds at most 2^-8 of that sum).  The calls use one rocBLAS handle per
 * device, created by fp8w_gemm_prepare or by the first GEMM call on the
 * device (rocBLAS allocates its own workspace then); if that first call's
 * stream is capturing, it fails with FP8W_ERR_CAPTURE and enqueues nothing,
 * and once the handle exists the calls may be captured.  Calls on one
 * device are serialized around its handle.  m, n, k <= 2^31 - 1.
 * Errors: NULL, SHAPE (also: workspace too small), ALIGN, OVERLAP, CAPTURE,
 * HIP. */
int64_t fp8w_gemm_workspace_bytes(int64_t n, int64_t k);

/* Create the current device's rocBLAS handle for the GEMM calls now, so that
 * later GEMM calls can be captured in a HIP graph.  Not for use under
 * capture; idempotent.  Errors: HIP (no device, or rocBLAS failed). */
fp8w_status fp8w_gemm_prepare(void);
fp8w_status fp8w_gemm_block(const uint16_t* x, int64_t m, const uint8_t* codes,
                            const float* scales, int64_t n, int64_t k, uint16_t* y,
                            void* workspace, int64_t workspace_bytes, void* stream);
fp8w_status fp8w_gemm_mx(const uint16_t* x, int64_t m, const uint8_t* codes,
                         const uint8_t* e8m0, int64_t n, int64_t k, uint16_t* y,
                         void* workspace, int64_t workspace_bytes, void* stream);

/* --------------------------------------------------------------- W8A8 -- */

/* Dynamic per-tensor activation quantization ("feat(qwen4_exp): load-time
 * per-tensor FP8 dense projections", What this adds: an amax pass, then the
 * cast; its perf(fp8) follow-up splits the amax block-parallel above 16384
 * elements with the same result).  One scale for the whole x [m, k]:
 * scale = amax/448 in fp32 (1.0 if amax == 0), codes = enc(x/scale) in
 * fp32 -- the block quantizer's rule on a single tile covering the tensor.
 *   x         : bf16 [m, k]                                  input
 *   codes     : u8 [m, k]                                    output
 *   scale     : f32 [1] (4-byte aligned)                     output
 *   workspace : >= fp8w_quantize_act_workspace_bytes() bytes, 4-byte
 *               aligned, when m * k > 16384 (partial maxima); may be NULL
 *               otherwise
 * Up to 16384 elements: one launch; above: two, the second reducing the
 * partials itself.  Both paths give the same bits.
 * Errors: NULL, SHAPE (also: workspace too small), ALIGN, OVERLAP, HIP. */
int64_t fp8w_quantize_act_workspace_bytes(void);
fp8w_status fp8w_quantize_act(const uint16_t* x, int64_t m, int64_t k, uint8_t* codes,
                              float* scale, void* workspace, int64_t workspace_bytes,
                              void* stream);

/* fp8w_quantize_act without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, result bits and errors as
 * fp8w_quantize_act, minus the workspace; any m * k (the partial maxima of
 * every size fit the array).  The partial maxima live in a file-scope device
 * array of 256 32-bit words (1 KiB) that each device holds until the process
 * ends; the first call on a device resolves that device's address of it
 * (hipGetSymbolAddress), so make that first call outside stream capture.
 * Every call on one device shares the array and leaves its partial maxima
 * in it: each launch writes every word it later reads, so nothing needs
 * clearing, but calls that overlap in time on one device (concurrent
 * streams, or host threads) race on it and must be serialized by the
 * caller.  Allocates nothing.  Errors: NULL, SHAPE, ALIGN, OVERLAP, HIP. */
fp8w_status fp8w_quantize_act_noalloc(const uint16_t* x, int64_t m, int64_t k, uint8_t* codes,
                                      float* scale, void* stream);

/* W8A8 GEMV on a quantized activation:
 *   y[i][j] = bf16_rne( x_scale * sum_k dec(x_codes[i][k]) * deq[j][k] )
 * with fp32 accumulation.  From m = 3 the products are fp8 x fp8 on the
 * matrix cores, block scales applied per 128-column block (MX scales inside
 * the instruction); at m <= 2 the activation codes are widened to bf16
 * (exact) and the products run on the vector units.
 *   x_codes : u8 [m, k], 16-byte aligned      input (fp8w_quantize_act)
 *   x_scale : f32 [1] on the device, 4-B aligned  input (read on the device)
 *   codes, scales / e8m0, n, k, y : as fp8w_gemv_block / fp8w_gemv_mx
 * Bound against the fp64 product of the same quantized operands:
 * |y - y_ref| <= 2^-7 * sum_k |x_scale dec(x_codes)| |deq| + 1e-6.
 * Requires 1 <= m <= 32, k >= 16, k % 16 == 0.
 * Errors: NULL, SHAPE, ALIGN, OVERLAP, HIP. */
fp8w_status fp8w_gemv_block_w8a8(const uint8_t* x_codes, const float* x_scale, int64_t m,
                                 const uint8_t* codes, const float* scales, int64_t n,
                                 int64_t k, uint16_t* y, void* stream);
fp8w_status fp8w_gemv_mx_w8a8(const uint8_t* x_codes, const float* x_scale, int64_t m,
                              const uint8_t* codes, const uint8_t* e8m0, int64_t n, int64_t k,
                              uint16_t* y, void* stream);

/* ----------------------------------------------------- generic formats -- */

/* GEMV in any format, with the same contract and bound as fp8w_gemv_block
 * (block scales multiply each 128-column block's partial sum; row and
 * tensor scales multiply each output).  fp8w_gemv_block / _mx and the _route
 * calls are this call with the format fixed. */
fp8w_status fp8w_gemv(const uint16_t* x, int64_t m, const uint8_t* codes, const void* scales,
                      fp8w_format format, int64_t n, int64_t k, uint16_t* y, fp8w_route route,
                      void* stream);

/* Dequantization in any format: bf16_rne(fl32(dec(code) * scale)). */
fp8w_status fp8w_dequantize(const uint8_t* codes, const void* scales, fp8w_format format,
                            int64_t n, int64_t k, uint16_t* w, void* stream);

/* The large-M route in any format (contract of fp8w_gemm_block). */
fp8w_status fp8w_gemm(const uint16_t* x, int64_t m, const uint8_t* codes, const void* scales,
                      fp8w_format format, int64_t n, int64_t k, uint16_t* y, void* workspace,
                      int64_t workspace_bytes, void* stream);

/* The W8A8 GEMV in any format (contract of fp8w_gemv_block_w8a8). */
fp8w_status fp8w_gemv_w8a8(const uint8_t* x_codes, const float* x_scale, int64_t m,
                           const uint8_t* codes, const void* scales, fp8w_format format,
                           int64_t n, int64_t k, uint16_t* y, void* stream);

/* ------------------------------------------------------------- grouped -- */

/* A group of independent GEMVs served by one kernel launch: the fixed cost
 * of a launch (about 1.7 us on MI355X) is paid once instead of per GEMV,
 * which matters when each GEMV streams only a few microseconds of weights
 * (the 96-GEMV decode pass of "feat(qwen4_exp): load-time per-tensor FP8
 * dense projections", Why; the grouped expert GEMM that reads [N/128,
 * K/128] fp32 block scales in "quantize_fp8_bs.rs", Atlas weight_map).  The
 * GEMVs of a group must not depend on one another (no y of one is the x of
 * another); all share m, the scale format (any fp8w_format) and the route.
 * Each GEMV meets the same error bound as the single call (the summation
 * order may differ, so the last bit of y may too). */

/* One GEMV of a group; the same layout rules as fp8w_gemv.  scales points
 * at the group's format's scale buffer (f32 grid, e8m0 bytes, bf16 grid,
 * f32 per row or one f32). */
typedef struct fp8w_gemv_desc {
  const uint16_t* x;     /* bf16 [m, k], 16-byte aligned       */
  const uint8_t* codes;  /* e4m3fn [n, k], 16-byte aligned     */
  const void* scales;    /* the format's scale buffer, aligned to its element */
  uint16_t* y;           /* bf16 [m, n], output                */
  int64_t n, k;          /* n >= 1, k >= 16, k % 16 == 0       */
} fp8w_gemv_desc;

/* What fp8w_grouped_plan_init fills in; pass it to fp8w_gemv_grouped. */
typedef struct fp8w_grouped_plan {
  const void* table;       /* the caller's device table buffer            */
  int32_t count;           /* GEMVs in the group                          */
  int32_t m;               /* activation rows, shared by the group        */
  int32_t format;          /* fp8w_format                                 */
  int32_t route;           /* fp8w_route resolved for m (VALU or MFMA)    */
  int64_t blocks;          /* workgroups of one launch                    */
  int64_t tiles;           /* row tiles of all GEMVs together             */
  int32_t tiles_per_block; /* 0: one tile per workgroup; else a contiguous
                              run of tiles per workgroup (streaming kernels) */
  int32_t seg_cols;        /* MFMA route: K columns of x staged per pass
                              (a multiple of 256; m <= 16: m * seg_cols * 2
                              bytes within 48 KB, m > 16: exactly 256).
                              VALU route: 0, or 4096 for m = 1 plans
                              without streaming whose tiles walk K in
                              4096-column segments                        */
  int32_t mx_packed8;      /* MFMA route, MX format: 1 when every GEMV's
                              exponent rows start 8-byte aligned
                              (ceil(k/32) % 8 == 0, 8-byte aligned array),
                              so its kernel reads 8 exponents per load;
                              0 otherwise                                  */
} fp8w_grouped_plan;

/* Bytes of device memory a table for `count` GEMVs needs (0 if count < 1). */
int64_t fp8w_grouped_table_bytes(int64_t count);

/* Set-up call (not for graph capture): validates every descriptor as the
 * single call would, rejects any output that overlaps another GEMV's
 * inputs or outputs, and writes the group's table into `device_table`
 * (caller-owned device memory of fp8w_grouped_table_bytes(count) bytes,
 * 16-byte aligned) with a blocking host-to-device copy.  The descriptors are
 * not retained.  Errors: NULL, SHAPE (count < 1, m out of range, too many
 * workgroups), ALIGN, UNSUPPORTED, OVERLAP, HIP. */
fp8w_status fp8w_grouped_plan_init(const fp8w_gemv_desc* descs, int64_t count, int64_t m,
                                   fp8w_format format, fp8w_route route, void* device_table,
                                   fp8w_grouped_plan* plan);

/* Enqueue every GEMV of the plan in one launch on `stream`.  Asynchronous,
 * allocation-free and safe to capture in a HIP graph; the buffers the
 * descriptors named must still be live.  Errors: NULL, SHAPE (a plan not
 * produced by fp8w_grouped_plan_init), HIP. */
fp8w_status fp8w_gemv_grouped(const fp8w_grouped_plan* plan, void* stream);

/* ---------------------------------------------------- grouped quantize -- */

/* Load-time quantization of many weights in one kernel launch: every bf16
 * weight of a checkpoint is requantized when it is loaded ("Load-time MXFP8
 * requantization of bf16 dense, hyper-connection and lm_head weights",
 * Proposed solution), and a launch per weight pays a fixed cost (about
 * 1.7 us on MI355X) that is as long as the whole of a small weight's pass.
 * One grouped launch streams the set as one large weight.  Each weight's
 * codes and scales are bit-identical to those of fp8w_quantize in the same
 * format.  Formats: BLOCK, BLOCK_BF16 and MX; ROW and TENSOR are
 * UNSUPPORTED. */
typedef struct fp8w_quant_desc {
  const uint16_t* w;     /* bf16 [n, k], 2-byte aligned              input  */
  uint8_t* codes;        /* e4m3fn [n, k]                             output */
  void* scales;          /* the format's scale buffer, aligned to its element
                            (f32 or bf16 block grid, e8m0 [n, ceil(k/32)]) output */
  int64_t n, k;          /* n, k >= 1                                        */
} fp8w_quant_desc;

/* What fp8w_quant_plan_init fills in; pass it to fp8w_quantize_grouped. */
typedef struct fp8w_quant_plan {
  const void* table;     /* the caller's device table buffer      */
  int32_t count;         /* weights in the group                  */
  int32_t format;        /* fp8w_format                           */
  int64_t blocks;        /* workgroups of one launch              */
} fp8w_quant_plan;

/* Bytes of device memory a table for `count` weights needs (0 if count < 1). */
int64_t fp8w_quant_table_bytes(int64_t count);

/* Set-up call (not for graph capture): validates every descriptor as
 * fp8w_quantize would, rejects any output that overlaps another output or
 * any input (the bf16 weights and the table), and writes the group's table
 * into `device_table` (caller-owned device memory of
 * fp8w_quant_table_bytes(count) bytes, 16-byte aligned) with a blocking
 * host-to-device copy.  The descriptors are not retained.
 * Errors: NULL, SHAPE (count < 1, n or k out of range, too many
 * workgroups), ALIGN, UNSUPPORTED (format), OVERLAP, HIP. */
fp8w_status fp8w_quant_plan_init(const fp8w_quant_desc* descs, int64_t count, fp8w_format format,
                                 void* device_table, fp8w_quant_plan* plan);

/* Enqueue the quantization of every weight of the plan in one launch on
 * `stream`.  Asynchronous, allocation-free and safe to capture in a HIP
 * graph; the buffers the descriptors named must still be live.
 * Errors: NULL, SHAPE (a plan not produced by fp8w_quant_plan_init), HIP. */
fp8w_status fp8w_quantize_grouped(const fp8w_quant_plan* plan, void* stream);

/* ------------------------------------------------------------- helpers -- */

/* Number of fp32 block scales for [n, k]: ceil(n/128) * ceil(k/128); 0 if
 * n < 1 or k < 1. */
int64_t fp8w_block_scale_count(int64_t n, int64_t k);

/* Number of e8m0 bytes for [n, k]: n * ceil(k/32); 0 if n < 1 or k < 1. */
int64_t fp8w_mx_scale_count(int64_t n, int64_t k);

/* Measurement aid, not part of the method: read `bytes` of device memory
 * at `buf` once, as the GEMV reads its weight stream (16-byte non-temporal
 * loads over a grid sized to the chip), and write one 32-bit XOR of the
 * data per workgroup to `out`.  The rate of this call is the practical HBM
 * read ceiling that the weight-streaming kernels are compared with, beside
 * the published peak.  `out` holds `out_words` words (caller-owned device
 * memory); the grid is min(out_words, ceil(bytes / 32768)) workgroups, and
 * 2048 words fill MI355X.  Asynchronous, allocation-free.  Errors: NULL,
 * SHAPE (bytes < 16, bytes % 16 != 0, out_words < 1), ALIGN (buf not
 * 16-byte or out not 4-byte aligned), OVERLAP, HIP. */
fp8w_status fp8w_read_ceiling(const void* buf, int64_t bytes, uint32_t* out, int64_t out_words,
                              void* stream);

/* Static, NUL-terminated name of a status code. */
const char* fp8w_status_string(fp8w_status status);

/* Library version, as major * 10000 + minor * 100 + patch. */
int fp8w_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8W_H_ */
