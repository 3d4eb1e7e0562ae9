/*
 * woq.h - group-wise 4-bit weight-only linear layers on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libwoq.so.  Every pointer argument is a plain address: "device"
 * pointers are HIP device memory (for example from hipMalloc or a PyTorch
 * tensor's data_ptr()), "host" pointers are ordinary process memory.  Sizes
 * are element counts unless a name ends in _bytes.  All tensors are dense and
 * row-major.  The caller owns every buffer; the library keeps no pointer after
 * a call returns.
 *
 * Streams: `stream` is a hipStream_t passed as void* (NULL = the legacy
 * default stream).  Calls marked ASYNC only enqueue work on that stream and
 * return; results are ready when the stream reaches them.  Calls marked SYNC
 * wait for their own work on that stream before returning.
 *
 * Errors: every entry point validates its arguments on the host before it
 * enqueues anything and returns a woq_status.  A call that returns anything
 * but WOQ_OK because of an argument check has enqueued nothing and written
 * nothing.  Data-dependent errors (WOQ_ENONFINITE, WOQ_ERANGE) are found on
 * the device; the outputs of such a call are then unspecified.
 *
 * Weight layout (linnet docs "Quantization", std.quant table, row
 * Int4GroupLinear; section "Group-wise 4-bit weights"): for a weight W[N, K]
 * (N outputs, K inputs) and a group size G dividing K,
 *   packed [N, K/G, G/2] uint8  - two 4-bit codes per byte, the code of the
 *                                 even input in the low nibble, the odd one in
 *                                 the high nibble (the packing sentence of the
 *                                 same page);
 *   scale  [N, K/G] float32;
 *   zero   [N, K/G] uint8      - each 0..15;
 * and W_hat[n, k] = (q[n, k] - zero[n, k/G]) * scale[n, k/G].
 */
#ifndef WOQ_H
#define WOQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  WOQ_OK = 0,
  WOQ_EINVAL = 1,        /* a required pointer is NULL, a size is negative, an enum is unknown */
  WOQ_ESHAPE = 2,        /* sizes inconsistent with each other (odd count, K odd, ...) */
  WOQ_EGROUP = 3,        /* group < 1, group does not divide K, or odd where the layout needs even */
  WOQ_ENONFINITE = 4,    /* a weight is NaN or infinite (data-dependent) */
  WOQ_ERANGE = 5,        /* a code exceeds 15 (data-dependent) */
  WOQ_EWORKSPACE = 6,    /* workspace missing or smaller than woq_linear_workspace_bytes() */
  WOQ_EUNSUPPORTED = 7,  /* valid input this build has no kernel for (group size, sizes >= 2^31) */
  WOQ_EALIGN = 8,        /* a pointer lacks the alignment stated for it below */
  WOQ_EHIP = 9,          /* the HIP runtime reported an error */
  WOQ_ENOTPD = 10        /* GPTQ: the damped calibration matrix is not positive definite (data-dependent) */
} woq_status;

typedef enum { WOQ_F32 = 0, WOQ_BF16 = 1 } woq_dtype;

/* Short English description of a status code (static storage, never NULL). */
const char* woq_status_str(int32_t status);

/* Library version as major*10000 + minor*100 + patch. */
int32_t woq_version(void);

/*
 * Group quantizer, round to nearest with ties to even.  SYNC.
 *   Asymmetric (symmetric = 0): the GPTQ/AWQ-style scheme with a zero point
 *     ("4.8 Quantization II", section "Per-Group INT4": unsigned codes 0..15
 *     with a zero point; linnet "Quantization", section "Group-wise 4-bit
 *     weights").  Per group: range = max - min (float64);
 *     scale = float32(range / 15); zero = clamp(rint(-15*min/range), 0, 15);
 *     q = clamp(rint(15*w/range) + zero, 0, 15).  A group with range 0 gets
 *     scale 1, zero = clamp(rint(-min), 0, 15), q = clamp(rint(w) + zero, 0, 15)
 *     (an all-zero group gets scale 1: "20. Quantization", the edge cases
 *     after quantize_groupwise).
 *   Symmetric (symmetric = 1): "20. Quantization", section "Symmetric
 *     quantization, from scratch", with Q = 7: a = max|w|;
 *     scale = float32(a / 7); c = clamp(rint(7*w/a), -7, 7); stored unsigned as
 *     q = c + 8 with zero = 8.  An all-zero group gets scale 1 and c = 0.
 *   Every quotient is one correctly rounded float64 division of the exact
 *   operands, so the rounding decision is taken on the real quotient.
 * Arguments: w [n, k] float32 (device, 4-byte aligned); group >= 1 divides k;
 *   outputs q [n, k] uint8 (codes, unpacked), scale [n, k/group] float32,
 *   zero [n, k/group] uint8 (device).
 * Errors: WOQ_EINVAL, WOQ_EGROUP, WOQ_ENONFINITE (any NaN or infinity in w),
 *   WOQ_EUNSUPPORTED (n*k >= 2^40), WOQ_EHIP.
 */
int32_t woq_quantize_groups(const float* w, int64_t n, int64_t k, int32_t group,
                            int32_t symmetric, uint8_t* q, float* scale, uint8_t* zero,
                            void* stream);

/*
 * Pack 4-bit codes two per byte: packed[i] = q[2i] | q[2i+1] << 4 (linnet
 * "Quantization", packing sentence; tinyllm L8.5 section 2 "Principles",
 * Packing).  SYNC (it reports codes above 15).
 * Arguments: q [count] uint8 (device), count even; packed [count/2] uint8 (device).
 * Errors: WOQ_EINVAL, WOQ_ESHAPE (odd count), WOQ_ERANGE (a code > 15), WOQ_EHIP.
 */
int32_t woq_pack_uint4(const uint8_t* q, int64_t count, uint8_t* packed, void* stream);

/*
 * Unpack unsigned nibbles: q[2i] = packed[i] & 15, q[2i+1] = packed[i] >> 4
 * (linnet "Quantization", std.quant table, unpack_uint4).  ASYNC.
 * Arguments: packed [count/2] uint8 (device); count even; q [count] uint8 (device).
 * Errors: WOQ_EINVAL, WOQ_ESHAPE (odd count), WOQ_EHIP.
 */
int32_t woq_unpack_uint4(const uint8_t* packed, int64_t count, uint8_t* q, void* stream);

/*
 * Group dequantization W_hat = (q - zero) * scale (linnet "Quantization",
 * std.quant table, dequantize_int4_groups).  The product is formed in float32
 * (one rounding of the exact value); with out_dtype = WOQ_BF16 that float32 is
 * then rounded to bfloat16, ties to even.  ASYNC.
 * Arguments: packed [n, k/2] uint8, scale [n, k/group] float32,
 *   zero [n, k/group] uint8 (device); group even, divides k;
 *   w_hat [n, k] of out_dtype (device).
 * Errors: WOQ_EINVAL, WOQ_EGROUP, WOQ_EUNSUPPORTED (n*k >= 2^40), WOQ_EHIP.
 */
int32_t woq_dequantize_int4_groups(const uint8_t* packed, const float* scale,
                                   const uint8_t* zero, int64_t n, int64_t k, int32_t group,
                                   int32_t out_dtype, void* w_hat, void* stream);

/*
 * Workspace the linear layer needs for these sizes, in bytes (0 when none).
 * Pure host function.  has_order != 0 when an act-order gather will be passed.
 */
size_t woq_linear_workspace_bytes(int64_t m, int64_t n, int64_t k, int32_t group,
                                  int32_t has_order);

/*
 * Linear layer over group-wise 4-bit weights (linnet "Quantization", std.quant
 * table, linear_int4_groups; section "Importing GPTQ and AWQ" for the
 * act-order gather):
 *   y[m, n] = sum_k x'[m, k] * W_hat[n, k] + bias[n],
 *   x'[m, k] = order ? x[m, order[k]] : x[m, k].
 * x is bfloat16; products and sums are float32; the sum over each group is
 * multiplied by that group's scale in float32; bias is added in float32; a
 * bfloat16 y is rounded once from that float32 value, ties to even.  Where
 * woq_linear_plan reports k_splits > 1 (the tiled GEMM on narrow layers), K is
 * cut into that many ranges whose float32 partial sums go through the
 * workspace and are added in range order (the same result on every run).
 * ASYNC.
 * Arguments:
 *   x_bf16 [m, k] bfloat16 (device, 16-byte aligned);
 *   packed [n, k/2] uint8 (device, 16-byte aligned); scale [n, k/group] float32
 *   (device, 16-byte aligned); zero [n, k/group] uint8 (device, 16-byte aligned);
 *   bias [n] float32 (device) or NULL; order [k] int32 (device, 16-byte
 *   aligned) or NULL - every
 *   entry must lie in [0, k) (entries outside are clamped into range, never read
 *   out of bounds; the result is then unspecified);
 *   group in {32, 64, 128, 256}, dividing k;
 *   y [m, n] of y_dtype (device, 4-byte aligned for float32, 2-byte for bfloat16),
 *   which must not overlap any input;
 *   workspace (device, 256-byte aligned) of at least
 *   woq_linear_workspace_bytes(m, n, k, group, order != NULL) bytes, or NULL
 *   when that is 0.  The workspace holds only scratch; it need not be cleared.
 * m == 0 or n == 0 is a no-op; k == 0 gives y = bias (or 0).
 * Errors: WOQ_EINVAL, WOQ_EGROUP, WOQ_EUNSUPPORTED (group outside the list,
 *   m, n or k >= 2^31, or k >= 2^24 on the tiled GEMM path: m > 128, or
 *   m > 64 on layers of fewer than 800 16-row tiles), WOQ_EALIGN,
 *   WOQ_EWORKSPACE, WOQ_EHIP.
 */
int32_t woq_linear_int4_groups(const void* x_bf16, int64_t m, const uint8_t* packed,
                               const float* scale, const uint8_t* zero, const float* bias,
                               const int32_t* order, int64_t n, int64_t k, int32_t group,
                               int32_t y_dtype, void* y, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * Prepared weights.  The linnet "Quantization" page runs its fused int4
 * kernels on weights re-ordered once at load time ("--prepare"); the order is
 * not given there, and the one below is this library's: the layout of a
 * 16x16x32 MFMA operand, so that one 16-byte load per lane fills a fragment
 * and a wave reads each 128-input step of 16 outputs as one contiguous
 * kilobyte.
 *   For W[n, k] (k a multiple of 32): blocks of 16 outputs x 128 inputs, 1024
 *   bytes each, ordered tile t = 0 .. ceil(n/16)-1, then step
 *   s = 0 .. ceil(k/128)-1 inside a tile; 16-byte slot l (0..63) of block
 *   (t, s) holds output row 16t + l % 16, packed bytes 64 s + 16 (l / 16) ..
 *   +16 of that row (inputs 128 s + 32 (l / 16) .. +32, nibbles as in the
 *   canonical layout).  Rows past n and bytes past k/2 are zero.
 *   Scale and zero keep the canonical [n, k/group] layout.
 * woq_prepared_bytes: size of that layout, ceil(n/16) * ceil(k/128) * 1024;
 *   0 for invalid sizes (negative, k not a multiple of 32, n or k >= 2^31).
 *   Pure host function.
 */
size_t woq_prepared_bytes(int64_t n, int64_t k);

/*
 * Canonical packed [n, k/2] -> prepared layout (above).  ASYNC.
 * Arguments: packed (device, 16-byte aligned); prepared (device, 16-byte
 *   aligned) of woq_prepared_bytes(n, k) bytes; the two must not overlap.
 * Errors: WOQ_EINVAL (negative size, NULL pointer), WOQ_ESHAPE (k not a
 *   multiple of 32), WOQ_EUNSUPPORTED (n or k >= 2^31, n*k >= 2^40),
 *   WOQ_EALIGN, WOQ_EHIP.
 */
int32_t woq_prepare_int4(const uint8_t* packed, int64_t n, int64_t k, uint8_t* prepared,
                         void* stream);

/*
 * Prepared layout -> canonical packed [n, k/2] (the inverse, for validation and
 * export).  ASYNC.  Same arguments and errors as woq_prepare_int4.
 */
int32_t woq_unprepare_int4(const uint8_t* prepared, int64_t n, int64_t k, uint8_t* packed,
                           void* stream);

/*
 * woq_linear_int4_groups without a caller workspace and without allocating:
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid it).  The workspace is a
 * fixed device array of woq_linear_noalloc_max_workspace_bytes() bytes
 * (32 MiB) inside the library; every device the library runs on holds its own
 * copy until the process ends.  ASYNC.
 * Arguments, results and errors: as woq_linear_int4_groups without workspace
 * and workspace_bytes.  Where woq_linear_workspace_bytes exceeds the array
 * because the plan splits K (its float32 partial outputs), the call runs the
 * same tiles with K whole instead (slower on narrow layers, equal up to float32
 * summation order); sizes whose workspace exceeds the array even then return
 * WOQ_EWORKSPACE before anything is enqueued (for example m = 2048 with
 * k = 14336).
 * Calls that overlap on one device (concurrent streams, or host threads) share
 * that device's array and race: serialize them.  The array keeps the last
 * call's contents; nothing in it needs to start cleared.
 */
size_t woq_linear_noalloc_max_workspace_bytes(void);
int32_t woq_linear_int4_groups_noalloc(const void* x_bf16, int64_t m, const uint8_t* packed,
                                       const float* scale, const uint8_t* zero, const float* bias,
                                       const int32_t* order, int64_t n, int64_t k, int32_t group,
                                       int32_t y_dtype, void* y, void* stream);

/*
 * woq_linear_int4_groups over prepared weights: identical arguments, results
 * and errors, except that `prepared` (device, 16-byte aligned, at least
 * woq_prepared_bytes(n, k) bytes) replaces `packed`.  The result equals that
 * of woq_linear_int4_groups on the canonical weights the buffer was prepared
 * from.  woq_linear_workspace_bytes and woq_linear_plan apply unchanged.
 */
int32_t woq_linear_int4_groups_prepared(const void* x_bf16, int64_t m, const uint8_t* prepared,
                                        const float* scale, const uint8_t* zero,
                                        const float* bias, const int32_t* order, int64_t n,
                                        int64_t k, int32_t group, int32_t y_dtype, void* y,
                                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Several linear layers over the same activations in one call (for example the
 * q, k and v projections of an attention block, or the gate and up projections
 * of an MLP): for i < count,
 *   y[i][m, n[i]] = x[m, k] . W_hat_i^T + bias[i],
 * each exactly as woq_linear_int4_groups (or, with prepared = 1,
 * woq_linear_int4_groups_prepared) would compute it with the same launch plan;
 * results agree with the separate calls within floating-point rounding (the
 * grouped call plans for the summed row count).  At m <= 4 all the matrices
 * share one decode launch, which saves a kernel launch per extra matrix;
 * other m run the matrices one after another.  ASYNC.
 * Arguments:
 *   x_bf16 [m, k] bfloat16 (device, 16-byte aligned), shared by every matrix;
 *   count in 1 .. 4;
 *   packed, scale, zero, y: host arrays of count device pointers, element i
 *     laid out and aligned as in woq_linear_int4_groups for n[i] rows
 *     (packed[i] holds the prepared layout when prepared = 1);
 *   bias: host array of count device pointers (an element may be NULL), or NULL;
 *   n: host array of count row counts; k, group, y_dtype as in
 *     woq_linear_int4_groups;
 *   workspace of at least the largest woq_linear_workspace_bytes(m, n[i], k,
 *     group, 0), or NULL when that is 0.
 *   No output may overlap an input or another output.  The act-order gather is
 *   not offered here.
 * Errors: as woq_linear_int4_groups for each matrix, checked for all of them
 *   before anything is enqueued; WOQ_EINVAL for count outside 1 .. 4, NULL
 *   arrays or prepared not 0 or 1.
 */
int32_t woq_linear_int4_groups_grouped(const void* x_bf16, int64_t m, int32_t count,
                                       const uint8_t* const* packed, const float* const* scale,
                                       const uint8_t* const* zero, const float* const* bias,
                                       const int64_t* n, int64_t k, int32_t group,
                                       int32_t prepared, int32_t y_dtype, void* const* y,
                                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * ---- Signed int4 groups with float16 scales ----
 * The int4 group format of tinyllm L8.5 ("Quantization: int8, int4 group
 * (packed), fp8, KV quant", section 2 "Principles", "int4 per group" and
 * "Packing"): symmetric codes c in -8..7 stored as 4-bit two's complement,
 * two per byte with the even input in the low nibble, [n, k/2] uint8; one
 * float16 scale per group of `group` consecutive inputs, [n, k/group]; no zero
 * point.  W_hat = c * scale.
 */

/*
 * Quantizer.  SYNC (it reports bad weights).  Per group: amax = max|w|;
 * s16 = float16(amax / 7), the quotient a float32 division then rounded to
 * float16, ties to even; c = clamp(rint(w / s16), -8, 7), the quotient a
 * float32 division against the stored float16 value, ties to even.  A group
 * whose s16 is 0 (all zero, or amax / 7 below float16's smallest subnormal)
 * gets codes 0 and scale 0.
 * Arguments: w [n, k] float32 (device, 4-byte aligned); group even, divides k;
 *   outputs codes [n, k] int8 (device), scale16 [n, k/group] float16 bits
 *   (device, 2-byte aligned).
 * Errors: WOQ_EINVAL, WOQ_EGROUP, WOQ_ENONFINITE (a NaN or infinity in w),
 *   WOQ_ERANGE (an s16 that overflows float16), WOQ_EUNSUPPORTED (n*k >= 2^40),
 *   WOQ_EHIP.  On an error the outputs of the offending groups are not written.
 */
int32_t woq_quantize_int4_sym_f16(const float* w, int64_t n, int64_t k, int32_t group,
                                  int8_t* codes, uint16_t* scale16, void* stream);

/*
 * Pack signed codes two per byte: packed[i] = (c[2i] & 15) | (c[2i+1] & 15) << 4.
 * SYNC (it reports codes outside -8..7).
 * Arguments: codes [count] int8 (device), count even; packed [count/2] uint8 (device).
 * Errors: WOQ_EINVAL, WOQ_ESHAPE (odd count), WOQ_ERANGE (a code outside -8..7), WOQ_EHIP.
 */
int32_t woq_pack_int4(const int8_t* codes, int64_t count, uint8_t* packed, void* stream);

/*
 * Unpack signed nibbles, each sign-extended (a nibble v >= 8 is v - 16).  ASYNC.
 * Arguments: packed [count/2] uint8 (device); count even; codes [count] int8 (device).
 * Errors: WOQ_EINVAL, WOQ_ESHAPE (odd count), WOQ_EHIP.
 */
int32_t woq_unpack_int4(const uint8_t* packed, int64_t count, int8_t* codes, void* stream);

/*
 * Dequantize W_hat = c * s16, exact in float32; with out_dtype = WOQ_BF16 that
 * float32 is rounded to bfloat16, ties to even.  ASYNC.
 * Arguments: packed [n, k/2] uint8, scale16 [n, k/group] float16 bits (device,
 *   2-byte aligned); group even, divides k; w_hat [n, k] of out_dtype (device).
 * Errors: WOQ_EINVAL, WOQ_EGROUP, WOQ_EUNSUPPORTED (n*k >= 2^40), WOQ_EHIP.
 */
int32_t woq_dequantize_int4_sym_f16(const uint8_t* packed, const uint16_t* scale16, int64_t n,
                                    int64_t k, int32_t group, int32_t out_dtype, void* w_hat,
                                    void* stream);

/*
 * Linear layer over signed int4 groups with float16 scales:
 *   y[m, n] = sum_k x'[m, k] * c[n, k] * s16[n, k / group] + bias[n],
 *   x'[m, k] = order ? x[m, order[k]] : x[m, k].
 * The same kernels, paths, workspace (woq_linear_workspace_bytes), plan
 * (woq_linear_plan), float32 arithmetic and error bound as
 * woq_linear_int4_groups: a signed nibble v is read as the unsigned code v ^ 8
 * with zero point 8, so each group is folded as scale * (sum - 8 * sum of x).
 * ASYNC.
 * Arguments: as woq_linear_int4_groups, with scale16 [n, k/group] float16 bits
 *   (device, 16-byte aligned) in place of scale and zero.
 * Errors: as woq_linear_int4_groups.
 */
int32_t woq_linear_int4_sym_f16(const void* x_bf16, int64_t m, const uint8_t* packed,
                                const uint16_t* scale16, const float* bias, const int32_t* order,
                                int64_t n, int64_t k, int32_t group, int32_t y_dtype, void* y,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * woq_linear_int4_sym_f16 over weights prepared with woq_prepare_int4 (the
 * byte order of the prepared layout does not depend on what the nibbles mean).
 * Arguments, results and errors as woq_linear_int4_sym_f16, with `prepared`
 * (device, 16-byte aligned, woq_prepared_bytes(n, k) bytes) replacing `packed`.
 */
int32_t woq_linear_int4_sym_f16_prepared(const void* x_bf16, int64_t m, const uint8_t* prepared,
                                         const uint16_t* scale16, const float* bias,
                                         const int32_t* order, int64_t n, int64_t k, int32_t group,
                                         int32_t y_dtype, void* y, void* workspace,
                                         size_t workspace_bytes, void* stream);

/*
 * ---- Int4Linear: signed int4 with one float32 scale a row ----
 * linnet "Quantization", std.quant table: Int4Linear weight [Out, In/2] of
 * signed 4-bit codes (two's complement nibbles, the even input in the low
 * nibble) and, as the page's Mlp example declares, scale [Out] float32;
 * dequantize_int4 = unpack, then dequantize: W_hat = c * scale[row].
 */

/*
 * Quantizer (tinyllm L8.5 section 2, symmetric scaling with q_max = 7 and one
 * scale a row).  SYNC.  s = amax / 7 (a float32 division); c = clamp(rint(w / s),
 * -8, 7), the quotient a float32 division, ties to even; a zero row gets s = 0
 * and codes 0.
 * Arguments: w [n, k] float32 (device, 4-byte aligned), k even; outputs codes
 *   [n, k] int8 (pack with woq_pack_int4), scale [n] float32 (device, 4-byte
 *   aligned).
 * Errors: WOQ_EINVAL, WOQ_ESHAPE (odd k), WOQ_ENONFINITE, WOQ_EUNSUPPORTED
 *   (n*k >= 2^40), WOQ_EHIP.
 */
int32_t woq_quantize_int4_rows(const float* w, int64_t n, int64_t k, int8_t* codes, float* scale,
                               void* stream);

/*
 * Dequantize W_hat = c * scale[row], rounded once to float32; with
 * out_dtype = WOQ_BF16 that float32 is rounded to bfloat16.  ASYNC.
 * Arguments: packed [n, k/2] uint8, scale [n] float32 (device); w_hat [n, k].
 * Errors: WOQ_EINVAL, WOQ_ESHAPE (odd k), WOQ_EUNSUPPORTED, WOQ_EHIP.
 */
int32_t woq_dequantize_int4_rows(const uint8_t* packed, const float* scale, int64_t n, int64_t k,
                                 int32_t out_dtype, void* w_hat, void* stream);

/*
 * Workspace woq_linear_int4_rows needs (0 when none).  Pure host function.
 */
size_t woq_linear_int4_rows_workspace_bytes(int64_t m, int64_t n, int64_t k, int32_t has_order);

/*
 * Linear layer over Int4Linear weights:
 *   y[m, n] = sum_k x'[m, k] * c[n, k] * scale[n] + bias[n],
 *   x'[m, k] = order ? x[m, order[k]] : x[m, k].
 * The kernels of woq_linear_int4_sym_f16, run in groups of the largest of 256,
 * 128, 64 and 32 that divides k, every group with the row's scale.  ASYNC.
 * Arguments: as woq_linear_int4_groups, with scale [n] float32 (device, 16-byte
 *   aligned) in place of scale and zero and no group; k a multiple of 32;
 *   workspace of woq_linear_int4_rows_workspace_bytes bytes.
 * Errors: as woq_linear_int4_groups; WOQ_ESHAPE for odd k, WOQ_EUNSUPPORTED for
 *   k not a multiple of 32.
 */
int32_t woq_linear_int4_rows(const void* x_bf16, int64_t m, const uint8_t* packed, const float* scale,
                             const float* bias, const int32_t* order, int64_t n, int64_t k,
                             int32_t y_dtype, void* y, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * ---- MXFP4 ----
 * linnet "Quantization" (std.quant table, dequantize_mxfp4: E2M1 values in
 * blocks of 32, one E8M0 scale byte a block) and tinyllm L8.5 section 2
 * ("MXFP4": a power-of-two scale X per block, elements 0, 0.5, 1, 1.5, 2, 3, 4, 6
 * times X, values above 6X saturate).  Layout: blocks [n, k/32, 16] uint8, two
 * E2M1 codes a byte (bit 3 the sign), the even input in the low nibble; scales
 * [n, k/32] uint8, X = 2^(e - 127).  W_hat = value(code) * X.
 */

/*
 * Quantizer.  SYNC.  Per block of 32: X = 2^(floor(log2 amax) - 2) (the OCP
 * Microscaling rule; 2 is the largest E2M1 exponent), e = clamp(floor(log2 amax)
 * - 2 + 127, 0, 254), e = 0 for a zero block; each element w / X (exact) rounds
 * to the nearest E2M1 magnitude, ties to the even code, saturating at 6, with the
 * sign of w (a negative value that rounds to 0 gives code 8).
 * Arguments: w [n, k] float32 (device, 4-byte aligned), k a multiple of 32;
 *   outputs codes [n, k] uint8 (0..15, pack them with woq_pack_uint4), scales
 *   [n, k/32] uint8 (device).
 * Errors: WOQ_EINVAL, WOQ_EGROUP (k not a multiple of 32), WOQ_ENONFINITE,
 *   WOQ_EUNSUPPORTED (n*k >= 2^40), WOQ_EHIP.
 */
int32_t woq_quantize_mxfp4(const float* w, int64_t n, int64_t k, uint8_t* codes, uint8_t* scales,
                           void* stream);

/*
 * Dequantize W_hat = value(code) * 2^(e - 127), exact in float32 for the scales
 * the quantizer writes; with out_dtype = WOQ_BF16 that float32 is rounded to
 * bfloat16, ties to even.  ASYNC.
 * Arguments: blocks [n, k/2] uint8, scales [n, k/32] uint8 (device); k a
 *   multiple of 32; w_hat [n, k] of out_dtype (device).
 * Errors: WOQ_EINVAL, WOQ_EGROUP, WOQ_EUNSUPPORTED (n*k >= 2^40), WOQ_EHIP.
 */
int32_t woq_dequantize_mxfp4(const uint8_t* blocks, const uint8_t* scales, int64_t n, int64_t k,
                             int32_t out_dtype, void* w_hat, void* stream);

/*
 * Linear layer over MXFP4 weights: y[m, n] = sum_k x[m, k] * W_hat[n, k] + bias[n].
 * x bfloat16, float32 accumulation.  Each lane's 16 weight bytes are one block,
 * converted with v_cvt_scalef32_pk_bf16_fp4 into bf16 values already multiplied
 * by the block's scale (exact: a power of two times a 2-bit significand), so
 * the products go straight into the MFMA accumulators: m <= 32 on the small-M
 * kernel, larger m on the tiled GEMM (with its activation pre-pass; workspace as
 * woq_linear_workspace_bytes(m, n, k, 32, 0)).  A block scale of 255 (not a
 * number in E8M0) gives NaN outputs.  ASYNC.
 * Arguments: x_bf16 [m, k] bfloat16 (device, 16-byte aligned); blocks [n, k/2]
 *   uint8 (device, 16-byte aligned); scales [n, k/32] uint8 (device, 16-byte
 *   aligned); bias [n] float32 or NULL; k a multiple of 32; y_dtype, y,
 *   workspace as woq_linear_int4_groups.
 * Errors: as woq_linear_int4_groups with group 32.
 */
int32_t woq_linear_mxfp4(const void* x_bf16, int64_t m, const uint8_t* blocks, const uint8_t* scales,
                         const float* bias, int64_t n, int64_t k, int32_t y_dtype, void* y,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * ---- Packed 4-bit zero points ----
 * linnet "Quantization": Int4GroupLinear's layout is ONNX Runtime's
 * MatMulNBits, whose zero points are 4-bit values two a byte.  Per row, the
 * zero points of groups 2j and 2j+1 share byte j, group 2j in the low nibble;
 * a row with an odd number of groups ends in a byte whose high nibble is 0
 * (ignored when read).  Packed size: n * ceil(ngroups / 2) bytes.
 */

/*
 * zero [n, ngroups] uint8 (0..15) -> zero_packed [n, ceil(ngroups/2)] (device,
 * no alignment needed).  SYNC.
 * Errors: WOQ_EINVAL, WOQ_ERANGE (a value above 15; the output is then
 *   undefined), WOQ_EUNSUPPORTED (n*ngroups >= 2^40), WOQ_EHIP.
 */
int32_t woq_pack_zero_points(const uint8_t* zero, int64_t n, int64_t ngroups, uint8_t* zero_packed,
                             void* stream);

/*
 * Inverse of woq_pack_zero_points: zero_packed [n, ceil(ngroups/2)] -> zero
 * [n, ngroups] uint8 (device).  ASYNC.  Load-time use: unpack once and call
 * woq_linear_int4_groups, which then costs nothing extra per call.
 * Errors: WOQ_EINVAL, WOQ_EUNSUPPORTED, WOQ_EHIP.
 */
int32_t woq_unpack_zero_points(const uint8_t* zero_packed, int64_t n, int64_t ngroups, uint8_t* zero,
                               void* stream);

/*
 * woq_linear_int4_groups with packed zero points: the row-streaming, small-M
 * and GEMM kernels read the nibbles where they read zero bytes otherwise (no
 * extra launch); only the tile GEMV (m <= 4 when the WOQ_DECODE_MFMA tuning
 * variable is set) first unpacks them into the head of the workspace.  Arguments, results and errors as
 * woq_linear_int4_groups, with zero_packed [n, ceil((k/group)/2)] uint8
 * (device, no alignment needed) replacing zero, and a workspace (256-byte
 * aligned) of woq_linear_int4_groups_zp4_workspace_bytes() bytes (may be 0).
 * Results are bit-identical to woq_linear_int4_groups over the unpacked zero
 * points.
 */
int32_t woq_linear_int4_groups_zp4(const void* x_bf16, int64_t m, const uint8_t* packed, const float* scale,
                                   const uint8_t* zero_packed, const float* bias, const int32_t* order, int64_t n,
                                   int64_t k, int32_t group, int32_t y_dtype, void* y, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * Workspace woq_linear_int4_groups_zp4 needs: woq_linear_workspace_bytes(...),
 * plus the unpacked zero points (n * k/group bytes rounded up to 256) when the
 * call runs on the tile GEMV.  Pure host function; 0 for invalid shapes or an
 * empty problem.
 */
size_t woq_linear_int4_groups_zp4_workspace_bytes(int64_t m, int64_t n, int64_t k, int32_t group,
                                                  int32_t has_order);

/*
 * ---- GPTQ: error-compensating quantization of one layer ----
 * "20. Quantization" (inference book), stretch exercise 4: H = 2 X^T X from
 * calibration inputs; the columns are quantized one at a time and each
 * column's error is spread over the columns not yet quantized through the
 * Cholesky factor of H^-1.  linnet "Importing GPTQ and AWQ": quantized in
 * activation order, the layer keeps an `order` it gathers its inputs through.
 * The steps the pages leave open follow the published method (Frantar et al.):
 *   - columns with H_jj = 0 get H_jj = 1 and their weights set to 0;
 *   - act_order visits the columns by decreasing H_jj (stable: equal H_jj keep
 *     column order);
 *   - H += damp * mean(diag H) * I; U = upper Cholesky factor of H^-1;
 *   - a group's (scale, zero) come from its current (already updated) weights
 *     when its first column comes up, by the asymmetric rule of
 *     woq_quantize_int4_groups (scale = float32(range / 15), zero =
 *     clamp(rint(-15 min / range), 0, 15));
 *   - code = clamp(rint(15 w / range) + zero, 0, 15); err = (w - (code - zero) *
 *     scale) / U_ii; the later weights w_j -= err * U_ij.
 * All arithmetic is float64 on the device.  SYNC (allocates and frees its
 * float64 working set: 3 K^2 + (N + 2) K + 256 N doubles).
 * Arguments: w [n, k] float32 (device, 4-byte aligned); x_bf16 [t, k] bfloat16
 *   calibration inputs (device, may be NULL when t = 0); group divides k, at
 *   most 256; act_order 0 or 1; damp >= 0 (0.01 in the method).
 *   Outputs (device): codes [n, k] uint8 in 0..15, scale [n, k/group] float32
 *   (4-byte aligned), zero [n, k/group] uint8, all with their columns in
 *   visiting order (pack the codes with woq_pack_uint4); order [k] int32
 *   (4-byte aligned), written only when act_order = 1 (the visiting order, to
 *   pass to the linear calls), may be NULL otherwise.
 * Errors: WOQ_EINVAL (NULL pointer, negative size, act_order not 0/1, damp
 *   negative or not finite), WOQ_EGROUP (group < 1 or not dividing k),
 *   WOQ_EUNSUPPORTED (group > 256, k >= 2^20), WOQ_ENONFINITE (a weight NaN or
 *   infinite), WOQ_ENOTPD (a Cholesky pivot of the damped, reordered matrix
 *   is not positive or its root is not finite: damp = 0 with fewer
 *   calibration rows than inputs can do this; codes, scales and zeros are
 *   then unspecified), WOQ_EALIGN, WOQ_EHIP.
 */
int32_t woq_gptq_quantize(const float* w, const void* x_bf16, int64_t t, int64_t n, int64_t k, int32_t group,
                          int32_t act_order, double damp, uint8_t* codes, float* scale, uint8_t* zero,
                          int32_t* order, void* stream);

/*
 * ---- AWQ: activation-aware scale search for one layer ----
 * "20. Quantization" (inference book), stretch exercise 3: a per-input-channel
 * scale s_j = mean|x_j|^alpha, alpha searched over [0, 1] for the least
 * calibration output error after 4-bit quantization of W diag(s); the page's
 * scaling identity X W^T = (X S^-1)(W S)^T: the scaled layer computes with
 * X S^-1, which the caller folds into the operation that produces x.
 *   - alpha = i / n_grid for i = 0 .. n_grid (20 in the published method);
 *   - s_j = float32(max(mean_t |x_tj|^alpha, 1e-4));
 *   - the scaled weights float32(w * s) are quantized by the asymmetric group
 *     rule of woq_quantize_int4_groups;
 *   - the error of a grid point is ||X (W - W_hat)^T||_F^2 with
 *     W_hat = (q - zero) * scale / s, in float64; the first least error wins.
 * SYNC (allocates and frees its working set: about 9 bytes per weight).
 * Arguments: w [n, k] float32 (device, 4-byte aligned); x_bf16 [t, k] bfloat16
 *   calibration inputs (device, t >= 1); group divides k; n_grid in 1..1000.
 *   Outputs (device): codes [n, k] uint8 0..15, scale [n, k/group] float32,
 *   zero [n, k/group] uint8 of the scaled weights at the chosen alpha (pack the
 *   codes with woq_pack_uint4); s [k] float32 (4-byte aligned); losses
 *   [n_grid + 1] float64 (8-byte aligned), the error of every grid point, or
 *   NULL; best (host) the chosen grid index, or NULL.
 * Errors: WOQ_EINVAL (NULL pointer, negative size, t < 1, n_grid out of
 *   range), WOQ_EGROUP, WOQ_EUNSUPPORTED (sizes >= 2^31, t >= 2^25),
 *   WOQ_ENONFINITE (a scaled weight NaN or infinite), WOQ_EALIGN, WOQ_EHIP.
 */
int32_t woq_awq_search(const float* w, const void* x_bf16, int64_t t, int64_t n, int64_t k, int32_t group,
                       int32_t n_grid, uint8_t* codes, float* scale, uint8_t* zero, float* s, double* losses,
                       int32_t* best, void* stream);

/*
 * Describe the kernel plan the linear calls use for these sizes: the path
 * (row-streaming decode "rows_dot2" for m <= 4 over canonical weights, tile
 * GEMV "gemv_mfma" for prepared weights at m <= 4; small-M MFMA
 * "skinny_mfma" up to 64 rows, and up to 128 on layers of at least 800
 * 16-row tiles; tiled MFMA GEMM "gemm_mfma" above), tiles, waves, the
 * number of K ranges of a split tiled GEMM (k_splits) and which input
 * pre-pass runs.  Writes a NUL-terminated
 * string of at most len bytes into buf (host).  Pure host function.
 * Errors: WOQ_EINVAL (buf NULL, len 0), plus the shape errors of the linear call.
 */
int32_t woq_linear_plan(int64_t m, int64_t n, int64_t k, int32_t group, int32_t has_order,
                        char* buf, size_t len);

#ifdef __cplusplus
}
#endif

#endif /* WOQ_H */
