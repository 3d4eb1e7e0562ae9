// Internal declarations shared by the translation units of libwoq.so.
// Not part of the public ABI (that is include/woq.h).
#pragma once

#include <hip/hip_runtime.h>
#include <atomic>
#include <stddef.h>
#include <stdint.h>

#include "../../include/woq.h"

namespace woq {

// ---------------------------------------------------------------------------
// Host-side helpers
// ---------------------------------------------------------------------------

inline int32_t hip_status(hipError_t e) { return e == hipSuccess ? WOQ_OK : WOQ_EHIP; }

// Raise a kernel's dynamic-LDS limit to `bytes` on the current device, once per
// device for each `done` (one bit per device; safe under concurrent callers).
inline int32_t raise_lds_limit(const void* fn, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return WOQ_EHIP;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t)1 << dev : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return WOQ_OK;
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess) return WOQ_EHIP;
  done.fetch_or(bit, std::memory_order_acq_rel);
  return WOQ_OK;
}

#define WOQ_HIP_TRY(expr)                         \
  do {                                            \
    hipError_t woq_e_ = (expr);                   \
    if (woq_e_ != hipSuccess) return WOQ_EHIP;    \
  } while (0)

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Workspace carve-up of the linear layer (all offsets 256-byte aligned).
struct LinearWorkspace {
  size_t xg_off = 0, xg_bytes = 0;   // gathered and/or pair-permuted activations, bf16 [M, kpad]
  size_t xs_off = 0, xs_bytes = 0;   // per-piece activation sums, f32 [K/min(G,128)][Mpad]
  size_t sz_off = 0, sz_bytes = 0;   // (scale, -(128 + zero)) pairs, f32x2 [K/G][N rounded to 256]
  size_t part_off = 0, part_bytes = 0;   // split-K partial outputs, f32 [splits][M][N]
  size_t total = 0;
};

// Which kernel family runs a linear call, and with what launch shape.
struct LinearPlan {
  int path = 0;          // 0 none, 1 small-M MFMA (m <= 128), 2 tiled MFMA GEMM, 3 bias only (k == 0),
                         // 4 decode GEMV (m <= 4), 5 row-streaming decode (m <= 4),
                         // 6 small-M MFMA with the activation slice in LDS (5 <= m <= 64)
  int mt = 1;            // 16-row activation tiles (small-M path)
  int fold_rows = 4;     // accumulator rows folded per tile (1 when m == 1)
  int ns = 1;            // 16-row weight tiles per workgroup (small-M path; per wave on path 6)
  int wm = 1;            // small-M path: wave groups along the activation rows
  int waves = 4;         // waves per workgroup
  int gb = 4;            // 32-wide k blocks per quantization group inside a 128-wide k step (1, 2, 4)
  int prep = 0;          // 1 = an input pre-pass kernel runs first
  int64_t grid = 0;      // workgroups
  int bm = 0, bn = 0;    // tile of the GEMM path
  int64_t mpad = 0;      // rows of the per-group sum table (GEMM path)
  int cnt = 0;           // 128-input steps per wave (decode and small-M paths; per K range on path 6)
  int64_t tail_n = 0;    // GEMM path: trailing output columns left to a second launch of
                         // 64-row tiles, so that the last round of workgroups is not half empty
  int rows_u = 0;        // row-streaming decode path (path 5): rows per workgroup
  int xfrag = 0;         // small-M path: a pre-pass writes the activations in MFMA fragment order
  int splits = 1;        // GEMM path and path 6: K ranges over separate workgroups (partials summed after)
  int sps = 0;           // GEMM path: 128-input steps per K range when splits > 1
};

// Compute units of one MI355X (gfx950): the GEMM path sizes its grid in rounds of this many
// workgroups (one workgroup per compute unit at a time).
constexpr int64_t kComputeUnits = 256;

// split_ok = false: the tiled GEMM keeps K whole (no partial-output buffer).
LinearWorkspace linear_workspace_layout(int64_t m, int64_t n, int64_t k, int32_t group,
                                        bool has_order, bool split_ok = true);
// rows_ok: the weights are canonical packed rows (unsigned or signed codes, or
// MXFP4 blocks; not prepared), which the row-streaming decode path can read.
LinearPlan linear_plan(int64_t m, int64_t n, int64_t k, int32_t group, bool has_order, bool rows_ok = true,
                       bool split_ok = true);

// ---------------------------------------------------------------------------
// Launchers (defined next to their kernels).  All enqueue on `stream` and
// return a woq_status.  Arguments are already validated.
// ---------------------------------------------------------------------------

int32_t launch_quantize(const float* w, int64_t n, int64_t k, int32_t group, int32_t symmetric,
                        uint8_t* q, float* scale, uint8_t* zero, uint32_t* flag,
                        hipStream_t stream);
int32_t launch_pack(const uint8_t* q, int64_t count, uint8_t* packed, uint32_t* flag,
                    hipStream_t stream);
int32_t launch_unpack(const uint8_t* packed, int64_t count, uint8_t* q, hipStream_t stream);
int32_t launch_pack_zero_points(const uint8_t* zero, int64_t n, int64_t ngroups, uint8_t* packed, uint32_t* flag,
                                hipStream_t stream);
int32_t launch_unpack_zero_points(const uint8_t* packed, int64_t n, int64_t ngroups, uint8_t* zero,
                                  hipStream_t stream);
int32_t launch_dequantize(const uint8_t* packed, const float* scale, const uint8_t* zero,
                          int64_t n, int64_t k, int32_t group, int32_t out_dtype, void* w_hat,
                          hipStream_t stream);
// Prepared weights: 1 KB blocks of 16 outputs x 128 inputs (see woq.h).
inline int64_t prepared_bytes(int64_t n, int64_t k) { return (n + 15) / 16 * ((k + 127) / 128) * 1024; }
int32_t launch_prepare(const uint8_t* packed, int64_t n, int64_t k, uint8_t* prepared,
                       hipStream_t stream);
int32_t launch_unprepare(const uint8_t* prepared, int64_t n, int64_t k, uint8_t* packed,
                         hipStream_t stream);

struct LinearArgs {
  const uint16_t* x;       // bf16 bits [M, K] (possibly the gathered copy)
  const uint8_t* packed;   // [N, K/2], or prepared blocks when `prepared`
  const float* scale;      // [N, K/G]
  const uint8_t* zero;     // [N, K/G]
  const float* bias;       // [N] or null
  void* y;                 // [M, N]
  const float* xs;         // per-piece sums [K/min(G,128)][mpad] (GEMM path)
  int32_t m, n, k, group;
  int32_t y_bf16;
  int32_t kpad;            // row stride of x (K rounded up to 128 on the GEMM path)
  int64_t mpad;
  int32_t prepared;        // 1: weights in the prepared (fragment-ordered) layout
  int32_t sym16;           // 1: signed two's complement codes, float16 scales, no zero point
  const uint16_t* scale16; // [N, K/G] float16 bits when sym16
  int32_t mx;              // 1: MXFP4 (E2M1 codes, E8M0 scale per block of 32; group = 32)
  const uint8_t* scale8;   // [N, K/32] E8M0 scale bytes when mx
  int32_t row_scale;       // 1 (with sym16): one float32 scale a row in `scale` [N] (Int4Linear)
  int32_t zp4;             // 1: `zero` holds packed 4-bit zero points [N, ceil(K/G / 2)], group 2j
                           //    in the low nibble of byte j (row-streaming, small-M and GEMM paths)
  float* part;             // GEMM path with splits > 1: f32 partial outputs [splits][M][N]
};

// Weight formats of the linear kernels' instantiations.
enum : int { kFmtU4 = 0, kFmtS16 = 1, kFmtMX = 2 };

// Signed int4 groups with float16 scales (quantize syncs through `flag`).
int32_t launch_quantize_s16(const float* w, int64_t n, int64_t k, int32_t group, int8_t* codes,
                            uint16_t* scale16, uint32_t* flag, hipStream_t stream);
int32_t launch_pack_s4(const int8_t* c, int64_t count, uint8_t* packed, uint32_t* flag,
                       hipStream_t stream);
int32_t launch_unpack_s4(const uint8_t* packed, int64_t count, int8_t* c, hipStream_t stream);
int32_t launch_dequantize_s16(const uint8_t* packed, const uint16_t* scale16, int64_t n, int64_t k,
                              int32_t group, int32_t out_dtype, void* w_hat, hipStream_t stream);

// MXFP4 (quantize syncs through `flag`).
int32_t launch_quantize_mx(const float* w, int64_t n, int64_t k, uint8_t* codes, uint8_t* scales,
                           uint32_t* flag, hipStream_t stream);
int32_t launch_dequantize_mx(const uint8_t* blocks, const uint8_t* scales, int64_t n, int64_t k,
                             int32_t out_dtype, void* w_hat, hipStream_t stream);

// Int4Linear: signed int4 with one float32 scale a row (quantize syncs through `flag`).
int32_t launch_quantize_rows(const float* w, int64_t n, int64_t k, int8_t* codes, float* scale,
                             uint32_t* flag, hipStream_t stream);
int32_t launch_dequantize_rows(const uint8_t* packed, const float* scale, int64_t n, int64_t k,
                               int32_t out_dtype, void* w_hat, hipStream_t stream);

// GPTQ (gptq.hip): columns per sweep block for a group size (0 if unsupported),
// and the whole quantization, synchronous.
int32_t gptq_block_cols(int32_t group);
int32_t run_gptq(const float* w, const uint16_t* x, int64_t t, int64_t n, int64_t k, int32_t group,
                 int32_t act_order, double damp, uint8_t* q, float* scale, uint8_t* zero, int32_t* order,
                 hipStream_t s);

// AWQ scale search (awq.hip), synchronous.
int32_t run_awq(const float* w, const uint16_t* x, int64_t t, int64_t n, int64_t k, int32_t group, int32_t n_grid,
                uint8_t* q, float* scale, uint8_t* zero, float* s_out, double* losses_out, int32_t* best_out,
                hipStream_t st);

int32_t launch_prep(const uint16_t* x, const int32_t* order, int32_t m, int32_t k, int32_t kpad,
                    int32_t group, int32_t permute, uint16_t* xg, float* xs, int64_t mpad,
                    hipStream_t stream);
int32_t launch_skinny(const LinearArgs& a, const LinearPlan& p, hipStream_t stream);
// Small-M pre-pass: x (gathered through `order` when given) in the small-M
// kernel's fragment order, [ceil(m/16)][ceil(k/128)][4][64 lanes] 16-byte
// chunks, pair-ordered unless `natural` (MXFP4); rows past m and inputs past k
// are zero.
size_t xfrag_bytes(int64_t m, int64_t k);
int32_t launch_xfrag(const uint16_t* x, const int32_t* order, int32_t m, int32_t k, int32_t group,
                     int32_t natural, uint16_t* out, hipStream_t stream);
// Decode path (m <= 4): LDS layout of one workgroup of `waves` waves with
// `cnt` steps each.
struct GemvLayout {
  int32_t xs_off = 0, sz_off = 0, wave_lds = 0, red_off = 0;
  size_t total = 0;
};
GemvLayout gemv_layout(int64_t m, int64_t k, int64_t group, int waves, int cnt);
int gemv_cnt_class(int cnt);   // the kernel variant serving `cnt` steps per wave (4, 8, 16; 0: none)
int32_t launch_gemv(const LinearArgs& a, const LinearPlan& p, hipStream_t stream);
// Up to kMaxGrouped matrices with the same m, k, group, layout and activations in
// one decode launch; `p` is the plan for their summed row count.
constexpr int kMaxGrouped = 4;
int32_t launch_gemv_grouped(const LinearArgs* args, int count, const LinearPlan& p,
                            hipStream_t stream);
// Small-M path: LDS of one workgroup of `waves` waves, `tiles` 16-row weight
// tiles and `cnt` steps per wave (per-wave (scale, zero) staging, then the
// cross-wave reduction area).
struct SkinnyLds {
  int32_t ngw = 0, sz_bytes = 0;
  int64_t red_off = 0;
  size_t total = 0;
};
SkinnyLds skinny_lds_layout(int64_t m, int64_t k, int64_t group, int waves, int tiles, int cnt);
constexpr size_t kSkinnyLdsLimit = 160 * 1024;   // LDS per CU
size_t gemm_sz_bytes(int64_t n, int64_t k, int32_t group);
constexpr int64_t kGemmMaxK = (int64_t)1 << 24;   // tile offsets of the GEMM path are 32-bit
// The GEMM path's inputs in one launch: x gathered/reordered into xg with its
// piece sums in xs (a.mpad rows, a.kpad stride) and the (scale, -(128 + zero))
// table into sz_ws; then launch_gemm, which reads them.
int32_t launch_gemm_prep(const LinearArgs& a, const int32_t* order, uint16_t* xg, float* xs, void* sz_ws,
                         hipStream_t stream);
int32_t launch_gemm(const LinearArgs& a, const LinearPlan& p, void* sz_ws, hipStream_t stream);
// Split-K second pass: y = the [splits][m][n] float32 partials summed in
// slice order, + bias, in y's type.
int32_t launch_splitk_reduce(const float* part, int32_t splits, int32_t m, int32_t n, const float* bias,
                             int32_t y_bf16, void* y, hipStream_t stream);
// Small-M path with the activation slice in LDS (path 6): LDS bytes of one
// workgroup (mt activation tiles, `steps` per K range, `tiles` weight tiles
// per wave), and the launch (kernel, then the split-K pass when the plan has
// more than one K range; a.part is the partial buffer).
size_t sm_lds_bytes(int mt, int steps, int tiles, int32_t group, bool mx);
int32_t launch_sm(const LinearArgs& a, const LinearPlan& p, hipStream_t stream);
int32_t launch_fill_bias(const float* bias, int32_t m, int32_t n, int32_t y_bf16, void* y,
                         hipStream_t stream);
// Row-streaming decode path (m <= 4, canonical weights): whether it takes
// (m, k), its rows per workgroup for n output rows in all, its waves per
// workgroup, and the launch over up to kMaxGrouped matrices sharing x.
bool rows_supported(int64_t m, int64_t k);
int rows_per_group(int64_t m, int64_t n, int64_t k);
int rows_waves(int64_t k);
int32_t launch_rows(const LinearArgs* args, int count, int u, hipStream_t stream);

}  // namespace woq
