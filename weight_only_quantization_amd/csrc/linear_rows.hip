// Decode path over weights in the canonical layout (1 <= m <= 4):
// y = x . dequant(W)^T + bias for group-wise 4-bit weights (linnet docs
// "Quantization", std.quant table, linear_int4_groups; the layout is the
// Int4GroupLinear row of the same table).
//
// At these row counts the layer is a stream of packed bytes, and two things
// decide how close a launch gets to the plain-read time of those bytes: how
// each load instruction touches memory, and how much work a wave still has
// to do after its last bytes arrive.  This kernel is shaped by both:
//
// * Every weight load is one contiguous kilobyte: lane l of a wave reads
//   bytes 16l .. 16l+15 of one row's 1 KB chunk, i.e. inputs
//   2048c + 32l .. +32 of that row (chunk c).  (A 16-row tile read as 16 rows
//   x 64 bytes per instruction streams measurably slower from HBM.)
// * A workgroup owns U rows (outputs) and all of K; its wave c takes chunk c
//   of each of those rows.  The wave issues its activation, scale and zero
//   loads first and then all U weight loads at once, so the whole matrix is in
//   flight within the first microsecond and each row is computed as soon as
//   its kilobyte arrives.
// * A lane's 32 inputs always lie in one quantization group (G >= 32), so the
//   lane holds one (scale, zero) pair per row and folds its own partial sum:
//   with bf16 codes (128 + q) (one AND-OR per code pair, exact) and
//   v_dot2_f32_bf16 against the activations,
//     part = s * (sum x (128 + q) - (128 + z) * sum x).
//   With G >= 64 a pair serves G / 32 lanes; the wave loads each pair once
//   and passes it to those lanes with ds_bpermute.
// * The U row partials of the 64 lanes are reduced in registers: lane-pair
//   swaps (v_permlane32_swap, v_permlane16_swap) and DPP moves halve the set
//   of rows held per lane at each distance, so the whole reduction costs
//   about two instructions per row; then the waves' partials meet in LDS in
//   wave order (deterministic), and the bias is added in float32.
// Signed codes with float16 scales (tinyllm L8.5, "int4 per group") and
// Int4Linear's one float32 scale a row run through the same arithmetic: a
// signed nibble v is the unsigned code v ^ 8 with zero point 8.
#include <cstdlib>

#include "woq_internal.h"

namespace woq {
namespace {

constexpr int kChunk = 2048;                  // inputs per wave and row (1 KB of codes)
constexpr int kMaxWaves = 16;                 // K <= 32768
constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr uint32_t kOffsetOOB = 0x80000000u;  // a buffer offset no descriptor covers
constexpr uint32_t kSignFlip = 0x88888888u;   // two's complement nibble v -> v ^ 8 (zero point 8)
constexpr uint32_t kOnes2 = 0x3F803F80u;      // bf16 pair (1.0, 1.0)

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

struct RowsProblem {
  const uint8_t* packed;
  const void* scale;      // float32 per group, float16 per group, or float32 per row
  const uint8_t* zero;    // unsigned codes only
  const float* bias;
  void* y;
  int32_t n;
  int32_t tile_begin;     // first workgroup of this matrix
};

struct RowsParams {
  const uint16_t* x;
  int32_t m, k, y_bf16;
  int32_t ngroups, group_shift;
  int32_t row_scale;      // signed codes with one float32 scale a row
  int32_t zp4;            // zero points packed two a byte (group 2j in the low nibble of byte j)
  int32_t zrow;           // zero-point bytes per row: ngroups, or ceil(ngroups / 2) with zp4
  uint32_t nib_mask, nib_offset;
  int32_t nprob;
  RowsProblem prob[kMaxGrouped];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, (int)kRsrcWord3);
}

__device__ __forceinline__ u32x4_t bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
// Weight loads: every packed byte is read once per call, in whole cache lines.
// Cache policy nt (non-temporal) with sc1 (agent scope): the lines stream
// through L2 without displacing the activations and scales that other
// workgroups re-read, and are not kept in the compute unit's vector L1.
constexpr int kStreamPolicy = 0x12;   // sc1 | nt
__device__ __forceinline__ u32x4_t bload16_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kStreamPolicy));
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// A copy of `v` the optimizer cannot fold into a constant (an identity DPP
// move), so that (d & mask) | offset is selected as one v_and_or_b32.
__device__ __forceinline__ uint32_t vgpr_copy(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xE4, 0xF, 0xF, false);
}

// 8 consecutive bf16 activations (4 dwords) -> the unpacker's pair order
// (x0, x4), (x1, x5), (x2, x6), (x3, x7).
__device__ __forceinline__ void pair_order(u32x4_t raw, uint32_t* o) {
  o[0] = __builtin_amdgcn_perm(raw[2], raw[0], 0x05040100u);
  o[1] = __builtin_amdgcn_perm(raw[2], raw[0], 0x07060302u);
  o[2] = __builtin_amdgcn_perm(raw[3], raw[1], 0x05040100u);
  o[3] = __builtin_amdgcn_perm(raw[3], raw[1], 0x07060302u);
}

// DPP moves inside 16-lane rows: 0 quad_perm [1,0,3,2], 1 quad_perm [2,3,0,1],
// 2 row_half_mirror, 3 row_ror:8.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  constexpr int kCtrl = CTRL == 0 ? 0xB1 : CTRL == 1 ? 0x4E : CTRL == 2 ? 0x141 : 0x128;
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false));
}

// a (lanes 0-31 kept, 32-63 taken from b's lanes 0-31) + b (the other halves):
// lanes below 32 get a_lo + a_hi, lanes from 32 get b_lo + b_hi.  The pair is
// read into scalars first (this compiler resolves a bit_cast of one element of
// a vector lvalue to element 0).
__device__ __forceinline__ float swap_add32(float a, float b) {
  const auto s = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), false, false);
  const uint32_t e0 = s[0], e1 = s[1];
  return __builtin_bit_cast(float, e0) + __builtin_bit_cast(float, e1);
}
// The same between neighbouring 16-lane rows (rows 0/1 and 2/3).
__device__ __forceinline__ float swap_add16(float a, float b) {
  const auto s = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), false, false);
  const uint32_t e0 = s[0], e1 = s[1];
  return __builtin_bit_cast(float, e0) + __builtin_bit_cast(float, e1);
}

// Sum v[0..U) over the 64 lanes.  Each halving step pairs lanes at one
// distance (32, 16, 8, 4) and keeps half of the rows: afterwards lane l holds
// the total of row l >> (6 - log2 U), added in a fixed order.
template <int U>
__device__ __forceinline__ float reduce_rows(float* v, int lane) {
  static_assert(U == 4 || U == 8 || U == 16, "rows per workgroup");
#pragma unroll
  for (int j = 0; j < U / 2; ++j) v[j] = swap_add32(v[j], v[j + U / 2]);
#pragma unroll
  for (int j = 0; j < U / 4; ++j) v[j] = swap_add16(v[j], v[j + U / 4]);
  if constexpr (U >= 8) {   // distance 8 (row_ror:8): lanes with bit 3 set keep the upper rows
    const bool hi = (lane >> 3) & 1;
#pragma unroll
    for (int t = 0; t < U / 8; ++t) {
      const float keep = hi ? v[t + U / 8] : v[t];
      const float give = hi ? v[t] : v[t + U / 8];
      v[t] = keep + dpp<3>(give);
    }
  }
  if constexpr (U >= 16) {  // distance 4 (row_half_mirror pairs lane i with 7 - i): by bit 2
    const bool hi = (lane >> 2) & 1;
    const float keep = hi ? v[1] : v[0];
    const float give = hi ? v[0] : v[1];
    v[0] = keep + dpp<2>(give);
  }
  float r = v[0];
  if constexpr (U == 4) {   // the remaining 16 lanes
    r += dpp<3>(r);
    r += dpp<2>(r);
    r += dpp<1>(r);
    r += dpp<0>(r);
  } else if constexpr (U == 8) {   // the remaining 8 lanes
    r += dpp<2>(r);
    r += dpp<1>(r);
    r += dpp<0>(r);
  } else {   // the remaining 4 lanes
    r += dpp<0>(r);
    r += dpp<1>(r);
  }
  return r;
}

// U: rows per workgroup (4, 8, 16); MR: activation rows computed (1, 2 or 4;
// rows past m repeat the last one and are not stored); FMT: unsigned codes,
// signed codes (kFmtS16) or MXFP4 (kFmtMX: a lane's 32 inputs are one block,
// whose E2M1 codes v_cvt_scalef32_pk_bf16_fp4 turns into bf16 already
// multiplied by the block's power-of-two scale, exactly, in natural input
// order: no fold and no activation sum); GRP: several matrices in one launch.
// SG (64, 128 or 256; 0: off): groups of SG inputs (scales per group), where
// the SG / 32 lanes of a group would load the same (scale, zero) pairs.  A
// wave instead loads 64 distinct entries per instruction, SG / 32 rows of its
// chunk's 2048 / SG groups, and hands them to the lanes that need them with
// ds_bpermute: U / (SG / 32) loads of each instead of U.
template <int U, int MR, int FMT, bool GRP, int SG = 0>
__global__ __launch_bounds__(1024) void rows_kernel(RowsParams p) {
  constexpr bool S16 = FMT == kFmtS16, MX = FMT == kFmtMX;
  static_assert(SG == 0 || (!MX && (SG == 64 || SG == 128 || SG == 256)), "shared (scale, zero) loads");
  constexpr int kShift = U == 16 ? 2 : (U == 8 ? 3 : 4);   // lane l holds row l >> kShift after the reduction
  __shared__ float red[kMaxWaves * 4 * 16];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int W = __builtin_amdgcn_readfirstlane((int)(blockDim.x >> 6));
  // This workgroup's matrix.  A single matrix is read straight from the
  // arguments; a grouped launch first finds its entry, which costs one more
  // round of argument loads before the first weight load.
  int pi = 0;
  if constexpr (GRP) {
#pragma unroll
    for (int i = 1; i < kMaxGrouped; ++i)
      if (i < p.nprob && (int)blockIdx.x >= p.prob[i].tile_begin) pi = i;
  }
  const RowsProblem& pr = p.prob[pi];
  const int M = p.m, N = pr.n, K = p.k, ng = p.ngroups;
  const int row0 = ((int)blockIdx.x - pr.tile_begin) * U;
  const int rows = min(U, N - row0);
  const uint32_t row_bytes = (uint32_t)K / 2;
  const int kin = wave * kChunk + 32 * lane;          // first input of this lane
  const uint32_t dead = kin >= K ? kOffsetOOB : 0u;   // lanes past K load zeros
  const int g = kin >> p.group_shift;
  const bool row_scale = S16 && SG == 0 && p.row_scale != 0;    // uniform

  const __amdgpu_buffer_rsrc_t rw = rsrc(pr.packed + (int64_t)row0 * row_bytes, (uint32_t)rows * row_bytes);
  const __amdgpu_buffer_rsrc_t rx = rsrc(p.x, (uint32_t)(M * K) * 2u);
  const uint32_t sbytes = MX ? 1u : (S16 && !row_scale ? 2u : 4u);
  const int srow = row_scale ? 1 : ng;
  const __amdgpu_buffer_rsrc_t rs =
      rsrc(static_cast<const char*>(pr.scale) + (int64_t)row0 * srow * sbytes, (uint32_t)(rows * srow) * sbytes);
  const int zrow = p.zrow;
  const __amdgpu_buffer_rsrc_t rz =
      rsrc(S16 || MX ? nullptr : pr.zero + (int64_t)row0 * zrow, S16 || MX ? 0u : (uint32_t)(rows * zrow));
  const bool zp4 = p.zp4 != 0;   // uniform
  const uint32_t zsh = zp4 ? 4u * (uint32_t)(g & 1) : 0u;   // the lane's zero point: bits [zsh, zsh + zbits)
  const uint32_t zbits = zp4 ? 4u : 8u;

  // 1. Activations, scales and zero points first, then every weight load of
  //    the wave: rows past N and lanes past K read zero.
  u32x4_t xr[MR][4];
#pragma unroll
  for (int mm = 0; mm < MR; ++mm) {
    const int xm = min(mm, M - 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) xr[mm][i] = bload16(rx, ((uint32_t)(xm * K + kin) * 2u + 16u * i) | dead);
  }
  uint32_t sr[U];   // float32 scale bits as loaded (unsigned codes; Int4Linear's row scale)
  uint32_t zr[U];   // zero-point byte as loaded; float16 scale bits for signed codes
  // Both are converted after the weight loads are out: a conversion, or a
  // select between two loads, here would make the wave wait for these loads
  // before it issues the weight loads.  Signed codes issue both scale loads,
  // the one their layout does not use at an offset no descriptor covers.
  // SG: lane l of load j holds the entry of row kRpl j + l / kNgw and group
  // kNgw wave + l % kNgw; rows past N and groups past K read zero.
  constexpr int kRpl = SG ? SG / 32 : 1;   // rows per load = lanes per group
  constexpr int kNgw = 64 / kRpl;          // groups in a wave's chunk
  constexpr int kPk = SG ? (U + kRpl - 1) / kRpl : 1;
  uint32_t spk[kPk], zpk[kPk];
  if constexpr (SG != 0) {
#pragma unroll
    for (int j = 0; j < kPk; ++j) {
      const int r = kRpl * j + lane / kNgw, gg = kNgw * wave + lane % kNgw;
      const bool in = r < rows && gg < ng;
      const uint32_t e = (uint32_t)(r * ng + gg);
      if constexpr (S16) {   // float16 scale bits
        spk[j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, (int)(in ? e * 2u : kOffsetOOB), 0, 0);
        zpk[j] = 0u;
      } else {
        const uint32_t ze = zp4 ? (uint32_t)(r * zrow + (gg >> 1)) : e;
        spk[j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, (int)(in ? e * 4u : kOffsetOOB), 0, 0);
        zpk[j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rz, (int)(in ? ze : kOffsetOOB), 0, 0);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if constexpr (SG != 0) break;
    const uint32_t e = (uint32_t)(u * ng + g);
    if constexpr (MX) {
      sr[u] = 0u;
      zr[u] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs, (int)(e | dead), 0, 0);   // E8M0 scale byte
    } else if constexpr (S16) {
      sr[u] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, (int)(row_scale ? ((uint32_t)u * 4u) | dead : kOffsetOOB), 0, 0);
      zr[u] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, (int)(row_scale ? kOffsetOOB : (e * 2u) | dead), 0, 0);
    } else {
      sr[u] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, (int)((e * 4u) | dead), 0, 0);
      const uint32_t ze = zp4 ? (uint32_t)(u * zrow + (g >> 1)) : e;
      zr[u] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rz, (int)(ze | dead), 0, 0);
    }
  }
  u32x4_t w[U];
  const uint32_t woff = ((uint32_t)kin / 2u) | dead;
#pragma unroll
  for (int u = 0; u < U; ++u) w[u] = bload16_stream(rw, woff + (uint32_t)u * row_bytes);
  // Every load above is issued before any of them is waited for: without
  // this the scheduler delays weight loads behind the activation math to save
  // registers, and the stream starts late.
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (SG != 0 && S16) {
    // As below; the float16 scales of two loads travel together.
    constexpr int kHw = (kPk + 1) / 2;
    uint32_t hall[kHw];
#pragma unroll
    for (int w2 = 0; w2 < kHw; ++w2) hall[w2] = 0;
#pragma unroll
    for (int j = 0; j < kPk; ++j) hall[j / 2] |= (spk[j] & 0xFFFFu) << (16 * (j % 2));
#pragma unroll
    for (int c = 0; c < kRpl; ++c) {
      if (c >= U) break;
      const int src = 4 * (kNgw * c + lane / kRpl);
#pragma unroll
      for (int w2 = 0; w2 < kHw; ++w2) {
        const uint32_t h = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)hall[w2]);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int u = kRpl * (2 * w2 + t) + c;
          if (u < U) { sr[u] = 0u; zr[u] = h >> (16 * t); }
        }
      }
    }
  } else if constexpr (SG != 0) {
    // Row u = kRpl j + c's entry for this lane's group (lane / kRpl of the
    // chunk) sits in lane kNgw c + lane / kRpl of load j.  The zero bytes of
    // four loads travel together, byte j % 4 from load j.
    constexpr int kZw = (kPk + 3) / 4;
    uint32_t zall[kZw];
#pragma unroll
    for (int w4 = 0; w4 < kZw; ++w4) zall[w4] = 0;
#pragma unroll
    for (int j = 0; j < kPk; ++j) zall[j / 4] |= (zpk[j] & 0xFFu) << (8 * (j % 4));
#pragma unroll
    for (int c = 0; c < kRpl; ++c) {
      if (c >= U) break;
      const int src = 4 * (kNgw * c + lane / kRpl);
      uint32_t zc[kZw];
#pragma unroll
      for (int w4 = 0; w4 < kZw; ++w4) zc[w4] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)zall[w4]);
#pragma unroll
      for (int j = 0; j < kPk; ++j) {
        if (kRpl * j + c >= U) break;
        sr[kRpl * j + c] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)spk[j]);
        zr[kRpl * j + c] = zc[j / 4] >> (8 * (j % 4));
      }
    }
  }

  // 2. The lane's activations in the unpacker's pair order, and their sum
  //    (MXFP4: in natural order, no sum).
  uint32_t xp[MR][16];
  float X[MR];
#pragma unroll
  for (int mm = 0; mm < MR; ++mm) {
    if constexpr (MX) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4_t r = xr[mm][i];
        xp[mm][4 * i + 0] = r[0]; xp[mm][4 * i + 1] = r[1]; xp[mm][4 * i + 2] = r[2]; xp[mm][4 * i + 3] = r[3];
      }
      X[mm] = 0.f;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) pair_order(xr[mm][i], xp[mm] + 4 * i);
      float t = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) t = dot2(xp[mm][i], kOnes2, t);
      X[mm] = t;
    }
  }

  // 3. Per row: codes as bf16 (128 + q), dot with the activations, fold.
  const uint32_t off = vgpr_copy(p.nib_offset);
  const uint32_t mask = p.nib_mask;
  float v[MR][U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if constexpr (MX) {
      // 2^(e - 127) of the block's E8M0 byte e (e = 0: 2^-127, a float32 subnormal)
      const uint32_t eb = zr[u] & 0xFFu;
      const float bs = __builtin_bit_cast(float, eb == 0 ? 0x00400000u : eb << 23);
#pragma unroll
      for (int mm = 0; mm < MR; ++mm) {
        float r0 = 0.f, r1 = 0.f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t wd = w[u][d];
          r0 = dot2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, bs, 0)), xp[mm][4 * d + 0], r0);
          r1 = dot2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, bs, 1)), xp[mm][4 * d + 1], r1);
          r0 = dot2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, bs, 2)), xp[mm][4 * d + 2], r0);
          r1 = dot2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, bs, 3)), xp[mm][4 * d + 3], r1);
        }
        v[mm][u] = r0 + r1;
      }
      continue;
    }
    // -(128 + zero): the codes enter the dot product as 128 + q
    const float nz = S16 ? -136.f : -128.f - (float)__builtin_amdgcn_ubfe(zr[u], zsh, zbits);
    const float su = S16 && !row_scale ? (float)__builtin_bit_cast(_Float16, (uint16_t)zr[u])
                                       : __builtin_bit_cast(float, sr[u]);
#pragma unroll
    for (int mm = 0; mm < MR; ++mm) {
      float r0 = 0.f, r1 = 0.f;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t wd = S16 ? w[u][d] ^ kSignFlip : w[u][d];
        r0 = dot2((wd & mask) | off, xp[mm][4 * d + 0], r0);
        r1 = dot2(((wd >> 4) & mask) | off, xp[mm][4 * d + 1], r1);
        r0 = dot2(((wd >> 8) & mask) | off, xp[mm][4 * d + 2], r0);
        r1 = dot2(((wd >> 12) & mask) | off, xp[mm][4 * d + 3], r1);
      }
      v[mm][u] = su * fmaf(nz, X[mm], r0 + r1);
    }
  }

  // 4. Reduce over the lanes, combine the waves in wave order, add the bias, store.
  const int rr = lane >> kShift;
  const bool lead = (lane & ((1 << kShift) - 1)) == 0;
  float t[MR];
#pragma unroll
  for (int mm = 0; mm < MR; ++mm) t[mm] = reduce_rows<U>(v[mm], lane);
  auto store = [&](int mm, int r, float o) {
    const int n = row0 + r;
    o += pr.bias ? pr.bias[n] : 0.f;
    if (p.y_bf16)
      reinterpret_cast<uint16_t*>(pr.y)[(int64_t)mm * N + n] = __builtin_bit_cast(uint16_t, (__bf16)o);
    else
      reinterpret_cast<float*>(pr.y)[(int64_t)mm * N + n] = o;
  };
  if (W == 1) {
    if (lead && rr < rows) {
#pragma unroll
      for (int mm = 0; mm < MR; ++mm)
        if (mm < M) store(mm, rr, t[mm]);
    }
    return;
  }
  if (lead) {
#pragma unroll
    for (int mm = 0; mm < MR; ++mm) red[(wave * 4 + mm) * 16 + rr] = t[mm];
  }
  __syncthreads();
  if (wave == 0 && lane < MR * U) {
    const int mm = lane / U, r = lane % U;
    if (mm < M && r < rows) {
      float o = 0.f;
      for (int i = 0; i < W; ++i) o += red[(i * 4 + mm) * 16 + r];
      store(mm, r, o);
    }
  }
}

// Groups of 128 or 256 (64 with 16-row workgroups; measured: 4-row ones are
// 2% slower there) load each (scale, zero) pair once a wave.
template <int U, int MR, int FMT, bool GRP>
void launch_fmt(const RowsParams& rp, dim3 g, dim3 b, hipStream_t stream) {
  if constexpr (FMT != kFmtMX) {
    const bool shared = !(FMT == kFmtS16 && rp.row_scale);
    if (shared && rp.group_shift == 7) {
      hipLaunchKernelGGL((rows_kernel<U, MR, FMT, GRP, 128>), g, b, 0, stream, rp);
      return;
    }
    if (shared && rp.group_shift == 8) {
      hipLaunchKernelGGL((rows_kernel<U, MR, FMT, GRP, 256>), g, b, 0, stream, rp);
      return;
    }
    if constexpr (U == 16) {
      if (shared && rp.group_shift == 6) {
        hipLaunchKernelGGL((rows_kernel<U, MR, FMT, GRP, 64>), g, b, 0, stream, rp);
        return;
      }
    }
  }
  hipLaunchKernelGGL((rows_kernel<U, MR, FMT, GRP>), g, b, 0, stream, rp);
}

template <int U, int MR>
int32_t launch_u(const RowsParams& rp, int64_t grid, int waves, int fmt, hipStream_t stream) {
  const dim3 g((unsigned)grid), b(64 * waves);
  if (rp.nprob > 1)   // grouped launches carry unsigned codes only
    launch_fmt<U, MR, kFmtU4, true>(rp, g, b, stream);
  else if (fmt == kFmtS16)
    launch_fmt<U, MR, kFmtS16, false>(rp, g, b, stream);
  else if (fmt == kFmtMX)
    launch_fmt<U, MR, kFmtMX, false>(rp, g, b, stream);
  else
    launch_fmt<U, MR, kFmtU4, false>(rp, g, b, stream);
  return hip_status(hipGetLastError());
}

// Four activation rows keep 4 rows per workgroup and two at most 8: wider
// ones would not fit in the 128 registers a 1024-thread workgroup leaves each
// lane.
template <int MR>
int32_t launch_mr(const RowsParams& rp, int u, int64_t grid, int waves, int fmt, hipStream_t stream) {
  if constexpr (MR > 2) {
    return launch_u<4, MR>(rp, grid, waves, fmt, stream);
  } else if constexpr (MR == 2) {
    return u == 4 ? launch_u<4, MR>(rp, grid, waves, fmt, stream) : launch_u<8, MR>(rp, grid, waves, fmt, stream);
  } else {
    switch (u) {
      case 4: return launch_u<4, MR>(rp, grid, waves, fmt, stream);
      case 8: return launch_u<8, MR>(rp, grid, waves, fmt, stream);
      case 16: return launch_u<16, MR>(rp, grid, waves, fmt, stream);
      default: return WOQ_EUNSUPPORTED;
    }
  }
}

}  // namespace

bool rows_supported(int64_t m, int64_t k) { return m >= 1 && m <= 4 && k > 0 && k <= (int64_t)kChunk * kMaxWaves; }

// Rows per workgroup (4 when m > 2, at most 8 when m = 2).  Long rows (four or more waves) take 16
// rows when that still gives a thousand waves, otherwise 4 (measured at m = 1
// on the Llama-3-8B decode shapes 14336x4096, 4096x14336, 4096x4096 and
// 1024x4096 with 4, 8 and 16 rows).  WOQ_ROWS_U forces 4, 8
// or 16 (a tuning aid, read on every call).
int rows_per_group(int64_t m, int64_t n, int64_t k) {
  if (m > 2) return 4;
  if (const char* e = std::getenv("WOQ_ROWS_U")) {
    const int u = std::atoi(e);
    if (u == 4 || u == 8 || u == 16) return m == 2 && u == 16 ? 8 : u;
  }
  const int64_t waves = (k + kChunk - 1) / kChunk;
  auto total = [&](int64_t u) { return (n + u - 1) / u * waves; };
  if (m == 1 && waves >= 4 && total(16) >= 1024) return 16;
  return 4;
}

int rows_waves(int64_t k) { return (int)((k + kChunk - 1) / kChunk); }

int32_t launch_rows(const LinearArgs* args, int count, int u, hipStream_t stream) {
  const LinearArgs& a = args[0];
  if (!rows_supported(a.m, a.k) || a.prepared || (a.mx && (count != 1 || a.group != 32))) return WOQ_EUNSUPPORTED;
  int32_t gshift = 0;
  while ((1 << gshift) < a.group) ++gshift;
  RowsParams rp{};
  rp.x = a.x;
  rp.m = a.m;
  rp.k = a.k;
  rp.y_bf16 = a.y_bf16;
  rp.ngroups = a.k / a.group;
  rp.group_shift = gshift;
  rp.row_scale = a.row_scale;
  rp.zp4 = a.zp4;
  rp.zrow = a.zp4 ? (rp.ngroups + 1) / 2 : rp.ngroups;
  rp.nib_mask = 0x000F000Fu;    // one nibble in each bf16 half
  rp.nib_offset = 0x43004300u;  // bf16 pair (128, 128): OR-ing a nibble n gives 128 + n
  rp.nprob = count;
  int64_t tb = 0;
  for (int i = 0; i < count; ++i) {
    const LinearArgs& ai = args[i];
    rp.prob[i] = RowsProblem{ai.packed,
                             ai.mx ? static_cast<const void*>(ai.scale8)
                                   : ai.sym16 && !ai.row_scale ? static_cast<const void*>(ai.scale16)
                                                               : static_cast<const void*>(ai.scale),
                             ai.zero, ai.bias, ai.y, ai.n, (int32_t)tb};
    tb += (ai.n + u - 1) / u;
  }
  if (tb == 0) return WOQ_OK;
  const int waves = rows_waves(a.k);
  const int fmt = a.mx ? kFmtMX : a.sym16 ? kFmtS16 : kFmtU4;
  switch (a.m) {
    case 1: return launch_mr<1>(rp, u, tb, waves, fmt, stream);
    case 2: return launch_mr<2>(rp, u, tb, waves, fmt, stream);
    default: return launch_mr<4>(rp, u, tb, waves, fmt, stream);
  }
}

}  // namespace woq
