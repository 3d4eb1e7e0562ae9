// Device helpers shared by the two MFMA linear paths.
//
// MFMA operand convention used throughout (v_mfma_f32_16x16x32_bf16, wave64):
// lanes are numbered l = 16*q + c (q = lane group 0..3, c = 0..15).  Each lane
// supplies 8 bf16 "slots" for A and for B; slot s of A-lane (q, i) is
// multiplied with slot s of B-lane (q, j) and all 32 (q, s) products are
// summed into D[i][j].  Lane (q, j) of the result holds D[4q + r][j] in its
// register r (r = 0..3).  Which k a (q, s) pair stands for is our choice, as
// long as A and B agree; the kernels below pick it so that nibble unpacking is
// cheap.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace woq {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// bf16 bit pattern 0x4300 is 128.0; OR-ing a nibble n into its low mantissa
// bits gives exactly 128 + n.  Two such values per dword.
constexpr uint32_t kNibPairMask = 0x000F000Fu;
constexpr uint32_t kBf16Offset2 = 0x43004300u;
constexpr float kNibOffset = 128.0f;
constexpr uint32_t kBf16One2 = 0x3F803F80u;   // bf16 pair (1.0, 1.0)

// A copy of `v` the optimizer cannot fold back into a constant: an identity
// DPP move.  Holding the bf16 offset this way leaves the nibble mask as the
// only scalar operand of (d & mask) | offset, which instruction selection
// then emits as a single v_and_or_b32 (gfx9 reads one scalar per VOP3).
__device__ __forceinline__ uint32_t vgpr_copy(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xE4, 0xF, 0xF, false);
}

// One packed dword holds the codes of 8 consecutive inputs k..k+7, input k+e
// in bits 4e..4e+3.  Expand it to 8 bf16 values 128 + code in slot order
// (k, k+4, k+1, k+5, k+2, k+6, k+3, k+7): dword v of the result pairs inputs
// k+v and k+v+4.  `mask` is kNibPairMask and `offset` kBf16Offset2, the
// latter best held in a vector register (vgpr_copy) by the caller.
__device__ __forceinline__ bf16x8_t unpack_codes(uint32_t d, uint32_t mask, uint32_t offset) {
  u32x4_t r;
  r[0] = (d & mask) | offset;
  r[1] = ((d >> 4) & mask) | offset;
  r[2] = ((d >> 8) & mask) | offset;
  r[3] = ((d >> 12) & mask) | offset;
  return __builtin_bit_cast(bf16x8_t, r);
}

// MXFP4: one dword holds 8 consecutive E2M1 codes (the even input in the low
// nibble of each byte).  v_cvt_scalef32_pk_bf16_fp4 turns the two codes of one
// byte into two bf16 values multiplied by `scale`; with a power-of-two scale
// (an E8M0 block scale) the product is exact.  The result is in natural input
// order.
__device__ __forceinline__ bf16x8_t fp4x8_to_bf16(uint32_t d, float scale) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  u32x4_t r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 3));
  return __builtin_bit_cast(bf16x8_t, r);
}

// Reorder 8 consecutive bf16 activations (natural order, as 4 dwords) into the
// slot order of unpack_codes.
__device__ __forceinline__ bf16x8_t pair_order(u32x4_t raw) {
  u32x4_t r;
  r[0] = __builtin_amdgcn_perm(raw[2], raw[0], 0x05040100u);   // (x0, x4)
  r[1] = __builtin_amdgcn_perm(raw[2], raw[0], 0x07060302u);   // (x1, x5)
  r[2] = __builtin_amdgcn_perm(raw[3], raw[1], 0x05040100u);   // (x2, x6)
  r[3] = __builtin_amdgcn_perm(raw[3], raw[1], 0x07060302u);   // (x3, x7)
  return __builtin_bit_cast(bf16x8_t, r);
}

// Transpose a 4x4 matrix of dwords spread over the four 16-lane groups: on
// entry lane group q holds row q in d[0..3]; on exit it holds column q.
// Two gfx950 lane-swap stages: swap the off-diagonal 2x2 blocks between lane
// halves (distance 32), then the off-diagonal elements inside each block
// between neighbouring lane groups (distance 16).
__device__ __forceinline__ void transpose4_lanegroups(uint32_t& d0, uint32_t& d1, uint32_t& d2,
                                                      uint32_t& d3) {
  {
    auto s = __builtin_amdgcn_permlane32_swap(d0, d2, false, false);
    d0 = s[0]; d2 = s[1];
    auto t = __builtin_amdgcn_permlane32_swap(d1, d3, false, false);
    d1 = t[0]; d3 = t[1];
  }
  {
    auto s = __builtin_amdgcn_permlane16_swap(d0, d1, false, false);
    d0 = s[0]; d1 = s[1];
    auto t = __builtin_amdgcn_permlane16_swap(d2, d3, false, false);
    d2 = t[0]; d3 = t[1];
  }
}

__device__ __forceinline__ f32x4_t mfma_bf16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ u32x4_t load16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

}  // namespace woq
