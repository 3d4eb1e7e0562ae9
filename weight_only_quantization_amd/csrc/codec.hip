// Quantize / pack / unpack / dequantize kernels for the Int4GroupLinear layout
// (linnet docs "Quantization", std.quant table).  None of these is on the
// linear layer's hot path; they are load-time and inspection kernels, written
// for exactness first: every rounding decision is the same one the float64
// rule in the public header describes.
#include "woq_internal.h"

#pragma clang fp contract(off)

namespace woq {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ bool finite_f32(float v) {
  return (__float_as_uint(v) & 0x7f800000u) != 0x7f800000u;
}

// Per-group parameters of the asymmetric rule (min/max range, zero point) or
// of the symmetric rule (absmax, zero fixed at 8).  `den` is the float64
// divisor of Q*w, `qmax` the code limit Q.
struct GroupRule {
  double den;     // range (asymmetric) or absmax (symmetric); 1 for a flat group
  double zero;    // zero point as a float64 integer
  float scale;
  bool flat;
};

__device__ __forceinline__ GroupRule asym_rule(double mn, double mx) {
  GroupRule r;
  const double d = mx - mn;
  r.flat = (d == 0.0);
  if (r.flat) {
    r.den = 1.0;
    r.scale = 1.0f;
    r.zero = fmin(fmax(__builtin_rint(-mn), 0.0), 15.0);
  } else {
    r.den = d;
    r.scale = (float)(d / 15.0);
    r.zero = fmin(fmax(__builtin_rint((-15.0 * mn) / d), 0.0), 15.0);
  }
  return r;
}

__device__ __forceinline__ GroupRule sym_rule(double a) {
  GroupRule r;
  r.flat = (a == 0.0);
  r.den = r.flat ? 1.0 : a;
  r.scale = r.flat ? 1.0f : (float)(a / 7.0);
  r.zero = 8.0;
  return r;
}

__device__ __forceinline__ uint32_t asym_code(const GroupRule& r, float w) {
  const double wd = (double)w;
  const double t = r.flat ? __builtin_rint(wd) : __builtin_rint((15.0 * wd) / r.den);
  const double q = fmin(fmax(t + r.zero, 0.0), 15.0);
  return (uint32_t)q;
}

__device__ __forceinline__ uint32_t sym_code(const GroupRule& r, float w) {
  if (r.flat) return 8u;
  const double c = fmin(fmax(__builtin_rint((7.0 * (double)w) / r.den), -7.0), 7.0);
  return (uint32_t)(int)(c + 8.0);
}

// L lanes cooperate on one group of 4*L consecutive weights (float4 per lane).
template <int L>
__global__ __launch_bounds__(kThreads) void quantize_coop_kernel(
    const float* __restrict__ w, int64_t ngroups, int32_t symmetric, int32_t q_aligned,
    uint8_t* __restrict__ q, float* __restrict__ scale, uint8_t* __restrict__ zero,
    uint32_t* __restrict__ flag) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x; t < ngroups * L; t += stride) {
    const int64_t gi = t / L;
    const int li = (int)(t % L);
    const int64_t base = gi * (4 * L) + 4 * li;
    const float4 v = *reinterpret_cast<const float4*>(w + base);
    int bad = (finite_f32(v.x) && finite_f32(v.y) && finite_f32(v.z) && finite_f32(v.w)) ? 0 : 1;
    float lo = fminf(fminf(v.x, v.y), fminf(v.z, v.w));
    float hi = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
    float am = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
#pragma unroll
    for (int off = L / 2; off > 0; off >>= 1) {
      lo = fminf(lo, __shfl_xor(lo, off, L));
      hi = fmaxf(hi, __shfl_xor(hi, off, L));
      am = fmaxf(am, __shfl_xor(am, off, L));
      bad |= __shfl_xor(bad, off, L);   // every lane takes part in every shuffle
    }
    if (bad) {
      if (li == 0) atomicOr(flag, 1u);
      continue;
    }
    const GroupRule r = symmetric ? sym_rule((double)am) : asym_rule((double)lo, (double)hi);
    uint32_t c0, c1, c2, c3;
    if (symmetric) {
      c0 = sym_code(r, v.x); c1 = sym_code(r, v.y); c2 = sym_code(r, v.z); c3 = sym_code(r, v.w);
    } else {
      c0 = asym_code(r, v.x); c1 = asym_code(r, v.y); c2 = asym_code(r, v.z); c3 = asym_code(r, v.w);
    }
    if (q_aligned) {
      *reinterpret_cast<uint32_t*>(q + base) = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
    } else {
      q[base] = (uint8_t)c0; q[base + 1] = (uint8_t)c1; q[base + 2] = (uint8_t)c2; q[base + 3] = (uint8_t)c3;
    }
    if (li == 0) {
      scale[gi] = r.scale;
      zero[gi] = (uint8_t)r.zero;
    }
  }
}

// One thread per group: any group size, any alignment.
__global__ __launch_bounds__(kThreads) void quantize_thread_kernel(
    const float* __restrict__ w, int64_t ngroups, int32_t group, int32_t symmetric,
    uint8_t* __restrict__ q, float* __restrict__ scale, uint8_t* __restrict__ zero,
    uint32_t* __restrict__ flag) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t gi = (int64_t)blockIdx.x * kThreads + threadIdx.x; gi < ngroups; gi += stride) {
    const float* g = w + gi * group;
    bool bad = false;
    float lo = g[0], hi = g[0], am = 0.0f;
    for (int e = 0; e < group; ++e) {
      const float v = g[e];
      bad = bad || !finite_f32(v);
      lo = fminf(lo, v);
      hi = fmaxf(hi, v);
      am = fmaxf(am, fabsf(v));
    }
    if (bad) {
      atomicOr(flag, 1u);
      continue;
    }
    const GroupRule r = symmetric ? sym_rule((double)am) : asym_rule((double)lo, (double)hi);
    uint8_t* qo = q + gi * group;
    for (int e = 0; e < group; ++e)
      qo[e] = (uint8_t)(symmetric ? sym_code(r, g[e]) : asym_code(r, g[e]));
    scale[gi] = r.scale;
    zero[gi] = (uint8_t)r.zero;
  }
}

// 16 codes -> 8 bytes per iteration; a code above 15 sets the flag.
__global__ __launch_bounds__(kThreads) void pack_vec_kernel(const uint4* __restrict__ q, int64_t nvec,
                                                            uint2* __restrict__ packed,
                                                            uint32_t* __restrict__ flag) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  bool bad = false;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += stride) {
    const uint4 v = q[i];
    bad = bad || ((v.x | v.y | v.z | v.w) & 0xF0F0F0F0u) != 0u;
    // byte j of a 4-code word holds code j; fold pairs (2i, 2i+1) into one byte
    auto fold = [](uint32_t a) -> uint32_t {   // 4 codes -> 2 packed bytes in the low 16 bits
      const uint32_t even = a & 0x000F000Fu;           // codes 0 and 2
      const uint32_t odd = (a >> 4) & 0x00F000F0u;     // codes 1 and 3, moved to the high nibble
      const uint32_t b = even | odd;                   // byte 0 = c0|c1<<4, byte 2 = c2|c3<<4
      return (b & 0xFFu) | ((b >> 8) & 0xFF00u);
    };
    uint2 o;
    o.x = fold(v.x) | (fold(v.y) << 16);
    o.y = fold(v.z) | (fold(v.w) << 16);
    packed[i] = o;
  }
  if (bad) atomicOr(flag, 1u);
}

__global__ __launch_bounds__(kThreads) void pack_byte_kernel(const uint8_t* __restrict__ q, int64_t nbytes,
                                                             uint8_t* __restrict__ packed,
                                                             uint32_t* __restrict__ flag) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  bool bad = false;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nbytes; i += stride) {
    const uint32_t lo = q[2 * i], hi = q[2 * i + 1];
    bad = bad || lo > 15u || hi > 15u;
    packed[i] = (uint8_t)((lo & 15u) | ((hi & 15u) << 4));
  }
  if (bad) atomicOr(flag, 1u);
}

// 8 packed bytes -> 16 codes per iteration.
__global__ __launch_bounds__(kThreads) void unpack_vec_kernel(const uint2* __restrict__ packed, int64_t nvec,
                                                              uint4* __restrict__ q) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += stride) {
    const uint2 p = packed[i];
    auto spread = [](uint32_t two) -> uint32_t {   // 2 packed bytes (low 16 bits) -> 4 codes
      const uint32_t b = (two & 0xFFu) | ((two & 0xFF00u) << 8);   // bytes at positions 0 and 2
      return (b & 0x000F000Fu) | ((b << 4) & 0x0F000F00u);
    };
    uint4 o;
    o.x = spread(p.x & 0xFFFFu);
    o.y = spread(p.x >> 16);
    o.z = spread(p.y & 0xFFFFu);
    o.w = spread(p.y >> 16);
    q[i] = o;
  }
}

__global__ __launch_bounds__(kThreads) void unpack_byte_kernel(const uint8_t* __restrict__ packed, int64_t nbytes,
                                                               uint8_t* __restrict__ q) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nbytes; i += stride) {
    const uint32_t b = packed[i];
    q[2 * i] = (uint8_t)(b & 15u);
    q[2 * i + 1] = (uint8_t)(b >> 4);
  }
}

__device__ __forceinline__ uint16_t bf16_bits_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);   // v_cvt_pk_bf16_f32: round to nearest even
}

__device__ __forceinline__ float dq(uint32_t code, float z, float s) {
  return ((float)code - z) * s;   // (q - zero) is exact; one float32 rounding of the product
}

// 4 packed bytes (8 codes of one group) per iteration; group % 8 == 0.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void dequant_vec_kernel(
    const uint32_t* __restrict__ packed, const float* __restrict__ scale,
    const uint8_t* __restrict__ zero, int64_t nwords, int64_t words_per_row, int32_t group,
    void* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const int64_t groups_per_row = words_per_row * 8 / group;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nwords; i += stride) {
    const int64_t row = i / words_per_row;
    const int64_t col = (i % words_per_row) * 8;            // first k of this word
    const int64_t gi = row * groups_per_row + col / group;
    const float s = scale[gi];
    const float z = (float)zero[gi];
    const uint32_t d = packed[i];
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = dq((d >> (4 * e)) & 15u, z, s);
    if (BF16) {
      uint4 o;
      o.x = bf16_bits_rne(v[0]) | ((uint32_t)bf16_bits_rne(v[1]) << 16);
      o.y = bf16_bits_rne(v[2]) | ((uint32_t)bf16_bits_rne(v[3]) << 16);
      o.z = bf16_bits_rne(v[4]) | ((uint32_t)bf16_bits_rne(v[5]) << 16);
      o.w = bf16_bits_rne(v[6]) | ((uint32_t)bf16_bits_rne(v[7]) << 16);
      reinterpret_cast<uint4*>(out)[i] = o;
    } else {
      float4* o = reinterpret_cast<float4*>(out) + 2 * i;
      o[0] = make_float4(v[0], v[1], v[2], v[3]);
      o[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
  }
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void dequant_byte_kernel(
    const uint8_t* __restrict__ packed, const float* __restrict__ scale,
    const uint8_t* __restrict__ zero, int64_t nbytes, int64_t bytes_per_row, int32_t group,
    void* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const int64_t groups_per_row = bytes_per_row * 2 / group;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nbytes; i += stride) {
    const int64_t row = i / bytes_per_row;
    const int64_t col = (i % bytes_per_row) * 2;
    const int64_t gi = row * groups_per_row + col / group;
    const float s = scale[gi];
    const float z = (float)zero[gi];
    const uint32_t b = packed[i];
    const float v0 = dq(b & 15u, z, s), v1 = dq(b >> 4, z, s);
    if (BF16) {
      uint16_t* o = reinterpret_cast<uint16_t*>(out);
      o[2 * i] = bf16_bits_rne(v0);
      o[2 * i + 1] = bf16_bits_rne(v1);
    } else {
      float* o = reinterpret_cast<float*>(out);
      o[2 * i] = v0;
      o[2 * i + 1] = v1;
    }
  }
}

// ---- signed int4 groups with float16 scales (tinyllm L8.5, "int4 per group") ----
// s16 = float16(amax / 7), the quotient a float32 division rounded once more
// to float16 (ties to even); codes rint(w / s16), the quotient again in
// float32 against the stored float16 value, clamped to -8..7; a group whose
// s16 is 0 gets codes 0.  Flag bit 0: a non-finite weight; bit 1: an s16 that
// overflows float16.  One thread per group.
__global__ __launch_bounds__(kThreads) void quantize_s16_kernel(
    const float* __restrict__ w, int64_t ngroups, int32_t group, int8_t* __restrict__ codes,
    uint16_t* __restrict__ scale16, uint32_t* __restrict__ flag) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t gi = (int64_t)blockIdx.x * kThreads + threadIdx.x; gi < ngroups; gi += stride) {
    const float* g = w + gi * group;
    bool bad = false;
    float am = 0.0f;
    for (int e = 0; e < group; ++e) {
      const float v = g[e];
      bad = bad || !finite_f32(v);
      am = fmaxf(am, fabsf(v));
    }
    if (bad) {
      atomicOr(flag, 1u);
      continue;
    }
    const _Float16 h = (_Float16)(am / 7.0f);   // float32 quotient, then float16 (round to nearest even)
    const float s = (float)h;
    if (!finite_f32(s)) {
      atomicOr(flag, 2u);
      continue;
    }
    int8_t* co = codes + gi * group;
    for (int e = 0; e < group; ++e) {
      const float c = s > 0.0f ? fminf(fmaxf(__builtin_rintf(g[e] / s), -8.0f), 7.0f) : 0.0f;
      co[e] = (int8_t)c;
    }
    scale16[gi] = __builtin_bit_cast(uint16_t, h);
  }
}

// Two signed codes per byte, 4-bit two's complement, even element low.  A code
// outside -8..7 sets the flag.
__global__ __launch_bounds__(kThreads) void pack_s4_kernel(const int8_t* __restrict__ c, int64_t nbytes,
                                                           uint8_t* __restrict__ packed,
                                                           uint32_t* __restrict__ flag) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  bool bad = false;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nbytes; i += stride) {
    const int lo = c[2 * i], hi = c[2 * i + 1];
    bad = bad || lo < -8 || lo > 7 || hi < -8 || hi > 7;
    packed[i] = (uint8_t)((lo & 15) | ((hi & 15) << 4));
  }
  if (bad) atomicOr(flag, 1u);
}

// Each nibble sign-extended to a byte (v >= 8 is v - 16).
__global__ __launch_bounds__(kThreads) void unpack_s4_kernel(const uint8_t* __restrict__ packed, int64_t nbytes,
                                                             int8_t* __restrict__ c) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nbytes; i += stride) {
    const int b = packed[i];
    c[2 * i] = (int8_t)(((b & 15) ^ 8) - 8);
    c[2 * i + 1] = (int8_t)(((b >> 4) ^ 8) - 8);
  }
}

// W_hat = c * s16: exact in float32 (a 4-bit integer times an 11-bit significand).
template <bool BF16>
__global__ __launch_bounds__(kThreads) void dequant_s16_kernel(
    const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scale16, int64_t nbytes,
    int64_t bytes_per_row, int32_t group, void* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const int64_t groups_per_row = bytes_per_row * 2 / group;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nbytes; i += stride) {
    const int64_t row = i / bytes_per_row;
    const int64_t col = (i % bytes_per_row) * 2;
    const float s = (float)__builtin_bit_cast(_Float16, scale16[row * groups_per_row + col / group]);
    const int b = packed[i];
    const float v0 = (float)(((b & 15) ^ 8) - 8) * s, v1 = (float)(((b >> 4) ^ 8) - 8) * s;
    if (BF16) {
      uint16_t* o = reinterpret_cast<uint16_t*>(out);
      o[2 * i] = bf16_bits_rne(v0);
      o[2 * i + 1] = bf16_bits_rne(v1);
    } else {
      float* o = reinterpret_cast<float*>(out);
      o[2 * i] = v0;
      o[2 * i + 1] = v1;
    }
  }
}

// ---- MXFP4: E2M1 codes in blocks of 32 with an E8M0 scale ----
// X = 2^(floor(log2 amax) - 2), stored as e = clamp(floor(log2 amax) - 2 + 127,
// 0, 254) (0 for a zero block); codes: w / X (exact) rounded to the nearest of
// 0, 0.5, 1, 1.5, 2, 3, 4, 6 with ties to the even code, saturating at 6, sign in
// bit 3.  One thread per block; flag bit 0: a non-finite weight.
__device__ __forceinline__ float e8m0_value(uint32_t e) {
  return e == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(e << 23);   // 2^(e - 127)
}

__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = fabsf(v);
  const uint32_t mag = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
                     : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.0f ? 6u : 7u;
  return mag | ((__float_as_uint(v) >> 28) & 8u);
}

__global__ __launch_bounds__(kThreads) void quantize_mx_kernel(const float* __restrict__ w, int64_t nblocks,
                                                               uint8_t* __restrict__ codes,
                                                               uint8_t* __restrict__ scales,
                                                               uint32_t* __restrict__ flag) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t bi = (int64_t)blockIdx.x * kThreads + threadIdx.x; bi < nblocks; bi += stride) {
    const float* g = w + bi * 32;
    bool bad = false;
    float am = 0.0f;
    for (int e = 0; e < 32; ++e) {
      bad = bad || !finite_f32(g[e]);
      am = fmaxf(am, fabsf(g[e]));
    }
    if (bad) {
      atomicOr(flag, 1u);
      continue;
    }
    const int ex = (int)((__float_as_uint(am) >> 23) & 0xFFu);   // biased exponent; 0 for zero and subnormals
    const uint32_t e = (uint32_t)min(max(ex - 2, 0), 254);
    const float inv = __uint_as_float((uint32_t)(254 - e) << 23);  // 1 / X = 2^(127 - e), exact
    uint8_t* co = codes + bi * 32;
    for (int k = 0; k < 32; ++k) co[k] = (uint8_t)e2m1_code(g[k] * inv);
    scales[bi] = (uint8_t)e;
  }
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void dequant_mx_kernel(const uint8_t* __restrict__ blocks,
                                                              const uint8_t* __restrict__ scales,
                                                              int64_t nbytes, void* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nbytes; i += stride) {
    const float x = e8m0_value(scales[i / 16]);
    const uint32_t b = blocks[i];
    auto val = [&](uint32_t c) {   // E2M1: exponent bits 2..1, mantissa bit 0 (subnormal at exponent 0)
      const uint32_t ee = (c >> 1) & 3u, mm = c & 1u;
      const float m = ee == 0 ? 0.5f * (float)mm : (float)(1u << (ee - 1u)) * (mm ? 1.5f : 1.0f);
      return ((c & 8u) ? -m : m) * x;
    };
    const float v0 = val(b & 15u), v1 = val(b >> 4);
    if (BF16) {
      uint16_t* o = reinterpret_cast<uint16_t*>(out);
      o[2 * i] = bf16_bits_rne(v0);
      o[2 * i + 1] = bf16_bits_rne(v1);
    } else {
      float* o = reinterpret_cast<float*>(out);
      o[2 * i] = v0;
      o[2 * i + 1] = v1;
    }
  }
}

// ---- Int4Linear: signed int4 codes with one float32 scale a row ----
// s = amax / 7 (a float32 division), codes clamp(rint(w / s), -8, 7) with the
// quotient in float32; a zero row gets s = 0 and codes 0.  One wave per row;
// flag bit 0: a non-finite weight.
__global__ __launch_bounds__(kThreads) void quantize_rows_kernel(const float* __restrict__ w, int64_t n,
                                                                 int64_t k, int8_t* __restrict__ codes,
                                                                 float* __restrict__ scale,
                                                                 uint32_t* __restrict__ flag) {
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (kThreads / 64);
  for (int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); row < n; row += waves) {
    const float* g = w + row * k;
    bool bad = false;
    float am = 0.0f;
    for (int64_t e = lane; e < k; e += 64) {
      bad = bad || !finite_f32(g[e]);
      am = fmaxf(am, fabsf(g[e]));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      am = fmaxf(am, __shfl_xor(am, off, 64));
      bad |= __shfl_xor((int)bad, off, 64) != 0;
    }
    if (bad) {
      if (lane == 0) atomicOr(flag, 1u);
      continue;
    }
    const float s = am / 7.0f;
    int8_t* co = codes + row * k;
    for (int64_t e = lane; e < k; e += 64)
      co[e] = (int8_t)(s > 0.0f ? fminf(fmaxf(__builtin_rintf(g[e] / s), -8.0f), 7.0f) : 0.0f);
    if (lane == 0) scale[row] = s;
  }
}

// W_hat = c * s, one float32 rounding.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void dequant_rows_kernel(const uint8_t* __restrict__ packed,
                                                                const float* __restrict__ scale,
                                                                int64_t nbytes, int64_t bytes_per_row,
                                                                void* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nbytes; i += stride) {
    const float s = scale[i / bytes_per_row];
    const int b = packed[i];
    const float v0 = (float)(((b & 15) ^ 8) - 8) * s, v1 = (float)(((b >> 4) ^ 8) - 8) * s;
    if (BF16) {
      uint16_t* o = reinterpret_cast<uint16_t*>(out);
      o[2 * i] = bf16_bits_rne(v0);
      o[2 * i + 1] = bf16_bits_rne(v1);
    } else {
      float* o = reinterpret_cast<float*>(out);
      o[2 * i] = v0;
      o[2 * i + 1] = v1;
    }
  }
}

// Packed 4-bit zero points (the MatMulNBits layout): per row, groups 2j and
// 2j+1 share byte j, group 2j in the low nibble; an odd row ends in a byte
// whose high nibble is 0.  One thread per output byte / per zero point.
__global__ __launch_bounds__(kThreads) void pack_zp_kernel(const uint8_t* __restrict__ zero, int64_t n,
                                                           int64_t ng, uint8_t* __restrict__ packed,
                                                           uint32_t* __restrict__ flag) {
  const int64_t nb = (ng + 1) / 2;
  bool bad = false;
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < n * nb; e += (int64_t)gridDim.x * kThreads) {
    const int64_t r = e / nb, j = e % nb;
    const uint32_t lo = zero[r * ng + 2 * j];
    const uint32_t hi = 2 * j + 1 < ng ? zero[r * ng + 2 * j + 1] : 0u;
    bad |= (lo | hi) > 15u;
    packed[e] = (uint8_t)((lo & 15u) | ((hi & 15u) << 4));
  }
  if (bad) atomicOr(flag, 1u);
}

__global__ __launch_bounds__(kThreads) void unpack_zp_kernel(const uint8_t* __restrict__ packed, int64_t n,
                                                             int64_t ng, uint8_t* __restrict__ zero) {
  const int64_t nb = (ng + 1) / 2;
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < n * ng; e += (int64_t)gridDim.x * kThreads) {
    const int64_t r = e / ng, g = e % ng;
    const uint32_t b = packed[r * nb + g / 2];
    zero[e] = (uint8_t)((g & 1) ? (b >> 4) : (b & 15u));
  }
}

unsigned grid_for(int64_t items) {
  const int64_t blocks = (items + kThreads - 1) / kThreads;
  return (unsigned)(blocks < 1 ? 1 : (blocks > 65536 ? 65536 : blocks));
}

// Prepared (fragment-ordered) weights: blocks of 16 outputs x 128 inputs
// (1024 bytes), tile-major then step-major; 16-byte slot l of block (t, s)
// holds row 16t + l % 16, packed bytes 64 s + 16 (l / 16) .. +16.  One thread
// per 16-byte slot; rows past n and bytes past k/2 are zero.
__global__ __launch_bounds__(kThreads) void prepare_kernel(const uint8_t* __restrict__ packed, int64_t n,
                                                           int64_t row_bytes, int64_t nsteps,
                                                           int64_t nslots, uint4* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nslots; i += stride) {
    const int64_t b = i >> 6;
    const int l = (int)(i & 63);
    const int64_t t = b / nsteps, st = b - t * nsteps;
    const int64_t row = 16 * t + (l & 15);
    const int64_t byte = 64 * st + 16 * (l >> 4);
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (row < n && byte < row_bytes) v = *reinterpret_cast<const uint4*>(packed + row * row_bytes + byte);
    out[i] = v;
  }
}

// Inverse: one thread per 16-byte chunk of the canonical rows.
__global__ __launch_bounds__(kThreads) void unprepare_kernel(const uint4* __restrict__ prepared,
                                                             int64_t row_bytes, int64_t nsteps,
                                                             int64_t nchunks, uint8_t* __restrict__ packed) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const int64_t cpr = row_bytes / 16;
  for (int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x; j < nchunks; j += stride) {
    const int64_t row = j / cpr, cc = j - row * cpr;
    const int64_t st = cc >> 2;
    const int l = (int)(16 * (cc & 3) + (row & 15));
    *reinterpret_cast<uint4*>(packed + row * row_bytes + 16 * cc) = prepared[((row >> 4) * nsteps + st) * 64 + l];
  }
}

}  // namespace

int32_t launch_quantize(const float* w, int64_t n, int64_t k, int32_t group, int32_t symmetric,
                        uint8_t* q, float* scale, uint8_t* zero, uint32_t* flag,
                        hipStream_t stream) {
  const int64_t ngroups = n * (k / group);
  if (ngroups == 0) return WOQ_OK;
  const bool coop = (group % 4 == 0) && group >= 4 && group <= 256 &&
                    ((group / 4) & (group / 4 - 1)) == 0 && aligned(w, 16);
  if (coop) {
    const int L = group / 4;
    const int32_t qa = aligned(q, 4) ? 1 : 0;
    const unsigned grid = grid_for(ngroups * L);
#define WOQ_Q(LL) \
    case LL: hipLaunchKernelGGL(quantize_coop_kernel<LL>, dim3(grid), dim3(kThreads), 0, stream, \
                                w, ngroups, symmetric, qa, q, scale, zero, flag); break;
    switch (L) {
      WOQ_Q(1) WOQ_Q(2) WOQ_Q(4) WOQ_Q(8) WOQ_Q(16) WOQ_Q(32) WOQ_Q(64)
      default: return WOQ_EUNSUPPORTED;
    }
#undef WOQ_Q
  } else {
    hipLaunchKernelGGL(quantize_thread_kernel, dim3(grid_for(ngroups)), dim3(kThreads), 0, stream,
                       w, ngroups, group, symmetric, q, scale, zero, flag);
  }
  return hip_status(hipGetLastError());
}

int32_t launch_pack(const uint8_t* q, int64_t count, uint8_t* packed, uint32_t* flag,
                    hipStream_t stream) {
  if (count == 0) return WOQ_OK;
  if (count % 16 == 0 && aligned(q, 16) && aligned(packed, 8)) {
    const int64_t nvec = count / 16;
    hipLaunchKernelGGL(pack_vec_kernel, dim3(grid_for(nvec)), dim3(kThreads), 0, stream,
                       reinterpret_cast<const uint4*>(q), nvec, reinterpret_cast<uint2*>(packed), flag);
  } else {
    hipLaunchKernelGGL(pack_byte_kernel, dim3(grid_for(count / 2)), dim3(kThreads), 0, stream,
                       q, count / 2, packed, flag);
  }
  return hip_status(hipGetLastError());
}

int32_t launch_unpack(const uint8_t* packed, int64_t count, uint8_t* q, hipStream_t stream) {
  if (count == 0) return WOQ_OK;
  if (count % 16 == 0 && aligned(q, 16) && aligned(packed, 8)) {
    const int64_t nvec = count / 16;
    hipLaunchKernelGGL(unpack_vec_kernel, dim3(grid_for(nvec)), dim3(kThreads), 0, stream,
                       reinterpret_cast<const uint2*>(packed), nvec, reinterpret_cast<uint4*>(q));
  } else {
    hipLaunchKernelGGL(unpack_byte_kernel, dim3(grid_for(count / 2)), dim3(kThreads), 0, stream,
                       packed, count / 2, q);
  }
  return hip_status(hipGetLastError());
}

int32_t launch_dequantize(const uint8_t* packed, const float* scale, const uint8_t* zero,
                          int64_t n, int64_t k, int32_t group, int32_t out_dtype, void* w_hat,
                          hipStream_t stream) {
  const int64_t nbytes = n * (k / 2);
  if (nbytes == 0) return WOQ_OK;
  const bool bf16 = out_dtype == WOQ_BF16;
  const bool vec = group % 8 == 0 && aligned(packed, 4) && aligned(w_hat, 16);
  if (vec) {
    const int64_t nwords = nbytes / 4, wpr = k / 8;
    if (bf16)
      hipLaunchKernelGGL(dequant_vec_kernel<true>, dim3(grid_for(nwords)), dim3(kThreads), 0, stream,
                         reinterpret_cast<const uint32_t*>(packed), scale, zero, nwords, wpr, group, w_hat);
    else
      hipLaunchKernelGGL(dequant_vec_kernel<false>, dim3(grid_for(nwords)), dim3(kThreads), 0, stream,
                         reinterpret_cast<const uint32_t*>(packed), scale, zero, nwords, wpr, group, w_hat);
  } else {
    if (bf16)
      hipLaunchKernelGGL(dequant_byte_kernel<true>, dim3(grid_for(nbytes)), dim3(kThreads), 0, stream,
                         packed, scale, zero, nbytes, k / 2, group, w_hat);
    else
      hipLaunchKernelGGL(dequant_byte_kernel<false>, dim3(grid_for(nbytes)), dim3(kThreads), 0, stream,
                         packed, scale, zero, nbytes, k / 2, group, w_hat);
  }
  return hip_status(hipGetLastError());
}

int32_t launch_prepare(const uint8_t* packed, int64_t n, int64_t k, uint8_t* prepared,
                       hipStream_t stream) {
  const int64_t nsteps = (k + 127) / 128;
  const int64_t nslots = (n + 15) / 16 * nsteps * 64;
  if (nslots == 0) return WOQ_OK;
  hipLaunchKernelGGL(prepare_kernel, dim3(grid_for(nslots)), dim3(kThreads), 0, stream,
                     packed, n, k / 2, nsteps, nslots, reinterpret_cast<uint4*>(prepared));
  return hip_status(hipGetLastError());
}

int32_t launch_unprepare(const uint8_t* prepared, int64_t n, int64_t k, uint8_t* packed,
                         hipStream_t stream) {
  const int64_t nsteps = (k + 127) / 128;
  const int64_t nchunks = n * (k / 32);
  if (nchunks == 0) return WOQ_OK;
  hipLaunchKernelGGL(unprepare_kernel, dim3(grid_for(nchunks)), dim3(kThreads), 0, stream,
                     reinterpret_cast<const uint4*>(prepared), k / 2, nsteps, nchunks, packed);
  return hip_status(hipGetLastError());
}

int32_t launch_quantize_s16(const float* w, int64_t n, int64_t k, int32_t group, int8_t* codes,
                            uint16_t* scale16, uint32_t* flag, hipStream_t stream) {
  const int64_t ngroups = n * (k / group);
  if (ngroups == 0) return WOQ_OK;
  hipLaunchKernelGGL(quantize_s16_kernel, dim3(grid_for(ngroups)), dim3(kThreads), 0, stream,
                     w, ngroups, group, codes, scale16, flag);
  return hip_status(hipGetLastError());
}

int32_t launch_pack_s4(const int8_t* c, int64_t count, uint8_t* packed, uint32_t* flag,
                       hipStream_t stream) {
  if (count == 0) return WOQ_OK;
  hipLaunchKernelGGL(pack_s4_kernel, dim3(grid_for(count / 2)), dim3(kThreads), 0, stream,
                     c, count / 2, packed, flag);
  return hip_status(hipGetLastError());
}

int32_t launch_unpack_s4(const uint8_t* packed, int64_t count, int8_t* c, hipStream_t stream) {
  if (count == 0) return WOQ_OK;
  hipLaunchKernelGGL(unpack_s4_kernel, dim3(grid_for(count / 2)), dim3(kThreads), 0, stream,
                     packed, count / 2, c);
  return hip_status(hipGetLastError());
}

int32_t launch_dequantize_s16(const uint8_t* packed, const uint16_t* scale16, int64_t n, int64_t k,
                              int32_t group, int32_t out_dtype, void* w_hat, hipStream_t stream) {
  const int64_t nbytes = n * (k / 2);
  if (nbytes == 0) return WOQ_OK;
  if (out_dtype == WOQ_BF16)
    hipLaunchKernelGGL(dequant_s16_kernel<true>, dim3(grid_for(nbytes)), dim3(kThreads), 0, stream,
                       packed, scale16, nbytes, k / 2, group, w_hat);
  else
    hipLaunchKernelGGL(dequant_s16_kernel<false>, dim3(grid_for(nbytes)), dim3(kThreads), 0, stream,
                       packed, scale16, nbytes, k / 2, group, w_hat);
  return hip_status(hipGetLastError());
}

int32_t launch_quantize_mx(const float* w, int64_t n, int64_t k, uint8_t* codes, uint8_t* scales,
                           uint32_t* flag, hipStream_t stream) {
  const int64_t nblocks = n * (k / 32);
  if (nblocks == 0) return WOQ_OK;
  hipLaunchKernelGGL(quantize_mx_kernel, dim3(grid_for(nblocks)), dim3(kThreads), 0, stream,
                     w, nblocks, codes, scales, flag);
  return hip_status(hipGetLastError());
}

int32_t launch_dequantize_mx(const uint8_t* blocks, const uint8_t* scales, int64_t n, int64_t k,
                             int32_t out_dtype, void* w_hat, hipStream_t stream) {
  const int64_t nbytes = n * (k / 2);
  if (nbytes == 0) return WOQ_OK;
  if (out_dtype == WOQ_BF16)
    hipLaunchKernelGGL(dequant_mx_kernel<true>, dim3(grid_for(nbytes)), dim3(kThreads), 0, stream,
                       blocks, scales, nbytes, w_hat);
  else
    hipLaunchKernelGGL(dequant_mx_kernel<false>, dim3(grid_for(nbytes)), dim3(kThreads), 0, stream,
                       blocks, scales, nbytes, w_hat);
  return hip_status(hipGetLastError());
}

int32_t launch_quantize_rows(const float* w, int64_t n, int64_t k, int8_t* codes, float* scale,
                             uint32_t* flag, hipStream_t stream) {
  if (n == 0) return WOQ_OK;
  const int64_t blocks = (n + kThreads / 64 - 1) / (kThreads / 64);
  hipLaunchKernelGGL(quantize_rows_kernel, dim3((unsigned)(blocks > 65536 ? 65536 : blocks)), dim3(kThreads), 0,
                     stream, w, n, k, codes, scale, flag);
  return hip_status(hipGetLastError());
}

int32_t launch_dequantize_rows(const uint8_t* packed, const float* scale, int64_t n, int64_t k,
                               int32_t out_dtype, void* w_hat, hipStream_t stream) {
  const int64_t nbytes = n * (k / 2);
  if (nbytes == 0) return WOQ_OK;
  if (out_dtype == WOQ_BF16)
    hipLaunchKernelGGL(dequant_rows_kernel<true>, dim3(grid_for(nbytes)), dim3(kThreads), 0, stream,
                       packed, scale, nbytes, k / 2, w_hat);
  else
    hipLaunchKernelGGL(dequant_rows_kernel<false>, dim3(grid_for(nbytes)), dim3(kThreads), 0, stream,
                       packed, scale, nbytes, k / 2, w_hat);
  return hip_status(hipGetLastError());
}

int32_t launch_pack_zero_points(const uint8_t* zero, int64_t n, int64_t ngroups, uint8_t* packed, uint32_t* flag,
                                hipStream_t stream) {
  if (n == 0 || ngroups == 0) return WOQ_OK;
  hipLaunchKernelGGL(pack_zp_kernel, dim3(grid_for(n * ((ngroups + 1) / 2))), dim3(kThreads), 0, stream, zero, n,
                     ngroups, packed, flag);
  return hip_status(hipGetLastError());
}

int32_t launch_unpack_zero_points(const uint8_t* packed, int64_t n, int64_t ngroups, uint8_t* zero,
                                  hipStream_t stream) {
  if (n == 0 || ngroups == 0) return WOQ_OK;
  hipLaunchKernelGGL(unpack_zp_kernel, dim3(grid_for(n * ngroups)), dim3(kThreads), 0, stream, packed, n, ngroups,
                     zero);
  return hip_status(hipGetLastError());
}

}  // namespace woq
