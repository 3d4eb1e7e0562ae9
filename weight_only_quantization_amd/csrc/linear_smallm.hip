// Small-M linear path with the activations shared through LDS: y = x .
// dequant(W)^T + bias for group-wise 4-bit weights (linnet docs
// "Quantization", std.quant table, linear_int4_groups), for 5 to 64
// activation rows (by default from 16, or from 8 with groups of 128 or more
// when K >= 8192 or N <= 1024, on layers under 800 tiles of 16 rows).  At these row counts the layer is bound by the weight
// stream, and what decides the time is how little else moves: the
// activations are read by every workgroup that covers a K range, so each
// workgroup owns many weight rows and only a slice of K.
//
// * Workgroup (b, r) owns 8 T tiles of 16 weight rows (wave w takes tiles
//   8 T b + T w .. + T) and the K range r of S 128-input steps.  Every
//   workgroup of a range reads the same activation slice; ranges go round
//   robin over the workgroup index, so with 2, 4 or 8 ranges each XCD (one L2)
//   sees the slices of few ranges.
// * The workgroup loads its activation slice once, 16 bytes a thread, rows
//   past M and inputs past K as zero, and writes it to LDS in the MFMA
//   operand order of the 16x16x32 instruction (chunk e of lane (q, c) of
//   activation tile mt at step i holds the 8 inputs its weight dword e meets,
//   in the unpacker's pair order), so that an operand is one contiguous
//   ds_read_b128; each 16-byte slot is XOR-swizzled by (step, chunk) so the
//   slice stores spread over all banks.  The sums of x over every group piece come from the same
//   loads: 8 values per thread in a fixed order, then a butterfly of lane
//   exchanges (each lane of a piece ends with the same bits).
// * Every wave issues its slice loads, then its (scale, zero) loads, then all
//   of its weight loads (T tiles x S steps, 16 bytes a lane: lane (q, c) reads
//   inputs [32q, 32q + 32) of row c of a step), and only then waits, for its
//   slice loads alone, to store the slice: the whole layer is in flight early.
// * Per step and tile: nibbles become bf16 (128 + code) with one AND-OR per
//   pair; per group piece the MFMAs give sum x (128 + code), and the fold
//   acc += scale * (that - (128 + zero) * sum x) applies the zero point and
//   scale (the dequantization (q - zero) * scale of each weight, never
//   materialized).  Groups under 128 inputs transpose the weight dwords
//   across lane groups so each MFMA stays inside one group; MXFP4 converts
//   each lane's block with its E8M0 scale (exact) and needs no fold.
// * (scale, -(128 + zero)) pairs of the wave's rows and the range's groups
//   are staged per wave in LDS after the slice barrier (a wave reads only its
//   own area, so its stores need no barrier).
// * One K range: bias added, y stored.  More: the float32 partial tile goes
//   to slice r of a [ranges][M][N] workspace buffer and a second pass adds
//   the slices in range order (the same bits on every run), adds the bias
//   and converts.
#include "woq_internal.h"
#include "mfma_common.h"

namespace woq {
namespace {

constexpr int kStepK = 128;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr uint32_t kOffsetOOB = 0x80000000u;   // a buffer offset no descriptor covers
constexpr int kStageBatch = 8;                 // staged (scale, zero) entries per lane and batch
constexpr uint32_t kSignFlip = 0x88888888u;    // two's complement nibble v -> unsigned v ^ 8 (zero point 8)

struct SmParams {
  const uint16_t* x;      // bf16 [M, K] (possibly the gathered copy)
  const uint8_t* packed;  // [N, K/2], or prepared 1 KB blocks
  const void* scale;      // float32, float16 for signed codes, E8M0 bytes for MXFP4
  const uint8_t* zero;    // unused for signed codes and MXFP4
  const float* bias;
  void* y;                // [M, N] when there is one K range
  float* part;            // [ranges][M][N] float32 partials when there are more
  int32_t m, n, k, y_bf16;
  int32_t nsteps, ngroups, prepared, ranges;
  uint32_t nib_mask, nib_offset;
  int32_t row_scale;      // signed codes with one float32 scale a row (Int4Linear)
  int32_t zp4;            // zero points packed two a byte (group 2j in the low nibble of byte j)
  int32_t zrow;           // zero-point bytes per row
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, (int)kRsrcWord3);
}

__device__ __forceinline__ u32x4_t bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// Sum of 8 bf16 values (natural order, 4 dwords) in float32, in a fixed order.
__device__ __forceinline__ float sum8_bf16(u32x4_t v) {
  float s[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
    s[d] = __uint_as_float(v[d] << 16) + __uint_as_float(v[d] & 0xFFFF0000u);
  return (s[0] + s[1]) + (s[2] + s[3]);
}

// 16-byte slot of lane `l`'s operand chunk e of step i inside its kilobyte.
// One store instruction of the slice writes a single activation row (fixed
// lane l mod 16) across 4 steps and the 16 (lane group, chunk) pairs; without
// the XOR all 64 of its chunks would fall in the same 4 of the 64 LDS banks.
// The read of an operand (fixed i and e, every lane) stays one contiguous,
// conflict-free kilobyte.
__device__ __forceinline__ int slot(int i, int e, int l) { return l ^ ((e + 4 * i) & 15); }

template <int G, int S, bool MX>
struct SmShape {
  static constexpr int GB = G >= 128 ? 4 : G / 32;   // 32-input blocks per group piece
  static constexpr int NP = 4 / GB;                  // group pieces per step
  static constexpr int NGW = S * kStepK / G;         // groups (MXFP4: blocks) of one K range
};

// G: group size; MT: 16-row activation tiles; T: 16-row weight tiles per
// wave; FMT: weight format (kFmtS16: signed codes with float16 scales, run as
// unsigned codes v ^ 8 with zero point 8; kFmtMX: MXFP4); S: steps per range.
template <int G, int MT, int T, int FMT, int S>
__global__ __launch_bounds__(kThreads) void sm_kernel(SmParams p) {
  constexpr bool S16 = FMT == kFmtS16, MX = FMT == kFmtMX;
  static_assert(!MX || G == 32, "MXFP4 blocks hold 32 inputs");
  using Sh = SmShape<G, S, MX>;
  constexpr int GB = Sh::GB, NP = Sh::NP, NGW = Sh::NGW;
  constexpr int PC = 4 * GB;                 // 16-byte activation chunks per group piece
  constexpr bool kTranspose = GB < 4 && !MX;
  constexpr int kXC = MT * S * 256 / kThreads;   // activation chunks per thread
  static_assert(kXC * kThreads == MT * S * 256, "whole chunks per thread");
  constexpr int kRowChunks = 16 * S;         // 16-byte chunks of one activation row in a range
  constexpr int kXsOff = MT * S * 4096;
  constexpr int kSzOff = kXsOff + (MX ? 0 : MT * S * NP * 64);
  constexpr int kSzEntries = 16 * T * NGW;
  constexpr int kSzWave = kSzEntries * 8;
  constexpr int kSzBatches = (kSzEntries + 64 * kStageBatch - 1) / (64 * kStageBatch);
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4;
  const int c = lane & 15;
  const int M = p.m, N = p.n, K = p.k;
  const int nsteps = p.nsteps;
  const int range = __builtin_amdgcn_readfirstlane((int)(blockIdx.x % (unsigned)p.ranges));
  const int nb = __builtin_amdgcn_readfirstlane((int)(blockIdx.x / (unsigned)p.ranges));
  const int s0 = range * S;
  const int live = __builtin_amdgcn_readfirstlane(min(S, nsteps - s0));
  const int tile0 = __builtin_amdgcn_readfirstlane((nb * kWaves + wave) * T);
  const int rows = __builtin_amdgcn_readfirstlane(max(0, min(16 * T, N - 16 * tile0)));
  const uint32_t row_bytes = (uint32_t)K / 2;
  const bool prep = p.prepared != 0;

  // 1. the activation slice: chunk J = thread + 512 j is row J / (16 S),
  //    inputs s0 * 128 + 8 (J % (16 S)) .. + 8; issued first, so waiting for
  //    them waits for nothing else.
  const __amdgpu_buffer_rsrc_t rx = rsrc(p.x, (uint32_t)M * (uint32_t)K * 2u);
  u32x4_t xv[kXC];
#pragma unroll
  for (int j = 0; j < kXC; ++j) {
    const int J = (int)threadIdx.x + kThreads * j;
    const int r = J / kRowChunks, kc = J % kRowChunks;
    const int kin = s0 * kStepK + 8 * kc;
    const bool in = r < M && kin < K;   // K is a multiple of 32: the 8 inputs are all in range
    xv[j] = bload16(rx, in ? (uint32_t)(r * K + kin) * 2u : kOffsetOOB);
  }

  // 2. (scale, -(128 + zero)) of this wave's rows and the range's groups,
  //    [row][group] float pairs; groups past the row read zero.
  const int gb = s0 * kStepK / G;   // first group of the range (ranges start on group boundaries)
  const bool row_scale = S16 && p.row_scale != 0;   // uniform
  const uint32_t sbytes = MX ? 1u : (S16 && !row_scale ? 2u : 4u);
  const int32_t srow = row_scale ? 1 : p.ngroups;
  const __amdgpu_buffer_rsrc_t rs =
      rsrc(static_cast<const char*>(p.scale) + (int64_t)tile0 * 16 * srow * sbytes, (uint32_t)(rows * srow) * sbytes);
  const int zrow = p.zrow;
  const bool zp4 = p.zp4 != 0;   // uniform
  const __amdgpu_buffer_rsrc_t rz = rsrc(S16 || MX ? nullptr : p.zero + (int64_t)tile0 * 16 * zrow,
                                         S16 || MX ? 0u : (uint32_t)(rows * zrow));
  uint32_t sv[kSzBatches][kStageBatch];
  uint32_t zv[kSzBatches][kStageBatch];
  uint32_t zs[kSzBatches][kStageBatch];   // bit offset of the zero point in its loaded byte
#pragma unroll
  for (int bt = 0; bt < kSzBatches; ++bt) {
#pragma unroll
    for (int b = 0; b < kStageBatch; ++b) {
      const int e = lane + 64 * (bt * kStageBatch + b);
      const int r = e / NGW, g = e % NGW;
      const bool in = e < kSzEntries && r < rows && gb + g < p.ngroups;
      const uint32_t idx = (uint32_t)(r * p.ngroups + gb + g);
      if constexpr (MX) {
        sv[bt][b] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs, in ? idx : kOffsetOOB, 0, 0);
        zv[bt][b] = 0u;
        zs[bt][b] = 0u;
      } else if constexpr (S16) {
        if (row_scale)
          sv[bt][b] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, in ? (uint32_t)r * 4u : kOffsetOOB, 0, 0);
        else
          sv[bt][b] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, in ? idx * 2u : kOffsetOOB, 0, 0);
        zv[bt][b] = 8u;
        zs[bt][b] = 0u;
      } else {
        sv[bt][b] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, in ? idx * 4u : kOffsetOOB, 0, 0);
        const uint32_t zidx = zp4 ? (uint32_t)(r * zrow + ((gb + g) >> 1)) : idx;
        zs[bt][b] = zp4 ? 4u * (uint32_t)((gb + g) & 1) : 0u;
        zv[bt][b] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rz, in ? zidx : kOffsetOOB, 0, 0);
      }
    }
  }

  // 3. the weight stream: all S steps of the T tiles.  Canonical rows [N, K/2]
  //    (lane (q, c): row c, bytes 64 s + 16 q of step s) or prepared 1 KB
  //    blocks (slot = lane); rows past N and steps past the range read zero.
  const int wtiles = (rows + 15) / 16;
  const __amdgpu_buffer_rsrc_t rb =
      prep ? rsrc(p.packed + (int64_t)tile0 * nsteps * 1024, (uint32_t)(wtiles * nsteps) * 1024u)
           : rsrc(p.packed + (int64_t)tile0 * 16 * row_bytes, (uint32_t)rows * row_bytes);
  const uint32_t wstep = prep ? 1024u : 64u;
  u32x4_t wb[S][T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const uint32_t woff = prep ? (uint32_t)(t * nsteps + s0) * 1024u + 16u * (uint32_t)lane
                               : (uint32_t)(16 * t + c) * row_bytes + (uint32_t)s0 * 64u + 16u * (uint32_t)q;
#pragma unroll
    for (int i = 0; i < S; ++i)
      wb[i][t] = bload16(rb, i < live ? woff + (uint32_t)i * wstep : kOffsetOOB);
  }


  // 4. activations to LDS in operand order, and their piece sums
  float* xsl = reinterpret_cast<float*>(lds + kXsOff);
#pragma unroll
  for (int j = 0; j < kXC; ++j) {
    const int J = (int)threadIdx.x + kThreads * j;
    const int r = J / kRowChunks, kc = J % kRowChunks;
    const int i = kc >> 4, u = kc & 15;
    const u32x4_t v = xv[j];
    if constexpr (!MX) {
      float sm = sum8_bf16(v);
#pragma unroll
      for (int off = PC / 2; off >= 1; off >>= 1) sm += __shfl_xor(sm, off);
      if (kc % PC == 0) xsl[(((r >> 4) * S + i) * NP + u / PC) * 16 + (r & 15)] = sm;
    }
    const int qq = kTranspose ? (u & 3) : (u >> 2);
    const int e = kTranspose ? (u >> 2) : (u & 3);
    *reinterpret_cast<u32x4_t*>(lds + (((r >> 4) * S + i) * 4 + e) * 1024 + slot(i, e, (qq << 4) + (r & 15)) * 16) =
        MX ? v : __builtin_bit_cast(u32x4_t, pair_order(v));
  }

  // 5. the slice is complete once every wave's LDS writes are (LDS-only
  //    fences: the weight loads in flight are not waited for here)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  if (rows == 0) return;   // uniform: a wave past N only helped load the slice

  // 6. the staged pairs (each wave reads only its own area: no barrier)
  unsigned char* szl = lds + kSzOff + wave * kSzWave;
#pragma unroll
  for (int bt = 0; bt < kSzBatches; ++bt) {
#pragma unroll
    for (int b = 0; b < kStageBatch; ++b) {
      const int e = lane + 64 * (bt * kStageBatch + b);
      if (e < kSzEntries) {
        if constexpr (MX) {   // (2^(e - 127), unused)
          const uint32_t eb = sv[bt][b] & 0xFFu;
          const float sc = __uint_as_float(eb == 0 ? 0x00400000u : eb << 23);
          *reinterpret_cast<f32x2_t*>(szl + e * 8) = f32x2_t{sc, 0.f};
        } else {
          const float sc = S16 && !row_scale ? (float)__builtin_bit_cast(_Float16, (uint16_t)sv[bt][b])
                                             : __builtin_bit_cast(float, sv[bt][b]);
          const uint32_t zq = __builtin_amdgcn_ubfe(zv[bt][b], zs[bt][b], zp4 ? 4u : 8u);
          *reinterpret_cast<f32x2_t*>(szl + e * 8) = f32x2_t{sc, -(kNibOffset + (float)zq)};
        }
      }
    }
  }


  // 7. the steps
  const uint32_t nib_offset = vgpr_copy(p.nib_offset);
  f32x4_t acc[MT][T];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < T; ++t) acc[mt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < S; ++i) {
    if (i >= live) break;   // uniform
    bf16x8_t af[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        af[mt][e] = *reinterpret_cast<const bf16x8_t*>(lds + ((mt * S + i) * 4 + e) * 1024 + slot(i, e, lane) * 16);
    if constexpr (MX) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const float xs = reinterpret_cast<const f32x2_t*>(szl + ((16 * t + c) * NGW + 4 * i + q) * 8)->x;
        bf16x8_t bw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) bw[e] = fp4x8_to_bf16(wb[i][t][e], xs);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[mt][t] = mfma_bf16(af[mt][e], bw[e], acc[mt][t]);
      }
      continue;
    }
    // piece sums of rows 16 mt + 4q + r: the accumulator layout
    f32x4_t xsum[MT][NP];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int pc = 0; pc < NP; ++pc)
        xsum[mt][pc] = *reinterpret_cast<const f32x4_t*>(xsl + ((mt * S + i) * NP + pc) * 16 + 4 * q);
#pragma unroll
    for (int t = 0; t < T; ++t) {
      bf16x8_t bw[4];
      if constexpr (kTranspose) {
        uint32_t d0 = wb[i][t][0], d1 = wb[i][t][1], d2 = wb[i][t][2], d3 = wb[i][t][3];
        if constexpr (S16) {
          d0 ^= kSignFlip; d1 ^= kSignFlip; d2 ^= kSignFlip; d3 ^= kSignFlip;
        }
        transpose4_lanegroups(d0, d1, d2, d3);
        bw[0] = unpack_codes(d0, p.nib_mask, nib_offset);
        bw[1] = unpack_codes(d1, p.nib_mask, nib_offset);
        bw[2] = unpack_codes(d2, p.nib_mask, nib_offset);
        bw[3] = unpack_codes(d3, p.nib_mask, nib_offset);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          bw[e] = unpack_codes(S16 ? wb[i][t][e] ^ kSignFlip : wb[i][t][e], p.nib_mask, nib_offset);
      }
#pragma unroll
      for (int pc = 0; pc < NP; ++pc) {
        const int g = (i * kStepK + 32 * GB * pc) / G;   // group inside the range
        const f32x2_t sz = *reinterpret_cast<const f32x2_t*>(szl + ((16 * t + c) * NGW + g) * 8);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          f32x4_t cg = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int e = 0; e < GB; ++e) cg = mfma_bf16(af[mt][pc * GB + e], bw[pc * GB + e], cg);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[mt][t][r] = fmaf(sz.x, fmaf(sz.y, xsum[mt][pc][r], cg[r]), acc[mt][t][r]);
        }
      }
    }
  }

  // 8. results: lane (q, c) of tile t holds rows 16 mt + 4q + r of output
  //    16 (tile0 + t) + c
  const bool one = p.ranges == 1;
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int n = (tile0 + t) * 16 + c;
    if (n >= N) continue;
    const float bv = one && p.bias ? p.bias[n] : 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * mt + 4 * q + r;
        if (row >= M) continue;
        const float o = acc[mt][t][r] + bv;
        if (!one)
          p.part[((int64_t)range * M + row) * N + n] = o;
        else if (p.y_bf16)
          reinterpret_cast<uint16_t*>(p.y)[(int64_t)row * N + n] = f32_to_bf16_bits(o);
        else
          reinterpret_cast<float*>(p.y)[(int64_t)row * N + n] = o;
      }
    }
  }
}

template <int G, int MT, int T, int FMT, int S>
int32_t launch_one(const SmParams& sp, const LinearPlan& pl, size_t lds, hipStream_t stream) {
  auto kern = sm_kernel<G, MT, T, FMT, S>;
  if (lds > 64 * 1024) {
    static std::atomic<uint64_t> raised{0};   // per instantiation, one bit per device
    const int32_t st = raise_lds_limit(reinterpret_cast<const void*>(kern), 160 * 1024, raised);
    if (st != WOQ_OK) return st;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)pl.grid), dim3(kThreads), lds, stream, sp);
  return hip_status(hipGetLastError());
}

template <int G, int MT, int FMT, int S>
int32_t dispatch_t(const SmParams& sp, const LinearPlan& pl, size_t lds, hipStream_t s) {
  switch (pl.ns) {
    case 1: return launch_one<G, MT, 1, FMT, S>(sp, pl, lds, s);
    case 2: return launch_one<G, MT, 2, FMT, S>(sp, pl, lds, s);
    default: return WOQ_EUNSUPPORTED;
  }
}

template <int G, int MT, int FMT>
int32_t dispatch_s(const SmParams& sp, const LinearPlan& pl, size_t lds, hipStream_t s) {
  switch (pl.cnt) {
    case 4: return dispatch_t<G, MT, FMT, 4>(sp, pl, lds, s);
    case 8: return dispatch_t<G, MT, FMT, 8>(sp, pl, lds, s);
    default: return WOQ_EUNSUPPORTED;
  }
}

template <int G, int FMT>
int32_t dispatch_mt(const SmParams& sp, const LinearPlan& pl, size_t lds, hipStream_t s) {
  switch (pl.mt) {
    case 1: return dispatch_s<G, 1, FMT>(sp, pl, lds, s);
    case 2: return dispatch_s<G, 2, FMT>(sp, pl, lds, s);
    case 4: return dispatch_s<G, 4, FMT>(sp, pl, lds, s);
    default: return WOQ_EUNSUPPORTED;
  }
}

}  // namespace

size_t sm_lds_bytes(int mt, int steps, int tiles, int32_t group, bool mx) {
  const int gb = group >= 128 ? 4 : group / 32;
  const int np = 4 / gb;
  const int ngw = steps * kStepK / group;
  return (size_t)mt * steps * 4096 + (mx ? 0 : (size_t)mt * steps * np * 64) + (size_t)kWaves * 16 * tiles * ngw * 8;
}

int32_t launch_sm(const LinearArgs& a, const LinearPlan& pl, hipStream_t stream) {
  const size_t lds = sm_lds_bytes(pl.mt, pl.cnt, pl.ns, a.group, a.mx != 0);
  SmParams sp{a.x, a.packed,
              a.mx ? static_cast<const void*>(a.scale8)
                   : a.sym16 && !a.row_scale ? static_cast<const void*>(a.scale16) : static_cast<const void*>(a.scale),
              a.zero, a.bias, a.y, a.part, a.m, a.n, a.k, a.y_bf16,
              (a.k + kStepK - 1) / kStepK, a.k / a.group, a.prepared, pl.splits,
              kNibPairMask, kBf16Offset2, a.row_scale, a.zp4,
              a.zp4 ? (a.k / a.group + 1) / 2 : a.k / a.group};
  int32_t st;
  if (a.mx) {
    st = a.group == 32 ? dispatch_mt<32, kFmtMX>(sp, pl, lds, stream) : WOQ_EUNSUPPORTED;
  } else if (a.sym16) {
    switch (a.group) {
      case 32: st = dispatch_mt<32, kFmtS16>(sp, pl, lds, stream); break;
      case 64: st = dispatch_mt<64, kFmtS16>(sp, pl, lds, stream); break;
      case 128: st = dispatch_mt<128, kFmtS16>(sp, pl, lds, stream); break;
      case 256: st = dispatch_mt<256, kFmtS16>(sp, pl, lds, stream); break;
      default: st = WOQ_EUNSUPPORTED;
    }
  } else {
    switch (a.group) {
      case 32: st = dispatch_mt<32, kFmtU4>(sp, pl, lds, stream); break;
      case 64: st = dispatch_mt<64, kFmtU4>(sp, pl, lds, stream); break;
      case 128: st = dispatch_mt<128, kFmtU4>(sp, pl, lds, stream); break;
      case 256: st = dispatch_mt<256, kFmtU4>(sp, pl, lds, stream); break;
      default: st = WOQ_EUNSUPPORTED;
    }
  }
  if (st != WOQ_OK || pl.splits <= 1) return st;
  return launch_splitk_reduce(a.part, pl.splits, a.m, a.n, a.bias, a.y_bf16, a.y, stream);
}

}  // namespace woq
