// Decode path (1 <= m <= 4): y = x . dequant(W)^T + bias for group-wise
// 4-bit weights (linnet docs "Quantization", std.quant table,
// linear_int4_groups).  The layer is bound by the weight stream, and at these
// sizes a wave's own instruction stream is the other limit: a lone wave issues
// about one instruction every four cycles, so every instruction per 128-input
// step, and every instruction a wave runs before and after its steps, shows
// up in the time per call.  The kernel is organised around that:
//
// * A workgroup owns 16 weight rows (outputs).  Its W waves split K into
//   contiguous ranges of `cnt` 128-input steps, and each wave stages only what
//   its own steps need: its slice of the activations (in LDS, already in the
//   unpacker's slot order, zero past K), the sum of that slice over every
//   group piece, and the (scale, -(128 + zero)) pairs of its groups.  No wave
//   waits for another until the final reduction.
// * Per step and lane one 16-byte buffer load of the lane's weight row (lane
//   group q reads inputs [k0+32q, k0+32q+32)); loads past the wave's range use
//   an offset no buffer descriptor covers and read zero, so the ring of PF
//   steps has no branches and exact vmcnt waits.
// * Nibbles become bf16 (128 + code) with one AND-OR per pair and feed
//   v_mfma_f32_16x16x32_bf16.  For groups of 128 and more MFMA e takes dword e
//   of every lane's load (inputs k0+32q+8e .. +8); smaller groups regroup the
//   dwords with a 4x4 transpose across lane groups so that each MFMA stays in
//   one group.
// * Per group piece: acc += scale * (sum + (-(128 + zero)) * piece_sum_of_x).
// * The waves' partial sums of the rows that exist (m <= 4) meet in LDS and
//   one wave adds the bias and stores.
#include "woq_internal.h"
#include "mfma_common.h"

namespace woq {
namespace {

constexpr int kStepK = 128;
constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr uint32_t kOffsetOOB = 0x80000000u;   // a buffer offset no descriptor covers
constexpr int kSzPerBatch = 16;    // (scale, zero) entries per row staged by one load batch
constexpr uint32_t kSignFlip = 0x88888888u;   // two's complement nibble v -> unsigned v ^ 8 (zero point 8)

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// One weight matrix of a launch.  A launch serves up to kMaxGrouped matrices
// that share the activations (and so K and the group size): workgroups
// [tile_begin, next tile_begin) take the 16-row tiles of matrix i.
struct GemvProblem {
  const uint8_t* packed;
  const void* scale;      // float32, or float16 for signed codes
  const uint8_t* zero;    // unused for signed codes
  const float* bias;
  void* y;
  int32_t n;
  int32_t tile_begin;
};

struct GemvParams {
  const uint16_t* x;
  int32_t m, k, y_bf16;
  int32_t nsteps;       // 128-input steps covering k
  int32_t cnt;          // steps owned by each wave, a multiple of 4
  int32_t ngroups;      // groups per row
  int32_t group_shift;  // log2(group)
  int32_t x_batches;    // activation staging batches of XL loads per lane
  int32_t z_bytewise;   // 1 when a row's groups do not fill whole dwords
  int32_t prepared;     // 1: weights in the prepared layout
  int32_t wave_lds;     // LDS bytes per wave
  int32_t xs_off;       // offsets inside a wave's region: piece sums
  int32_t sz_off;       //   (scale, -(128 + zero)) pairs
  int32_t red_off;      // offset of the cross-wave reduction area
  // The nibble mask and the bf16 offset pattern arrive as arguments so they sit
  // in registers: one v_and_or_b32 per pair then expands two codes.
  uint32_t nib_mask, nib_offset;
  int32_t row_scale;    // signed codes with one float32 scale a row (Int4Linear)
  int32_t nprob;
  GemvProblem prob[kMaxGrouped];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, (int)kRsrcWord3);
}

__device__ __forceinline__ u32x4_t bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
// Prepared weights are read once per call as whole 1 KB blocks: cache policy
// nt (non-temporal) with sc1 (agent scope) streams them through L2 without
// displacing the activations, and skips the compute unit's vector L1.
// Canonical rows are read 64 bytes a step, so each cache line serves two
// steps and keeps the default policy.
constexpr int kStreamPolicy = 0x12;   // sc1 | nt
__device__ __forceinline__ u32x4_t bload16_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kStreamPolicy));
}

// Sum of the 8 bf16 values of a 16-byte chunk, in float32.  (The whole
// vector is bit-cast: this compiler resolves a bit_cast of one element of a
// vector lvalue to element 0.)
__device__ __forceinline__ float chunk_sum(u32x4_t v) {
  const bf16x2_t one2 = __builtin_bit_cast(bf16x2_t, kBf16One2);
  const bf16x8_t h = __builtin_bit_cast(bf16x8_t, v);
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) s = __builtin_amdgcn_fdot2_f32_bf16(bf16x2_t{h[2 * e], h[2 * e + 1]}, one2, s, false);
  return s;
}

__device__ __forceinline__ float dpp_f32(float v, int ctrl_id) {
  const int b = __builtin_bit_cast(int, v);
  int r;
  switch (ctrl_id) {
    case 0: r = __builtin_amdgcn_update_dpp(0, b, 0xB1, 0xF, 0xF, false); break;    // quad_perm [1,0,3,2]
    case 1: r = __builtin_amdgcn_update_dpp(0, b, 0x4E, 0xF, 0xF, false); break;    // quad_perm [2,3,0,1]
    case 2: r = __builtin_amdgcn_update_dpp(0, b, 0x141, 0xF, 0xF, false); break;   // row_half_mirror
    default: r = __builtin_amdgcn_update_dpp(0, b, 0x140, 0xF, 0xF, false); break;  // row_mirror
  }
  return __builtin_bit_cast(float, r);
}

// Sum over aligned groups of L lanes (L = 2, 4, 8 or 16) inside each 16-lane
// row; every lane of a group ends with the group's sum, added in a fixed order.
template <int L>
__device__ __forceinline__ float lane_group_sum(float v) {
  if constexpr (L >= 2) v += dpp_f32(v, 0);
  if constexpr (L >= 4) v += dpp_f32(v, 1);
  if constexpr (L >= 8) v += dpp_f32(v, 2);
  if constexpr (L >= 16) v += dpp_f32(v, 3);
  return v;
}

// GB: 32-wide blocks per group piece inside a step (1, 2 or 4); FR:
// accumulator rows folded and stored (1 when m == 1, else 4); CC: the most
// steps a wave owns (4, 8 or 16); PF: steps of weight loads in flight; FMT:
// the weight format.  kFmtS16: signed two's complement codes with float16
// scales and no zero point (tinyllm L8.5, "int4 per group"); a signed nibble v
// is the unsigned code v ^ 8 with zero point 8, so those weights go through the
// same arithmetic after one XOR per dword.  kFmtMX: MXFP4 (GB = 1: blocks of
// 32 inputs, one E8M0 scale each); a lane's 16 loaded bytes are one block,
// converted by v_cvt_scalef32_pk_bf16_fp4 into bf16 values already multiplied
// by the block's power-of-two scale (exact), so the MFMAs accumulate straight
// into the outputs with the activations in natural order and no fold.
template <int GB, int FR, int CC, int PF, int FMT, bool GRP, bool PREP>
__global__ __launch_bounds__(1024) void gemv_kernel(GemvParams p) {
  constexpr bool S16 = FMT == kFmtS16, MX = FMT == kFmtMX;
  static_assert(!MX || GB == 1, "MXFP4 blocks hold 32 inputs");
  constexpr int NP = 4 / GB;              // group pieces per step
  constexpr int XL = FR == 1 ? CC / 4 : 4;                        // activation loads per batch
  constexpr int SZB = CC * NP / kSzPerBatch > 1 ? CC * NP / kSzPerBatch : 1;
  constexpr int kSzEntries = SZB * kSzPerBatch;                   // staged entries per row
  constexpr int kPieceLanes = 4 * GB;     // 8-input chunks per piece
  constexpr bool kTranspose = GB < 4 && !MX;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int W = __builtin_amdgcn_readfirstlane((int)(blockDim.x >> 6));
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4;
  const int c = lane & 15;
  // this workgroup's matrix (uniform)
  // (a single matrix is read straight from the arguments; only a grouped
  // launch pays a second round of argument loads to find its entry)
  int pi = 0;
  if constexpr (GRP) {
#pragma unroll
    for (int i = 1; i < kMaxGrouped; ++i)
      if (i < p.nprob && (int)blockIdx.x >= p.prob[i].tile_begin) pi = i;
  }
  const GemvProblem& pr = p.prob[pi];
  const int tile = (int)blockIdx.x - pr.tile_begin;
  const int M = p.m, N = pr.n, K = p.k;
  const int cnt = p.cnt;
  const uint32_t row_bytes = (uint32_t)K / 2;
  const int row0 = tile * 16;
  const int rows = min(16, N - row0);
  const int s0 = wave * cnt;                       // first step of this wave
  const int live = min(cnt, p.nsteps - s0);        // <= 0 for a wave past K
  const uint32_t wbase = (uint32_t)(wave * p.wave_lds);

  // Weights: canonical rows [N, K/2], or prepared 1 KB blocks (16 rows x one
  // 128-input step, tile-major) whose 16-byte slot l is exactly lane l's share
  // of a step, so a step is one contiguous kilobyte.
  constexpr bool prep = PREP;   // p.prepared != 0
  const __amdgpu_buffer_rsrc_t rb =
      prep ? rsrc(pr.packed + (int64_t)tile * p.nsteps * 1024, (uint32_t)p.nsteps * 1024u)
           : rsrc(pr.packed + (int64_t)row0 * row_bytes, (uint32_t)rows * row_bytes);
  // scale element bytes and entries per row: float32 per group, float16 per
  // group (S16), one float32 per row (S16 with row_scale: Int4Linear), a byte
  // per block (MX)
  const bool row_scale = S16 && p.row_scale != 0;   // uniform
  const uint32_t sbytes = MX ? 1u : (S16 && !row_scale ? 2u : 4u);
  const int32_t srow = row_scale ? 1 : p.ngroups;
  const __amdgpu_buffer_rsrc_t rs =
      rsrc(static_cast<const char*>(pr.scale) + (int64_t)row0 * srow * sbytes, (uint32_t)(rows * srow) * sbytes);
  const __amdgpu_buffer_rsrc_t rz = rsrc(S16 || MX ? nullptr : pr.zero + (int64_t)row0 * p.ngroups,
                                         S16 || MX ? 0u : (uint32_t)(rows * p.ngroups));
  const __amdgpu_buffer_rsrc_t rx = rsrc(p.x, (uint32_t)M * (uint32_t)K * 2u);

  // ---- staging loads: activations, then scales and zero points -----------------
  // Load j covers four steps of one activation row: lane l holds the 8-input
  // chunk l % 16 of step l / 16.  Loads past the last row or past K read zero.
  const int lpr = cnt >> 2;                        // loads per activation row
  int xrow = 0, xst = 0;                           // (row, step / 4) of the next load
  u32x4_t xb[XL];
  int xr[XL], xs4[XL];
  auto load_x = [&]() {
#pragma unroll
    for (int j = 0; j < XL; ++j) {
      const int step = s0 + 4 * xst + q;
      const int inp = step * kStepK + 8 * c;
      const bool in = xrow < M && inp < K;
      xb[j] = bload16(rx, in ? (uint32_t)(xrow * K + inp) * 2u : kOffsetOOB);
      xr[j] = xrow;
      xs4[j] = xst;
      if (++xst == lpr) { xst = 0; ++xrow; }
    }
  };
  // x chunk -> LDS in pair order, and its share of the piece sums
  const uint32_t xs_base = wbase + (uint32_t)p.xs_off;
  auto put_x = [&]() {
#pragma unroll
    for (int j = 0; j < XL; ++j) {
      if (xr[j] < M) {   // uniform
        const int lstep = 4 * xs4[j] + q;
        if constexpr (MX) {   // natural order, and no piece sums
          *reinterpret_cast<u32x4_t*>(lds + wbase + (uint32_t)((xr[j] * cnt + lstep) * 256 + 16 * c)) = xb[j];
          continue;
        }
        *reinterpret_cast<bf16x8_t*>(lds + wbase + (uint32_t)((xr[j] * cnt + lstep) * 256 + 16 * c)) = pair_order(xb[j]);
        const float sm = lane_group_sum<kPieceLanes>(chunk_sum(xb[j]));
        if ((c & (kPieceLanes - 1)) == 0) {
          const int piece = c / kPieceLanes;
          *reinterpret_cast<float*>(lds + xs_base + (uint32_t)(((lstep * NP + piece) * 4 + xr[j]) * 4)) = sm;
        }
      }
    }
  };
  // (scale, -(128 + zero)) of the tile's rows and groups [gb, gb + 16 SZB):
  // lane l stages row l % 16, entries gb + 4 (l / 16) + 16 b .. +4 of batch b.
  // Entries past the last group or row read zero.
  const int gb = ((s0 * kStepK) >> p.group_shift) & ~3;
  const uint32_t sz_base = wbase + (uint32_t)p.sz_off;
  u32x4_t sv[SZB];
  uint32_t zv[SZB];
  auto load_sz = [&](int b) {
    const int g = gb + 4 * q + kSzPerBatch * b;
    const uint32_t e0 = (uint32_t)(c * p.ngroups + g);
    if constexpr (MX) {   // four E8M0 scale bytes
      zv[b] = 0u;
      sv[b] = u32x4_t{0u, 0u, 0u, 0u};
      if (!p.z_bytewise) {
        const bool in = c < rows && g < p.ngroups;
        sv[b][0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, in ? e0 : kOffsetOOB, 0, 0);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool ie = c < rows && g + e < p.ngroups;
          sv[b][0] |= (uint32_t)(uint8_t)__builtin_amdgcn_raw_buffer_load_b8(rs, ie ? e0 + e : kOffsetOOB, 0, 0) << (8 * e);
        }
      }
    } else if constexpr (S16) {   // four float16 scales, kept as raw halves until put_sz
      zv[b] = 0x08080808u;
      sv[b] = u32x4_t{0u, 0u, 0u, 0u};
      if (row_scale) {   // the row's one float32 scale, for every group
        const uint32_t v = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, c < rows ? (uint32_t)c * 4u : kOffsetOOB, 0, 0);
        sv[b] = u32x4_t{v, v, v, v};
      } else if (!p.z_bytewise) {   // uniform: whole 8-byte runs of scales
        const bool in = c < rows && g < p.ngroups;
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, in ? e0 * 2u : kOffsetOOB, 0, 0);
        sv[b][0] = v[0];
        sv[b][1] = v[1];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool ie = c < rows && g + e < p.ngroups;
          const uint32_t h = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, ie ? (e0 + e) * 2u : kOffsetOOB, 0, 0);
          sv[b][e >> 1] |= h << (16 * (e & 1));
        }
      }
    } else if (!p.z_bytewise) {   // uniform: whole dwords of zero points
      const bool in = c < rows && g < p.ngroups;
      sv[b] = bload16(rs, in ? e0 * 4u : kOffsetOOB);
      zv[b] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rz, in ? e0 : kOffsetOOB, 0, 0);
    } else {
      zv[b] = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool ie = c < rows && g + e < p.ngroups;
        sv[b][e] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, ie ? (e0 + e) * 4u : kOffsetOOB, 0, 0);
        zv[b] |= (uint32_t)(uint8_t)__builtin_amdgcn_raw_buffer_load_b8(rz, ie ? e0 + e : kOffsetOOB, 0, 0) << (8 * e);
      }
    }
  };
  auto put_sz = [&](int b) {
    // (bit_cast of the whole vector: this compiler resolves a bit_cast of one
    // element of a vector lvalue to element 0)
    f32x4_t sf;
    if constexpr (MX) {   // 2^(e - 127) of each E8M0 byte
      const u32x4_t raw = sv[b];
      const uint32_t w4 = raw[0];
      uint32_t bits[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t eb = (w4 >> (8 * e)) & 0xFFu;
        bits[e] = eb == 0 ? 0x00400000u : eb << 23;
      }
      sf = f32x4_t{__uint_as_float(bits[0]), __uint_as_float(bits[1]), __uint_as_float(bits[2]),
                   __uint_as_float(bits[3])};
    } else if constexpr (S16) {
      const u32x4_t raw = sv[b];
      const uint32_t h01 = raw[0], h23 = raw[1];
      if (row_scale)
        sf = __builtin_bit_cast(f32x4_t, raw);
      else
        sf = f32x4_t{(float)__builtin_bit_cast(_Float16, (uint16_t)(h01 & 0xFFFFu)),
                   (float)__builtin_bit_cast(_Float16, (uint16_t)(h01 >> 16)),
                   (float)__builtin_bit_cast(_Float16, (uint16_t)(h23 & 0xFFFFu)),
                   (float)__builtin_bit_cast(_Float16, (uint16_t)(h23 >> 16))};
    } else {
      sf = __builtin_bit_cast(f32x4_t, sv[b]);
    }
    const uint32_t z = zv[b];
    f32x4_t* dst = reinterpret_cast<f32x4_t*>(lds + sz_base + (uint32_t)((c * kSzEntries + 4 * q + kSzPerBatch * b) * 8));
    if constexpr (MX) {
      dst[0] = f32x4_t{sf[0], 0.f, sf[1], 0.f};
      dst[1] = f32x4_t{sf[2], 0.f, sf[3], 0.f};
      return;
    }
    dst[0] = f32x4_t{sf[0], -(kNibOffset + (float)(z & 0xFFu)), sf[1], -(kNibOffset + (float)((z >> 8) & 0xFFu))};
    dst[1] = f32x4_t{sf[2], -(kNibOffset + (float)((z >> 16) & 0xFFu)), sf[3], -(kNibOffset + (float)(z >> 24))};
  };

  // ---- weight ring --------------------------------------------------------------
  // Steps past this wave's range load nothing: their offsets get bit 31.
  u32x4_t bq[PF];
  const uint32_t bstep = prep ? 1024u : (uint32_t)(kStepK / 2);   // bytes per step and lane group
  const uint32_t boff = prep ? 16u * (uint32_t)lane + (uint32_t)s0 * 1024u
                             : (uint32_t)c * row_bytes + 16u * (uint32_t)q + (uint32_t)s0 * (kStepK / 2);
  auto issue = [&](int slot, int i) {
    const uint32_t dead = (uint32_t)(live - 1 - i) & kOffsetOOB;    // uniform
    const uint32_t off = (boff + (uint32_t)i * bstep) | dead;
    if constexpr (PREP)
      bq[slot] = bload16_stream(rb, off);
    else
      bq[slot] = bload16(rb, off);
  };

  load_x();
#pragma unroll
  for (int b = 0; b < SZB; ++b) load_sz(b);
#pragma unroll
  for (int u = 0; u < PF; ++u) issue(u, u);        // the weight stream starts now
#pragma unroll
  for (int b = 0; b < SZB; ++b) put_sz(b);
  put_x();
  if constexpr (FR != 1) {   // m == 1 always stages its activations in one batch
    for (int b = 1; b < p.x_batches; ++b) {
      load_x();
      put_x();
    }
  }

  // ---- main loop ------------------------------------------------------------------
  // Each wave reads only what it wrote itself, and LDS operations of one wave
  // complete in order, so no barrier is needed before the loop.
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // Activation operand of lane (q, i): row i, clamped to the last row (the
  // extra rows' outputs are never stored).  MFMA e reads the chunk of inputs
  // k0+32q+8e (no transpose) or k0+32e+8q (transpose).
  const uint32_t a_lane = wbase + (uint32_t)(min(c, M - 1) * cnt * 256) + (kTranspose ? 16u : 64u) * (uint32_t)q;
  constexpr uint32_t kAStride = kTranspose ? 64 : 16;
  const uint32_t sz_lane = sz_base + (uint32_t)(c * kSzEntries * 8);
  const uint32_t nib_offset = vgpr_copy(p.nib_offset);
  const int nsteps_run = (max(live, 0) + PF - 1) / PF * PF;

  // Step i takes its weights out of ring slot `slot`, refills the slot with
  // step i + PF as soon as the bytes are out of it, and only then computes;
  // the scheduling barrier keeps the compiler from sinking the refill below
  // the arithmetic.  A step past the wave's range multiplies zero activations
  // by zero weights and adds exactly nothing.
  auto step_mx = [&](int slot, int i) {
    const uint32_t a_addr = a_lane + (uint32_t)i * 256u;
    bf16x8_t af[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) af[e] = *reinterpret_cast<const bf16x8_t*>(lds + a_addr + kAStride * e);
    // this lane's block: 4 i + q of the wave's range
    const float xsc = *reinterpret_cast<const float*>(lds + sz_lane + (uint32_t)(4 * i + q) * 8u);
    bf16x8_t bw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) bw[e] = fp4x8_to_bf16(bq[slot][e], xsc);
    issue(slot, i + PF);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = mfma_bf16(af[e], bw[e], acc);
  };
  auto step = [&](int slot, int i) {
    if constexpr (MX) {
      step_mx(slot, i);
      return;
    }
    const uint32_t a_addr = a_lane + (uint32_t)i * 256u;
    bf16x8_t af[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) af[e] = *reinterpret_cast<const bf16x8_t*>(lds + a_addr + kAStride * e);
    f32x2_t sz[NP];
    f32x4_t xs[NP];
#pragma unroll
    for (int pc = 0; pc < NP; ++pc) {
      const int g = (((s0 + i) * kStepK + 32 * GB * pc) >> p.group_shift) - gb;   // uniform
      sz[pc] = *reinterpret_cast<const f32x2_t*>(lds + sz_lane + (uint32_t)g * 8u);
      const uint32_t xa = xs_base + (uint32_t)((i * NP + pc) * 16);
      if constexpr (FR == 1)
        xs[pc][0] = *reinterpret_cast<const float*>(lds + xa);
      else
        xs[pc] = *reinterpret_cast<const f32x4_t*>(lds + xa);
    }
    bf16x8_t bw[4];
    if constexpr (kTranspose) {
      // The lane swaps work on copies, so the slot's registers stay free for
      // the refill (no copy of a register a load is still writing).
      uint32_t d0 = vgpr_copy(bq[slot][0]), d1 = vgpr_copy(bq[slot][1]);
      uint32_t d2 = vgpr_copy(bq[slot][2]), d3 = vgpr_copy(bq[slot][3]);
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
      for (int e = 0; e < 4; ++e) bw[e] = unpack_codes(S16 ? bq[slot][e] ^ kSignFlip : bq[slot][e], p.nib_mask, nib_offset);
    }
    issue(slot, i + PF);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int pc = 0; pc < NP; ++pc) {
      f32x4_t cg = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < GB; ++e) cg = mfma_bf16(af[pc * GB + e], bw[pc * GB + e], cg);
#pragma unroll
      for (int r = 0; r < FR; ++r) acc[r] = fmaf(sz[pc].x, fmaf(sz[pc].y, xs[pc][r], cg[r]), acc[r]);
    }
  };

  for (int i0 = 0; i0 < nsteps_run; i0 += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) step(u, i0 + u);
  }

  // ---- combine the waves, add the bias, store ---------------------------------------
  // Lane c < 16 holds output column row0 + c for activation rows r < 4 in acc[r].
  const int n = row0 + c;
  auto store = [&](const f32x4_t& v) {
    if (lane < 16 && n < N) {
      const float bv = pr.bias ? pr.bias[n] : 0.f;
#pragma unroll
      for (int r = 0; r < FR; ++r) {
        if (r < M) {
          const float o = v[r] + bv;
          if (p.y_bf16)
            reinterpret_cast<uint16_t*>(pr.y)[(int64_t)r * N + n] = f32_to_bf16_bits(o);
          else
            reinterpret_cast<float*>(pr.y)[(int64_t)r * N + n] = o;
        }
      }
    }
  };
  if (W == 1) {
    store(acc);
    return;
  }
  float* red = reinterpret_cast<float*>(lds + p.red_off);   // [W][16][FR]
  if (lane < 16) {
#pragma unroll
    for (int r = 0; r < FR; ++r) red[(wave * 16 + lane) * FR + r] = acc[r];
  }
  // LDS-only fences: the waves' partials are visible after the barrier, and
  // no wait for the (empty) weight loads still in flight is added.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  if (wave == 0) {
    f32x4_t v = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (lane < 16) {
      for (int w = 0; w < W; ++w)
#pragma unroll
        for (int r = 0; r < FR; ++r) v[r] += red[(w * 16 + lane) * FR + r];
    }
    store(v);
  }
}

template <int GB, int FR, int CC, int FMT>
int32_t launch_one(const GemvParams& gp, const LinearPlan& pl, size_t lds, hipStream_t stream) {
  const bool grp = gp.nprob > 1;
  const bool prep = gp.prepared != 0;
  auto kern = grp ? (prep ? gemv_kernel<GB, FR, CC, 4, FMT, true, true> : gemv_kernel<GB, FR, CC, 4, FMT, true, false>)
                  : (prep ? gemv_kernel<GB, FR, CC, 4, FMT, false, true> : gemv_kernel<GB, FR, CC, 4, FMT, false, false>);
  if (lds > 64 * 1024) {
    static std::atomic<uint64_t> raised[4] = {{0}, {0}, {0}, {0}};   // per kernel, one bit per device
    const int32_t st = raise_lds_limit(reinterpret_cast<const void*>(kern), 160 * 1024,
                                       raised[(grp ? 1 : 0) + (prep ? 2 : 0)]);
    if (st != WOQ_OK) return st;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)pl.grid), dim3(64 * pl.waves), lds, stream, gp);
  return hip_status(hipGetLastError());
}

template <int GB, int FR, int FMT>
int32_t dispatch_cc(const GemvParams& gp, const LinearPlan& pl, size_t lds, hipStream_t stream) {
  const int cc = gemv_cnt_class(pl.cnt);
  switch (cc) {
    case 4: return launch_one<GB, FR, 4, FMT>(gp, pl, lds, stream);
    case 8: return launch_one<GB, FR, 8, FMT>(gp, pl, lds, stream);
    case 16: return launch_one<GB, FR, 16, FMT>(gp, pl, lds, stream);
    default: return WOQ_EUNSUPPORTED;
  }
}

template <int FR, int FMT>
int32_t dispatch_gb(const GemvParams& gp, const LinearPlan& pl, size_t lds, hipStream_t stream) {
  switch (pl.gb) {
    case 1: return dispatch_cc<1, FR, FMT>(gp, pl, lds, stream);
    case 2: return dispatch_cc<2, FR, FMT>(gp, pl, lds, stream);
    case 4: return dispatch_cc<4, FR, FMT>(gp, pl, lds, stream);
    default: return WOQ_EUNSUPPORTED;
  }
}

}  // namespace

int gemv_cnt_class(int cnt) { return cnt <= 4 ? 4 : (cnt <= 8 ? 8 : (cnt <= 16 ? 16 : 0)); }

GemvLayout gemv_layout(int64_t m, int64_t k, int64_t group, int waves, int cnt) {
  GemvLayout l;
  const int64_t piece = group < kStepK ? group : kStepK;
  const int64_t np = kStepK / piece;
  const int cc = gemv_cnt_class(cnt);
  const int64_t szb = cc * np / kSzPerBatch > 1 ? cc * np / kSzPerBatch : 1;
  l.xs_off = (int32_t)(m * cnt * 256);
  l.sz_off = l.xs_off + (int32_t)(cnt * np * 16);
  l.wave_lds = l.sz_off + (int32_t)(16 * szb * kSzPerBatch * 8);
  l.red_off = l.wave_lds * waves;
  l.total = (size_t)l.red_off + (size_t)waves * 16 * 4 * 4;
  return l;
}

int32_t launch_gemv_grouped(const LinearArgs* args, int count, const LinearPlan& pl,
                            hipStream_t stream) {
  const LinearArgs& a = args[0];
  int32_t gshift = 0;
  while ((1 << gshift) < a.group) ++gshift;
  const GemvLayout l = gemv_layout(a.m, a.k, a.group, pl.waves, pl.cnt);
  const int32_t nsteps = (a.k + kStepK - 1) / kStepK;
  const int32_t ngroups = a.k / a.group;
  const int cc = gemv_cnt_class(pl.cnt);
  const int32_t xl = pl.fold_rows == 1 ? cc / 4 : 4;
  const int32_t loads = (a.m * pl.cnt / 4 + xl - 1) / xl;
  GemvParams gp{a.x, a.m, a.k, a.y_bf16, nsteps, pl.cnt, ngroups, gshift, loads,
                ngroups % 4 != 0 ? 1 : 0, a.prepared, l.wave_lds, l.xs_off, l.sz_off, l.red_off,
                kNibPairMask, kBf16Offset2, a.row_scale, count, {}};
  int32_t tb = 0;
  for (int i = 0; i < count; ++i) {
    gp.prob[i] = GemvProblem{args[i].packed,
                             a.mx ? static_cast<const void*>(args[i].scale8)
                                  : a.sym16 && !a.row_scale ? static_cast<const void*>(args[i].scale16)
                                                            : static_cast<const void*>(args[i].scale),
                             args[i].zero, args[i].bias, args[i].y, args[i].n, tb};
    tb += (args[i].n + 15) / 16;
  }
  LinearPlan p2 = pl;
  p2.grid = tb;
  if (a.mx) {
    if (pl.gb != 1) return WOQ_EUNSUPPORTED;
    return pl.fold_rows == 1 ? dispatch_cc<1, 1, kFmtMX>(gp, p2, l.total, stream)
                             : dispatch_cc<1, 4, kFmtMX>(gp, p2, l.total, stream);
  }
  if (a.sym16)
    return pl.fold_rows == 1 ? dispatch_gb<1, kFmtS16>(gp, p2, l.total, stream)
                             : dispatch_gb<4, kFmtS16>(gp, p2, l.total, stream);
  return pl.fold_rows == 1 ? dispatch_gb<1, kFmtU4>(gp, p2, l.total, stream)
                           : dispatch_gb<4, kFmtU4>(gp, p2, l.total, stream);
}

int32_t launch_gemv(const LinearArgs& a, const LinearPlan& pl, hipStream_t stream) {
  return launch_gemv_grouped(&a, 1, pl, stream);
}

}  // namespace woq
