// Small-M linear path (up to 64 activation rows by default, 128 when forced,
// and the decode shapes the row kernel cannot take): y = x . dequant(W)^T +
// bias for group-wise 4-bit weights (linnet docs "Quantization", std.quant
// table, linear_int4_groups).  At these row counts the layer is bound by the
// weight stream; what matters is that each packed byte is read once, that the
// activations it meets cost little next to it, and that enough bytes are in
// flight.
//
// * A workgroup owns T tiles of 16 weight rows (outputs) and all of K; its W
//   waves form WM groups along the activation rows (each takes MT tiles of 16
//   rows; WM > 1 only above 32 rows) times WK contiguous K ranges of `cnt`
//   128-input steps.
// * Per step a lane issues one 16-byte load per weight tile (lane group q
//   reads inputs [k0 + 32q, k0 + 32q + 32) of row c) and four 16-byte loads
//   per 16-row activation tile: the activations go straight from memory (they
//   are small and stay in the caches) into the MFMA operand registers, so no
//   LDS staging and no barrier precede the stream.  The T weight tiles of a
//   wave share those activation operands.  Two steps of loads are in flight.
// * Nibbles become bf16 (128 + code) with one AND-OR per pair and meet the
//   activations, reordered into the unpacker's pair order, in
//   v_mfma_f32_16x16x32_bf16.  For groups of 128 and more MFMA e takes dword e
//   of every lane's load; smaller groups transpose the dwords across lane
//   groups so that each MFMA stays inside one group, and load the activation
//   chunks in the matching order.
// * Per group piece: acc += scale * (sum x(128 + code) - (128 + zero) * sum x);
//   the sums of x come from the same MFMA unit against a ones operand, already
//   in the accumulator layout.  Each wave stages the (scale, -(128 + zero))
//   pairs of its rows and groups in its own LDS area; those loads go out just
//   before the first steps of the stream and are converted behind them.
// * Per step the activation registers are refilled as soon as they are
//   converted, and each weight tile's as soon as it is unpacked, so one tile's
//   operands are live at a time.
// * The waves' partial tiles meet in LDS (fixed order); bias, then y.
#include "woq_internal.h"
#include "mfma_common.h"

namespace woq {
namespace {

constexpr int kStepK = 128;
constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr uint32_t kOffsetOOB = 0x80000000u;   // a buffer offset no descriptor covers
constexpr int kStageBatch = 8;   // staged (scale, zero) entries per lane and batch
constexpr int kPF = 2;           // steps of loads in flight per wave
constexpr uint32_t kSignFlip = 0x88888888u;   // two's complement nibble v -> unsigned v ^ 8 (zero point 8)

struct SkinnyParams {
  const uint16_t* x;
  const uint8_t* packed;
  const void* scale;      // float32, or float16 for signed codes
  const uint8_t* zero;    // unused for signed codes
  const float* bias;
  void* y;
  int32_t m, n, k, y_bf16;
  int32_t nsteps, ngroups, prepared;
  int32_t cnt;        // steps per wave
  int32_t ngw;        // groups staged per row and wave
  int32_t sz_bytes;   // LDS bytes of one wave's staging area
  int32_t red_off;    // LDS offset of the reduction area
  // The nibble mask and the bf16 offset pattern arrive as arguments so they sit
  // in registers: one v_and_or_b32 per pair then expands two codes.
  uint32_t nib_mask, nib_offset;
  int32_t row_scale;  // signed codes with one float32 scale a row (Int4Linear)
  int32_t wm;         // wave groups along the activation rows (each takes MT tiles of 16 rows)
  int32_t zp4;        // zero points packed two a byte (group 2j in the low nibble of byte j)
  int32_t zrow;       // zero-point bytes per row: ngroups, or ceil(ngroups / 2) with zp4
  int32_t mtiles;     // 16-row activation tiles in the fragment-ordered copy (XF)
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, (int)kRsrcWord3);
}

__device__ __forceinline__ u32x4_t bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// G: group size; MT: 16-row activation tiles; T: 16-row weight tiles per
// workgroup; FMT: the weight format.  kFmtS16: signed two's complement codes
// with float16 scales and no zero point (tinyllm L8.5, "int4 per group"), run
// as unsigned codes v ^ 8 with zero point 8 after one XOR per dword.  kFmtMX:
// MXFP4 (G = 32, E2M1 codes, one E8M0 scale per block): each lane's 16 loaded
// bytes are one block, which v_cvt_scalef32_pk_bf16_fp4 turns into bf16 values
// already multiplied by the block's power-of-two scale (exact), so the MFMAs
// accumulate straight into the outputs, in natural input order, with no
// per-group fold.
// XF: x is the fragment-ordered copy the pre-pass wrote (x_frag_kernel): the
// four chunks of a step are four contiguous kilobytes, already pair-ordered.
template <int G, int MT, int T, int FMT, bool XF>
__global__ __launch_bounds__(512) void skinny_kernel(SkinnyParams p) {
  constexpr bool S16 = FMT == kFmtS16, MX = FMT == kFmtMX;
  static_assert(!MX || G == 32, "MXFP4 blocks hold 32 inputs");
  constexpr int GB = G >= 128 ? 4 : G / 32;   // 32-input blocks per group piece
  constexpr int NP = 4 / GB;                  // group pieces per step
  constexpr bool kTranspose = GB < 4 && !MX;
  // inputs, and bytes, between the activation chunks of MFMA e and e + 1
  constexpr int kXEIn = kTranspose ? 32 : 8;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int W = __builtin_amdgcn_readfirstlane((int)(blockDim.x >> 6));
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4;
  const int c = lane & 15;
  // Waves are a WM x WK grid: wave group wm takes activation tiles
  // [wm MT, wm MT + MT), K range wk takes `cnt` steps.
  const int WM = p.wm;
  const int wm = __builtin_amdgcn_readfirstlane(wave % WM);
  const int wk = __builtin_amdgcn_readfirstlane(wave / WM);
  const int M = p.m, N = p.n, K = p.k;
  const int nsteps = p.nsteps;
  const uint32_t row_bytes = (uint32_t)K / 2;
  const int tile0 = blockIdx.x * T;
  const int wg_rows = __builtin_amdgcn_readfirstlane(min(16 * T, N - 16 * tile0));
  const int cnt = p.cnt;
  const int s0 = __builtin_amdgcn_readfirstlane(wk * cnt);
  const int live = __builtin_amdgcn_readfirstlane(max(0, min(cnt, nsteps - s0)));
  const bool prep = p.prepared != 0;

  // 1. (scale, -(128 + zero)) of this wave's groups [gb, gb + ngw) for the
  //    workgroup's rows, [row][group] float pairs; groups past the row read zero.
  //    The first batch of staging loads goes out before the weight stream and is
  //    converted after it, so the two latencies overlap.
  const int gb = (s0 * kStepK) / G;
  const int ngw = p.ngw;
  // one staging area per K range: the WM waves of a range write the same
  // values there, and each reads only entries it wrote itself
  unsigned char* szl = lds + wk * p.sz_bytes;
  // float32 per group, float16 per group (S16), one float32 per row (S16 with
  // row_scale: Int4Linear), a byte per block (MX)
  const bool row_scale = S16 && p.row_scale != 0;   // uniform
  const uint32_t sbytes = MX ? 1u : (S16 && !row_scale ? 2u : 4u);
  const int32_t srow = row_scale ? 1 : p.ngroups;
  const __amdgpu_buffer_rsrc_t rs =
      rsrc(static_cast<const char*>(p.scale) + (int64_t)tile0 * 16 * srow * sbytes,
           (uint32_t)(wg_rows * srow) * sbytes);
  const int zrow = p.zrow;
  const bool zp4 = p.zp4 != 0;   // uniform
  const __amdgpu_buffer_rsrc_t rz = rsrc(S16 || MX ? nullptr : p.zero + (int64_t)tile0 * 16 * zrow,
                                         S16 || MX ? 0u : (uint32_t)(wg_rows * zrow));
  const int sz_total = 16 * T * ngw;
  uint32_t sv[kStageBatch];   // float32 bits, or float16 bits for S16 (converted when stored)
  uint32_t zv[kStageBatch];
  uint32_t zs[kStageBatch];   // bit offset of the zero point in its loaded byte
  auto stage_load = [&](int base) {
#pragma unroll
    for (int b = 0; b < kStageBatch; ++b) {
      const int e = base + lane + 64 * b;
      const int r = e / ngw, g = e % ngw;
      const bool in = e < sz_total && r < wg_rows && gb + g < p.ngroups;
      const uint32_t idx = (uint32_t)(r * p.ngroups + gb + g);
      if constexpr (MX) {
        sv[b] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs, in ? idx : kOffsetOOB, 0, 0);
        zv[b] = 0u;
        zs[b] = 0u;
      } else if constexpr (S16) {
        if (row_scale)
          sv[b] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, in ? (uint32_t)r * 4u : kOffsetOOB, 0, 0);
        else
          sv[b] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, in ? idx * 2u : kOffsetOOB, 0, 0);
        zv[b] = 8u;
        zs[b] = 0u;
      } else {
        sv[b] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, in ? idx * 4u : kOffsetOOB, 0, 0);
        const uint32_t zidx = zp4 ? (uint32_t)(r * zrow + ((gb + g) >> 1)) : idx;
        zs[b] = zp4 ? 4u * (uint32_t)((gb + g) & 1) : 0u;
        zv[b] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rz, in ? zidx : kOffsetOOB, 0, 0);
      }
    }
  };
  auto stage_store = [&](int base) {
#pragma unroll
    for (int b = 0; b < kStageBatch; ++b) {
      const int e = base + lane + 64 * b;
      if constexpr (MX) {   // (2^(e - 127), unused)
        const uint32_t eb = sv[b] & 0xFFu;
        const float sc = __uint_as_float(eb == 0 ? 0x00400000u : eb << 23);
        if (e < sz_total) *reinterpret_cast<f32x2_t*>(szl + e * 8) = f32x2_t{sc, 0.f};
      } else {
        const float sc = S16 && !row_scale ? (float)__builtin_bit_cast(_Float16, (uint16_t)sv[b])
                                           : __builtin_bit_cast(float, sv[b]);
        const uint32_t zq = __builtin_amdgcn_ubfe(zv[b], zs[b], zp4 ? 4u : 8u);
        if (e < sz_total)
          *reinterpret_cast<f32x2_t*>(szl + e * 8) = f32x2_t{sc, -(kNibOffset + (float)zq)};
      }
    }
  };
  stage_load(0);

  // 2. the streams.  Weights: canonical rows [N, K/2] (lane (q, c): row c,
  //    bytes 64 s + 16 q of step s) or prepared 1 KB blocks (slot = lane).
  //    Activations: lane (q, c) of tile mt reads row 16 mt + c; loads past the
  //    rows, past K or past the wave's steps read zero.
  const int wg_tiles = (wg_rows + 15) / 16;
  const __amdgpu_buffer_rsrc_t rb =
      prep ? rsrc(p.packed + (int64_t)tile0 * nsteps * 1024, (uint32_t)(wg_tiles * nsteps) * 1024u)
           : rsrc(p.packed + (int64_t)tile0 * 16 * row_bytes, (uint32_t)wg_rows * row_bytes);
  const __amdgpu_buffer_rsrc_t rx =
      rsrc(p.x, XF ? (uint32_t)p.mtiles * (uint32_t)nsteps * 4096u : (uint32_t)M * (uint32_t)K * 2u);
  const uint32_t wstep = prep ? 1024u : 64u;
  uint32_t woff[T];
#pragma unroll
  for (int t = 0; t < T; ++t)
    woff[t] = prep ? (uint32_t)(t * nsteps + s0) * 1024u + 16u * (uint32_t)lane
                   : (uint32_t)(16 * t + c) * row_bytes + (uint32_t)s0 * 64u + 16u * (uint32_t)q;
  const int in0 = s0 * kStepK + (kTranspose ? 8 * q : 32 * q);   // first input of this lane's chunk 0
  const int xlim = K - in0;                                       // inputs left from there
  uint32_t xoff[MT];
  bool xrow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int row = 16 * (wm * MT + mt) + c;
    xrow[mt] = row < M;
    xoff[mt] = (uint32_t)(min(row, M - 1) * K + in0) * 2u;
  }
  u32x4_t wb[kPF][T];
  u32x4_t xb[kPF][MT][4];
  auto issue_w = [&](int slot, int t, int i) {
    const uint32_t dead = (uint32_t)(live - 1 - i) & kOffsetOOB;
    wb[slot][t] = bload16(rb, (woff[t] + (uint32_t)i * wstep) | dead);
  };
  auto issue_x = [&](int slot, int i) {
    const uint32_t dead = (uint32_t)(live - 1 - i) & kOffsetOOB;
    if constexpr (XF) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int tile = wm * MT + mt;
        const uint32_t base = (uint32_t)((tile * nsteps + s0 + i) * 4) * 1024u + 16u * (uint32_t)lane;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          xb[slot][mt][e] = bload16(rx, tile < p.mtiles ? (base + 1024u * (uint32_t)e) | dead : kOffsetOOB);
      }
      return;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool in_k = i * kStepK + kXEIn * e < xlim;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        xb[slot][mt][e] = bload16(rx, xrow[mt] && in_k ? (xoff[mt] + (uint32_t)(i * kStepK + kXEIn * e) * 2u) | dead
                                                       : kOffsetOOB);
    }
  };
  auto issue = [&](int slot, int i) {
#pragma unroll
    for (int t = 0; t < T; ++t) issue_w(slot, t, i);
    issue_x(slot, i);
  };
#pragma unroll
  for (int u = 0; u < kPF; ++u) issue(u, u);
  stage_store(0);
  for (int base = 64 * kStageBatch; base < sz_total; base += 64 * kStageBatch) {
    stage_load(base);
    stage_store(base);
  }

  const uint32_t nib_offset = vgpr_copy(p.nib_offset);
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4_t{kBf16One2, kBf16One2, kBf16One2, kBf16One2});
  f32x4_t acc[MT][T];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < T; ++t) acc[mt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Step i: operands out of ring slot `slot`, the slot refilled with step
  // i + kPF once its bytes are out (the scheduling barrier keeps the refill
  // ahead of the arithmetic).  A step past the wave's range multiplies zero
  // activations with zero-byte weights and adds nothing.
  auto step_mx = [&](int slot, int i) {
    // activations in natural input order; lane (q, c) of weight tile t holds
    // block 4 i + q of row 16 t + c
    bf16x8_t af[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) af[mt][e] = __builtin_bit_cast(bf16x8_t, xb[slot][mt][e]);
    issue_x(slot, i + kPF);
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float xs = reinterpret_cast<const f32x2_t*>(szl + ((16 * t + c) * ngw + 4 * i + q) * 8)->x;
      bf16x8_t bw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) bw[e] = fp4x8_to_bf16(wb[slot][t][e], xs);
      issue_w(slot, t, i + kPF);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[mt][t] = mfma_bf16(af[mt][e], bw[e], acc[mt][t]);
    }
  };
  auto step = [&](int slot, int i) {
    if constexpr (MX) {
      step_mx(slot, i);
      return;
    }
    // activation operands in pair order, and their piece sums: lane (q, c)
    // gets the sums of rows 16 mt + 4q + r, the layout of the accumulators
    bf16x8_t af[MT][4];
    f32x4_t xsum[MT][NP];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        af[mt][e] = XF ? __builtin_bit_cast(bf16x8_t, xb[slot][mt][e]) : pair_order(xb[slot][mt][e]);
#pragma unroll
      for (int pc = 0; pc < NP; ++pc) {
        f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < GB; ++e) s = mfma_bf16(af[mt][pc * GB + e], ones, s);
        xsum[mt][pc] = s;
      }
    }
    issue_x(slot, i + kPF);
#pragma unroll
    for (int t = 0; t < T; ++t) {
      bf16x8_t bw[4];
      if constexpr (kTranspose) {
        // the lane swaps work on copies, so the slot's registers are free for the refill
        uint32_t d0 = vgpr_copy(wb[slot][t][0]), d1 = vgpr_copy(wb[slot][t][1]);
        uint32_t d2 = vgpr_copy(wb[slot][t][2]), d3 = vgpr_copy(wb[slot][t][3]);
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
          bw[e] = unpack_codes(S16 ? wb[slot][t][e] ^ kSignFlip : wb[slot][t][e], p.nib_mask, nib_offset);
      }
      issue_w(slot, t, i + kPF);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int pc = 0; pc < NP; ++pc) {
        const int g = (i * kStepK + 32 * GB * pc) / G;   // group inside the wave's range
        const f32x2_t sz = *reinterpret_cast<const f32x2_t*>(szl + ((16 * t + c) * ngw + g) * 8);
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
  };
  const int nrun = (live + kPF - 1) / kPF * kPF;   // <= cnt: the host keeps cnt a multiple of kPF
  for (int i0 = 0; i0 < nrun; i0 += kPF) {
#pragma unroll
    for (int u = 0; u < kPF; ++u) step(u, i0 + u);
  }

  // 3. combine the K ranges: red[wave][mt][t][lane] (4 floats each); wave w
  //    then finishes the (wave group, mt, t) tiles w, w + W, ..., adding the K
  //    ranges in order
  float* red = reinterpret_cast<float*>(lds + p.red_off);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < T; ++t)
      *reinterpret_cast<f32x4_t*>(red + (((wave * MT + mt) * T + t) * 64 + lane) * 4) = acc[mt][t];
  // LDS-only fences: the waves' partials are visible after the barrier, and
  // no wait for the (empty) weight loads still in flight is added.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  const int WK = W / WM;
  for (int pr = wave; pr < WM * MT * T; pr += W) {
    const int pm = pr / (MT * T), mt = (pr / T) % MT, t = pr % T;
    f32x4_t v = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int kk = 0; kk < WK; ++kk) {
      const int w = kk * WM + pm;
      const f32x4_t a = *reinterpret_cast<const f32x4_t*>(red + (((w * MT + mt) * T + t) * 64 + lane) * 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] += a[r];
    }
    const int n = (tile0 + t) * 16 + c;
    if (n < N) {
      const float bv = p.bias ? p.bias[n] : 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * (pm * MT + mt) + 4 * q + r;
        if (row < M) {
          const float o = v[r] + bv;
          if (p.y_bf16)
            reinterpret_cast<uint16_t*>(p.y)[(int64_t)row * N + n] = f32_to_bf16_bits(o);
          else
            reinterpret_cast<float*>(p.y)[(int64_t)row * N + n] = o;
        }
      }
    }
  }
}

// Pre-pass for m > 16: one thread per 16-byte chunk of the fragment-ordered
// copy, enumerated in its storage order (tile, step, chunk e, lane), so the
// writes are contiguous.  Lane (q, c) of tile t holds, for chunk e of step s,
// the 8 inputs from s*128 + 32q + 8e (groups of 128 and more, and MXFP4) or
// s*128 + 8q + 32e (smaller groups) of activation row 16t + c: the inputs the
// kernel's weight fragments of that lane meet.  The act-order gather happens
// here too (indices clamped into range, as in the other pre-pass).
template <bool TR, bool NATURAL>
__global__ __launch_bounds__(256) void x_frag_kernel(const uint16_t* __restrict__ x,
                                                     const int32_t* __restrict__ order, int32_t m,
                                                     int32_t k, int32_t nsteps, int64_t total,
                                                     uint16_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
    const int lane = (int)(t & 63), e = (int)((t >> 6) & 3);
    const int64_t ts = t >> 8;
    const int step = (int)(ts % nsteps), tile = (int)(ts / nsteps);
    const int q = lane >> 4, c = lane & 15;
    const int row = 16 * tile + c;
    const int in = step * kStepK + (TR ? 8 * q + 32 * e : 32 * q + 8 * e);
    u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
    if (row < m && in < k) {   // k is a multiple of 32, so the 8 inputs are all in range
      const uint16_t* xr = x + (int64_t)row * k;
      if (order) {
        uint32_t h[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int32_t src = order[in + i];
          h[i] = xr[src < 0 ? 0 : (src >= k ? k - 1 : src)];
        }
        v = u32x4_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
      } else {
        v = load16(xr + in);
      }
    }
    *reinterpret_cast<u32x4_t*>(out + t * 8) = NATURAL ? v : __builtin_bit_cast(u32x4_t, pair_order(v));
  }
}

template <int G, int MT, int T, int FMT, bool XF>
int32_t launch_one(const SkinnyParams& sp, const LinearPlan& pl, size_t lds, hipStream_t stream) {
  auto kern = skinny_kernel<G, MT, T, FMT, XF>;
  if (lds > 64 * 1024) {
    static std::atomic<uint64_t> raised{0};   // per instantiation, one bit per device
    const int32_t st = raise_lds_limit(reinterpret_cast<const void*>(kern), 160 * 1024, raised);
    if (st != WOQ_OK) return st;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)pl.grid), dim3(64 * pl.waves), lds, stream, sp);
  return hip_status(hipGetLastError());
}

template <int G, int MT, int FMT, bool XF>
int32_t dispatch_t(const SkinnyParams& sp, const LinearPlan& pl, size_t lds, hipStream_t s) {
  switch (pl.ns) {
    case 1: return launch_one<G, MT, 1, FMT, XF>(sp, pl, lds, s);
    case 2: return launch_one<G, MT, 2, FMT, XF>(sp, pl, lds, s);
    case 4: return launch_one<G, MT, 4, FMT, XF>(sp, pl, lds, s);
    default: return WOQ_EUNSUPPORTED;
  }
}

// The fragment-ordered activations serve two activation tiles per wave (m > 16).
template <int G, int FMT>
int32_t dispatch_mt(const SkinnyParams& sp, const LinearPlan& pl, size_t lds, hipStream_t s) {
  switch (pl.mt) {
    case 1: return pl.xfrag ? WOQ_EUNSUPPORTED : dispatch_t<G, 1, FMT, false>(sp, pl, lds, s);
    case 2: return pl.xfrag ? dispatch_t<G, 2, FMT, true>(sp, pl, lds, s) : dispatch_t<G, 2, FMT, false>(sp, pl, lds, s);
    default: return WOQ_EUNSUPPORTED;
  }
}

}  // namespace

int64_t mt_total(int64_t m) { return (m + 15) / 16; }

size_t xfrag_bytes(int64_t m, int64_t k) {
  return (size_t)mt_total(m) * (size_t)((k + kStepK - 1) / kStepK) * 4096u;
}

int32_t launch_xfrag(const uint16_t* x, const int32_t* order, int32_t m, int32_t k, int32_t group,
                     int32_t natural, uint16_t* out, hipStream_t stream) {
  const int32_t nsteps = (k + kStepK - 1) / kStepK;
  const int64_t total = mt_total(m) * (int64_t)nsteps * 256;
  if (total == 0) return WOQ_OK;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  const bool tr = group < kStepK && !natural;   // the kernel's lane-group transpose for groups under 128
  const dim3 g((unsigned)blocks), b(256);
  if (natural)
    hipLaunchKernelGGL((x_frag_kernel<false, true>), g, b, 0, stream, x, order, m, k, nsteps, total, out);
  else if (tr)
    hipLaunchKernelGGL((x_frag_kernel<true, false>), g, b, 0, stream, x, order, m, k, nsteps, total, out);
  else
    hipLaunchKernelGGL((x_frag_kernel<false, false>), g, b, 0, stream, x, order, m, k, nsteps, total, out);
  return hip_status(hipGetLastError());
}

SkinnyLds skinny_lds_layout(int64_t m, int64_t k, int64_t group, int waves, int tiles, int cnt) {
  SkinnyLds l;
  const int64_t mt = (m + 15) / 16 > 1 ? 2 : 1;   // activation tiles per wave
  l.ngw = (int32_t)((cnt * kStepK + group - 1) / group + 1);   // a range may straddle one more group
  l.sz_bytes = 16 * tiles * l.ngw * 8;
  const int64_t wm = (mt_total(m) + mt - 1) / mt;        // wave groups along the rows
  const int64_t wk = (waves + wm - 1) / wm;               // K ranges
  l.red_off = (wk * l.sz_bytes + 255) / 256 * 256;
  l.total = (size_t)l.red_off + (size_t)waves * mt * tiles * 64 * 16;
  (void)k;
  return l;
}

int32_t launch_skinny(const LinearArgs& a, const LinearPlan& pl, hipStream_t stream) {
  const SkinnyLds l = skinny_lds_layout(a.m, a.k, a.group, pl.waves, pl.ns, pl.cnt);
  SkinnyParams sp{a.x, a.packed,
                  a.mx ? static_cast<const void*>(a.scale8)
                       : a.sym16 && !a.row_scale ? static_cast<const void*>(a.scale16)
                                                 : static_cast<const void*>(a.scale),
                  a.zero, a.bias, a.y, a.m, a.n, a.k, a.y_bf16,
                  (a.k + kStepK - 1) / kStepK, a.k / a.group, a.prepared, pl.cnt, l.ngw,
                  l.sz_bytes, (int32_t)l.red_off, kNibPairMask, kBf16Offset2, a.row_scale, pl.wm, a.zp4,
                  a.zp4 ? (a.k / a.group + 1) / 2 : a.k / a.group, (int32_t)mt_total(a.m)};
  if (a.mx) return a.group == 32 ? dispatch_mt<32, kFmtMX>(sp, pl, l.total, stream) : WOQ_EUNSUPPORTED;
  if (a.sym16) {
    switch (a.group) {
      case 32: return dispatch_mt<32, kFmtS16>(sp, pl, l.total, stream);
      case 64: return dispatch_mt<64, kFmtS16>(sp, pl, l.total, stream);
      case 128: return dispatch_mt<128, kFmtS16>(sp, pl, l.total, stream);
      case 256: return dispatch_mt<256, kFmtS16>(sp, pl, l.total, stream);
      default: return WOQ_EUNSUPPORTED;
    }
  }
  switch (a.group) {
    case 32: return dispatch_mt<32, kFmtU4>(sp, pl, l.total, stream);
    case 64: return dispatch_mt<64, kFmtU4>(sp, pl, l.total, stream);
    case 128: return dispatch_mt<128, kFmtU4>(sp, pl, l.total, stream);
    case 256: return dispatch_mt<256, kFmtU4>(sp, pl, l.total, stream);
    default: return WOQ_EUNSUPPORTED;
  }
}

}  // namespace woq
