// Skinny linear path (1 <= m <= 16): y = x . dequant(W)^T + bias for
// group-wise 4-bit weights (linnet docs "Quantization", std.quant table,
// linear_int4_groups).  At these row counts the layer is bound by the weight
// stream, so the kernel is organised around reading each packed byte once and
// keeping many bytes in flight:
//
// * A workgroup owns NS tiles of 16 weight rows (outputs) and all of K; its
//   W waves split K into 128-wide steps (wave w takes steps w, w+W, ...).
// * The activations x[M, K] are staged once per workgroup in LDS, already in
//   the slot order of the nibble unpacker and zero-padded to whole steps; the
//   scales and zero points of the workgroup's rows are staged next to them,
//   so the weight bytes are the only per-step global loads.
// * Per step and tile, each lane issues one 16-byte buffer load of its weight
//   row: lane group q reads inputs [k0+32q, k0+32q+32).  Buffer loads return
//   zero outside the workgroup's rows, so the stream has no branches and the
//   compiler can keep PF steps of loads in flight with exact vmcnt waits.
// * Which input each MFMA operand slot stands for is free as long as the
//   activation and weight operands agree.  When a group spans the whole step
//   (G >= 128), MFMA e takes dword e of every lane's load (inputs
//   k0+32q+8e .. +8), so the loaded bytes are used where they land.  Smaller
//   groups need each MFMA inside one group: a 4x4 transpose across lane groups
//   (two gfx950 lane-swap stages) gives MFMA e the 32 inputs of block e.
// * Nibbles become bf16 (128 + code) with one AND-OR per pair.  The MFMA sums
//   x*(128+code) over each group piece and the piece adds
//   scale * (sum - (128 + zero) * sum_of_x); the activation sums come from the
//   same MFMA unit against ones, the pair (scale, -(128 + zero)) from LDS.
// * Partial sums of the waves meet in LDS; one pass adds the bias and stores.
#include <type_traits>

#include "woq_internal.h"
#include "mfma_common.h"

namespace woq {
namespace {

constexpr int kStepK = 128;
constexpr int kBlockK = 32;
// LDS starts with a junk block, which absorbs the writes of out-of-range
// staging chunks, and a zero block, the activations of steps past a wave's last.
constexpr int kJunkBytes = 256;
constexpr int kZeroOff = 256;
constexpr int kXOff = 512;
constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr uint32_t kOffsetOOB = 0x80000000u;   // a buffer offset no descriptor covers
// s_waitcnt immediate that waits for LDS traffic only: lgkmcnt(0), vmcnt and
// expcnt at their maxima
constexpr int kWaitLdsOnly = 0xC07F;
// staging chunks per thread and batch: activations (8 inputs each) and
// scale / zero-point pairs (4 entries each)
constexpr int kStageX = 8, kStageS = 4;

struct SkinnyParams {
  const uint16_t* x;
  const uint8_t* packed;
  const float* scale;
  const uint8_t* zero;
  const float* bias;
  void* y;
  int32_t m, n, k, group, y_bf16;
  int32_t group_shift; // log2(group)
  int32_t kpad;        // K rounded up to a whole step
  int32_t xrow;        // LDS row stride of the staged activations, bytes
  int32_t sz_off;       // LDS offset of the staged (scale, -(128 + zero)) pairs
  int32_t z_bytewise;    // 1 when a row's zero points do not fill whole dwords
  int32_t t_rows, t_cols;  // workgroup size split into activation rows and 16-byte chunks
  int32_t prepared;        // 1: weights in the prepared layout
  // The nibble mask and the bf16 offset pattern arrive as arguments so they sit
  // in registers: one v_and_or_b32 per pair then expands two codes.
  uint32_t nib_mask, nib_offset;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, (int)kRsrcWord3);
}

__device__ __forceinline__ u32x4_t bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// NS: 16-row weight tiles per workgroup; GB: 32-wide blocks per quantization
// group inside a step (1, 2 or 4); PF: steps of weight loads in flight;
// FR: accumulator registers folded (1 when m == 1, else 4).
template <int NS, int GB, int PF, int FR>
__global__ __launch_bounds__(512) void skinny_kernel(SkinnyParams p) {
  constexpr int NP = 4 / GB;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int W = blockDim.x >> 6;
  const int T = blockDim.x;
  const int tid = threadIdx.x;
  // wave index made explicitly uniform: everything derived from it (step
  // offsets, counts, clamps) is then scalar work
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int q = lane >> 4;
  const int c = lane & 15;
  const int K = p.k, M = p.m, N = p.n;
  const int nsteps = p.kpad / kStepK;
  const int ngroups = K / p.group;
  const uint32_t row_bytes = (uint32_t)K / 2;
  const int row0 = blockIdx.x * NS * 16;
  const int rows = min(NS * 16, N - row0);
  const int cnt = wave < nsteps ? (nsteps - wave + W - 1) / W : 0;

  // Weights: canonical rows, or prepared 1 KB blocks (16 rows x one step,
  // tile-major) whose 16-byte slot l is lane l's share of a step.
  const bool prep = p.prepared != 0;   // uniform
  const int tile0 = blockIdx.x * NS;
  const int ptiles = min(NS, (N + 15) / 16 - tile0);
  const __amdgpu_buffer_rsrc_t rb =
      prep ? rsrc(p.packed + (int64_t)tile0 * nsteps * 1024, (uint32_t)(ptiles * nsteps) * 1024u)
           : rsrc(p.packed + (int64_t)row0 * row_bytes, (uint32_t)rows * row_bytes);
  const __amdgpu_buffer_rsrc_t rs = rsrc(p.scale + (int64_t)row0 * ngroups, (uint32_t)rows * ngroups * 4);
  const __amdgpu_buffer_rsrc_t rz = rsrc(p.zero + (int64_t)row0 * ngroups, (uint32_t)rows * ngroups);
  const __amdgpu_buffer_rsrc_t rx = rsrc(p.x, (uint32_t)M * (uint32_t)K * 2);

  // ---- weight stream: PF steps in flight ------------------------------------
  // Steps past this wave's last one load nothing: their offsets get bit 31,
  // which no descriptor covers.  Computed arithmetically so the stream stays
  // free of branches (and of the conservative waits a branch would force).
  u32x4_t bq[PF][NS];
  uint32_t boff[NS];              // per-lane byte offset of its row and lane group
#pragma unroll
  for (int t = 0; t < NS; ++t)
    boff[t] = prep ? (uint32_t)(t * nsteps) * 1024u + 16u * (uint32_t)lane
                   : (uint32_t)(16 * t + c) * row_bytes + (uint32_t)(16 * q);
  const uint32_t bstep = prep ? 1024u : (uint32_t)(kStepK / 2);
  auto issue = [&](int slot, int i) {
    const uint32_t dead = (uint32_t)(cnt - 1 - i) & kOffsetOOB;
    const uint32_t step_off = (uint32_t)(wave + i * W) * bstep | dead;   // uniform
#pragma unroll
    for (int t = 0; t < NS; ++t) bq[slot][t] = bload16(rb, boff[t] + step_off);
  };

  // ---- stage activations, scales and zero points in LDS ----------------------
  // Layout: [junk][zeros][x rows, pair order, zero-padded][(scale, -(128+zero))
  // float pairs of the workgroup's rows].  Common case: one batch of staging
  // loads per thread, issued before the weight prefetch, so the waits for them
  // leave the weight loads in flight.  Every staging load and LDS write is
  // unconditional (out-of-range loads use an offset no descriptor covers and
  // read zero; their writes land in the junk block): a load whose register is
  // consumed on only some paths would make the compiler drain the whole weight
  // stream inside the main loop.  Larger staging (long rows, many activation
  // rows, zero-point rows that end inside a dword) runs first, with its own
  // waits, before the stream starts.
  const int cpr = p.kpad / 8;                     // 8-input chunks per activation row
  const int xchunks = M * cpr;
  const int entries = rows * ngroups;
  const int szchunks = (entries + 3) / 4;
  const bool slow = xchunks > kStageX * T || szchunks > kStageS * T || p.z_bytewise;  // uniform
  u32x4_t xb[kStageX], sb[kStageS];
  uint32_t xr[kStageX], zb[kStageS];
  // Thread tid stages the chunks tid, tid+T, ... of the row-major chunk grid
  // [M][cpr]; (row, col) advance by (t_rows, t_cols) per chunk with one wrap,
  // so no division runs per chunk.  Each workgroup starts its columns at a
  // different offset, spreading the shared activation reads over L2 channels.
  const int rotc = (int)((blockIdx.x * 64u) % (uint32_t)cpr);
  auto load_x = [&](int batch, int limit) {
    const int ch0 = tid + batch * kStageX * T;       // one division per batch
    int row = ch0 / cpr, col = ch0 - row * cpr;
#pragma unroll
    for (int u = 0; u < kStageX; ++u) {
      int cr = col + rotc;
      cr = cr >= cpr ? cr - cpr : cr;
      const bool in = ch0 + T * u < limit;
      xb[u] = bload16(rx, in && cr * 8 < K ? (uint32_t)(row * K + cr * 8) * 2 : kOffsetOOB);
      xr[u] = in ? (uint32_t)(kXOff + row * p.xrow + cr * 16) : 0u;
      col += p.t_cols;
      row += p.t_rows;
      if (col >= cpr) { col -= cpr; ++row; }
    }
  };
  auto put_x = [&]() {
#pragma unroll
    for (int u = 0; u < kStageX; ++u) *reinterpret_cast<bf16x8_t*>(lds + xr[u]) = pair_order(xb[u]);
  };
  // chunk ch: entries 4ch .. 4ch+3 (entry = row * ngroups + group), 16 bytes
  // of scales and one dword of zero points
  auto load_sz = [&](int base, int limit, auto bytewise) {
#pragma unroll
    for (int u = 0; u < kStageS; ++u) {
      const int ch = base + tid + T * u;
      const bool in = ch < limit;
      sb[u] = bload16(rs, in ? (uint32_t)ch * 16 : kOffsetOOB);
      if constexpr (decltype(bytewise)::value) {
        // range checks work on whole dwords: the last row may end inside one
        uint32_t z = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          z |= (uint32_t)(uint8_t)__builtin_amdgcn_raw_buffer_load_b8(rz, in ? (uint32_t)(4 * ch + e) : kOffsetOOB, 0, 0) << (8 * e);
        zb[u] = z;
      } else {
        zb[u] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rz, in ? (uint32_t)ch * 4 : kOffsetOOB, 0, 0);
      }
    }
  };
  auto put_sz = [&](int base, int limit) {
#pragma unroll
    for (int u = 0; u < kStageS; ++u) {
      const int ch = base + tid + T * u;
      // (bit_cast of the whole vector: this compiler resolves a bit_cast of
      // one element of a vector lvalue to element 0)
      const f32x4_t sv = __builtin_bit_cast(f32x4_t, sb[u]);
      float f[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[2 * e] = sv[e];
        f[2 * e + 1] = -(kNibOffset + (float)((zb[u] >> (8 * e)) & 0xFFu));
      }
      f32x4_t* dst = reinterpret_cast<f32x4_t*>(lds + (ch < limit ? p.sz_off + ch * 32 : 0));
      dst[0] = f32x4_t{f[0], f[1], f[2], f[3]};
      dst[1] = f32x4_t{f[4], f[5], f[6], f[7]};
    }
  };
  if (slow) {
    for (int batch = 0; batch * kStageX * T < xchunks; ++batch) {
      load_x(batch, xchunks);
      put_x();
    }
    for (int base = 0; base < szchunks; base += kStageS * T) {
      load_sz(base, szchunks, std::true_type{});
      put_sz(base, szchunks);
    }
  }
  // the common case; after slow staging it only touches the junk block
  const int xlim = slow ? 0 : xchunks, szlim = slow ? 0 : szchunks;
  load_x(0, xlim);
  load_sz(0, szlim, std::false_type{});
#pragma unroll
  for (int u = 0; u < PF; ++u) issue(u, u);       // the weight stream starts now
  if (tid < 16) *reinterpret_cast<u32x4_t*>(lds + kZeroOff + 16 * tid) = u32x4_t{0u, 0u, 0u, 0u};
  put_x();
  put_sz(0, szlim);
  // The staging writes must be visible to the workgroup, but the weight loads
  // issued above stay in flight across the barrier (__syncthreads would wait
  // for every outstanding load, draining the ring before the first step).
  __builtin_amdgcn_s_waitcnt(kWaitLdsOnly);
  __builtin_amdgcn_s_barrier();

  // ---- main loop --------------------------------------------------------------
  constexpr bool kTranspose = GB < 4;
  f32x4_t acc[NS];
#pragma unroll
  for (int t = 0; t < NS; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // Activation operand of lane (q, i): row i (lanes past the last row repeat
  // row M-1; their outputs are never stored).  MFMA e reads the chunk of
  // inputs k0+32q+8e (no transpose) or k0+32e+8q (transpose).
  const uint32_t a_lane = (uint32_t)(kXOff + min(c, M - 1) * p.xrow + (kTranspose ? 16 : 64) * q);
  const uint32_t a_zero = (uint32_t)(kZeroOff + (kTranspose ? 16 : 64) * q);
  constexpr int kAStride = kTranspose ? 64 : 16;
  const uint32_t sz_lane = (uint32_t)(p.sz_off + c * ngroups * 8);
  const uint32_t nib_offset = vgpr_copy(p.nib_offset);
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4_t{kBf16One2, kBf16One2, kBf16One2, kBf16One2});

  // Step i takes its weights out of ring slot `slot`, refills the slot with
  // step i + PF as soon as the bytes are out of it, and only then computes;
  // the scheduling barrier keeps the compiler from sinking the refill below
  // the arithmetic, which would let the stream run dry once per ring turn.
  // A step past the wave's last multiplies zero activations (the zero block)
  // by zero weights and adds exactly nothing.
  auto step = [&](int slot, int i) {
    const bool live = i < cnt;
    const int k0 = min(wave + max(min(i, cnt - 1), 0) * W, nsteps - 1) * kStepK;
    const uint32_t a_addr = live ? a_lane + (uint32_t)k0 * 2 : a_zero;
    bf16x8_t af[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) af[e] = *reinterpret_cast<const bf16x8_t*>(lds + a_addr + kAStride * e);
    // (scale, -(128 + zero)) of each tile row and group piece
    float2 sz[NS][NP];
#pragma unroll
    for (int t = 0; t < NS; ++t)
#pragma unroll
      for (int pc = 0; pc < NP; ++pc) {
        const int g = min((k0 + kBlockK * GB * pc) >> p.group_shift, ngroups - 1);
        sz[t][pc] = *reinterpret_cast<const float2*>(lds + sz_lane + (16 * t * ngroups + g) * 8);
      }
    bf16x8_t bw[NS][4];
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      if constexpr (kTranspose) {
        // The lane swaps work in place; on copies, the slot's registers stay
        // free for the refill and keep their place from one ring turn to the
        // next (no copy of a register a load is still writing).
        uint32_t d0 = vgpr_copy(bq[slot][t][0]), d1 = vgpr_copy(bq[slot][t][1]);
        uint32_t d2 = vgpr_copy(bq[slot][t][2]), d3 = vgpr_copy(bq[slot][t][3]);
        transpose4_lanegroups(d0, d1, d2, d3);
        bw[t][0] = unpack_codes(d0, p.nib_mask, nib_offset);
        bw[t][1] = unpack_codes(d1, p.nib_mask, nib_offset);
        bw[t][2] = unpack_codes(d2, p.nib_mask, nib_offset);
        bw[t][3] = unpack_codes(d3, p.nib_mask, nib_offset);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) bw[t][e] = unpack_codes(bq[slot][t][e], p.nib_mask, nib_offset);
      }
    }
    issue(slot, i + PF);
    __builtin_amdgcn_sched_barrier(0);
    // activation sums of each group piece, in the accumulator layout
    f32x4_t xs[NP];
#pragma unroll
    for (int pc = 0; pc < NP; ++pc) {
      f32x4_t v = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < GB; ++e) v = mfma_bf16(af[pc * GB + e], ones, v);
      xs[pc] = v;
    }
#pragma unroll
    for (int t = 0; t < NS; ++t) {
#pragma unroll
      for (int pc = 0; pc < NP; ++pc) {
        f32x4_t cg = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < GB; ++e) cg = mfma_bf16(af[pc * GB + e], bw[t][pc * GB + e], cg);
#pragma unroll
        for (int r = 0; r < FR; ++r)
          acc[t][r] = fmaf(sz[t][pc].x, fmaf(sz[t][pc].y, xs[pc][r], cg[r]), acc[t][r]);
      }
    }
  };

  for (int i0 = 0; i0 < cnt; i0 += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) step(u, i0 + u);
  }

  // ---- combine the waves, add the bias, store ----------------------------------
  constexpr int kTileElems = NS * 4 * 64;
  auto store = [&](int e, float v) {
    const int ln = e & 63;
    const int r = (e >> 6) & 3;
    const int t = e >> 8;
    const int m = 4 * (ln >> 4) + r;
    const int n = row0 + 16 * t + (ln & 15);
    if (m < M && n < N) {
      if (p.bias) v += p.bias[n];
      if (p.y_bf16)
        reinterpret_cast<uint16_t*>(p.y)[(int64_t)m * N + n] = f32_to_bf16_bits(v);
      else
        reinterpret_cast<float*>(p.y)[(int64_t)m * N + n] = v;
    }
  };
  if (W == 1) {
#pragma unroll
    for (int t = 0; t < NS; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) store((t * 4 + r) * 64 + lane, acc[t][r]);
    return;
  }
  __syncthreads();   // the activation area becomes the reduction area
  float* red = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int t = 0; t < NS; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave * kTileElems + (t * 4 + r) * 64 + lane] = acc[t][r];
  __syncthreads();
  for (int e = tid; e < kTileElems; e += T) {
    float v = 0.f;
    for (int w = 0; w < W; ++w) v += red[w * kTileElems + e];
    store(e, v);
  }
}

template <int NS, int GB, int PF, int FR>
int32_t launch_one(const SkinnyParams& sp, const LinearPlan& pl, size_t lds, hipStream_t stream) {
  auto kern = skinny_kernel<NS, GB, PF, FR>;
  if (lds > 64 * 1024) {
    static bool raised = false;   // raise the dynamic-LDS limit once per instantiation
    if (!raised) {
      if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                              hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess)
        return WOQ_EHIP;
      raised = true;
    }
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)pl.grid), dim3(64 * pl.waves), lds, stream, sp);
  return hip_status(hipGetLastError());
}

template <int NS, int FR>
int32_t dispatch_gb(const SkinnyParams& sp, const LinearPlan& pl, size_t lds, hipStream_t stream) {
  // Four steps in flight per wave: deeper rings measured slower on the decode
  // shapes (more outstanding requests delay every workgroup's staging).
  switch (pl.gb) {
    case 1:   // two tiles of 32-wide groups exceed the register budget
      if constexpr (NS == 1) return launch_one<1, 1, 4, FR>(sp, pl, lds, stream);
      return WOQ_EUNSUPPORTED;
    case 2: return launch_one<NS, 2, 4, FR>(sp, pl, lds, stream);
    case 4: return launch_one<NS, 4, 4, FR>(sp, pl, lds, stream);
    default: return WOQ_EUNSUPPORTED;
  }
}

}  // namespace

struct SkinnyLds {
  size_t sz_off, total;
};

SkinnyLds skinny_lds_layout(int64_t m, int64_t k, int64_t group, int waves, int ns) {
  const int64_t kpad = (k + kStepK - 1) / kStepK * kStepK;
  const int64_t entries = 16 * ns * (k / group);
  SkinnyLds l;
  l.sz_off = (size_t)kXOff + (size_t)(m * (kpad * 2 + 16));
  const size_t stage = l.sz_off + (size_t)((entries + 3) / 4 * 32);
  const size_t red = waves > 1 ? (size_t)waves * ns * 4 * 64 * 4 : 0;
  l.total = stage > red ? stage : red;
  return l;
}

size_t skinny_lds_bytes(int64_t m, int64_t k, int64_t group, int waves, int ns) {
  return skinny_lds_layout(m, k, group, waves, ns).total;
}

int32_t launch_skinny(const LinearArgs& a, const LinearPlan& pl, hipStream_t stream) {
  const int32_t kpad = (a.k + kStepK - 1) / kStepK * kStepK;
  int32_t gshift = 0;
  while ((1 << gshift) < a.group) ++gshift;
  const SkinnyLds l = skinny_lds_layout(a.m, a.k, a.group, pl.waves, pl.ns);
  SkinnyParams sp{a.x, a.packed, a.scale, a.zero, a.bias, a.y, a.m, a.n, a.k, a.group, a.y_bf16,
                  gshift, kpad, kpad * 2 + 16, (int32_t)l.sz_off,
                  (a.k / a.group) % 4 != 0 ? 1 : 0, 64 * pl.waves / (kpad / 8),
                  64 * pl.waves % (kpad / 8), a.prepared, kNibPairMask, kBf16Offset2};
  const size_t lds = l.total;
  const bool one = pl.fold_rows == 1;
  switch (pl.ns) {
    case 1: return one ? dispatch_gb<1, 1>(sp, pl, lds, stream) : dispatch_gb<1, 4>(sp, pl, lds, stream);
    case 2: return one ? dispatch_gb<2, 1>(sp, pl, lds, stream) : dispatch_gb<2, 4>(sp, pl, lds, stream);
    default: return WOQ_EUNSUPPORTED;
  }
}

}  // namespace woq
