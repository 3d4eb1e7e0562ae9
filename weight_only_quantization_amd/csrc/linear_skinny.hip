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
// * A 4x4 transpose across lane groups (two gfx950 lane-swap stages) turns the
//   loaded bytes into the operand layout of four v_mfma_f32_16x16x32_bf16, one
//   per 32-wide input block.  Nibbles become bf16 (128 + code) with one
//   AND-OR per pair.  The MFMA sums x*(128+code) over each quantization group
//   and the group's contribution is scale * (sum - (128 + zero) * sum_of_x),
//   with the activation sums taken from the same MFMA unit against ones.
// * Partial sums of the waves meet in LDS; one pass adds the bias and stores.
#include "woq_internal.h"
#include "mfma_common.h"

namespace woq {
namespace {

constexpr int kStepK = 128;
constexpr int kBlockK = 32;
constexpr int kZeroBytes = 256;          // zero block read by lanes without an activation row
constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr uint32_t kOffsetOOB = 0x80000000u;   // a buffer offset no descriptor covers
// 16-byte staging chunks per thread and batch: activations, scales, zero points
constexpr int kStageX = 8, kStageS = 4, kStageZ = 2;

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
  int32_t s_off, z_off;  // LDS offsets of the staged scales and zero points
  int32_t z_bytewise;    // 1 when a row's zero points do not fill whole dwords
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
  const int wave = tid >> 6;
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

  const __amdgpu_buffer_rsrc_t rb = rsrc(p.packed + (int64_t)row0 * row_bytes, (uint32_t)rows * row_bytes);
  const __amdgpu_buffer_rsrc_t rs = rsrc(p.scale + (int64_t)row0 * ngroups, (uint32_t)rows * ngroups * 4);
  const __amdgpu_buffer_rsrc_t rz = rsrc(p.zero + (int64_t)row0 * ngroups, (uint32_t)rows * ngroups);
  const __amdgpu_buffer_rsrc_t rx = rsrc(p.x, (uint32_t)M * (uint32_t)K * 2);

  // ---- weight stream: PF steps in flight ------------------------------------
  // Steps past this wave's last one load nothing: their offsets get bit 31,
  // which no descriptor covers.  Computed arithmetically so the stream stays
  // free of branches (and of the conservative waits a branch would force).
  u32x4_t bq[PF][NS];
  auto issue = [&](int slot, int i) {
    const uint32_t dead = (uint32_t)(cnt - 1 - i) & kOffsetOOB;
    const int k0 = (wave + i * W) * kStepK;
#pragma unroll
    for (int t = 0; t < NS; ++t)
      bq[slot][t] = bload16(rb, ((uint32_t)(16 * t + c) * row_bytes + (uint32_t)(k0 / 2 + 16 * q)) | dead);
  };

  // ---- stage activations, scales and zero points in LDS ----------------------
  // Layout: [zero block][x rows, pair order, zero-padded][scales][zero points].
  // All staging loads are issued before the weight prefetch, so the one wait
  // for them leaves the weight loads in flight.
  const int cpr = p.kpad / 8;                     // 16-byte chunks per activation row
  const int xchunks = M * cpr;
  const uint32_t sbytes = (uint32_t)rows * ngroups * 4, zbytes = (uint32_t)rows * ngroups;
  const int schunks = (int)((sbytes + 15) / 16), zchunks = (int)((zbytes + 15) / 16);
  unsigned char* const lds_s = lds + p.s_off;
  unsigned char* const lds_z = lds + p.z_off;
  u32x4_t xb[kStageX], sb[kStageS], zb[kStageZ];
  auto load_x = [&](int base) {
#pragma unroll
    for (int u = 0; u < kStageX; ++u) {
      const int ch = base + tid + T * u;
      const int row = ch / cpr, col = ch % cpr;
      const bool ok = ch < xchunks && col * 8 < K;
      xb[u] = bload16(rx, ok ? (uint32_t)(row * K + col * 8) * 2 : kOffsetOOB);
    }
  };
  auto put_x = [&](int base) {
#pragma unroll
    for (int u = 0; u < kStageX; ++u) {
      const int ch = base + tid + T * u;
      if (ch < xchunks) {
        const int row = ch / cpr, col = ch % cpr;
        *reinterpret_cast<bf16x8_t*>(lds + kZeroBytes + row * p.xrow + col * 16) = pair_order(xb[u]);
      }
    }
  };
  auto load_sz = [&](int sbase, int zbase) {
#pragma unroll
    for (int u = 0; u < kStageS; ++u) {
      const int ch = sbase + tid + T * u;
      sb[u] = bload16(rs, ch < schunks ? (uint32_t)ch * 16 : kOffsetOOB);
    }
    // Buffer range checks work on whole dwords; when the zero points end inside
    // a dword they are fetched byte by byte so none of them reads back as 0.
    if (p.z_bytewise) {
#pragma unroll
      for (int u = 0; u < kStageZ; ++u) {
        const int ch = zbase + tid + T * u;
        uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const uint32_t off = ch < zchunks ? (uint32_t)(ch * 16 + e) : kOffsetOOB;
          w[e >> 2] |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rz, (int)off, 0, 0) << (8 * (e & 3));
        }
        zb[u] = u32x4_t{w[0], w[1], w[2], w[3]};
      }
    } else {
#pragma unroll
      for (int u = 0; u < kStageZ; ++u) {
        const int ch = zbase + tid + T * u;
        zb[u] = bload16(rz, ch < zchunks ? (uint32_t)ch * 16 : kOffsetOOB);
      }
    }
  };
  auto put_sz = [&](int sbase, int zbase) {
#pragma unroll
    for (int u = 0; u < kStageS; ++u) {
      const int ch = sbase + tid + T * u;
      if (ch < schunks) *reinterpret_cast<u32x4_t*>(lds_s + ch * 16) = sb[u];
    }
#pragma unroll
    for (int u = 0; u < kStageZ; ++u) {
      const int ch = zbase + tid + T * u;
      if (ch < zchunks) *reinterpret_cast<u32x4_t*>(lds_z + ch * 16) = zb[u];
    }
  };
  load_x(0);
  load_sz(0, 0);
#pragma unroll
  for (int u = 0; u < PF; ++u) issue(u, u);       // the weight stream starts now
  if (tid < kZeroBytes / 16)
    *reinterpret_cast<u32x4_t*>(lds + tid * 16) = u32x4_t{0u, 0u, 0u, 0u};
  put_x(0);
  put_sz(0, 0);
  for (int base = kStageX * T; base < xchunks; base += kStageX * T) {
    load_x(base);
    put_x(base);
  }
  for (int sbase = kStageS * T, zbase = kStageZ * T; sbase < schunks || zbase < zchunks;
       sbase += kStageS * T, zbase += kStageZ * T) {
    load_sz(sbase, zbase);
    put_sz(sbase, zbase);
  }
  __syncthreads();

  // ---- main loop --------------------------------------------------------------
  f32x4_t acc[NS];
#pragma unroll
  for (int t = 0; t < NS; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint32_t row_mask = c < M ? 0xFFFFFFFFu : 0u;   // lanes without a row read the zero block
  const uint32_t a_lane = (uint32_t)(kZeroBytes + c * p.xrow + 16 * q);
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4_t{kBf16One2, kBf16One2, kBf16One2, kBf16One2});
  const uint32_t nib_offset = vgpr_copy(p.nib_offset);

  // A dead step (past the wave's last) reads the zero block and zero-filled
  // weights and scales, so it adds exactly nothing.
  auto compute = [&](int slot, int i) {
    const int k0 = (wave + i * W) * kStepK;
    const uint32_t live_mask = (uint32_t)((i - cnt) >> 31);   // all ones while i < cnt
    const uint32_t a_addr = (a_lane + (uint32_t)k0 * 2) & row_mask & live_mask;
    bf16x8_t af[4];
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
      af[jb] = *reinterpret_cast<const bf16x8_t*>(lds + a_addr + 64 * jb);
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
      uint32_t d0 = bq[slot][t][0], d1 = bq[slot][t][1], d2 = bq[slot][t][2], d3 = bq[slot][t][3];
      transpose4_lanegroups(d0, d1, d2, d3);
      const uint32_t dw[4] = {d0, d1, d2, d3};
      const int srow = (16 * t + c) * ngroups;
#pragma unroll
      for (int pc = 0; pc < NP; ++pc) {
        // group of this piece, clamped so padded and dead steps read a finite scale
        const int g = min((k0 + kBlockK * GB * pc) >> p.group_shift, ngroups - 1);
        const float s = *reinterpret_cast<const float*>(lds_s + (srow + g) * 4);
        const float zz = -(kNibOffset + (float)lds_z[srow + g]);
        f32x4_t cg = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < GB; ++e)
          cg = mfma_bf16(af[pc * GB + e], unpack_codes(dw[pc * GB + e], p.nib_mask, nib_offset), cg);
#pragma unroll
        for (int r = 0; r < FR; ++r) acc[t][r] = fmaf(s, fmaf(zz, xs[pc][r], cg[r]), acc[t][r]);
      }
    }
  };

  for (int i0 = 0; i0 < cnt; i0 += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      compute(u, i0 + u);
      issue(u, i0 + u + PF);
    }
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
  // Prefetch depth: 8 steps with one weight tile per workgroup, 4 with two.
  switch (pl.gb) {
    case 1:   // two tiles of 32-wide groups exceed the register budget
      if constexpr (NS == 1) return launch_one<1, 1, 8, FR>(sp, pl, lds, stream);
      return WOQ_EUNSUPPORTED;
    case 2: return launch_one<NS, 2, NS == 1 ? 8 : 4, FR>(sp, pl, lds, stream);
    case 4: return launch_one<NS, 4, NS == 1 ? 8 : 4, FR>(sp, pl, lds, stream);
    default: return WOQ_EUNSUPPORTED;
  }
}

}  // namespace

struct SkinnyLds {
  size_t x_off, s_off, z_off, total;
};

SkinnyLds skinny_lds_layout(int64_t m, int64_t k, int64_t group, int waves, int ns) {
  const int64_t kpad = (k + kStepK - 1) / kStepK * kStepK;
  const int64_t rows = 16 * ns, ngroups = k / group;
  SkinnyLds l;
  l.x_off = kZeroBytes;
  l.s_off = l.x_off + (size_t)(m * (kpad * 2 + 16));
  l.z_off = l.s_off + (size_t)((rows * ngroups * 4 + 15) / 16 * 16);
  const size_t stage = l.z_off + (size_t)((rows * ngroups + 15) / 16 * 16);
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
                  gshift, kpad, kpad * 2 + 16, (int32_t)l.s_off, (int32_t)l.z_off,
                  (a.k / a.group) % 4 != 0 ? 1 : 0, kNibPairMask, kBf16Offset2};
  const size_t lds = l.total;
  const bool one = pl.fold_rows == 1;
  switch (pl.ns) {
    case 1: return one ? dispatch_gb<1, 1>(sp, pl, lds, stream) : dispatch_gb<1, 4>(sp, pl, lds, stream);
    case 2: return one ? dispatch_gb<2, 1>(sp, pl, lds, stream) : dispatch_gb<2, 4>(sp, pl, lds, stream);
    default: return WOQ_EUNSUPPORTED;
  }
}

}  // namespace woq
