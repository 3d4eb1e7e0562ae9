// Skinny linear path (1 <= m <= 16): y = x . dequant(W)^T + bias for
// group-wise 4-bit weights (linnet docs "Quantization", std.quant table,
// linear_int4_groups).  At these row counts the layer is bound by the weight
// stream, so the kernel is organised around reading each packed byte once:
//
// * A workgroup owns NS tiles of 16 weight rows (outputs) and all of K; its
//   waves split K into 128-wide steps (wave w takes steps w, w+W, ...).
// * Per step and tile, each lane issues one 16-byte load of its row: lane
//   group q reads inputs [k0+32q, k0+32q+32).  A 4x4 transpose across lane
//   groups (two gfx950 lane-swap stages) turns that into the operand layout of
//   four v_mfma_f32_16x16x32_bf16, one per 32-wide input block.
// * Nibbles become bf16 (128 + code) with one AND-OR per pair; activations are
//   reordered to match.  The MFMA sums x*(128+code) over each quantization
//   group; the group's contribution is then
//       scale * (sum - (128 + zero) * sum_of_x)
//   with the activation sums taken from the same MFMA unit against ones.
// * Partial sums of the waves meet in LDS; one pass adds the bias and stores.
// Loads are prefetched PF steps ahead so each wave keeps several KB in flight.
#include "woq_internal.h"
#include "mfma_common.h"

namespace woq {
namespace {

constexpr int kStepK = 128;
constexpr int kBlockK = 32;

struct SkinnyParams {
  const uint16_t* x;
  const uint8_t* packed;
  const float* scale;
  const uint8_t* zero;
  const float* bias;
  void* y;
  int32_t m, n, k, group, y_bf16;
};

// MT: 16-row activation tiles; FR: accumulator registers folded (1 if m == 1);
// NS: 16-row weight tiles per workgroup; GB: 32-wide blocks per group within a
// step (1, 2 or 4); PF: steps of weight loads kept in flight (even).
template <int MT, int FR, int NS, int GB, int PF>
__global__ __launch_bounds__(1024) void skinny_kernel(SkinnyParams p) {
  constexpr int NP = 4 / GB;   // quantization-group pieces per step
  extern __shared__ float red[];
  const int W = blockDim.x >> 6;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4;
  const int c = lane & 15;
  const int K = p.k, M = p.m, N = p.n;
  const int nsteps = (K + kStepK - 1) / kStepK;
  const int ngroups = K / p.group;
  const int64_t row_bytes = K / 2;
  const int tile0 = blockIdx.x * NS;
  const int cnt = wave < nsteps ? (nsteps - wave + W - 1) / W : 0;

  f32x4_t acc[NS][MT];
#pragma unroll
  for (int t = 0; t < NS; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Per-lane weight row of each tile, and whether it exists.
  int nrow[NS];
  bool nok[NS];
#pragma unroll
  for (int t = 0; t < NS; ++t) {
    nrow[t] = 16 * (tile0 + t) + c;
    nok[t] = nrow[t] < N;
  }

  u32x4_t bq[PF][NS];
  float sq[PF][NS][NP];
  uint32_t zq[PF][NS];          // zero points of the NP pieces, one byte each
  u32x4_t aq[2][MT][4];

  auto issue_b = [&](u32x4_t (&b)[NS], float (&s)[NS][NP], uint32_t (&z)[NS], int i) {
    const int k0 = (wave + i * W) * kStepK;
    const int nb = min(4, (K - k0) / kBlockK);
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      if (nok[t] && q < nb) {
        b[t] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4_t*>(p.packed + (int64_t)nrow[t] * row_bytes + k0 / 2 + 16 * q));
      } else {
        b[t] = u32x4_t{0u, 0u, 0u, 0u};
      }
      z[t] = 0u;
#pragma unroll
      for (int pc = 0; pc < NP; ++pc) {
        const int jb0 = pc * GB;
        if (nok[t] && jb0 < nb) {
          const int64_t gi = (int64_t)nrow[t] * ngroups + (k0 + kBlockK * jb0) / p.group;
          s[t][pc] = p.scale[gi];
          z[t] |= (uint32_t)p.zero[gi] << (8 * pc);
        } else {
          s[t][pc] = 0.f;
        }
      }
    }
  };

  auto issue_a = [&](u32x4_t (&a)[MT][4], int i) {
    const int k0 = (wave + i * W) * kStepK;
    const int nb = min(4, (K - k0) / kBlockK);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = 16 * mt + c;
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        if (m < M && jb < nb)
          a[mt][jb] = load16(p.x + (int64_t)m * K + k0 + kBlockK * jb + 8 * q);
        else
          a[mt][jb] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  };

  auto compute = [&](const u32x4_t (&b)[NS], const float (&s)[NS][NP], const uint32_t (&z)[NS],
                     const u32x4_t (&a)[MT][4], int i) {
    const int k0 = (wave + i * W) * kStepK;
    const int nb = min(4, (K - k0) / kBlockK);
    const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4_t{kBf16One2, kBf16One2, kBf16One2, kBf16One2});
    bf16x8_t af[MT][4];
    f32x4_t xs[NP][MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) af[mt][jb] = pair_order(a[mt][jb]);
    // Activation sums of each group piece, in the accumulator layout.
#pragma unroll
    for (int pc = 0; pc < NP; ++pc)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4_t v = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < GB; ++e) v = mfma_bf16(af[mt][pc * GB + e], ones, v);
        xs[pc][mt] = v;
      }
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      uint32_t d0 = b[t][0], d1 = b[t][1], d2 = b[t][2], d3 = b[t][3];
      transpose4_lanegroups(d0, d1, d2, d3);
      const uint32_t dw[4] = {d0, d1, d2, d3};
#pragma unroll
      for (int pc = 0; pc < NP; ++pc) {
        if (pc * GB >= nb) break;
        f32x4_t cg[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) cg[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < GB; ++e) {
          const bf16x8_t bf = unpack_codes(dw[pc * GB + e]);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) cg[mt] = mfma_bf16(af[mt][pc * GB + e], bf, cg[mt]);
        }
        const float zz = -(kNibOffset + (float)((z[t] >> (8 * pc)) & 0xFFu));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < FR; ++r)
            acc[t][mt][r] = fmaf(s[t][pc], fmaf(zz, xs[pc][mt][r], cg[mt][r]), acc[t][mt][r]);
      }
    }
  };

  // Prologue: weight loads for the first PF steps, activations for the first.
#pragma unroll
  for (int u = 0; u < PF; ++u)
    if (u < cnt) issue_b(bq[u], sq[u], zq[u], u);
  if (cnt > 0) issue_a(aq[0], 0);

  for (int i0 = 0; i0 < cnt; i0 += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int i = i0 + u;
      if (i < cnt) {
        if (i + 1 < cnt) issue_a(aq[(u + 1) & 1], i + 1);
        compute(bq[u], sq[u], zq[u], aq[u & 1], i);
        if (i + PF < cnt) issue_b(bq[u], sq[u], zq[u], i + PF);
      }
    }
  }

  // Combine the waves' partial sums, add the bias, store.
  constexpr int kTileElems = NS * MT * 4 * 64;
  auto store = [&](int e, float v) {
    const int ln = e & 63;
    const int r = (e >> 6) & 3;
    const int mt = (e >> 8) % MT;
    const int t = (e >> 8) / MT;
    const int m = 16 * mt + 4 * (ln >> 4) + r;
    const int n = 16 * (tile0 + t) + (ln & 15);
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
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) store(((t * MT + mt) * 4 + r) * 64 + lane, acc[t][mt][r]);
    return;
  }
#pragma unroll
  for (int t = 0; t < NS; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        red[wave * kTileElems + ((t * MT + mt) * 4 + r) * 64 + lane] = acc[t][mt][r];
  __syncthreads();
  for (int e = threadIdx.x; e < kTileElems; e += blockDim.x) {
    float v = 0.f;
    for (int w = 0; w < W; ++w) v += red[w * kTileElems + e];
    store(e, v);
  }
}

template <int MT, int FR, int NS, int GB, int PF>
int32_t launch_one(const SkinnyParams& sp, const LinearPlan& pl, hipStream_t stream) {
  const size_t lds = pl.waves > 1 ? (size_t)pl.waves * NS * MT * 4 * 64 * sizeof(float) : 0;
  hipLaunchKernelGGL((skinny_kernel<MT, FR, NS, GB, PF>), dim3((unsigned)pl.grid),
                     dim3(64 * pl.waves), lds, stream, sp);
  return hip_status(hipGetLastError());
}

// Prefetch depth: 4 steps for one weight tile per workgroup, 2 for two; 2 for
// 32-wide groups, whose four pieces per step hold more scale state.
template <int MT, int FR, int NS>
int32_t dispatch_gb(const SkinnyParams& sp, const LinearPlan& pl, hipStream_t stream) {
  constexpr int PF = NS == 1 ? 4 : 2;
  switch (pl.gb) {
    case 1:
      if (NS != 1) return WOQ_EUNSUPPORTED;
      return launch_one<MT, FR, 1, 1, 2>(sp, pl, stream);
    case 2: return launch_one<MT, FR, NS, 2, PF>(sp, pl, stream);
    case 4: return launch_one<MT, FR, NS, 4, PF>(sp, pl, stream);
    default: return WOQ_EUNSUPPORTED;
  }
}

template <int MT, int FR>
int32_t dispatch_ns(const SkinnyParams& sp, const LinearPlan& pl, hipStream_t stream) {
  switch (pl.ns) {
    case 1: return dispatch_gb<MT, FR, 1>(sp, pl, stream);
    case 2: return dispatch_gb<MT, FR, 2>(sp, pl, stream);
    default: return WOQ_EUNSUPPORTED;
  }
}

}  // namespace

int32_t launch_skinny(const LinearArgs& a, const LinearPlan& pl, hipStream_t stream) {
  SkinnyParams sp{a.x, a.packed, a.scale, a.zero, a.bias, a.y, a.m, a.n, a.k, a.group, a.y_bf16};
  if (pl.mt == 1 && pl.fold_rows == 1) return dispatch_ns<1, 1>(sp, pl, stream);
  if (pl.mt == 1) return dispatch_ns<1, 4>(sp, pl, stream);
  return WOQ_EUNSUPPORTED;
}

}  // namespace woq
