// Tiled linear path (m > 32) and the activation pre-pass.
//
// Pre-pass: x' = x gathered through the act-order index when one is given
// (linnet docs "Quantization", section "Importing GPTQ and AWQ": the layer
// gathers its inputs first), optionally written in the slot order of the
// nibble unpacker, plus the float32 sum of x' over every "piece": the part of
// a quantization group inside one 128-wide k step (the whole group for
// groups of at most 128 inputs).
//
// GEMM: a workgroup of 8 waves computes a 128 x 256 tile of y.  The activation
// tile of each 128-wide k step is staged in LDS (double buffered, one barrier
// per step); every wave streams its own 64 weight rows straight from global
// memory into registers, transposes them across lane groups and expands the
// nibbles to bf16 (128 + code) for v_mfma_f32_16x16x32_bf16.  Per
// quantization group the MFMA sums are folded into float32 accumulators as
//   acc += scale * (sum - (128 + zero) * group_sum_of_x).
#include "woq_internal.h"
#include "mfma_common.h"

namespace woq {
namespace {

constexpr int kStepK = 128;
constexpr int kBlockK = 32;

// One thread per 8 consecutive inputs of a row (16 bytes).  The lanes of one
// piece (piece/8 of them, consecutive) add their partial sums in a fixed
// shuffle tree, so the sums are the same on every run.  Rows from m to mpad
// only get zero sums.
template <int LP>   // lanes per piece: piece / 8
__global__ __launch_bounds__(256) void prep_kernel(const uint16_t* __restrict__ x,
                                                   const int32_t* __restrict__ order, int32_t m,
                                                   int32_t k, int32_t permute,
                                                   uint16_t* __restrict__ xg, float* __restrict__ xs,
                                                   int64_t mpad) {
  const int cpr = k / 8;                       // chunks per row
  const int npieces = cpr / LP;
  const int64_t total = mpad * cpr;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
    const int64_t row = t / cpr;
    const int col = (int)(t % cpr);
    u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
    if (row < m) {
      const uint16_t* xr = x + row * k;
      if (order) {
        const u32x4_t i0 = load16(order + col * 8), i1 = load16(order + col * 8 + 4);
        const int32_t idx[8] = {(int32_t)i0[0], (int32_t)i0[1], (int32_t)i0[2], (int32_t)i0[3],
                                (int32_t)i1[0], (int32_t)i1[1], (int32_t)i1[2], (int32_t)i1[3]};
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int src = idx[e] < 0 ? 0 : (idx[e] >= k ? k - 1 : idx[e]);   // clamp bad indices
          h[e] = xr[src];
        }
        v = u32x4_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
      } else {
        v = load16(xr + col * 8);
      }
    }
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      sum += __builtin_bit_cast(float, v[e] << 16) + __builtin_bit_cast(float, v[e] & 0xFFFF0000u);
#pragma unroll
    for (int off = 1; off < LP; off <<= 1) sum += __shfl_xor(sum, off, LP);
    if (row < m && xg)
      *reinterpret_cast<u32x4_t*>(xg + row * k + col * 8) =
          permute ? __builtin_bit_cast(u32x4_t, pair_order(v)) : v;
    if (xs && (col % LP) == 0) xs[(int64_t)(col / LP) * mpad + row] = sum;
  }
}

__global__ __launch_bounds__(256) void fill_bias_kernel(const float* __restrict__ bias, int32_t m,
                                                        int32_t n, int32_t y_bf16, void* __restrict__ y) {
  const int64_t total = (int64_t)m * n;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
    const float v = bias ? bias[t % n] : 0.f;
    if (y_bf16)
      reinterpret_cast<uint16_t*>(y)[t] = f32_to_bf16_bits(v);
    else
      reinterpret_cast<float*>(y)[t] = v;
  }
}

constexpr int kBM = 128, kBN = 256;
constexpr int kWaves = 8;                 // 2 (m) x 4 (n), each wave 64 x 64
constexpr int kLdsRow = kStepK + 8;       // bf16 elements per LDS row (padding breaks bank aliasing)
constexpr int kStageElems = kBM * kLdsRow;

struct GemmParams {
  const uint16_t* xp;     // pair-ordered activations [M, K]
  const uint8_t* packed;
  const float* scale;
  const uint8_t* zero;
  const float* bias;
  const float* xs;        // [K/min(G,128)][mpad]
  void* y;
  int32_t m, n, k, group, y_bf16;
  int64_t mpad;
  int32_t tiles_m, tiles_n;
};

template <int GB>
__global__ __launch_bounds__(512) void gemm_kernel(GemmParams p) {
  constexpr int NP = 4 / GB;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * kStageElems];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int q = lane >> 4, c = lane & 15;
  const int wm = wave >> 2, wn = wave & 3;
  const int K = p.k, M = p.m, N = p.n;
  const int ngroups = K / p.group;
  const int64_t row_bytes = K / 2;

  // Workgroups are dealt to the 8 XCDs round robin; renumber so that the
  // workgroups of one XCD cover neighbouring tiles that share weight columns.
  const int nwg = p.tiles_m * p.tiles_n;
  int bid = blockIdx.x;
  const int full = (nwg / 8) * 8;
  if (bid < full) bid = (bid % 8) * (full / 8) + bid / 8;
  const int tm = bid % p.tiles_m, tn = bid / p.tiles_m;
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int nsteps = (K + kStepK - 1) / kStepK;

  f32x4_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  int nrow[4];
  bool nok[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    nrow[nt] = n0 + 64 * wn + 16 * nt + c;
    nok[nt] = nrow[nt] < N;
  }

  // Global -> register staging of the activation tile: 2048 chunks of 16 B,
  // 4 per thread.
  u32x4_t ga[4];
  auto load_a = [&](int step) {
    const int k0 = step * kStepK;
    const int kw = min(kStepK, K - k0);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int id = tid + 512 * u;
      const int row = id >> 4, col = (id & 15) * 8;
      if (m0 + row < M && col < kw)
        ga[u] = load16(p.xp + (int64_t)(m0 + row) * K + k0 + col);
      else
        ga[u] = u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  auto store_a = [&](int stage) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int id = tid + 512 * u;
      const int row = id >> 4, col = (id & 15) * 8;
      *reinterpret_cast<u32x4_t*>(&lds[stage * kStageElems + row * kLdsRow + col]) = ga[u];
    }
  };

  u32x4_t gb[4];
  auto load_b = [&](int step) {
    const int k0 = step * kStepK;
    const int nb = min(4, (K - k0) / kBlockK);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      if (nok[nt] && q < nb)
        gb[nt] = load16(p.packed + (int64_t)nrow[nt] * row_bytes + k0 / 2 + 16 * q);
      else
        gb[nt] = u32x4_t{0u, 0u, 0u, 0u};
    }
  };

  // The weights of this step leave gb through the transpose; the next step's
  // loads are issued into gb right after, to land during this step's MFMAs.
  const uint32_t nib_offset = vgpr_copy(kBf16Offset2);
  auto compute = [&](int stage, int step) {
    const int k0 = step * kStepK;
    const int nb = min(4, (K - k0) / kBlockK);
    uint32_t dw[4][4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      uint32_t d0 = gb[nt][0], d1 = gb[nt][1], d2 = gb[nt][2], d3 = gb[nt][3];
      transpose4_lanegroups(d0, d1, d2, d3);
      dw[nt][0] = d0; dw[nt][1] = d1; dw[nt][2] = d2; dw[nt][3] = d3;
    }
    if (step + 1 < nsteps) load_b(step + 1);
#pragma unroll
    for (int pc = 0; pc < NP; ++pc) {
      if (pc * GB >= nb) break;
      const int g = (k0 + kBlockK * pc * GB) / p.group;
      const int pi = (k0 + kBlockK * pc * GB) / (kBlockK * GB);
      // metadata of this piece: per-row activation sums, per-column scale and zero
      f32x4_t xsv[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        xsv[mt] = *reinterpret_cast<const f32x4_t*>(p.xs + (int64_t)pi * p.mpad + m0 + 64 * wm + 16 * mt + 4 * q);
      float sv[4], zv[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int64_t gi = (int64_t)(nok[nt] ? nrow[nt] : 0) * ngroups + g;
        sv[nt] = nok[nt] ? p.scale[gi] : 0.f;
        zv[nt] = -(kNibOffset + (float)(nok[nt] ? p.zero[gi] : 0));
      }
      bf16x8_t af[4][GB];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int e = 0; e < GB; ++e)
          af[mt][e] = __builtin_bit_cast(
              bf16x8_t, *reinterpret_cast<const u32x4_t*>(
                            &lds[stage * kStageElems + (64 * wm + 16 * mt + c) * kLdsRow +
                                 kBlockK * (pc * GB + e) + 8 * q]));
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        f32x4_t cg[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) cg[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < GB; ++e) {
          const bf16x8_t bf = unpack_codes(dw[nt][pc * GB + e], kNibPairMask, nib_offset);
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) cg[mt] = mfma_bf16(af[mt][e], bf, cg[mt]);
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[nt][mt][r] = fmaf(sv[nt], fmaf(zv[nt], xsv[mt][r], cg[mt][r]), acc[nt][mt][r]);
      }
    }
  };

  if (nsteps > 0) {
    load_a(0);
    load_b(0);
    store_a(0);
    __syncthreads();
  }
  for (int i0 = 0; i0 < nsteps; i0 += 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = i0 + u;
      if (i < nsteps) {
        const bool more = i + 1 < nsteps;
        if (more) load_a(i + 1);
        compute(u, i);
        if (more) store_a(u ^ 1);
        __syncthreads();
      }
    }
  }

#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int n = nrow[nt];
    if (!nok[nt]) continue;
    const float b = p.bias ? p.bias[n] : 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 64 * wm + 16 * mt + 4 * q + r;
        if (m < M) {
          const float v = acc[nt][mt][r] + b;
          if (p.y_bf16)
            reinterpret_cast<uint16_t*>(p.y)[(int64_t)m * N + n] = f32_to_bf16_bits(v);
          else
            reinterpret_cast<float*>(p.y)[(int64_t)m * N + n] = v;
        }
      }
  }
}

}  // namespace

int32_t launch_prep(const uint16_t* x, const int32_t* order, int32_t m, int32_t k, int32_t group,
                    int32_t permute, uint16_t* xg, float* xs, int64_t mpad, hipStream_t stream) {
  const int32_t piece = group < kStepK ? group : kStepK;
  const int64_t total = mpad * (k / 8);
  if (total == 0) return WOQ_OK;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  switch (piece / 8) {
    case 4: hipLaunchKernelGGL(prep_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, stream, x, order, m, k, permute, xg, xs, mpad); break;
    case 8: hipLaunchKernelGGL(prep_kernel<8>, dim3((unsigned)blocks), dim3(256), 0, stream, x, order, m, k, permute, xg, xs, mpad); break;
    case 16: hipLaunchKernelGGL(prep_kernel<16>, dim3((unsigned)blocks), dim3(256), 0, stream, x, order, m, k, permute, xg, xs, mpad); break;
    default: return WOQ_EUNSUPPORTED;
  }
  return hip_status(hipGetLastError());
}

int32_t launch_fill_bias(const float* bias, int32_t m, int32_t n, int32_t y_bf16, void* y,
                         hipStream_t stream) {
  const int64_t total = (int64_t)m * n;
  if (total == 0) return WOQ_OK;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_bias_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, bias, m, n,
                     y_bf16, y);
  return hip_status(hipGetLastError());
}

int32_t launch_gemm(const LinearArgs& a, const LinearPlan& pl, hipStream_t stream) {
  GemmParams gp{a.x, a.packed, a.scale, a.zero, a.bias, a.xs, a.y, a.m, a.n, a.k, a.group,
                a.y_bf16, a.mpad, (a.m + kBM - 1) / kBM, (a.n + kBN - 1) / kBN};
  const unsigned grid = (unsigned)(gp.tiles_m * gp.tiles_n);
  switch (pl.gb) {
    case 1: hipLaunchKernelGGL(gemm_kernel<1>, dim3(grid), dim3(512), 0, stream, gp); break;
    case 2: hipLaunchKernelGGL(gemm_kernel<2>, dim3(grid), dim3(512), 0, stream, gp); break;
    case 4: hipLaunchKernelGGL(gemm_kernel<4>, dim3(grid), dim3(512), 0, stream, gp); break;
    default: return WOQ_EUNSUPPORTED;
  }
  return hip_status(hipGetLastError());
}

}  // namespace woq
