// AWQ scale search for one layer ("20. Quantization", stretch exercise 3: a
// per-input-channel scale s_j = mean|x_j|^alpha, alpha searched over [0, 1] for
// the least calibration output error after 4-bit quantization of W diag(s); the
// page's scaling identity X W^T = (X S^-1)(W S)^T makes the scaled layer
// compute with X S^-1).  The grid is alpha = i / n_grid, i = 0 .. n_grid; the
// scales are float32(max(mean|x_j|^alpha, 1e-4)); the scaled weights float32(w * s)
// go through the group quantizer; the error of a grid point is
// ||X (W - W_hat)^T||_F^2 with W_hat = (q - zero) * scale / s, in float64; the
// first least error wins.
//
// Per grid point: the scales (K threads), the scaled weights, the group
// quantizer, and one float64 tile kernel for E = X (W - W_hat)^T that forms
// W - W_hat while it stages the weights and leaves each tile's sum of squares
// in a slot of its own; one workgroup adds the slots in a fixed order, so the
// errors do not depend on scheduling.
#include <vector>

#include "woq_internal.h"

#pragma clang fp contract(off)

namespace woq {
namespace {

constexpr double kAwqFloor = 1e-4;

__device__ __forceinline__ double bf16_bits_f64(uint16_t b) { return (double)__uint_as_float((uint32_t)b << 16); }

// m[j] = (sum_t |x[t][j]|) / T, the rows added in order.
__global__ __launch_bounds__(256) void awq_mean_kernel(const uint16_t* __restrict__ x, int64_t t, int64_t k,
                                                       double* __restrict__ m) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= k) return;
  double acc = 0.0;
  for (int64_t r = 0; r < t; ++r) acc += fabs(bf16_bits_f64(x[r * k + j]));
  m[j] = acc / (double)t;
}

__global__ __launch_bounds__(256) void awq_scale_kernel(const double* __restrict__ m, int64_t k, double alpha,
                                                        float* __restrict__ s) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j < k) s[j] = (float)fmax(pow(m[j], alpha), kAwqFloor);
}

// ws = float32(w * s[column]) (a float32 product: the exact product rounded once).
__global__ __launch_bounds__(256) void awq_scale_weights_kernel(const float* __restrict__ w,
                                                                const float* __restrict__ s, int64_t n, int64_t k,
                                                                float* __restrict__ ws) {
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n * k; e += (int64_t)gridDim.x * 256)
    ws[e] = w[e] * s[e % k];
}

// One 64 (calibration rows) x 64 (output rows) tile of E = X D^T, D = W - W_hat,
// 256 threads of 4 x 4 entries, 16 input channels per LDS stage; the tile's sum
// of E^2 goes to part[tile].
__global__ __launch_bounds__(256) void awq_error_kernel(const uint16_t* __restrict__ x, const float* __restrict__ w,
                                                        const uint8_t* __restrict__ q,
                                                        const float* __restrict__ scale,
                                                        const uint8_t* __restrict__ zero,
                                                        const float* __restrict__ s, int64_t t, int64_t n,
                                                        int64_t k, int32_t group, double* __restrict__ part) {
  __shared__ double xa[16][65];
  __shared__ double db[16][65];
  __shared__ double red[256];
  const int64_t t0 = (int64_t)blockIdx.y * 64, n0 = (int64_t)blockIdx.x * 64;
  const int ti = threadIdx.x / 16, tj = threadIdx.x % 16;
  const int64_t ng = k / group;
  double acc[4][4] = {};
  for (int64_t c0 = 0; c0 < k; c0 += 16) {
    for (int e = threadIdx.x; e < 16 * 64; e += 256) {
      const int row = e / 16, cc = e % 16;   // 16 consecutive channels of one row
      const int64_t c = c0 + cc;
      const int64_t tr = t0 + row, nr = n0 + row;
      xa[cc][row] = (tr < t && c < k) ? bf16_bits_f64(x[tr * k + c]) : 0.0;
      double d = 0.0;
      if (nr < n && c < k) {
        const int64_t g = nr * ng + c / group;
        const double w_hat = (((double)q[nr * k + c] - (double)zero[g]) * (double)scale[g]) / (double)s[c];
        d = (double)w[nr * k + c] - w_hat;
      }
      db[cc][row] = d;
    }
    __syncthreads();
    for (int cc = 0; cc < 16; ++cc) {
      double a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = xa[cc][4 * ti + u];
        b[u] = db[cc][4 * tj + u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = fma(a[u], b[v], acc[u][v]);
    }
    __syncthreads();
  }
  double sq = 0.0;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) sq += acc[u][v] * acc[u][v];   // rows and columns out of range hold 0
  red[threadIdx.x] = sq;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = red[0];
}

// loss = sum of the tile slots, one workgroup, a fixed order.
__global__ __launch_bounds__(256) void awq_sum_kernel(const double* __restrict__ part, int64_t count,
                                                      double* __restrict__ loss) {
  __shared__ double red[256];
  double acc = 0.0;
  for (int64_t e = threadIdx.x; e < count; e += 256) acc += part[e];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) *loss = red[0];
}

unsigned awq_grid(int64_t items) {
  const int64_t blocks = (items + 255) / 256;
  return (unsigned)(blocks < 1 ? 1 : (blocks > 65536 ? 65536 : blocks));
}

}  // namespace

int32_t run_awq(const float* w, const uint16_t* x, int64_t t, int64_t n, int64_t k, int32_t group, int32_t n_grid,
                uint8_t* q, float* scale, uint8_t* zero, float* s_out, double* losses_out, int32_t* best_out,
                hipStream_t st) {
  const int64_t ng = k / group;
  const unsigned tn = (unsigned)((n + 63) / 64), tt = (unsigned)((t + 63) / 64);
  const int64_t tiles = (int64_t)tn * tt;
  double *m = nullptr, *part = nullptr, *losses = nullptr;
  float *s = nullptr, *ws = nullptr, *sc = nullptr;
  uint8_t *qt = nullptr, *zt = nullptr;
  uint32_t* flag = nullptr;
  int32_t rc = WOQ_OK;
  auto alloc = [&](auto** p, size_t bytes) {
    if (rc == WOQ_OK) rc = hip_status(hipMallocAsync(reinterpret_cast<void**>(p), bytes, st));
  };
  alloc(&m, (size_t)k * 8);
  alloc(&part, (size_t)tiles * 8);
  alloc(&losses, (size_t)(n_grid + 1) * 8);
  alloc(&s, (size_t)k * 4);
  alloc(&ws, (size_t)n * k * 4);
  alloc(&sc, (size_t)n * ng * 4);
  alloc(&qt, (size_t)n * k);
  alloc(&zt, (size_t)n * ng);
  alloc(&flag, sizeof(uint32_t));
  std::vector<double> hl(n_grid + 1);
  uint32_t hflag = 0;
  if (rc == WOQ_OK) rc = hip_status(hipMemsetAsync(flag, 0, sizeof(uint32_t), st));
  if (rc == WOQ_OK) {
    hipLaunchKernelGGL(awq_mean_kernel, dim3(awq_grid(k)), dim3(256), 0, st, x, t, k, m);
    rc = hip_status(hipGetLastError());
  }
  for (int32_t i = 0; i <= n_grid && rc == WOQ_OK; ++i) {
    const double alpha = (double)i / (double)n_grid;
    hipLaunchKernelGGL(awq_scale_kernel, dim3(awq_grid(k)), dim3(256), 0, st, m, k, alpha, s);
    hipLaunchKernelGGL(awq_scale_weights_kernel, dim3(awq_grid(n * k)), dim3(256), 0, st, w, s, n, k, ws);
    rc = hip_status(hipGetLastError());
    if (rc == WOQ_OK) rc = launch_quantize(ws, n, k, group, 0, qt, sc, zt, flag, st);
    if (rc == WOQ_OK) {
      hipLaunchKernelGGL(awq_error_kernel, dim3(tn, tt), dim3(256), 0, st, x, w, qt, sc, zt, s, t, n, k, group,
                         part);
      hipLaunchKernelGGL(awq_sum_kernel, dim3(1), dim3(256), 0, st, part, tiles, losses + i);
      rc = hip_status(hipGetLastError());
    }
  }
  if (rc == WOQ_OK) rc = hip_status(hipMemcpyAsync(hl.data(), losses, hl.size() * 8, hipMemcpyDeviceToHost, st));
  if (rc == WOQ_OK) rc = hip_status(hipMemcpyAsync(&hflag, flag, sizeof(uint32_t), hipMemcpyDeviceToHost, st));
  if (rc == WOQ_OK) rc = hip_status(hipStreamSynchronize(st));
  if (rc == WOQ_OK && hflag) rc = WOQ_ENONFINITE;
  int32_t best = 0;
  if (rc == WOQ_OK) {
    for (int32_t i = 1; i <= n_grid; ++i)
      if (hl[i] < hl[best]) best = i;
    // the chosen grid point again, into the caller's buffers
    const double alpha = (double)best / (double)n_grid;
    hipLaunchKernelGGL(awq_scale_kernel, dim3(awq_grid(k)), dim3(256), 0, st, m, k, alpha, s_out);
    hipLaunchKernelGGL(awq_scale_weights_kernel, dim3(awq_grid(n * k)), dim3(256), 0, st, w, s_out, n, k, ws);
    rc = hip_status(hipGetLastError());
    if (rc == WOQ_OK) rc = launch_quantize(ws, n, k, group, 0, q, scale, zero, flag, st);
    if (rc == WOQ_OK && losses_out)
      rc = hip_status(hipMemcpyAsync(losses_out, losses, hl.size() * 8, hipMemcpyDeviceToDevice, st));
  }
  const int32_t sync = hip_status(hipStreamSynchronize(st));
  if (rc == WOQ_OK) rc = sync;
  if (rc == WOQ_OK && best_out) *best_out = best;
  for (void* p : {static_cast<void*>(m), static_cast<void*>(part), static_cast<void*>(losses), static_cast<void*>(s),
                  static_cast<void*>(ws), static_cast<void*>(sc), static_cast<void*>(qt), static_cast<void*>(zt),
                  static_cast<void*>(flag)})
    if (p) (void)hipFreeAsync(p, st);
  (void)hipStreamSynchronize(st);
  return rc;
}

}  // namespace woq
