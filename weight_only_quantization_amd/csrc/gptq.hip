// GPTQ for one layer ("20. Quantization", stretch exercise 4: H = 2 X^T X from
// calibration inputs, quantize column by column, spreading each column's error
// over the remaining columns with the Cholesky factor of H^-1; linnet
// "Importing GPTQ and AWQ": in activation order the layer gathers its inputs
// through `order`).  Everything runs in float64, so the codes are decided on
// the same values as a float64 reference up to the rounding of the factorization.
//
// * H = X^T X (the factor 2 scales the Cholesky factor and the errors inversely
//   and cancels).  Columns with H_jj = 0 get H_jj = 1 and zero weights; with
//   act_order the columns are visited by decreasing H_jj (a stable sort, on the
//   host); H += damp * mean(diag H) * I.
// * The upper Cholesky factor U of H^-1 (H^-1 = U^T U) without forming H^-1:
//   with J the reversal permutation, J H J = L L^T (lower Cholesky) gives
//   H = (J L J)(J L J)^T, so U = (J L J)^-1 = J L^-1 J.  A right-looking
//   Cholesky and triangular inverse in panels of 64 columns: one launch works
//   through a panel column by column, one tiled float64 update applies it to
//   the rest.
// * The sweep is independent for every output row: a row's codes, scales and
//   updates use only its own weights and the shared U.  Per block of whole
//   groups (at least 128 columns), four lanes per row keep the block's weights
//   in LDS, take a group's (scale, zero) from its current columns when the
//   group starts, code each column, and subtract err * U from the rest of the
//   block, err = (w - dequant) / U_ii; a second kernel applies the block's
//   errors to every later column.  Every weight takes its updates one at a time
//   in column order, each product rounded before the subtraction.
#include <algorithm>
#include <vector>

#include <cfloat>

#include "woq_internal.h"

#pragma clang fp contract(off)

namespace woq {
namespace {

constexpr int kSweepRows = 16;        // sweep: rows per workgroup, four lanes a row
constexpr int kSweepMinCols = 128;    // columns per sweep block: whole groups, at least this many
constexpr int kSweepMaxCols = 256;

__device__ __forceinline__ double bf16_to_f64(uint16_t b) {
  return (double)__uint_as_float((uint32_t)b << 16);
}

__global__ __launch_bounds__(256) void gptq_finite_kernel(const float* __restrict__ w, int64_t count,
                                                          uint32_t* __restrict__ flag) {
  bool bad = false;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < count; e += (int64_t)gridDim.x * 256)
    bad |= !isfinite(w[e]);
  if (bad) atomicOr(flag, 1u);
}

// H[i][j] = sum_t x[t][i] x[t][j] (float64; the bf16 products are exact): 64 x 64
// tiles, 256 threads of 4 x 4 entries, 16 calibration rows per LDS stage.
__global__ __launch_bounds__(256) void gptq_h_kernel(const uint16_t* __restrict__ x, int64_t t, int64_t k,
                                                     double* __restrict__ h) {
  __shared__ double xa[16][64];
  __shared__ double xb[16][64];
  const int64_t i0 = (int64_t)blockIdx.y * 64, j0 = (int64_t)blockIdx.x * 64;
  const int ti = threadIdx.x / 16, tj = threadIdx.x % 16;
  double acc[4][4] = {};
  for (int64_t r0 = 0; r0 < t; r0 += 16) {
    for (int e = threadIdx.x; e < 16 * 64; e += 256) {
      const int rr = e / 64, cc = e % 64;
      const int64_t r = r0 + rr;
      xa[rr][cc] = (r < t && i0 + cc < k) ? bf16_to_f64(x[r * k + i0 + cc]) : 0.0;
      xb[rr][cc] = (r < t && j0 + cc < k) ? bf16_to_f64(x[r * k + j0 + cc]) : 0.0;
    }
    __syncthreads();
    for (int rr = 0; rr < 16; ++rr) {
      double a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = xa[rr][4 * ti + u];
        b[u] = xb[rr][4 * tj + u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = fma(a[u], b[v], acc[u][v]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t i = i0 + 4 * ti + u, j = j0 + 4 * tj + v;
      if (i < k && j < k) h[i * k + j] = acc[u][v];
    }
}

__global__ __launch_bounds__(256) void gptq_diag_kernel(const double* __restrict__ h, int64_t k,
                                                        double* __restrict__ d) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < k) d[i] = h[i * k + i];
}

// A[a][b] = Hp[K-1-a][K-1-b] with Hp[u][v] = H[perm[u]][perm[v]] off the
// diagonal and pdiag[u] (dead columns set to 1, then damped) on it.
__global__ __launch_bounds__(256) void gptq_arrange_kernel(const double* __restrict__ h,
                                                           const int32_t* __restrict__ perm,
                                                           const double* __restrict__ pdiag, int64_t k,
                                                           double* __restrict__ a) {
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < k * k; e += (int64_t)gridDim.x * 256) {
    const int64_t u = k - 1 - e / k, v = k - 1 - e % k;
    a[e] = u == v ? pdiag[u] : h[(int64_t)perm[u] * k + perm[v]];
  }
}

// The weights in visiting order, column-major (wc[c][row]), dead columns zero.
__global__ __launch_bounds__(256) void gptq_weights_kernel(const float* __restrict__ w, const int32_t* __restrict__ perm,
                                                           const uint8_t* __restrict__ dead, int64_t n, int64_t k,
                                                           double* __restrict__ wc) {
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n * k; e += (int64_t)gridDim.x * 256) {
    const int64_t c = e / n, r = e % n;
    const int32_t src = perm[c];
    wc[e] = dead[src] ? 0.0 : (double)w[r * k + src];
  }
}

// Panel of columns [j0, j0 + b) done: A[i][c] -= A[i][t] A[c][t] for t = j0 .. j0+b-1
// in order, for i, c >= j0 + b.  kTT x kTT tiles on and below the diagonal (the
// part of a diagonal tile above it is updated too and never read), 8 x 8
// entries a thread, held in registers; the panel's rows of both tiles pass
// through LDS kChunk columns at a time (the column tile's rows stored as
// 16 v + tc for row 8 tc + v, so the 16 threads of a row group read distinct
// banks).
constexpr int kPanel = 64;
constexpr int kChunk = 16;
constexpr int kTT = 128;

__global__ __launch_bounds__(256) void gptq_chol_trail_kernel(double* __restrict__ a, int64_t k, int64_t j0,
                                                              int32_t b) {
  if (blockIdx.x > blockIdx.y) return;   // above the diagonal
  __shared__ double pi[kTT][kChunk + 1];
  __shared__ double pc[kTT][kChunk + 1];
  const int64_t base = j0 + b;
  const int64_t i0 = base + (int64_t)blockIdx.y * kTT, c0 = base + (int64_t)blockIdx.x * kTT;
  const int ti = threadIdx.x / 16, tc = threadIdx.x % 16;
  double acc[8][8];
#pragma unroll
  for (int u = 0; u < 8; ++u)
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const int64_t i = i0 + 8 * ti + u, c = c0 + 8 * tc + v;
      acc[u][v] = (i < k && c < k) ? a[i * k + c] : 0.0;
    }
  for (int t0 = 0; t0 < b; t0 += kChunk) {
    const int nt = min(kChunk, b - t0);
    for (int e = threadIdx.x; e < kTT * kChunk; e += 256) {
      const int r = e / kChunk, t = e % kChunk;
      pi[r][t] = (i0 + r < k && t < nt) ? a[(i0 + r) * k + j0 + t0 + t] : 0.0;
      pc[(r % 8) * 16 + r / 8][t] = (c0 + r < k && t < nt) ? a[(c0 + r) * k + j0 + t0 + t] : 0.0;
    }
    __syncthreads();
    for (int t = 0; t < nt; ++t) {
      double x[8], y[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = pi[8 * ti + u][t];
#pragma unroll
      for (int v = 0; v < 8; ++v) y[v] = pc[16 * v + tc][t];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int v = 0; v < 8; ++v) acc[u][v] -= x[u] * y[v];
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 8; ++u)
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const int64_t i = i0 + 8 * ti + u, c = c0 + 8 * tc + v;
      if (i < k && c < k) a[i * k + c] = acc[u][v];
    }
}

// Cholesky, a whole panel of columns [j0, j0 + b) in one launch (b <= kPanel):
// for j = j0 .. j0+b-1 in order, A[i][j] /= sqrt(A[j][j]) for i > j, then
// A[i][c] -= A[i][j] A[c][j] for j < c < j0 + b, c <= i; one thread per row
// i >= j0.  The values A[c][j] of the panel's own b rows are what every row
// needs, so each workgroup factors that b x b block in LDS itself (the same
// operations in the same order in every workgroup, hence the same values), and
// workgroup 0 writes it back with the roots.  Every entry takes the same
// operations in the same order as column by column.
__global__ __launch_bounds__(256) void gptq_chol_panel_kernel(double* __restrict__ a, int64_t k, int64_t j0,
                                                              int32_t b, double* __restrict__ dg,
                                                              uint32_t* __restrict__ flag) {
  __shared__ double blk[kPanel][kPanel + 1];   // blk[r][c] = A[j0 + r][j0 + c], c <= r
  __shared__ double root[kPanel];
  const int tid = threadIdx.x;
  for (int e = tid; e < kPanel * kPanel; e += 256) {
    const int r = e / kPanel, c = e % kPanel;
    blk[r][c] = (r < b && c <= r) ? a[(j0 + r) * k + j0 + c] : 0.0;
  }
  // this thread's row below the block: its b panel entries
  const int64_t i = j0 + b + (int64_t)blockIdx.x * 256 + tid;
  const bool mine = i < k;
  double v[kPanel];
#pragma unroll
  for (int c = 0; c < kPanel; ++c) v[c] = (mine && c < b) ? a[i * k + j0 + c] : 0.0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPanel; ++j) {
    if (j >= b) continue;   // uniform
    // the block's column j (threads 0 .. b-1 own its rows)
    if (tid == 0) {
      const double pv = blk[j][j];
      const double d = sqrt(pv);
      root[j] = d;
      if (blockIdx.x == 0) {
        dg[j0 + j] = d;
        if (!(pv > 0.0) || !(d <= DBL_MAX)) atomicOr(flag, 2u);
      }
    }
    __syncthreads();
    const double d = root[j];
    if (tid > j && tid < b) blk[tid][j] /= d;
    __syncthreads();
    if (tid > j && tid < b)
      for (int c = j + 1; c <= tid; ++c) blk[tid][c] -= blk[tid][j] * blk[c][j];
    // this thread's row: the same two operations against the block's column j
    v[j] /= d;
#pragma unroll
    for (int c = j + 1; c < kPanel; ++c)
      if (c < b) v[c] -= v[j] * blk[c][j];
    __syncthreads();
  }
  if (mine) {
#pragma unroll
    for (int c = 0; c < kPanel; ++c)
      if (c < b) a[i * k + j0 + c] = v[c];
  }
  if (blockIdx.x == 0)
    for (int e = tid; e < kPanel * kPanel; e += 256) {
      const int r = e / kPanel, c = e % kPanel;
      if (r < b && c < r) a[(j0 + r) * k + j0 + c] = blk[r][c];
    }
}

// Triangular inverse T = L^-1, a whole panel of rows [p0, p0 + b) in one launch:
// for r = p0 .. p0+b-1 in order, T[r][j] /= L[r][r] for j <= r, then
// T[i][j] -= L[i][r] T[r][j] for r < i < p0 + b, j <= r; one thread per column
// j < p0 + b, the column's b panel entries in registers.  Every entry takes the
// same operations in the same order as row by row.
__global__ __launch_bounds__(256) void gptq_tri_panel_kernel(double* __restrict__ tm, const double* __restrict__ a,
                                                             const double* __restrict__ dg, int64_t k, int64_t p0,
                                                             int32_t b) {
  __shared__ double lb[kPanel][kPanel + 1];    // lb[i][r] = L[p0 + i][p0 + r], r < i
  __shared__ double dgs[kPanel];
  const int tid = threadIdx.x;
  for (int e = tid; e < kPanel * kPanel; e += 256) {
    const int i = e / kPanel, r = e % kPanel;
    lb[i][r] = (i < b && r < i) ? a[(p0 + i) * k + p0 + r] : 0.0;
  }
  if (tid < kPanel) dgs[tid] = tid < b ? dg[p0 + tid] : 1.0;
  const int64_t j = (int64_t)blockIdx.x * 256 + tid;
  const bool mine = j < p0 + b;
  double t[kPanel];
#pragma unroll
  for (int r = 0; r < kPanel; ++r) t[r] = (mine && r < b) ? tm[(p0 + r) * k + j] : 0.0;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kPanel; ++r) {
    if (r >= b || j > p0 + r) continue;   // T[p0 + r][j] is final zero above the diagonal
    t[r] /= dgs[r];
#pragma unroll
    for (int i = r + 1; i < kPanel; ++i)
      if (i < b) t[i] -= lb[i][r] * t[r];
  }
  if (mine) {
#pragma unroll
    for (int r = 0; r < kPanel; ++r)
      if (r < b) tm[(p0 + r) * k + j] = t[r];
  }
}

__global__ __launch_bounds__(256) void gptq_identity_kernel(double* __restrict__ tm, int64_t k) {
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < k * k; e += (int64_t)gridDim.x * 256)
    tm[e] = (e / k == e % k) ? 1.0 : 0.0;
}

// Panel of rows [p0, p0 + b) final: T[i][j] -= L[i][r] T[r][j] for r = p0 .. p0+b-1
// in order, for i >= p0 + b, j < p0 + b (T[r][j] is 0 for j > r, which changes
// nothing).  kTT x kTT tiles, 8 x 8 entries a thread in registers; L's panel
// columns and T's panel rows pass through LDS kChunk at a time (T's columns
// stored as 16 v + tj for column 8 tj + v, as in the factor's update).
__global__ __launch_bounds__(256) void gptq_tri_trail_kernel(double* __restrict__ tm, const double* __restrict__ a,
                                                             int64_t k, int64_t p0, int32_t b) {
  __shared__ double li[kTT][kChunk + 1];
  __shared__ double tr[kChunk][kTT + 1];
  const int64_t pend = p0 + b;
  const int64_t i0 = pend + (int64_t)blockIdx.y * kTT, j0 = (int64_t)blockIdx.x * kTT;
  const int ti = threadIdx.x / 16, tj = threadIdx.x % 16;
  double acc[8][8];
#pragma unroll
  for (int u = 0; u < 8; ++u)
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const int64_t i = i0 + 8 * ti + u, j = j0 + 8 * tj + v;
      acc[u][v] = (i < k && j < pend) ? tm[i * k + j] : 0.0;
    }
  for (int t0 = 0; t0 < b; t0 += kChunk) {
    const int nt = min(kChunk, b - t0);
    for (int e = threadIdx.x; e < kTT * kChunk; e += 256) {
      const int r = e / kChunk, t = e % kChunk;
      li[r][t] = (i0 + r < k && t < nt) ? a[(i0 + r) * k + p0 + t0 + t] : 0.0;
      const int t2 = e / kTT, jj = e % kTT;
      tr[t2][(jj % 8) * 16 + jj / 8] = (t2 < nt && j0 + jj < pend) ? tm[(p0 + t0 + t2) * k + j0 + jj] : 0.0;
    }
    __syncthreads();
    for (int t = 0; t < nt; ++t) {
      double x[8], y[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = li[8 * ti + u][t];
#pragma unroll
      for (int v = 0; v < 8; ++v) y[v] = tr[t][16 * v + tj];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int v = 0; v < 8; ++v) acc[u][v] -= x[u] * y[v];
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 8; ++u)
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const int64_t i = i0 + 8 * ti + u, j = j0 + 8 * tj + v;
      if (i < k && j < pend) tm[i * k + j] = acc[u][v];
    }
}

// U[i][j] = T[K-1-i][K-1-j] (upper triangular: i <= j).
__device__ __forceinline__ double u_at(const double* __restrict__ tm, int64_t k, int64_t i, int64_t j) {
  return tm[(k - 1 - i) * k + (k - 1 - j)];
}

// Sweep of columns [c0, c0 + nb) (whole groups) for rows [16 b, 16 b + 16), four
// lanes a row: lane share p holds the row's block columns j with j % 4 == p (in
// LDS) and applies every update to them.  Column i's owner (share i % 4) codes
// it and passes its error to the row's other lanes; a group's min and max are
// each lane's over its columns, then over the four (exact, in any order).  The
// group rule is the asymmetric quantizer's: d = max - min over the group's
// current columns, scale = float32(d / 15), zero = clamp(rint(-15 min / d), 0, 15),
// codes clamp(rint(15 w / d) + zero, 0, 15); a flat group (d = 0) takes scale 1,
// zero clamp(rint(-min), 0, 15) and codes clamp(rint(w) + zero, 0, 15).  Every
// entry takes its updates one at a time in column order, as with one thread a row.
__global__ __launch_bounds__(4 * kSweepRows) void gptq_sweep_kernel(double* __restrict__ wc, const double* __restrict__ tm,
                                                                    int64_t n, int64_t k, int32_t group, int64_t c0,
                                                                    int32_t nb, uint8_t* __restrict__ q,
                                                                    float* __restrict__ scale, uint8_t* __restrict__ zero,
                                                                    double* __restrict__ err) {
  extern __shared__ double vals[];   // [nb][kSweepRows]
  const int lane = threadIdx.x;
  const int rl = lane >> 2, share = lane & 3;
  const int64_t row = (int64_t)blockIdx.x * kSweepRows + rl;
  const bool live = row < n;
  for (int j = share; j < nb; j += 4) vals[j * kSweepRows + rl] = live ? wc[(c0 + j) * n + row] : 0.0;
  const int64_t ng = k / group;
  double d_safe = 1.0, zr = 0.0, sc = 1.0;
  bool flat = true;
  for (int i = 0; i < nb; ++i) {
    const int64_t c = c0 + i;
    if (c % group == 0) {
      // this lane's columns of the group (none for a lane past a group of 2)
      double mn = INFINITY, mx = -INFINITY;
      for (int j = i + ((share - i) & 3); j < i + group; j += 4) {
        const double v = vals[j * kSweepRows + rl];
        mn = fmin(mn, v);
        mx = fmax(mx, v);
      }
      mn = fmin(mn, __shfl_xor(mn, 1));
      mx = fmax(mx, __shfl_xor(mx, 1));
      mn = fmin(mn, __shfl_xor(mn, 2));
      mx = fmax(mx, __shfl_xor(mx, 2));
      const double d = mx - mn;
      flat = d == 0.0;
      d_safe = flat ? 1.0 : d;
      sc = flat ? 1.0 : (double)(float)(d / 15.0);
      zr = fmin(fmax(__builtin_rint(flat ? -mn : (-15.0 * mn) / d_safe), 0.0), 15.0);
      if (live && share == 0) {
        scale[row * ng + c / group] = (float)sc;
        zero[row * ng + c / group] = (uint8_t)zr;
      }
    }
    const int owner = i & 3;
    double e = 0.0;
    if (share == owner) {
      const double v = vals[i * kSweepRows + rl];
      const double r = __builtin_rint(flat ? v : (15.0 * v) / d_safe);
      const double qi = fmin(fmax(r + zr, 0.0), 15.0);
      e = (v - (qi - zr) * sc) / u_at(tm, k, c, c);
      if (live) {
        q[row * k + c] = (uint8_t)qi;
        err[(int64_t)i * n + row] = e;
      }
    }
    e = __shfl(e, (lane & ~3) | owner);
    for (int j = i + 1 + ((share - i - 1) & 3); j < nb; j += 4) vals[j * kSweepRows + rl] -= e * u_at(tm, k, c, c0 + j);
  }
}

// The later columns take the block's errors, one column of the block at a time:
// wc[cc][row] -= err[i][row] * U[c0 + i][cc] for i = 0 .. nb-1, cc >= c0 + nb.
constexpr int kTrailCols = 16;

__global__ __launch_bounds__(256) void gptq_trailing_kernel(double* __restrict__ wc, const double* __restrict__ tm,
                                                            const double* __restrict__ err, int64_t n, int64_t k,
                                                            int64_t c0, int32_t nb) {
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t cc0 = c0 + nb + (int64_t)blockIdx.y * kTrailCols;
  if (row >= n) return;
  const int cols = (int)std::min<int64_t>(kTrailCols, k - cc0);
  double acc[kTrailCols];
#pragma unroll
  for (int u = 0; u < kTrailCols; ++u) acc[u] = u < cols ? wc[(cc0 + u) * n + row] : 0.0;
  for (int i = 0; i < nb; ++i) {
    const double e = err[(int64_t)i * n + row];
#pragma unroll
    for (int u = 0; u < kTrailCols; ++u)
      if (u < cols) acc[u] -= e * u_at(tm, k, c0 + i, cc0 + u);
  }
#pragma unroll
  for (int u = 0; u < kTrailCols; ++u)
    if (u < cols) wc[(cc0 + u) * n + row] = acc[u];
}

unsigned flat_grid(int64_t items) {
  const int64_t blocks = (items + 255) / 256;
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(blocks, 65536));
}

}  // namespace

int32_t gptq_block_cols(int32_t group) {
  if (group < 1 || group > kSweepMaxCols) return 0;
  return group * ((kSweepMinCols + group - 1) / group);
}

int32_t run_gptq(const float* w, const uint16_t* x, int64_t t, int64_t n, int64_t k, int32_t group,
                 int32_t act_order, double damp, uint8_t* q, float* scale, uint8_t* zero, int32_t* order,
                 hipStream_t s) {
  const int32_t bcols = gptq_block_cols(group);
  if (bcols == 0) return WOQ_EUNSUPPORTED;
  static std::atomic<uint64_t> raised{0};   // the sweep's dynamic-LDS limit, one bit per device
  if (const int32_t st = raise_lds_limit(reinterpret_cast<const void*>(gptq_sweep_kernel),
                                         (int)(kSweepMaxCols * kSweepRows * sizeof(double)), raised);
      st != WOQ_OK)
    return st;
  double *h = nullptr, *a = nullptr, *tm = nullptr, *wc = nullptr, *err = nullptr, *dg = nullptr, *dd = nullptr;
  int32_t* dperm = nullptr;
  uint8_t* ddead = nullptr;
  uint32_t* flag = nullptr;
  int32_t st = WOQ_OK;
  auto alloc = [&](auto** p, size_t bytes) {
    if (st == WOQ_OK) st = hip_status(hipMallocAsync(reinterpret_cast<void**>(p), bytes, s));
  };
  alloc(&h, (size_t)k * k * 8);
  alloc(&a, (size_t)k * k * 8);
  alloc(&tm, (size_t)k * k * 8);
  alloc(&wc, (size_t)n * k * 8);
  alloc(&err, (size_t)bcols * n * 8);
  alloc(&dg, (size_t)k * 8);
  alloc(&dd, (size_t)k * 8);
  alloc(&dperm, (size_t)k * 4);
  alloc(&ddead, (size_t)k);
  alloc(&flag, sizeof(uint32_t));
  std::vector<double> diag(k), pdiag(k);
  std::vector<int32_t> perm(k);
  std::vector<uint8_t> dead(k);
  uint32_t hflag = 0;
  if (st == WOQ_OK) st = hip_status(hipMemsetAsync(flag, 0, sizeof(uint32_t), s));
  if (st == WOQ_OK) {
    const unsigned tiles = (unsigned)((k + 63) / 64);
    hipLaunchKernelGGL(gptq_finite_kernel, dim3(flat_grid(n * k)), dim3(256), 0, s, w, n * k, flag);
    hipLaunchKernelGGL(gptq_h_kernel, dim3(tiles, tiles), dim3(256), 0, s, x, t, k, h);
    hipLaunchKernelGGL(gptq_diag_kernel, dim3(flat_grid(k)), dim3(256), 0, s, h, k, dd);
    st = hip_status(hipGetLastError());
  }
  if (st == WOQ_OK) st = hip_status(hipMemcpyAsync(diag.data(), dd, (size_t)k * 8, hipMemcpyDeviceToHost, s));
  if (st == WOQ_OK) st = hip_status(hipMemcpyAsync(&hflag, flag, sizeof(uint32_t), hipMemcpyDeviceToHost, s));
  if (st == WOQ_OK) st = hip_status(hipStreamSynchronize(s));
  if (st == WOQ_OK && hflag) st = WOQ_ENONFINITE;
  if (st == WOQ_OK) {
    double mean = 0.0;
    for (int64_t i = 0; i < k; ++i) {
      dead[i] = diag[i] == 0.0;
      if (dead[i]) diag[i] = 1.0;
      mean += diag[i];
    }
    mean /= (double)k;
    for (int64_t i = 0; i < k; ++i) perm[i] = (int32_t)i;
    if (act_order)
      std::stable_sort(perm.begin(), perm.end(), [&](int32_t u, int32_t v) { return diag[u] > diag[v]; });
    for (int64_t i = 0; i < k; ++i) pdiag[i] = diag[perm[i]] + damp * mean;
    st = hip_status(hipMemcpyAsync(dd, pdiag.data(), (size_t)k * 8, hipMemcpyHostToDevice, s));
    if (st == WOQ_OK) st = hip_status(hipMemcpyAsync(dperm, perm.data(), (size_t)k * 4, hipMemcpyHostToDevice, s));
    if (st == WOQ_OK) st = hip_status(hipMemcpyAsync(ddead, dead.data(), (size_t)k, hipMemcpyHostToDevice, s));
  }
  if (st == WOQ_OK) {
    hipLaunchKernelGGL(gptq_arrange_kernel, dim3(flat_grid(k * k)), dim3(256), 0, s, h, dperm, dd, k, a);
    hipLaunchKernelGGL(gptq_weights_kernel, dim3(flat_grid(n * k)), dim3(256), 0, s, w, dperm, ddead, n, k, wc);
    hipLaunchKernelGGL(gptq_identity_kernel, dim3(flat_grid(k * k)), dim3(256), 0, s, tm, k);
    st = hip_status(hipGetLastError());
    // Panels of kPanel columns: inside a panel the column kernels touch only the
    // panel; one tiled launch then applies the whole panel to the rest.  Every
    // entry takes the same updates in the same order as column by column.
    for (int64_t j0 = 0; j0 < k && st == WOQ_OK; j0 += kPanel) {
      const int64_t jend = std::min<int64_t>(k, j0 + kPanel);
      hipLaunchKernelGGL(gptq_chol_panel_kernel, dim3((unsigned)std::max<int64_t>(1, (k - jend + 255) / 256)), dim3(256),
                         0, s, a, k, j0, (int32_t)(jend - j0), dg, flag);
      if (jend < k) {
        const unsigned t = (unsigned)((k - jend + kTT - 1) / kTT);
        hipLaunchKernelGGL(gptq_chol_trail_kernel, dim3(t, t), dim3(256), 0, s, a, k, j0, (int32_t)(jend - j0));
      }
      st = hip_status(hipGetLastError());
    }
    // A factor with a non-positive pivot is not used: report it before the inverse.
    if (st == WOQ_OK) st = hip_status(hipMemcpyAsync(&hflag, flag, sizeof(uint32_t), hipMemcpyDeviceToHost, s));
    if (st == WOQ_OK) st = hip_status(hipStreamSynchronize(s));
    if (st == WOQ_OK && (hflag & 2u)) st = WOQ_ENOTPD;
    for (int64_t p0 = 0; p0 < k && st == WOQ_OK; p0 += kPanel) {
      const int64_t pend = std::min<int64_t>(k, p0 + kPanel);
      hipLaunchKernelGGL(gptq_tri_panel_kernel, dim3((unsigned)((pend + 255) / 256)), dim3(256), 0, s, tm, a, dg, k, p0,
                         (int32_t)(pend - p0));
      if (pend < k)
        hipLaunchKernelGGL(gptq_tri_trail_kernel, dim3((unsigned)((pend + kTT - 1) / kTT), (unsigned)((k - pend + kTT - 1) / kTT)),
                           dim3(256), 0, s, tm, a, k, p0, (int32_t)(pend - p0));
      st = hip_status(hipGetLastError());
    }
    for (int64_t c0 = 0; c0 < k && st == WOQ_OK; c0 += bcols) {
      const int32_t nb = (int32_t)std::min<int64_t>(bcols, k - c0);
      hipLaunchKernelGGL(gptq_sweep_kernel, dim3((unsigned)((n + kSweepRows - 1) / kSweepRows)), dim3(4 * kSweepRows),
                         (size_t)nb * kSweepRows * sizeof(double), s, wc, tm, n, k, group, c0, nb, q, scale, zero,
                         err);
      if (c0 + nb < k) {
        const unsigned gy = (unsigned)((k - c0 - nb + kTrailCols - 1) / kTrailCols);
        hipLaunchKernelGGL(gptq_trailing_kernel, dim3((unsigned)((n + 255) / 256), gy), dim3(256), 0, s, wc, tm, err,
                           n, k, c0, nb);
      }
      st = hip_status(hipGetLastError());
    }
  }
  if (st == WOQ_OK && act_order)
    st = hip_status(hipMemcpyAsync(order, dperm, (size_t)k * 4, hipMemcpyDeviceToDevice, s));
  // finish before the host vectors the copies read go out of scope
  const int32_t sync = hip_status(hipStreamSynchronize(s));
  if (st == WOQ_OK) st = sync;
  for (void* p : {static_cast<void*>(h), static_cast<void*>(a), static_cast<void*>(tm), static_cast<void*>(wc),
                  static_cast<void*>(err), static_cast<void*>(dg), static_cast<void*>(dd), static_cast<void*>(dperm),
                  static_cast<void*>(ddead), static_cast<void*>(flag)})
    if (p) (void)hipFreeAsync(p, s);
  (void)hipStreamSynchronize(s);
  return st;
}

}  // namespace woq
