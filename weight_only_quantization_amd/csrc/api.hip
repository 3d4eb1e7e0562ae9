// C ABI of libwoq.so: argument validation, kernel planning and dispatch.
// Every argument check runs on the host before anything is enqueued, so a call
// that fails validation has no effect.  Data-dependent errors (non-finite
// weights, codes above 15, a factorization that fails) are found by the
// kernels and reported after they ran; the outputs of such a call are then
// unspecified.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <atomic>
#include <mutex>

#include "woq_internal.h"

namespace woq {
namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;
constexpr int64_t kMaxElems = (int64_t)1 << 40;

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

// Error flags of the synchronous codec calls (non-finite weights, codes above
// 15): a file-scope device array, one slot per call taken round robin, so
// those calls allocate nothing.  Its address on a device is taken once, with
// that device current.  More than kFlagSlots codec calls in flight at once
// (from as many host threads) would share a slot.
constexpr int kFlagSlots = 256;
constexpr int kFlagDevices = 64;
__device__ __align__(256) uint32_t flag_pool[kFlagSlots];
void* flag_addr[kFlagDevices] = {};
std::mutex flag_mutex;
std::atomic<uint32_t> flag_next{0};

// Clear a slot, run launch(slot) on stream s, read the slot back (synchronizes).
template <class F>
int32_t with_flag(hipStream_t s, uint32_t* hflag, F launch) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kFlagDevices) return WOQ_EHIP;
  void* base = nullptr;
  {
    std::lock_guard<std::mutex> lock(flag_mutex);
    if (!flag_addr[dev]) {
      void* ptr = nullptr;
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(flag_pool)) != hipSuccess || !ptr) return WOQ_EHIP;
      flag_addr[dev] = ptr;
    }
    base = flag_addr[dev];
  }
  uint32_t* flag = static_cast<uint32_t*>(base) + flag_next.fetch_add(1, std::memory_order_relaxed) % kFlagSlots;
  int32_t st = hip_status(hipMemsetAsync(flag, 0, sizeof(uint32_t), s));
  if (st == WOQ_OK) st = launch(flag);
  if (st == WOQ_OK) st = hip_status(hipMemcpyAsync(hflag, flag, sizeof(uint32_t), hipMemcpyDeviceToHost, s));
  if (st == WOQ_OK) st = hip_status(hipStreamSynchronize(s));
  return st;
}

bool linear_group_ok(int32_t g) { return g == 32 || g == 64 || g == 128 || g == 256; }

int32_t check_linear_shape(int64_t m, int64_t n, int64_t k, int32_t group) {
  if (m < 0 || n < 0 || k < 0) return WOQ_EINVAL;
  if (group < 1) return WOQ_EGROUP;
  if (!linear_group_ok(group)) return (group % 2 || k % group) ? WOQ_EGROUP : WOQ_EUNSUPPORTED;
  if (k % group) return WOQ_EGROUP;
  if (m >= kMaxDim || n >= kMaxDim || k >= kMaxDim) return WOQ_EUNSUPPORTED;
  return WOQ_OK;
}

// Int4Linear has one scale a row; the kernels run it in groups of the largest
// supported size dividing k (each group sees the same row scale), 0 if none.
int32_t rows_group(int64_t k) {
  for (int32_t g : {256, 128, 64, 32})
    if (k > 0 && k % g == 0) return g;
  return 0;
}

// Optional tuning override of the small-M launch shape: WOQ_SKINNY="tiles,cnt"
// (16-row weight tiles per workgroup, 128-input steps per wave; read on every call).
bool skinny_override(int* tiles, int* cnt) {
  const char* e = std::getenv("WOQ_SKINNY");
  int a = 0, b = 0;
  if (!e || std::sscanf(e, "%d,%d", &a, &b) != 2) return false;
  if (!(a == 1 || a == 2 || a == 4) || b < 2 || b % 2 != 0) return false;
  *tiles = a;
  *cnt = b;
  return true;
}

// Small-M launch shape (m <= 128).  The waves of a workgroup form a WM x WK
// grid: each of the WM wave groups takes two 16-row activation tiles (one when
// m <= 16), each of the WK K ranges `cnt` consecutive 128-input steps (even,
// at least 2), with at most 8 waves; the workgroup takes 4 weight tiles when
// that still leaves about 200 workgroups (the tiles share each activation
// operand), else 2 or 1.  The per-range (scale, zero) staging must fit next to
// the reduction area in LDS; wider tiles give way first.  (Measured on
// 14336x4096, 4096x14336 and 4096x4096 at m = 5..128 and every group size.)
bool skinny_plan(int64_t m, int64_t n, int64_t k, int32_t group, LinearPlan* p) {
  const int64_t nsteps = (k + 127) / 128;
  const int64_t tiles = (n + 15) / 16;
  const int64_t mtt = (m + 15) / 16;
  const int64_t mt = mtt >= 2 ? 2 : 1;
  const int64_t wm = (mtt + mt - 1) / mt;
  if (wm > 8) return false;
  const int64_t wk_max = 8 / wm;
  int64_t cnt = (nsteps + wk_max - 1) / wk_max;
  if (cnt < 2) cnt = 2;
  cnt = (cnt + 1) / 2 * 2;
  int t = tiles >= 800 ? 4 : (tiles >= 400 ? 2 : 1);
  int o_t, o_c;
  const bool forced = skinny_override(&o_t, &o_c) && (nsteps + o_c - 1) / o_c <= wk_max;
  if (forced) {
    t = o_t;
    cnt = o_c;
  }
  // Above 64 rows only wide layers, whose workgroups share each activation
  // fragment among 4 weight tiles, beat the tiled GEMM.
  if (m > 64 && t < 4 && !forced) return false;
  const int64_t waves = wm * ((nsteps + cnt - 1) / cnt);
  if (waves > 8 || cnt >= ((int64_t)1 << 20)) return false;
  while (t > 1 && skinny_lds_layout(m, k, group, (int)waves, t, (int)cnt).total > kSkinnyLdsLimit) t /= 2;
  if (skinny_lds_layout(m, k, group, (int)waves, t, (int)cnt).total > kSkinnyLdsLimit) return false;
  p->path = 1;
  p->mt = (int)mt;
  p->wm = (int)wm;
  // From 24 rows (groups of 128 and more) or 33 rows (any group) the
  // activations go through a pre-pass into fragment order: contiguous
  // kilobyte loads and no in-kernel reordering, which outweigh the extra
  // launch there (measured on 14336x4096 at groups 32 and 128: 12 % faster at
  // 32 rows, 19 % at 64; 4 % slower at 17).  WOQ_SKINNY_XFRAG=0/1 overrides
  // (a tuning aid, read on every call).
  p->xfrag = mtt >= 2 && nsteps <= 8192 && (m > 32 || (m >= 24 && group >= 128)) ? 1 : 0;
  if (const char* e = std::getenv("WOQ_SKINNY_XFRAG"); e && (e[0] == '0' || e[0] == '1') && mtt >= 2 &&
                                                          nsteps <= 8192)
    p->xfrag = e[0] - '0';
  p->fold_rows = 4;
  p->ns = t;
  p->waves = (int)waves;
  p->cnt = (int)cnt;
  p->grid = (tiles + t - 1) / t;
  return true;
}

// Small-M launch shape with the activation slice in LDS (path 6, 5 <= m <= 64):
// workgroups of 8 waves with T weight tiles each (T in {1, 2}), K ranges of S
// steps (S in {4, 8}).  Ranges of 8 steps from K = 8192 (fewer, larger partials
// where K is long), else 4; two tiles a wave above 32 rows with 8-step ranges;
// a shape whose LDS does not fit gives way to one tile, and if that does not
// fit either the path declines (shorter ranges would double the partials).
// (Measured on 1024x4096, 4096x4096, 4096x14336 and 14336x4096 at 5..64 rows,
// groups 32, 128 and 256, against every shape.)  More than one range needs
// the partial buffer (split_ok).  WOQ_SM="T,S" forces a shape (a tuning aid,
// read on every call).
bool sm_plan(int64_t m, int64_t n, int64_t k, int32_t group, bool split_ok, LinearPlan* p) {
  if (m < 5 || m > 64 || k >= ((int64_t)1 << 24) || m * k * 2 >= ((int64_t)1 << 31)) return false;
  const int64_t nsteps = (k + 127) / 128;
  const int64_t tiles = (n + 15) / 16;
  const int mt = m <= 16 ? 1 : (m <= 32 ? 2 : 4);
  auto fits = [&](int t, int st) {
    const int64_t ranges = (nsteps + st - 1) / st;
    return (ranges == 1 || split_ok) && sm_lds_bytes(mt, st, t, group, false) <= kSkinnyLdsLimit;
  };
  int t = 0, st = 0;
  int ft = 0, fs = 0;
  const char* e = std::getenv("WOQ_SM");
  if (e && std::sscanf(e, "%d,%d", &ft, &fs) == 2 && (ft == 1 || ft == 2) && (fs == 4 || fs == 8)) {
    if (!fits(ft, fs)) return false;
    t = ft;
    st = fs;
  } else {
    const int s_pref = nsteps >= 64 ? 8 : 4;
    const int t_pref = s_pref == 8 && m > 32 ? 2 : 1;
    const int cand[2][2] = {{t_pref, s_pref}, {1, s_pref}};
    for (const auto& c : cand) {
      if (fits(c[0], c[1])) {
        t = c[0];
        st = c[1];
        break;
      }
    }
    if (t == 0) return false;
  }
  p->path = 6;
  p->mt = mt;
  p->ns = t;
  p->cnt = st;
  p->waves = 8;
  p->splits = (int)((nsteps + st - 1) / st);
  p->grid = (tiles + 8 * t - 1) / (8 * t) * p->splits;
  p->fold_rows = 4;
  return true;
}

// Decode GEMV launch shape.  Each wave takes `cnt` consecutive 128-input
// steps (4, 8, 12 or 16) and a workgroup of ceil(steps / cnt) waves (at most
// 16) covers K for 16 outputs.  A step costs the fewest instructions for
// m = 1 and groups of 128 or more (no lane transpose, one piece per step), so
// there long ranges (16 steps) amortize each wave's set-up best; 64-wide
// groups take 8, and 32-wide groups or m > 1 take 4 (more, shorter waves
// overlap the heavier steps).  Small grids give up range length until about
// 1536 waves cover the chip; the 16-wave limit per workgroup can force longer
// ranges.  (Measured on the 14336x4096, 4096x14336 and 4096x4096 decode
// shapes for every group size at m = 1 and 4.)  WOQ_GEMV_WAVES replaces the
// rule by "the smallest cnt whose grid has at most this many waves" (a
// tuning aid, read on every call).
bool gemv_plan(int64_t m, int64_t n, int64_t k, int32_t group, LinearPlan* p) {
  const int64_t nsteps = (k + 127) / 128;
  const int64_t tiles = (n + 15) / 16;
  auto waves = [&](int64_t c) { return (nsteps + c - 1) / c; };
  int64_t cnt;
  if (const char* e = std::getenv("WOQ_GEMV_WAVES"); e && std::strtol(e, nullptr, 10) > 0) {
    const int64_t target = std::strtol(e, nullptr, 10);
    cnt = 16;
    for (int64_t c = 4; c <= 16; c += 4) {
      if (waves(c) <= 16 && tiles * waves(c) <= target) {
        cnt = c;
        break;
      }
    }
  } else {
    cnt = (m == 1 && group >= 128) ? 16 : (m == 1 && group == 64) ? 8 : 4;
    while (cnt > 4 && tiles * waves(cnt) < 1536) cnt -= 4;
    while (cnt < 16 && waves(cnt) > 16) cnt += 4;
  }
  const int64_t w = waves(cnt);
  if (w > 16) return false;   // more than 1024 threads per workgroup
  if (gemv_layout(m, k, group, (int)w, (int)cnt).total > kSkinnyLdsLimit) return false;
  p->path = 4;
  p->fold_rows = m == 1 ? 1 : 4;
  p->waves = (int)w;
  p->cnt = (int)cnt;
  p->grid = tiles;
  return true;
}

}  // namespace

LinearPlan linear_plan(int64_t m, int64_t n, int64_t k, int32_t group, bool has_order, bool rows_ok,
                       bool split_ok) {
  LinearPlan p;
  if (m == 0 || n == 0) return p;
  if (k == 0) {
    p.path = 3;
    return p;
  }
  p.gb = group >= 128 ? 4 : group / 32;
  // Canonical rows at m <= 4 stream through the row kernel; WOQ_DECODE_MFMA
  // keeps them on the tile GEMV (a tuning and test aid, read on every call).
  // At 3 and 4 rows the row kernel is bound by its dot arithmetic (one v_dot2
  // per weight pair and row); on layers of at least 2^25 weights with groups
  // of 128 and more the small-M MFMA kernel is faster there (14336x4096 at
  // m = 4: 12.8 against 15.1 us; 4096x14336: 13.7 against 16.2 us).
  const bool decode_mfma = std::getenv("WOQ_DECODE_MFMA") != nullptr;
  const bool mfma_rows = rows_ok && !decode_mfma && (m >= 3 || (m == 2 && k >= 8192)) && group >= 128 &&
                         n * k >= ((int64_t)1 << 25);
  if (rows_ok && rows_supported(m, k) && !mfma_rows && !decode_mfma) {
    p.path = 5;
    p.rows_u = rows_per_group(m, n, k);
    p.waves = rows_waves(k);
    p.grid = (n + p.rows_u - 1) / p.rows_u;
    p.prep = has_order ? 1 : 0;
    return p;
  }
  const bool force_skinny = std::getenv("WOQ_FORCE_SKINNY") != nullptr;   // tuning aid, read on every call
  // The tile GEMV takes those 3-4 rows, and 2 rows, when K >= 8192: 4096x14336
  // at m = 4 13.0 against 14.5 us on the small-M kernel, at m = 2 10.7 against
  // 11.5 us on the row kernel; 8192x28672 at m = 2 32.3 against 43 us (on
  // 14336x4096 the small-M kernel stays ahead at m = 3-4, 12.8 against 13.7 us,
  // and the row kernel at m = 2, 10.6 against 12.5 us).
  const bool mfma_gemv = mfma_rows && k >= 8192;
  if (m <= 4 && !force_skinny && (!mfma_rows || mfma_gemv) && k < ((int64_t)1 << 26) &&
      gemv_plan(m, n, k, group, &p)) {
    p.prep = has_order ? 1 : 0;
    return p;
  }
  const bool force_tiled = std::getenv("WOQ_FORCE_TILED") != nullptr;   // tuning aid, read on every call
  // From 16 to 64 rows (from 8 with groups of 128 or more when K >= 8192 or
  // N <= 1024), layers narrower than 800 tiles
  // of 16 rows (where the small-M kernel below gives each workgroup fewer than
  // 4 tiles, so every workgroup re-reads x for few weight rows) run on the
  // path with the activation slice in LDS: 4096x14336 at 16 rows 23.1 -> 15.3
  // us, at 64 rows 37.9 -> 31.0 us, at 8 rows 16.3 -> 14.9 us; 1024x4096 at 16
  // rows 8.8 -> 6.9 us, at 8 and 12 rows 7.3 / 8.2 -> 6.8 us.  On wider layers,
  // and below 16 rows with groups of 32 or shorter K, the small-M kernel is as
  // fast or faster.  WOQ_SM="0" keeps
  // every call off it, "T,S" puts every call of 5..64 rows on it with that
  // shape, and a forced small-M shape (WOQ_SKINNY) keeps the rule from
  // applying (tuning aids, read on every call).
  {
    const char* e = std::getenv("WOQ_SM");
    const bool off = e && e[0] == '0';
    const bool forced = e && !off;
    const int64_t tiles = (n + 15) / 16;
    const bool rule = (m >= 16 || (m >= 8 && group >= 128 && (k >= 8192 || tiles <= 64))) && tiles < 800 &&
                      std::getenv("WOQ_SKINNY") == nullptr;
    if (!force_tiled && !off && (forced || rule) && sm_plan(m, n, k, group, split_ok, &p)) {
      p.prep = has_order ? 1 : 0;
      return p;
    }
  }
  // The small-M kernel takes up to 128 rows (from 65 rows only layers of at
  // least 800 weight tiles of 16 rows: 14336x4096 at 128 rows runs in 41 us
  // against the tiled GEMM's 46 us at group 128, 57 against 89 us at group 32).
  if (m <= 128 && !force_tiled && k < ((int64_t)1 << 26) && skinny_plan(m, n, k, group, &p)) {
    p.prep = has_order ? 1 : 0;
    return p;
  }
  p.path = 2;
  p.prep = 1;
  // Tile by the number of activation rows: at small M, narrow tiles keep the
  // grid wide enough to cover the chip.  Above 64 rows: 128 x 256 tiles unless
  // even split over K (below) they would fill at most half the chip, then
  // 128 x 64 ones.  Measured on 1024x4096, 4096x4096, 4096x14336 and
  // 14336x4096 at 256 and 512 rows against every tile width (64, 128, 256) and
  // 1, 2, 4 or 8 K ranges: the rule picks the fastest of the 12 in all 8.
  // WOQ_GEMM_BN (64, 128 or 256) forces the tile width above 64 rows and
  // WOQ_GEMM_SPLITS the number of K ranges (tuning aids, read on every call).
  const int64_t nsteps = (k + 127) / 128;
  auto ranges_for = [&](int64_t tiles) {
    return std::max<int64_t>(1, std::min<int64_t>({16, kComputeUnits / tiles, nsteps / 4}));
  };
  if (m > 64) {
    p.bm = 128;
    const int64_t t256 = ((m + 127) / 128) * ((n + 255) / 256);
    p.bn = t256 * ranges_for(t256) > kComputeUnits / 2 ? 256 : 64;
    if (const char* e = std::getenv("WOQ_GEMM_BN")) {
      const int bn = std::atoi(e);
      if (bn == 64 || bn == 128 || bn == 256) p.bn = bn;
    }
    p.waves = p.bn == 256 ? 8 : 4;
  } else if (m > 32) {
    p.bm = 64; p.bn = 64; p.waves = 4;
  } else {
    p.bm = 32; p.bn = 64; p.waves = 2;
  }
  p.mpad = ((m + 127) / 128) * 128;
  const int64_t tm = (m + p.bm - 1) / p.bm, tn = (n + p.bn - 1) / p.bn;
  p.grid = tm * tn;
  // Split-K: a grid under three quarters of the chip takes up to 16 K ranges
  // of at least 4 steps (an even count) each, as many as keep it within one
  // round of workgroups; the ranges' float32 partials are summed in order
  // afterwards.
  {
    const char* env_splits = std::getenv("WOQ_GEMM_SPLITS");
    const int64_t forced = env_splits ? std::atoi(env_splits) : 0;
    if (split_ok && (forced > 0 || p.grid < kComputeUnits * 3 / 4)) {
      int64_t s = forced > 0 ? std::min<int64_t>(forced, std::max<int64_t>(nsteps / 2, 1)) : ranges_for(p.grid);
      if (s >= 2) {
        int64_t sps = (nsteps + s - 1) / s;
        sps += sps & 1;
        s = (nsteps + sps - 1) / sps;
        if (s >= 2) {
          p.splits = (int)s;
          p.sps = (int)sps;
          p.grid *= s;
        }
      }
    }
  }
  if (p.bm == 128 && p.bn == 256) {
    // 128 x 256 tiles run one workgroup per compute unit.  When the last round
    // would be at most half full, the trailing tile columns that hold it go to
    // a second launch as 64-row tiles (half the work each, twice as many), so
    // that round takes about half as long.
    const int64_t rem = p.grid % kComputeUnits;
    if (p.grid > kComputeUnits && rem != 0 && 2 * rem <= kComputeUnits) {
      const int64_t cols = (rem + tm - 1) / tm;
      const int64_t tail_tiles = ((m + 63) / 64) * cols;
      if (cols < tn && tail_tiles <= kComputeUnits) {
        p.tail_n = n - (tn - cols) * 256;
        p.grid = tm * (tn - cols) + tail_tiles;
      }
    }
  }
  return p;
}

LinearWorkspace linear_workspace_layout(int64_t m, int64_t n, int64_t k, int32_t group,
                                        bool has_order, bool split_ok) {
  LinearWorkspace w;
  const LinearPlan p = linear_plan(m, n, k, group, has_order, true, split_ok);
  if (p.path == 1 && p.xfrag) {
    w.xg_off = 0;
    w.xg_bytes = round256(xfrag_bytes(m, k));
  } else if ((p.path == 1 || p.path == 4 || p.path == 5) && has_order) {
    w.xg_off = 0;
    w.xg_bytes = round256((size_t)m * (size_t)k * 2);
  } else if (p.path == 6) {
    w.xg_off = 0;
    w.xg_bytes = has_order ? round256((size_t)m * (size_t)k * 2) : 0;
    w.part_off = w.xg_bytes;
    w.part_bytes = p.splits > 1 ? round256((size_t)p.splits * (size_t)m * (size_t)n * 4) : 0;
  } else if (p.path == 2) {
    const int64_t kpad = (k + 127) / 128 * 128;
    w.xg_off = 0;
    w.xg_bytes = round256((size_t)m * (size_t)kpad * 2);
    w.xs_off = w.xg_bytes;
    const int64_t piece = group < 128 ? group : 128;   // sums per group part inside a k step
    w.xs_bytes = round256((size_t)(k / piece) * (size_t)p.mpad * 4);
    w.sz_off = w.xs_off + w.xs_bytes;
    w.sz_bytes = round256(gemm_sz_bytes(n, k, group));
    w.part_off = w.sz_off + w.sz_bytes;
    w.part_bytes = p.splits > 1 ? round256((size_t)p.splits * (size_t)m * (size_t)n * 4) : 0;
  }
  w.total = w.xg_bytes + w.xs_bytes + w.sz_bytes + w.part_bytes;
  return w;
}

}  // namespace woq

using namespace woq;

extern "C" {

const char* woq_status_str(int32_t status) {
  switch (status) {
    case WOQ_OK: return "ok";
    case WOQ_EINVAL: return "invalid argument (null pointer, negative size or unknown enum)";
    case WOQ_ESHAPE: return "inconsistent sizes";
    case WOQ_EGROUP: return "group size invalid for this layout (must be even where packed, >= 1, and divide K)";
    case WOQ_ENONFINITE: return "non-finite weight";
    case WOQ_ERANGE: return "code outside 0..15";
    case WOQ_EWORKSPACE: return "workspace missing or too small";
    case WOQ_EUNSUPPORTED: return "unsupported (group not in {32,64,128,256} or sizes too large)";
    case WOQ_EALIGN: return "pointer not aligned as required";
    case WOQ_EHIP: return "HIP runtime error";
    case WOQ_ENOTPD: return "calibration matrix not positive definite (raise the damping)";
    default: return "unknown status";
  }
}

int32_t woq_version(void) { return 100; }

int32_t woq_quantize_groups(const float* w, int64_t n, int64_t k, int32_t group,
                            int32_t symmetric, uint8_t* q, float* scale, uint8_t* zero,
                            void* stream) {
  if (n < 0 || k < 0) return WOQ_EINVAL;
  if (symmetric != 0 && symmetric != 1) return WOQ_EINVAL;
  if (group < 1 || (k > 0 && k % group)) return WOQ_EGROUP;
  if (n * k >= kMaxElems) return WOQ_EUNSUPPORTED;
  if (n == 0 || k == 0) return WOQ_OK;
  if (!w || !q || !scale || !zero) return WOQ_EINVAL;
  if (!aligned(w, 4) || !aligned(scale, 4)) return WOQ_EALIGN;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint32_t hflag = 0;
  const int32_t st = with_flag(s, &hflag, [&](uint32_t* flag) {
    return launch_quantize(w, n, k, group, symmetric, q, scale, zero, flag, s);
  });
  if (st != WOQ_OK) return st;
  return hflag ? WOQ_ENONFINITE : WOQ_OK;
}

int32_t woq_pack_uint4(const uint8_t* q, int64_t count, uint8_t* packed, void* stream) {
  if (count < 0) return WOQ_EINVAL;
  if (count % 2) return WOQ_ESHAPE;
  if (count >= kMaxElems) return WOQ_EUNSUPPORTED;
  if (count == 0) return WOQ_OK;
  if (!q || !packed) return WOQ_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint32_t hflag = 0;
  const int32_t st = with_flag(s, &hflag, [&](uint32_t* flag) {
    return launch_pack(q, count, packed, flag, s);
  });
  if (st != WOQ_OK) return st;
  return hflag ? WOQ_ERANGE : WOQ_OK;
}

int32_t woq_unpack_uint4(const uint8_t* packed, int64_t count, uint8_t* q, void* stream) {
  if (count < 0) return WOQ_EINVAL;
  if (count % 2) return WOQ_ESHAPE;
  if (count >= kMaxElems) return WOQ_EUNSUPPORTED;
  if (count == 0) return WOQ_OK;
  if (!q || !packed) return WOQ_EINVAL;
  return launch_unpack(packed, count, q, reinterpret_cast<hipStream_t>(stream));
}

int32_t woq_dequantize_int4_groups(const uint8_t* packed, const float* scale,
                                   const uint8_t* zero, int64_t n, int64_t k, int32_t group,
                                   int32_t out_dtype, void* w_hat, void* stream) {
  if (n < 0 || k < 0) return WOQ_EINVAL;
  if (out_dtype != WOQ_F32 && out_dtype != WOQ_BF16) return WOQ_EINVAL;
  if (group < 2 || group % 2 || (k > 0 && k % group)) return WOQ_EGROUP;
  if (n * k >= kMaxElems) return WOQ_EUNSUPPORTED;
  if (n == 0 || k == 0) return WOQ_OK;
  if (!packed || !scale || !zero || !w_hat) return WOQ_EINVAL;
  if (!aligned(scale, 4) || !aligned(w_hat, out_dtype == WOQ_F32 ? 4 : 2)) return WOQ_EALIGN;
  return launch_dequantize(packed, scale, zero, n, k, group, out_dtype, w_hat,
                           reinterpret_cast<hipStream_t>(stream));
}

int32_t woq_quantize_int4_sym_f16(const float* w, int64_t n, int64_t k, int32_t group,
                                  int8_t* codes, uint16_t* scale16, void* stream) {
  if (n < 0 || k < 0) return WOQ_EINVAL;
  if (group < 2 || group % 2 || (k > 0 && k % group)) return WOQ_EGROUP;
  if (n * k >= kMaxElems) return WOQ_EUNSUPPORTED;
  if (n == 0 || k == 0) return WOQ_OK;
  if (!w || !codes || !scale16) return WOQ_EINVAL;
  if (!aligned(w, 4) || !aligned(scale16, 2)) return WOQ_EALIGN;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint32_t hflag = 0;
  const int32_t st = with_flag(s, &hflag, [&](uint32_t* flag) {
    return launch_quantize_s16(w, n, k, group, codes, scale16, flag, s);
  });
  if (st != WOQ_OK) return st;
  if (hflag & 1u) return WOQ_ENONFINITE;
  return hflag ? WOQ_ERANGE : WOQ_OK;
}

int32_t woq_pack_int4(const int8_t* codes, int64_t count, uint8_t* packed, void* stream) {
  if (count < 0) return WOQ_EINVAL;
  if (count % 2) return WOQ_ESHAPE;
  if (count >= kMaxElems) return WOQ_EUNSUPPORTED;
  if (count == 0) return WOQ_OK;
  if (!codes || !packed) return WOQ_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint32_t hflag = 0;
  const int32_t st = with_flag(s, &hflag, [&](uint32_t* flag) {
    return launch_pack_s4(codes, count, packed, flag, s);
  });
  if (st != WOQ_OK) return st;
  return hflag ? WOQ_ERANGE : WOQ_OK;
}

int32_t woq_unpack_int4(const uint8_t* packed, int64_t count, int8_t* codes, void* stream) {
  if (count < 0) return WOQ_EINVAL;
  if (count % 2) return WOQ_ESHAPE;
  if (count >= kMaxElems) return WOQ_EUNSUPPORTED;
  if (count == 0) return WOQ_OK;
  if (!codes || !packed) return WOQ_EINVAL;
  return launch_unpack_s4(packed, count, codes, reinterpret_cast<hipStream_t>(stream));
}

int32_t woq_dequantize_int4_sym_f16(const uint8_t* packed, const uint16_t* scale16, int64_t n,
                                    int64_t k, int32_t group, int32_t out_dtype, void* w_hat,
                                    void* stream) {
  if (n < 0 || k < 0) return WOQ_EINVAL;
  if (out_dtype != WOQ_F32 && out_dtype != WOQ_BF16) return WOQ_EINVAL;
  if (group < 2 || group % 2 || (k > 0 && k % group)) return WOQ_EGROUP;
  if (n * k >= kMaxElems) return WOQ_EUNSUPPORTED;
  if (n == 0 || k == 0) return WOQ_OK;
  if (!packed || !scale16 || !w_hat) return WOQ_EINVAL;
  if (!aligned(scale16, 2) || !aligned(w_hat, out_dtype == WOQ_F32 ? 4 : 2)) return WOQ_EALIGN;
  return launch_dequantize_s16(packed, scale16, n, k, group, out_dtype, w_hat,
                               reinterpret_cast<hipStream_t>(stream));
}

int32_t woq_quantize_mxfp4(const float* w, int64_t n, int64_t k, uint8_t* codes, uint8_t* scales,
                           void* stream) {
  if (n < 0 || k < 0) return WOQ_EINVAL;
  if (k % 32) return WOQ_EGROUP;
  if (n * k >= kMaxElems) return WOQ_EUNSUPPORTED;
  if (n == 0 || k == 0) return WOQ_OK;
  if (!w || !codes || !scales) return WOQ_EINVAL;
  if (!aligned(w, 4)) return WOQ_EALIGN;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint32_t hflag = 0;
  const int32_t st = with_flag(s, &hflag, [&](uint32_t* flag) {
    return launch_quantize_mx(w, n, k, codes, scales, flag, s);
  });
  if (st != WOQ_OK) return st;
  return hflag ? WOQ_ENONFINITE : WOQ_OK;
}

int32_t woq_dequantize_mxfp4(const uint8_t* blocks, const uint8_t* scales, int64_t n, int64_t k,
                             int32_t out_dtype, void* w_hat, void* stream) {
  if (n < 0 || k < 0) return WOQ_EINVAL;
  if (out_dtype != WOQ_F32 && out_dtype != WOQ_BF16) return WOQ_EINVAL;
  if (k % 32) return WOQ_EGROUP;
  if (n * k >= kMaxElems) return WOQ_EUNSUPPORTED;
  if (n == 0 || k == 0) return WOQ_OK;
  if (!blocks || !scales || !w_hat) return WOQ_EINVAL;
  if (!aligned(w_hat, out_dtype == WOQ_F32 ? 4 : 2)) return WOQ_EALIGN;
  return launch_dequantize_mx(blocks, scales, n, k, out_dtype, w_hat, reinterpret_cast<hipStream_t>(stream));
}

int32_t woq_quantize_int4_rows(const float* w, int64_t n, int64_t k, int8_t* codes, float* scale,
                               void* stream) {
  if (n < 0 || k < 0) return WOQ_EINVAL;
  if (k % 2) return WOQ_ESHAPE;
  if (n * k >= kMaxElems) return WOQ_EUNSUPPORTED;
  if (n == 0) return WOQ_OK;
  if (!w || !codes || !scale) return WOQ_EINVAL;
  if (!aligned(w, 4) || !aligned(scale, 4)) return WOQ_EALIGN;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint32_t hflag = 0;
  const int32_t st = with_flag(s, &hflag, [&](uint32_t* flag) {
    return launch_quantize_rows(w, n, k, codes, scale, flag, s);
  });
  if (st != WOQ_OK) return st;
  return hflag ? WOQ_ENONFINITE : WOQ_OK;
}

int32_t woq_gptq_quantize(const float* w, const void* x_bf16, int64_t t, int64_t n, int64_t k, int32_t group,
                          int32_t act_order, double damp, uint8_t* codes, float* scale, uint8_t* zero,
                          int32_t* order, void* stream) {
  if (n < 0 || k < 0 || t < 0 || act_order < 0 || act_order > 1) return WOQ_EINVAL;
  if (!(damp >= 0.0) || !std::isfinite(damp)) return WOQ_EINVAL;
  if (group < 1 || (k > 0 && k % group)) return WOQ_EGROUP;
  if (gptq_block_cols(group) == 0) return WOQ_EUNSUPPORTED;
  if (k >= (int64_t)1 << 20 || n >= kMaxDim || t >= kMaxDim || n * k >= kMaxElems || t * k >= kMaxElems)
    return WOQ_EUNSUPPORTED;
  if (n == 0 || k == 0) return WOQ_OK;
  if (!w || (t > 0 && !x_bf16) || !codes || !scale || !zero || (act_order && !order)) return WOQ_EINVAL;
  if (!aligned(w, 4) || !aligned(x_bf16, 2) || !aligned(scale, 4) || (act_order && !aligned(order, 4)))
    return WOQ_EALIGN;
  return run_gptq(w, static_cast<const uint16_t*>(x_bf16), t, n, k, group, act_order, damp, codes, scale, zero,
                  order, reinterpret_cast<hipStream_t>(stream));
}

int32_t woq_awq_search(const float* w, const void* x_bf16, int64_t t, int64_t n, int64_t k, int32_t group,
                       int32_t n_grid, uint8_t* codes, float* scale, uint8_t* zero, float* s, double* losses,
                       int32_t* best, void* stream) {
  if (n < 0 || k < 0 || t < 1 || n_grid < 1 || n_grid > 1000) return WOQ_EINVAL;
  if (group < 1 || (k > 0 && k % group)) return WOQ_EGROUP;
  if (n >= kMaxDim || k >= kMaxDim || t >= kMaxDim / 64 || n * k >= kMaxElems || t * k >= kMaxElems)
    return WOQ_EUNSUPPORTED;
  if (n == 0 || k == 0) return WOQ_OK;
  if (!w || !x_bf16 || !codes || !scale || !zero || !s) return WOQ_EINVAL;
  if (!aligned(w, 4) || !aligned(x_bf16, 2) || !aligned(scale, 4) || !aligned(s, 4) ||
      (losses && !aligned(losses, 8)))
    return WOQ_EALIGN;
  return run_awq(w, static_cast<const uint16_t*>(x_bf16), t, n, k, group, n_grid, codes, scale, zero, s, losses,
                 best, reinterpret_cast<hipStream_t>(stream));
}

int32_t woq_dequantize_int4_rows(const uint8_t* packed, const float* scale, int64_t n, int64_t k,
                                 int32_t out_dtype, void* w_hat, void* stream) {
  if (n < 0 || k < 0) return WOQ_EINVAL;
  if (out_dtype != WOQ_F32 && out_dtype != WOQ_BF16) return WOQ_EINVAL;
  if (k % 2) return WOQ_ESHAPE;
  if (n * k >= kMaxElems) return WOQ_EUNSUPPORTED;
  if (n == 0 || k == 0) return WOQ_OK;
  if (!packed || !scale || !w_hat) return WOQ_EINVAL;
  if (!aligned(scale, 4) || !aligned(w_hat, out_dtype == WOQ_F32 ? 4 : 2)) return WOQ_EALIGN;
  return launch_dequantize_rows(packed, scale, n, k, out_dtype, w_hat, reinterpret_cast<hipStream_t>(stream));
}

size_t woq_linear_int4_rows_workspace_bytes(int64_t m, int64_t n, int64_t k, int32_t has_order) {
  const int32_t g = rows_group(k);
  return g ? woq_linear_workspace_bytes(m, n, k, g, has_order) : 0;
}

size_t woq_linear_int4_groups_zp4_workspace_bytes(int64_t m, int64_t n, int64_t k, int32_t group,
                                                  int32_t has_order) {
  if (check_linear_shape(m, n, k, group) != WOQ_OK) return 0;
  if (m == 0 || n == 0 || k == 0) return 0;
  const LinearPlan plan = linear_plan(m, n, k, group, has_order != 0);
  return (plan.path == 4 ? round256((size_t)n * (size_t)(k / group)) : 0) +
         linear_workspace_layout(m, n, k, group, has_order != 0).total;
}

int32_t woq_pack_zero_points(const uint8_t* zero, int64_t n, int64_t ngroups, uint8_t* packed, void* stream) {
  if (n < 0 || ngroups < 0) return WOQ_EINVAL;
  if (n * ngroups >= kMaxElems) return WOQ_EUNSUPPORTED;
  if (n == 0 || ngroups == 0) return WOQ_OK;
  if (!zero || !packed) return WOQ_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint32_t hflag = 0;
  const int32_t st = with_flag(s, &hflag, [&](uint32_t* flag) {
    return launch_pack_zero_points(zero, n, ngroups, packed, flag, s);
  });
  if (st != WOQ_OK) return st;
  return hflag ? WOQ_ERANGE : WOQ_OK;
}

int32_t woq_unpack_zero_points(const uint8_t* packed, int64_t n, int64_t ngroups, uint8_t* zero, void* stream) {
  if (n < 0 || ngroups < 0) return WOQ_EINVAL;
  if (n * ngroups >= kMaxElems) return WOQ_EUNSUPPORTED;
  if (n == 0 || ngroups == 0) return WOQ_OK;
  if (!zero || !packed) return WOQ_EINVAL;
  return launch_unpack_zero_points(packed, n, ngroups, zero, reinterpret_cast<hipStream_t>(stream));
}

size_t woq_linear_workspace_bytes(int64_t m, int64_t n, int64_t k, int32_t group,
                                  int32_t has_order) {
  if (check_linear_shape(m, n, k, group) != WOQ_OK) return 0;
  return linear_workspace_layout(m, n, k, group, has_order != 0).total;
}

}  // extern "C"

namespace {

// Shared body of the linear entry points; `prepared` selects the weight layout
// the kernels address, `scale16` (non-null) the signed codes with float16
// scales and no zero point.
int32_t linear_impl(const void* x_bf16, int64_t m, const uint8_t* packed, const float* scale,
                    const uint8_t* zero, const float* bias, const int32_t* order, int64_t n,
                    int64_t k, int32_t group, int32_t y_dtype, void* y, void* workspace,
                    size_t workspace_bytes, void* stream, int32_t prepared,
                    const uint16_t* scale16 = nullptr, const uint8_t* scale8 = nullptr,
                    const float* scale_row = nullptr, const uint8_t* zero_packed = nullptr,
                    bool split_ok = true) {
  const bool row = scale_row != nullptr;     // Int4Linear: signed codes, one float32 scale a row
  const bool zp4 = zero_packed != nullptr;   // packed 4-bit zero points
  const bool sym16 = scale16 != nullptr || row;
  const bool mx = scale8 != nullptr;
  int32_t st = check_linear_shape(m, n, k, group);
  if (st != WOQ_OK) return st;
  if (y_dtype != WOQ_F32 && y_dtype != WOQ_BF16) return WOQ_EINVAL;
  if (m == 0 || n == 0) return WOQ_OK;
  if (!y) return WOQ_EINVAL;
  if (!aligned(y, y_dtype == WOQ_F32 ? 4 : 2)) return WOQ_EALIGN;
  if (bias && !aligned(bias, 4)) return WOQ_EALIGN;
  if (k == 0)
    return launch_fill_bias(bias, (int32_t)m, (int32_t)n, y_dtype == WOQ_BF16, y,
                            reinterpret_cast<hipStream_t>(stream));
  if (!x_bf16 || !packed || (!sym16 && !mx && (!scale || (!zero && !zp4)))) return WOQ_EINVAL;
  if (!aligned(x_bf16, 16) || !aligned(packed, 16)) return WOQ_EALIGN;
  if (mx ? !aligned(scale8, 16)
         : row ? !aligned(scale_row, 16)
               : sym16 ? !aligned(scale16, 16) : (!aligned(scale, 16) || (!zp4 && !aligned(zero, 16))))
    return WOQ_EALIGN;
  const bool has_order = order != nullptr;
  if (has_order && !aligned(order, 16)) return WOQ_EALIGN;
  const LinearPlan plan = linear_plan(m, n, k, group, has_order, !prepared, split_ok);
  const LinearWorkspace ws = linear_workspace_layout(m, n, k, group, has_order, split_ok);
  // The tile GEMV reads one zero point a byte: packed ones are unpacked into the
  // head of the workspace first; every other path reads them as they are.
  const bool zp4_unpack = zp4 && plan.path == 4;
  const size_t zbytes = zp4_unpack ? round256((size_t)n * (size_t)(k / group)) : 0;
  if (plan.path == 2 && k >= kGemmMaxK) return WOQ_EUNSUPPORTED;
  if (ws.total + zbytes > 0) {
    if (!workspace || workspace_bytes < ws.total + zbytes) return WOQ_EWORKSPACE;
    if (!aligned(workspace, 256)) return WOQ_EALIGN;
  }
  char* wsb = static_cast<char*>(workspace) + zbytes;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (zp4_unpack) {
    st = launch_unpack_zero_points(zero_packed, n, k / group, static_cast<uint8_t*>(workspace), s);
    if (st != WOQ_OK) return st;
    zero = static_cast<const uint8_t*>(workspace);
  } else if (zp4) {
    zero = zero_packed;
  }
  LinearArgs a{};
  a.x = static_cast<const uint16_t*>(x_bf16);
  a.packed = packed;
  a.scale = scale;
  a.zero = zero;
  a.bias = bias;
  a.y = y;
  a.m = (int32_t)m;
  a.n = (int32_t)n;
  a.k = (int32_t)k;
  a.group = group;
  a.y_bf16 = y_dtype == WOQ_BF16;
  a.mpad = plan.mpad;
  a.kpad = a.k;
  a.prepared = prepared;
  a.sym16 = sym16 ? 1 : 0;
  a.scale16 = scale16;
  a.mx = mx ? 1 : 0;
  a.scale8 = scale8;
  a.row_scale = row ? 1 : 0;
  a.zp4 = zp4 && !zp4_unpack ? 1 : 0;
  if (row) a.scale = scale_row;
  if (plan.path == 1) {
    if (plan.xfrag) {
      uint16_t* xf = reinterpret_cast<uint16_t*>(wsb + ws.xg_off);
      st = launch_xfrag(a.x, order, a.m, a.k, group, mx ? 1 : 0, xf, s);
      if (st != WOQ_OK) return st;
      a.x = xf;
    } else if (has_order) {
      uint16_t* xg = reinterpret_cast<uint16_t*>(wsb + ws.xg_off);
      st = launch_prep(a.x, order, a.m, a.k, a.k, group, 0, xg, nullptr, m, s);
      if (st != WOQ_OK) return st;
      a.x = xg;
    }
    return launch_skinny(a, plan, s);
  }
  if (plan.path == 6) {
    if (has_order) {
      uint16_t* xg = reinterpret_cast<uint16_t*>(wsb + ws.xg_off);
      st = launch_prep(a.x, order, a.m, a.k, a.k, group, 0, xg, nullptr, m, s);
      if (st != WOQ_OK) return st;
      a.x = xg;
    }
    a.part = reinterpret_cast<float*>(wsb + ws.part_off);
    return launch_sm(a, plan, s);
  }
  if (plan.path == 4 || plan.path == 5) {
    if (has_order) {
      uint16_t* xg = reinterpret_cast<uint16_t*>(wsb + ws.xg_off);
      st = launch_prep(a.x, order, a.m, a.k, a.k, group, 0, xg, nullptr, m, s);
      if (st != WOQ_OK) return st;
      a.x = xg;
    }
    return plan.path == 5 ? launch_rows(&a, 1, plan.rows_u, s) : launch_gemv(a, plan, s);
  }
  uint16_t* xg = reinterpret_cast<uint16_t*>(wsb + ws.xg_off);
  float* xs = reinterpret_cast<float*>(wsb + ws.xs_off);
  a.kpad = (a.k + 127) / 128 * 128;
  // the activation pre-pass and the scale/zero table, one launch
  st = launch_gemm_prep(a, order, xg, xs, wsb + ws.sz_off, s);
  if (st != WOQ_OK) return st;
  a.x = xg;
  a.xs = xs;
  a.part = reinterpret_cast<float*>(wsb + ws.part_off);
  return launch_gemm(a, plan, wsb + ws.sz_off, s);
}

}  // namespace

extern "C" {

int32_t woq_linear_int4_groups(const void* x_bf16, int64_t m, const uint8_t* packed,
                               const float* scale, const uint8_t* zero, const float* bias,
                               const int32_t* order, int64_t n, int64_t k, int32_t group,
                               int32_t y_dtype, void* y, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return linear_impl(x_bf16, m, packed, scale, zero, bias, order, n, k, group, y_dtype, y,
                     workspace, workspace_bytes, stream, 0);
}

}  // extern "C"

namespace {

// Workspace of woq_linear_int4_groups_noalloc: a file-scope device array, so
// that call allocates nothing.  Each device holds its own copy from the load of
// the library until the process ends; its address on a device is taken once,
// with that device current, and kept in `scratch_addr`.
constexpr size_t kScratchBytes = (size_t)32 << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* scratch_addr[kMaxDevices] = {};
std::mutex scratch_mutex;

// The current device's copy of `scratch` (null with the status on failure).
void* device_scratch(int32_t* status) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *status = WOQ_EHIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_addr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      *status = WOQ_EHIP;
      return nullptr;
    }
    scratch_addr[dev] = ptr;
  }
  *status = WOQ_OK;
  return scratch_addr[dev];
}

}  // namespace

extern "C" {

size_t woq_linear_noalloc_max_workspace_bytes(void) { return kScratchBytes; }

int32_t woq_linear_int4_groups_noalloc(const void* x_bf16, int64_t m, const uint8_t* packed,
                                       const float* scale, const uint8_t* zero, const float* bias,
                                       const int32_t* order, int64_t n, int64_t k, int32_t group,
                                       int32_t y_dtype, void* y, void* stream) {
  const int32_t st = check_linear_shape(m, n, k, group);
  if (st != WOQ_OK) return st;
  const size_t need = linear_workspace_layout(m, n, k, group, order != nullptr).total;
  if (m == 0 || n == 0 || need == 0)
    return linear_impl(x_bf16, m, packed, scale, zero, bias, order, n, k, group, y_dtype, y, nullptr, 0,
                       stream, 0);
  // A split-K plan whose partial outputs do not fit runs with K whole.
  const bool split_ok = need <= kScratchBytes;
  if (!split_ok && linear_workspace_layout(m, n, k, group, order != nullptr, false).total > kScratchBytes)
    return WOQ_EWORKSPACE;
  int32_t dst = WOQ_OK;
  void* ws = device_scratch(&dst);
  if (dst != WOQ_OK) return dst;
  return linear_impl(x_bf16, m, packed, scale, zero, bias, order, n, k, group, y_dtype, y, ws, kScratchBytes,
                     stream, 0, nullptr, nullptr, nullptr, nullptr, split_ok);
}

int32_t woq_linear_int4_groups_zp4(const void* x_bf16, int64_t m, const uint8_t* packed, const float* scale,
                                   const uint8_t* zero_packed, const float* bias, const int32_t* order, int64_t n,
                                   int64_t k, int32_t group, int32_t y_dtype, void* y, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if (k > 0 && m > 0 && n > 0 && !zero_packed) return WOQ_EINVAL;
  return linear_impl(x_bf16, m, packed, scale, nullptr, bias, order, n, k, group, y_dtype, y, workspace,
                     workspace_bytes, stream, 0, nullptr, nullptr, nullptr, zero_packed);
}

int32_t woq_linear_int4_sym_f16(const void* x_bf16, int64_t m, const uint8_t* packed,
                                const uint16_t* scale16, const float* bias, const int32_t* order,
                                int64_t n, int64_t k, int32_t group, int32_t y_dtype, void* y,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (k > 0 && m > 0 && n > 0 && !scale16) return WOQ_EINVAL;
  return linear_impl(x_bf16, m, packed, nullptr, nullptr, bias, order, n, k, group, y_dtype, y,
                     workspace, workspace_bytes, stream, 0, scale16);
}

int32_t woq_linear_int4_sym_f16_prepared(const void* x_bf16, int64_t m, const uint8_t* prepared,
                                         const uint16_t* scale16, const float* bias,
                                         const int32_t* order, int64_t n, int64_t k, int32_t group,
                                         int32_t y_dtype, void* y, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  if (k > 0 && m > 0 && n > 0 && !scale16) return WOQ_EINVAL;
  return linear_impl(x_bf16, m, prepared, nullptr, nullptr, bias, order, n, k, group, y_dtype, y,
                     workspace, workspace_bytes, stream, 1, scale16);
}

int32_t woq_linear_int4_rows(const void* x_bf16, int64_t m, const uint8_t* packed, const float* scale,
                             const float* bias, const int32_t* order, int64_t n, int64_t k,
                             int32_t y_dtype, void* y, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (k > 0 && m > 0 && n > 0 && !scale) return WOQ_EINVAL;
  const int32_t g = rows_group(k);
  if (k > 0 && g == 0) return k % 2 ? WOQ_ESHAPE : WOQ_EUNSUPPORTED;
  return linear_impl(x_bf16, m, packed, nullptr, nullptr, bias, order, n, k, k > 0 ? g : 32, y_dtype,
                     y, workspace, workspace_bytes, stream, 0, nullptr, nullptr, scale);
}

int32_t woq_linear_mxfp4(const void* x_bf16, int64_t m, const uint8_t* blocks, const uint8_t* scales,
                         const float* bias, int64_t n, int64_t k, int32_t y_dtype, void* y,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (k > 0 && m > 0 && n > 0 && !scales) return WOQ_EINVAL;
  return linear_impl(x_bf16, m, blocks, nullptr, nullptr, bias, nullptr, n, k, 32, y_dtype, y,
                     workspace, workspace_bytes, stream, 0, nullptr, scales);
}

int32_t woq_linear_int4_groups_prepared(const void* x_bf16, int64_t m, const uint8_t* prepared,
                                        const float* scale, const uint8_t* zero,
                                        const float* bias, const int32_t* order, int64_t n,
                                        int64_t k, int32_t group, int32_t y_dtype, void* y,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  return linear_impl(x_bf16, m, prepared, scale, zero, bias, order, n, k, group, y_dtype, y,
                     workspace, workspace_bytes, stream, 1);
}

int32_t woq_linear_int4_groups_grouped(const void* x_bf16, int64_t m, int32_t count,
                                       const uint8_t* const* packed, const float* const* scale,
                                       const uint8_t* const* zero, const float* const* bias,
                                       const int64_t* n, int64_t k, int32_t group,
                                       int32_t prepared, int32_t y_dtype, void* const* y,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  if (count < 1 || count > kMaxGrouped || !packed || !scale || !zero || !n || !y) return WOQ_EINVAL;
  if (prepared != 0 && prepared != 1) return WOQ_EINVAL;
  if (y_dtype != WOQ_F32 && y_dtype != WOQ_BF16) return WOQ_EINVAL;
  // Every matrix is validated as the single call would before anything is enqueued.
  int64_t rows16 = 0;
  for (int i = 0; i < count; ++i) {
    const int32_t st = check_linear_shape(m, n[i], k, group);
    if (st != WOQ_OK) return st;
    if (m == 0 || n[i] == 0 || k == 0) continue;
    if (!x_bf16 || !packed[i] || !scale[i] || !zero[i] || !y[i]) return WOQ_EINVAL;
    if (!aligned(y[i], y_dtype == WOQ_F32 ? 4 : 2)) return WOQ_EALIGN;
    if (bias && bias[i] && !aligned(bias[i], 4)) return WOQ_EALIGN;
    if (!aligned(x_bf16, 16) || !aligned(packed[i], 16) || !aligned(scale[i], 16) || !aligned(zero[i], 16))
      return WOQ_EALIGN;
    rows16 += (n[i] + 15) / 16 * 16;
  }
  if (m == 0) return WOQ_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  LinearPlan plan;
  int64_t rows_total = 0;
  for (int i = 0; i < count; ++i) rows_total += n[i];
  const bool rows = k > 0 && !prepared && rows_supported(m, k) && rows_total > 0 &&
                    std::getenv("WOQ_DECODE_MFMA") == nullptr;
  if (rows || (k > 0 && m <= 4 && rows16 > 0 && rows16 < kMaxDim && k < ((int64_t)1 << 26) &&
               std::getenv("WOQ_FORCE_SKINNY") == nullptr && gemv_plan(m, rows16, k, group, &plan))) {
    // one decode launch over all the matrices
    LinearArgs args[kMaxGrouped];
    int used = 0;
    for (int i = 0; i < count; ++i) {
      if (n[i] == 0) continue;
      LinearArgs& a = args[used++];
      a = LinearArgs{};
      a.x = static_cast<const uint16_t*>(x_bf16);
      a.packed = packed[i];
      a.scale = scale[i];
      a.zero = zero[i];
      a.bias = bias ? bias[i] : nullptr;
      a.y = y[i];
      a.m = (int32_t)m;
      a.n = (int32_t)n[i];
      a.k = (int32_t)k;
      a.group = group;
      a.y_bf16 = y_dtype == WOQ_BF16;
      a.kpad = a.k;
      a.prepared = prepared;
    }
    if (!used) return WOQ_OK;
    if (rows) return launch_rows(args, used, rows_per_group(m, rows_total, k), s);
    plan.gb = group >= 128 ? 4 : group / 32;
    return launch_gemv_grouped(args, used, plan, s);
  }
  // otherwise one call per matrix, in order, sharing the workspace
  for (int i = 0; i < count; ++i) {
    const int32_t st = linear_impl(x_bf16, m, packed[i], scale[i], zero[i], bias ? bias[i] : nullptr,
                                   nullptr, n[i], k, group, y_dtype, y[i], workspace, workspace_bytes,
                                   stream, prepared);
    if (st != WOQ_OK) return st;
  }
  return WOQ_OK;
}

size_t woq_prepared_bytes(int64_t n, int64_t k) {
  if (n < 0 || k < 0 || k % 32 || n >= kMaxDim || k >= kMaxDim) return 0;
  return (size_t)prepared_bytes(n, k);
}

int32_t woq_prepare_int4(const uint8_t* packed, int64_t n, int64_t k, uint8_t* prepared,
                         void* stream) {
  if (n < 0 || k < 0) return WOQ_EINVAL;
  if (k % 32) return WOQ_ESHAPE;
  if (n >= kMaxDim || k >= kMaxDim || n * k >= kMaxElems) return WOQ_EUNSUPPORTED;
  if (n == 0 || k == 0) return WOQ_OK;
  if (!packed || !prepared) return WOQ_EINVAL;
  if (!aligned(packed, 16) || !aligned(prepared, 16)) return WOQ_EALIGN;
  return launch_prepare(packed, n, k, prepared, reinterpret_cast<hipStream_t>(stream));
}

int32_t woq_unprepare_int4(const uint8_t* prepared, int64_t n, int64_t k, uint8_t* packed,
                           void* stream) {
  if (n < 0 || k < 0) return WOQ_EINVAL;
  if (k % 32) return WOQ_ESHAPE;
  if (n >= kMaxDim || k >= kMaxDim || n * k >= kMaxElems) return WOQ_EUNSUPPORTED;
  if (n == 0 || k == 0) return WOQ_OK;
  if (!packed || !prepared) return WOQ_EINVAL;
  if (!aligned(packed, 16) || !aligned(prepared, 16)) return WOQ_EALIGN;
  return launch_unprepare(prepared, n, k, packed, reinterpret_cast<hipStream_t>(stream));
}

int32_t woq_linear_plan(int64_t m, int64_t n, int64_t k, int32_t group, int32_t has_order,
                        char* buf, size_t len) {
  if (!buf || len == 0) return WOQ_EINVAL;
  const int32_t st = check_linear_shape(m, n, k, group);
  if (st != WOQ_OK) return st;
  const LinearPlan p = linear_plan(m, n, k, group, has_order != 0);
  const size_t ws = linear_workspace_layout(m, n, k, group, has_order != 0).total;
  switch (p.path) {
    case 0: std::snprintf(buf, len, "path=none"); break;
    case 3: std::snprintf(buf, len, "path=bias_fill"); break;
    case 1:
      std::snprintf(buf, len,
                    "path=skinny_mfma act_tiles=%d wave_groups=%d weight_tiles=%d waves=%d steps_per_wave=%d "
                    "group_blocks=%d grid=%lld prep=%s workspace=%zu",
                    p.mt, p.wm, p.ns, p.waves, p.cnt, p.gb, (long long)p.grid,
                    p.xfrag ? (p.prep ? "gather+fragments" : "fragments") : (p.prep ? "gather" : "none"), ws);
      break;
    case 6:
      std::snprintf(buf, len,
                    "path=smallm_lds act_tiles=%d weight_tiles_per_wave=%d waves=%d steps_per_range=%d "
                    "k_ranges=%d group_blocks=%d grid=%lld prep=%s workspace=%zu",
                    p.mt, p.ns, p.waves, p.cnt, p.splits, p.gb, (long long)p.grid, p.prep ? "gather" : "none", ws);
      break;
    case 4:
      std::snprintf(buf, len,
                    "path=gemv_mfma fold_rows=%d waves=%d steps_per_wave=%d group_blocks=%d grid=%lld "
                    "prep=%s workspace=%zu",
                    p.fold_rows, p.waves, p.cnt, p.gb, (long long)p.grid, p.prep ? "gather" : "none", ws);
      break;
    case 5:
      std::snprintf(buf, len, "path=rows_dot2 rows_per_group=%d waves=%d grid=%lld prep=%s workspace=%zu",
                    p.rows_u, p.waves, (long long)p.grid, p.prep ? "gather" : "none", ws);
      break;
    default:
      std::snprintf(buf, len,
                    "path=gemm_mfma tile=%dx%d waves=%d group_blocks=%d tail_cols=%lld k_splits=%d grid=%lld "
                    "prep=%s workspace=%zu",
                    p.bm, p.bn, p.waves, p.gb, (long long)p.tail_n, p.splits, (long long)p.grid,
                    has_order ? "gather+reorder+groupsum" : "reorder+groupsum", ws);
  }
  return WOQ_OK;
}

}  // extern "C"
