// Tiled linear path (m > 16) and the activation pre-pass.
//
// Pre-pass: x' = x gathered through the act-order index when one is given
// (linnet docs "Quantization", section "Importing GPTQ and AWQ": the layer
// gathers its inputs first), optionally written in the slot order of the
// nibble unpacker with each row zero-padded to whole 128-input steps, plus the
// float32 sum of x' over every "piece": the part of a quantization group inside
// one 128-wide k step (the whole group for groups of at most 128 inputs).
// A second small pass lays the scales and zero points out per group as
// (scale, -(128 + zero)) float pairs, [K/G][N rounded up to 256].
//
// GEMM (linnet docs "Quantization", std.quant table, linear_int4_groups): a
// workgroup computes a BM x BN tile of y from 32 x 32 tiles of
// v_mfma_f32_32x32x16_bf16.  Large m takes 128 x 256 with 8 waves of 64 x 64
// (2 x 2 MFMA tiles); smaller m takes 128 x 64, 64 x 64 or 32 x 64 tiles
// (4, 4 and 2 waves) so that the grid still covers the chip.  Per 128-input
// step the workgroup streams the activation tile (BM x 256 bytes), the packed
// weight tile (BN x 64 bytes), the piece sums and the scale/zero pairs
// straight from memory into a ring of LDS stages (three, or two where three
// do not fit) with buffer-to-LDS loads, so the memory stream runs ahead
// without holding registers; one barrier per step hands a stage from the
// loads to the arithmetic.  Both tiles are stored XOR-swizzled so the
// reads of 8 neighbouring rows hit distinct banks.  Nibbles become bf16
// (128 + code) with one AND-OR per pair; each MFMA takes one dword of every
// lane's 16 loaded bytes (inputs u+32h+8b .. +8 of a 64-input unit u, h the
// lane half), which keeps every MFMA inside one group for groups of 64 and
// more; 32-input groups regroup the dwords between the lane halves with two
// v_permlane32_swap.  Per group piece the MFMA sums fold into float32
// accumulators as acc += scale * sum; the zero-point term
// -scale * (128 + zero) * piece_sum_of_x is an outer product and is added by
// float32 MFMAs (v_mfma_f32_32x32x2_f32), two pieces per instruction.
#include "woq_internal.h"
#include "mfma_common.h"


namespace woq {
namespace {

constexpr int kStepK = 128;
constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr uint32_t kOffsetOOB = 0x80000000u;   // a buffer offset no descriptor covers
constexpr uint32_t kSignFlip = 0x88888888u;    // two's complement nibble v -> unsigned v ^ 8 (zero point 8)

// One thread per 8 consecutive inputs of a row (16 bytes).  The lanes of one
// piece (piece/8 of them, consecutive) add their partial sums in a fixed
// shuffle tree, so the sums are the same on every run.  Rows from m to mpad
// only get zero sums; columns from k to kpad (the written row stride) get
// zeros.
struct PrepArgs {
  const uint16_t* x;
  const int32_t* order;
  int32_t m, k, kpad, permute;
  uint16_t* xg;
  float* xs;
  int64_t mpad;
};

// The grid-stride body, as workgroup `block` of `nblocks` (256 threads each).
template <int LP>   // lanes per piece: piece / 8
__device__ __forceinline__ void prep_body(const PrepArgs& a, int64_t block, int64_t nblocks) {
  const uint16_t* __restrict__ x = a.x;
  const int32_t* __restrict__ order = a.order;
  const int32_t m = a.m, k = a.k, kpad = a.kpad, permute = a.permute;
  uint16_t* __restrict__ xg = a.xg;
  float* __restrict__ xs = a.xs;
  const int64_t mpad = a.mpad;
  const int cpr = kpad / 8;                    // chunks per written row
  const int kc = k / 8;                        // chunks holding inputs
  const int64_t total = mpad * cpr;
  const int64_t stride = nblocks * 256;
  for (int64_t t = block * 256 + threadIdx.x; t < total; t += stride) {
    const int64_t row = t / cpr;
    const int col = (int)(t % cpr);
    u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
    if (row < m && col < kc) {
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
      *reinterpret_cast<u32x4_t*>(xg + row * kpad + col * 8) =
          permute ? __builtin_bit_cast(u32x4_t, pair_order(v)) : v;
    if (xs && col < kc && (col % LP) == 0) xs[(int64_t)(col / LP) * mpad + row] = sum;
  }
}

template <int LP>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a) {
  prep_body<LP>(a, blockIdx.x, gridDim.x);
}

// sz[g][c] = (scale[c][g], -(128 + zero[c][g])) for c < n, zeros up to npad.
// With signed codes the scale is float16 and the zero point 8 (the codes are
// read as v ^ 8); for MXFP4 (fmt 2) the entry is (2^(e - 127), 0) of the E8M0
// scale byte e.
struct SzArgs {
  const void* scale;
  const uint8_t* zero;
  int32_t n, ngroups, npad, fmt, row_scale, zp4;
  f32x2_t* sz;
};

__device__ __forceinline__ void sz_body(const SzArgs& a, int64_t block, int64_t nblocks) {
  const void* __restrict__ scale = a.scale;
  const uint8_t* __restrict__ zero = a.zero;
  const int32_t n = a.n, ngroups = a.ngroups, npad = a.npad, fmt = a.fmt, row_scale = a.row_scale, zp4 = a.zp4;
  f32x2_t* __restrict__ sz = a.sz;
  const int64_t total = (int64_t)ngroups * npad;
  const int64_t stride = nblocks * 256;
  for (int64_t t = block * 256 + threadIdx.x; t < total; t += stride) {
    const int64_t g = t / npad;
    const int c = (int)(t % npad);
    f32x2_t v = f32x2_t{0.f, 0.f};
    if (c < n) {
      const int64_t e = (int64_t)c * ngroups + g;
      if (fmt == kFmtMX) {
        const uint32_t eb = static_cast<const uint8_t*>(scale)[e];
        v = f32x2_t{__uint_as_float(eb == 0 ? 0x00400000u : eb << 23), 0.f};
      } else if (fmt == kFmtS16) {   // float16 per group, or one float32 per row (Int4Linear)
        const float sc = row_scale ? static_cast<const float*>(scale)[c]
                                   : (float)static_cast<const _Float16*>(scale)[e];
        v = f32x2_t{sc, -(kNibOffset + 8.0f)};
      } else {
        // packed zero points: group g in nibble g & 1 of byte g / 2 of the row
        const uint32_t zq = zp4 ? (zero[(int64_t)c * ((ngroups + 1) / 2) + g / 2] >> (4 * (g & 1))) & 15u
                                : zero[e];
        v = f32x2_t{static_cast<const float*>(scale)[e], -(kNibOffset + (float)zq)};
      }
    }
    sz[t] = v;
  }
}

// The activation pre-pass and the scale/zero table in one launch: workgroups
// below prep_blocks take the first, the rest the second.
template <int LP>
__global__ __launch_bounds__(256) void prep_sz_kernel(PrepArgs pa, SzArgs sa, int32_t prep_blocks) {
  if ((int)blockIdx.x < prep_blocks)
    prep_body<LP>(pa, blockIdx.x, prep_blocks);
  else
    sz_body(sa, (int64_t)blockIdx.x - prep_blocks, (int64_t)gridDim.x - prep_blocks);
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

// Split-K: y = sum over the K ranges of their float32 partials, in range
// order (the same result on every run), + bias, then y's type.  The slices
// are loaded kReduceBatch at a time before any is added, so a call waits for
// ceil(splits / kReduceBatch) memory round trips rather than one per range.
constexpr int kReduceBatch = 8;

__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int32_t splits,
                                                            int32_t m, int32_t n, const float* __restrict__ bias,
                                                            int32_t y_bf16, void* __restrict__ y) {
  const int64_t total = (int64_t)m * n;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
    float v = 0.f;
    for (int r0 = 0; r0 < splits; r0 += kReduceBatch) {
      float a[kReduceBatch];
#pragma unroll
      for (int j = 0; j < kReduceBatch; ++j) a[j] = r0 + j < splits ? part[(int64_t)(r0 + j) * total + t] : 0.f;
#pragma unroll
      for (int j = 0; j < kReduceBatch; ++j)
        if (r0 + j < splits) v = r0 + j == 0 ? a[j] : v + a[j];
    }
    if (bias) v += bias[t % n];
    if (y_bf16)
      reinterpret_cast<uint16_t*>(y)[t] = f32_to_bf16_bits(v);
    else
      reinterpret_cast<float*>(y)[t] = v;
  }
}

// The same, four consecutive outputs a thread (n a multiple of 4, so the four
// share a row; y aligned to four of its elements).
__global__ __launch_bounds__(256) void splitk_reduce4_kernel(const float* __restrict__ part, int32_t splits,
                                                             int32_t m, int32_t n, const float* __restrict__ bias,
                                                             int32_t y_bf16, void* __restrict__ y) {
  const int64_t total4 = (int64_t)m * n / 4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const f32x4_t* p4 = reinterpret_cast<const f32x4_t*>(part);
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total4; t += stride) {
    f32x4_t v = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // Each partial is read exactly once: non-temporal loads.
    for (int r0 = 0; r0 < splits; r0 += kReduceBatch) {
      f32x4_t a[kReduceBatch];
#pragma unroll
      for (int j = 0; j < kReduceBatch; ++j)
        a[j] = r0 + j < splits ? __builtin_nontemporal_load(p4 + (int64_t)(r0 + j) * total4 + t)
                               : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < kReduceBatch; ++j) {
        if (r0 + j >= splits) continue;
        if (r0 + j == 0) {
          v = a[j];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] += a[j][e];
        }
      }
    }
    if (bias) {
      const f32x4_t b = *reinterpret_cast<const f32x4_t*>(bias + (4 * t) % n);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += b[e];
    }
    if (y_bf16) {
      uint32_t lo = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
      uint32_t hi = (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
      reinterpret_cast<uint2*>(y)[t] = make_uint2(lo, hi);
    } else {
      reinterpret_cast<f32x4_t*>(y)[t] = v;
    }
  }
}

typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kJunk = 1024;                 // LDS that absorbs the loads of unused slots
constexpr int kNPad = 256;                  // column padding of the (scale, zero) table

// Workgroup tile: WM x WN waves, each holding MT x NT tiles of 32 x 32 outputs.
template <int WM_, int WN_, int MT_, int NT_>
struct Tile {
  static constexpr int WM = WM_, WN = WN_, MT = MT_, NT = NT_;
  static constexpr int kWaves = WM * WN;
  static constexpr int BM = 32 * MT * WM, BN = 32 * NT * WN;
  static constexpr int kABytes = BM * kStepK * 2;   // activation tile of one step, bf16
  static constexpr int kBBytes = BN * kStepK / 2;   // packed weight tile of one step
  static constexpr int kA = BM / 4;                 // 1 KB activation loads per stage
  static constexpr int kB = BN / 16;                // 1 KB weight loads per stage
  static constexpr int kAPer = (kA + kWaves - 1) / kWaves;
  static constexpr int kBPer = (kB + kWaves - 1) / kWaves;
  static constexpr int kSzParts = (BN + 127) / 128; // 1 KB (scale, zero) loads per piece
};

// s_waitcnt operand that waits until at most n vector-memory loads of this
// wave are outstanding (expcnt and lgkmcnt left at their maxima).
constexpr int wait_vmcnt(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, (int)kRsrcWord3);
}

// 16 bytes per lane from the buffer straight into LDS: lane l's bytes land at
// dst + 16 * l (dst is the same for the whole wave).  A device-only function:
// inside a kernel's lambdas the builtin keeps the host compiler from emitting
// the kernel's launch stub.
__device__ __forceinline__ void bload16_lds(__amdgpu_buffer_rsrc_t r, unsigned char* dst, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, off, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// float32 32x32x2: lane l supplies row (or column) l % 32 of input l / 32
__device__ __forceinline__ f32x16_t mfma32f(float a, float b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

struct GemmParams {
  const uint16_t* xp;     // pair-ordered activations [M, kpad], zero past K
  const uint8_t* packed;  // [N, K/2], or prepared blocks
  const float* xs;        // piece sums [K/piece][mpad]
  const f32x2_t* sz;      // (scale, -(128 + zero)) [K/G][npad]
  const float* bias;
  void* y;
  int32_t m, n, k, kpad, group, y_bf16;
  int64_t mpad;
  int32_t npad, ngroups, npieces;
  int32_t tiles_m, tiles_n;
  int32_t n_base, n_cols; // this launch computes output columns [n_base, n_base + n_cols)
  int32_t prepared;       // 1: packed holds prepared 1 KB blocks
  int32_t vec_out;        // 1: y is 16-byte aligned and its rows are whole 16-byte chunks
  int32_t sym16;          // 1: signed two's complement codes (float16 scales in the table)
  int32_t mx;             // 1: MXFP4 (E2M1 codes; the table holds (2^(e - 127), 0) per block)
  int32_t sps;            // 128-input steps per K range (split-K), or nsteps
  float* part;            // split-K: workgroup (tile, r) writes its float32 partial tile, no
                          // bias, to part + r * M * N; null: the whole sum goes to y
};

// Tl: workgroup tile; GB: 32-input blocks per group piece inside a step (1, 2
// or 4); S: LDS stages; S16: signed two's complement codes (read as v ^ 8,
// one XOR per dword; the scale table already holds zero point 8).
template <class Tl, int GB, int S, int FMT>
__global__ __launch_bounds__(64 * Tl::kWaves) void gemm_kernel(GemmParams p) {
  constexpr bool S16 = FMT == kFmtS16, MX = FMT == kFmtMX;
  static_assert(!MX || GB == 1, "MXFP4 blocks hold 32 inputs");
  constexpr int MT = Tl::MT, NT = Tl::NT, kWaves = Tl::kWaves;
  constexpr int BM = Tl::BM, BN = Tl::BN;
  constexpr int kABytes = Tl::kABytes, kBBytes = Tl::kBBytes;
  constexpr int NP = 4 / GB;                    // group pieces per step
  constexpr int kPiece = 32 * GB;               // inputs per piece
  constexpr int kXsOff = kABytes + kBBytes;     // NP x 1 KB of piece sums (512 B used each)
  constexpr int kSzOff = kXsOff + NP * 1024;    // NP x kSzParts KB of (scale, -(128 + zero)) pairs
  constexpr int kSzStride = Tl::kSzParts * 1024;
  constexpr int kStage = kSzOff + NP * kSzStride;
  constexpr int kMetaTotal = NP * (1 + Tl::kSzParts);
  constexpr int kMeta = (kMetaTotal + kWaves - 1) / kWaves;   // metadata loads per wave and stage
  constexpr int kLoads = Tl::kAPer + Tl::kBPer + kMeta;      // loads per wave and stage
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  unsigned char* const junk = lds + S * kStage;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int h = lane >> 5, j = lane & 31;
  const int wm = wave / Tl::WN, wn = wave % Tl::WN;
  const int K = p.k, M = p.m, N = p.n;
  const uint32_t row_bytes = (uint32_t)K / 2;

  // Workgroup r * tiles + t computes tile t over K range r (steps [s0, s1)).
  // Workgroups are dealt to the 8 XCDs round robin; renumber so that the
  // workgroups of one XCD cover neighbouring tiles that share weight columns.
  const int nwg = p.tiles_m * p.tiles_n;
  const int split = (int)blockIdx.x / nwg;
  int bid = (int)blockIdx.x - split * nwg;
  const int full = (nwg / 8) * 8;
  if (bid < full) bid = (bid % 8) * (full / 8) + bid / 8;
  const int tm = bid % p.tiles_m, tn = bid / p.tiles_m;
  const int m0 = tm * BM, n0 = p.n_base + tn * BN;
  const int nsteps = (K + kStepK - 1) / kStepK;
  const int s0 = split * p.sps;
  const int s1 = min(nsteps, s0 + p.sps);

  // Weights: canonical rows, or prepared 1 KB blocks (16 rows x one step,
  // tile-major; slot l of a block holds row l % 16, quarter l / 16 of the step).
  const bool prep = p.prepared != 0;   // uniform
  const int ptiles = min(BN / 16, (N + 15) / 16 - n0 / 16);
  const int gshift = __builtin_ctz((unsigned)p.group);   // groups are powers of two

  // ---- one stage of loads: this wave's share, the same count for every wave --
  // Activation tile: BM/4 loads of 4 rows x 256 bytes; lane l of load a fills
  // LDS row 4a + l/16, position l%16 with chunk (l%16) ^ (row & 7) of that row.
  // Weight tile: BN/16 loads of 16 rows x 64 bytes; position l%4 of row
  // 16b + l/4 holds chunk (l%4) ^ ((row >> 1) & 3).  Metadata: per piece one
  // load of 128 piece sums (lanes 0..31) and 128 (scale, zero) pairs per load.
  // Load slots past the tile's count read nothing into the junk block.
  //
  // A lane's byte offsets do not change from step to step: each step moves
  // the base of its buffer descriptors instead and shrinks their size to
  // what is left past the base, so rows past M or N, pieces and groups past K
  // and steps past the range (size 0) still read zero.  The offsets below
  // are relative to the step's bases; kOffsetOOB marks a slot with nothing
  // to load.
  uint32_t voa[Tl::kAPer], vob[Tl::kBPer], vom[kMeta];
#pragma unroll
  for (int u = 0; u < Tl::kAPer; ++u) {
    const int a = wave * Tl::kAPer + u;       // uniform
    const int row = 4 * a + (lane >> 4);
    const int c = (lane & 15) ^ (row & 7);
    voa[u] = a < Tl::kA ? ((uint32_t)row * (uint32_t)p.kpad + (uint32_t)(8 * c)) * 2u : kOffsetOOB;
  }
#pragma unroll
  for (int u = 0; u < Tl::kBPer; ++u) {
    const int b = wave * Tl::kBPer + u;       // uniform
    const int row = 16 * b + (lane >> 2);
    const int c = (lane & 3) ^ ((row >> 1) & 3);
    vob[u] = b >= Tl::kB ? kOffsetOOB
             : prep      ? (uint32_t)(b * nsteps) * 1024u + 16u * (uint32_t)(16 * c + (lane >> 2))
                         : (uint32_t)row * row_bytes + (uint32_t)(16 * c);
  }
#pragma unroll
  for (int u = 0; u < kMeta; ++u) {
    const int mi = wave * kMeta + u;          // uniform
    const int pc = mi / (1 + Tl::kSzParts), part = mi - (1 + Tl::kSzParts) * pc;
    uint32_t off = kOffsetOOB;
    if (pc < NP && part == 0) {               // piece pc of the step: its sums for rows m0 + 4 lane ..
      if (lane < 32) off = (uint32_t)(((int64_t)pc * p.mpad + m0 + 4 * lane) * 4);
    } else if (pc < NP) {                     // its group: pc pieces on when groups are one piece
      const int pg = (pc * kPiece) >> gshift;
      off = (uint32_t)(((int64_t)pg * p.npad + n0 + 128 * (part - 1) + 2 * lane) * 8);
    }
    vom[u] = off;
  }
  const uint16_t* const xbase = p.xp + (int64_t)m0 * p.kpad;
  const uint32_t xbytes = (uint32_t)min(BM, M - m0) * (uint32_t)p.kpad * 2u;
  const uint8_t* const wbase = prep ? p.packed + (int64_t)(n0 / 16) * nsteps * 1024 : p.packed + (int64_t)n0 * row_bytes;
  const uint32_t wbytes = prep ? (uint32_t)(ptiles * nsteps) * 1024u : (uint32_t)min(BN, N - n0) * row_bytes;
  const bool ktail = !prep && K % kStepK != 0;   // canonical rows whose last step is partial
  auto issue_stage = [&](int slot, int step) {
    unsigned char* st = lds + slot * kStage;
    const int k0 = step * kStepK;
    const bool live = step < s1;              // uniform
    const __amdgpu_buffer_rsrc_t ra = rsrc(xbase + k0, live ? xbytes - (uint32_t)k0 * 2u : 0u);
    const uint32_t wstep = prep ? (uint32_t)step * 1024u : (uint32_t)k0 / 2u;
    // The last step of canonical rows with a partial step keeps the rows'
    // own ends: its lanes past the end of a row read zero, not the next row.
    const bool wlast = ktail && k0 + kStepK > K;   // uniform
    const __amdgpu_buffer_rsrc_t rb = rsrc(wbase + (wlast ? 0u : wstep), !live ? 0u : wlast ? wbytes : wbytes - wstep);
    const int pi0 = k0 / kPiece, g0 = k0 >> gshift;
    const __amdgpu_buffer_rsrc_t rx =
        rsrc(p.xs + (int64_t)pi0 * p.mpad, live && !MX && pi0 < p.npieces ? (uint32_t)((int64_t)(p.npieces - pi0) * p.mpad * 4) : 0u);
    const __amdgpu_buffer_rsrc_t rz =
        rsrc(p.sz + (int64_t)g0 * p.npad, live && g0 < p.ngroups ? (uint32_t)((int64_t)(p.ngroups - g0) * p.npad * 8) : 0u);
#pragma unroll
    for (int u = 0; u < Tl::kAPer; ++u) {
      const int a = wave * Tl::kAPer + u;     // uniform
      bload16_lds(ra, a < Tl::kA ? st + a * 1024 : junk, voa[u]);
    }
#pragma unroll
    for (int u = 0; u < Tl::kBPer; ++u) {
      const int b = wave * Tl::kBPer + u;     // uniform
      uint32_t off = vob[u];
      if (wlast) {
        const int c = (lane & 3) ^ (((16 * b + (lane >> 2)) >> 1) & 3);
        off = (uint32_t)(k0 / 2 + 16 * c) < row_bytes ? off + (uint32_t)k0 / 2u : kOffsetOOB;
      }
      bload16_lds(rb, b < Tl::kB ? st + kABytes + b * 1024 : junk, off);
    }
#pragma unroll
    for (int u = 0; u < kMeta; ++u) {
      const int mi = wave * kMeta + u;       // uniform
      const int pc = mi / (1 + Tl::kSzParts), part = mi - (1 + Tl::kSzParts) * pc;
      unsigned char* dst = pc >= NP ? junk : part == 0 ? st + kXsOff + pc * 1024 : st + kSzOff + pc * kSzStride + (part - 1) * 1024;
      bload16_lds(pc < NP && part == 0 ? rx : rz, dst, vom[u]);
    }
  };

  f32x16_t acc[MT][NT];
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
  const f32x16_t zero16 = {};

  const uint32_t nib_offset = vgpr_copy(kBf16Offset2);
  // this lane's activation row (A operand) and weight row (B operand) per tile
  int arow[MT], brow[NT];
#pragma unroll
  for (int t = 0; t < MT; ++t) arow[t] = 32 * MT * wm + 32 * t + j;
#pragma unroll
  for (int t = 0; t < NT; ++t) brow[t] = 32 * NT * wn + 32 * t + j;
  // This lane's LDS offsets inside a stage, so that every read of a step adds
  // only a constant to one of them.  Activation fragment (unit L, dword b,
  // tile mt): row arow[mt] = arow[0] + 32 mt, chunk (8 L + cin) ^ (row & 7) =
  // 8 L + (cin ^ (j & 7)), cin the 8-input chunk that matches dword b of this
  // lane half.  Weight dwords (unit L, tile nt): row brow[0] + 32 nt, chunk
  // (2 L + h) ^ ((j >> 1) & 3).
  int aofs[4], wofs[2];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int cin = GB == 1 && !MX ? 4 * (b >> 1) + 2 * h + (b & 1) : 4 * h + b;
    aofs[b] = arow[0] * 256 + 16 * (cin ^ (j & 7));
  }
#pragma unroll
  for (int L = 0; L < 2; ++L) wofs[L] = brow[0] * 64 + 16 * ((2 * L + h) ^ ((j >> 1) & 3));

  // zero-point operands carried from an even step to the next (one piece per step)
  float zpa[MT] = {}, zpb[NT] = {};
  // MFMA sums of the current group piece, and the fold of the last finished
  // piece still to be added (its scales)
  f32x16_t cg[MT][NT];
  float fold_sv[NT] = {};
  bool fold_pending = false;

  auto compute = [&](int slot, int step) {
    const unsigned char* st = lds + slot * kStage;
    const int k0 = step * kStepK;
    // The zero-point part of a piece, -scale * (128 + zero) * piece_sum_of_x,
    // is an outer product of a column factor and a row factor: it goes
    // through the matrix unit, two pieces per float32 MFMA.  Operands for
    // piece pc: row factor -sum_of_x of this lane's activation row, column
    // factor scale * (128 + zero) of its weight row (zero past the inputs).
    auto zp_operands = [&](int pc, float (&a)[MT], float (&b)[NT]) {
      const bool in = k0 + pc * kPiece < K;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const float xv = *reinterpret_cast<const float*>(st + kXsOff + pc * 1024 + arow[mt] * 4);
        a[mt] = in ? -xv : 0.f;
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const f32x2_t v = *reinterpret_cast<const f32x2_t*>(st + kSzOff + pc * kSzStride + brow[nt] * 8);
        b[nt] = -v[0] * v[1];
      }
    };
    auto correct = [&]() {
      if constexpr (NP == 1) {
        // One piece per step: lane half h carries the pieces of steps with
        // parity h; the MFMA runs after every odd step.
        float a[MT], b[NT];
        zp_operands(0, a, b);
        const bool mine = h == (step & 1);
#pragma unroll
        for (int t = 0; t < MT; ++t) zpa[t] = mine ? a[t] : zpa[t];
#pragma unroll
        for (int t = 0; t < NT; ++t) zpb[t] = mine ? b[t] : zpb[t];
        if (step & 1) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mfma32f(zpa[mt], zpb[nt], acc[mt][nt]);
        }
      } else {
#pragma unroll
        for (int pp = 0; pp < NP; pp += 2) {
          float a[MT], b[NT];
          zp_operands(pp + h, a, b);       // lane half h: piece pp + h
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mfma32f(a[mt], b[nt], acc[mt][nt]);
        }
      }
    };
    // All weight bytes of the step, then the activation fragments one 16-input
    // block ahead of the MFMAs that use them.
    uint32_t bd[2][NT][4];
#pragma unroll
    for (int L = 0; L < 2; ++L)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        u32x4_t v = *reinterpret_cast<const u32x4_t*>(st + kABytes + wofs[L] + 2048 * nt);
        if constexpr (S16) v ^= u32x4_t{kSignFlip, kSignFlip, kSignFlip, kSignFlip};
        bd[L][nt][0] = v[0]; bd[L][nt][1] = v[1]; bd[L][nt][2] = v[2]; bd[L][nt][3] = v[3];
        if constexpr (GB == 1 && !MX) {
          // Regroup for 32-input groups: the lower lanes keep their inputs
          // 0..15 and take the upper lanes' 32..47; the upper lanes end with
          // 16..31 and 48..63.  Dwords 0, 1 then lie in the unit's first
          // group on both halves, dwords 2, 3 in its second.
          auto s0 = __builtin_amdgcn_permlane32_swap(bd[L][nt][0], bd[L][nt][2], false, false);
          bd[L][nt][0] = s0[0]; bd[L][nt][2] = s0[1];
          auto s1 = __builtin_amdgcn_permlane32_swap(bd[L][nt][1], bd[L][nt][3], false, false);
          bd[L][nt][1] = s1[0]; bd[L][nt][3] = s1[1];
        }
      }
    auto load_af = [&](int blk, bf16x8_t (&af)[MT]) {
      const int L = blk >> 2, b = blk & 3;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        af[mt] = *reinterpret_cast<const bf16x8_t*>(st + aofs[b] + 128 * L + 8192 * mt);
    };
    // Fold of one group piece, acc += scale * sum (the zero-point part is added
    // by correct()), deferred to the first block of the next piece: there the
    // fold of each 32x32 tile sits right before that tile's first MFMA of the
    // new piece, so the matrix unit works on one tile while the vector unit
    // folds the next.  The scales of a finished piece are read at its end (the
    // stage may be refilled before the next piece starts).
    auto fold_tile = [&](int mt, int nt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mt][nt][r] = fmaf(fold_sv[nt], cg[mt][nt][r], acc[mt][nt][r]);
    };
    bf16x8_t afc[MT], afn[MT];
    if constexpr (MX) {
      // MXFP4: lane half h of 64-input unit L holds block 2L + h of its row,
      // converted with that block's scale into exact bf16 weights; the MFMAs
      // accumulate straight into the outputs (no fold, no zero point).
      float xsc[2][NT];
#pragma unroll
      for (int L = 0; L < 2; ++L)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          xsc[L][nt] = *reinterpret_cast<const float*>(st + kSzOff + (2 * L + h) * kSzStride + brow[nt] * 8);
      __builtin_amdgcn_s_setprio(1);
      load_af(0, afc);
#pragma unroll
      for (int blk = 0; blk < 8; ++blk) {
        const int L = blk >> 2, b = blk & 3;
        if (blk + 1 < 8) load_af(blk + 1, afn);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const bf16x8_t bf = fp4x8_to_bf16(bd[L][nt][b], xsc[L][nt]);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[mt][nt] = mfma32(afc[mt], bf, acc[mt][nt]);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) afc[mt] = afn[mt];
      }
      __builtin_amdgcn_s_setprio(0);
      return;
    }
    // The two waves of a SIMD leave the barrier together; raising this wave's
    // priority for its MFMA phase lets one of them run ahead, so that one
    // folds (VALU) while the other keeps the matrix unit busy.
    // In 8-wave tiles waves w and w + 4 share a SIMD; the second tile row's
    // waves get the higher priority: the first row's are older and win
    // equal-priority issue, and otherwise finish their step first and wait at
    // the next barrier (measured: 1-2 % faster at groups of 128, 4 % at 32).
    if (kWaves == 8 && wm) __builtin_amdgcn_s_setprio(2); else __builtin_amdgcn_s_setprio(1);
    load_af(0, afc);
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
      const int L = blk >> 2, b = blk & 3;
      constexpr int kBlocksPerPiece = 8 / NP;
      const bool first = blk % kBlocksPerPiece == 0;      // a new piece starts
      const bool folding = first && fold_pending;          // uniform
      if (blk + 1 < 8) load_af(blk + 1, afn);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const bf16x8_t bf = unpack_codes(bd[L][nt][b], kNibPairMask, nib_offset);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if (folding) fold_tile(mt, nt);
          cg[mt][nt] = mfma32(afc[mt], bf, first ? zero16 : cg[mt][nt]);
        }
      }
      if (blk % kBlocksPerPiece == kBlocksPerPiece - 1) {
        // this piece's fold is pending (pieces past the end of the inputs add nothing)
        const int pc = blk / kBlocksPerPiece;
        fold_pending = k0 + pc * kPiece < K;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          fold_sv[nt] = *reinterpret_cast<const float*>(st + kSzOff + pc * kSzStride + brow[nt] * 8);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) afc[mt] = afn[mt];
    }
    __builtin_amdgcn_s_setprio(0);
    correct();
  };

  // ---- the ring: stage i lives in slot i % S --------------------------------
#pragma unroll
  for (int s = 0; s < S; ++s) issue_stage(s, s0 + s);
  int slot = 0;
  for (int i = s0; i < s1; ++i) {
    // this wave's loads of stage i have landed ...
    if (i == s0)
      __builtin_amdgcn_s_waitcnt(wait_vmcnt((S - 1) * kLoads));
    else
      __builtin_amdgcn_s_waitcnt(wait_vmcnt((S - 2) * kLoads));
    // ... and everyone's have; everyone has also finished step i - 1, so its
    // slot takes step i - 1 + S.  A plain barrier: a __syncthreads fence would
    // also wait for the loads still streaming into the other stages.  The empty
    // asm statements keep the compiler from moving LDS accesses across it.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (i > s0) issue_stage(slot == 0 ? S - 1 : slot - 1, i - 1 + S);
    compute(slot, i);
    slot = slot == S - 1 ? 0 : slot + 1;
  }
  __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
  if (fold_pending) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mt][nt][r] = fmaf(fold_sv[nt], cg[mt][nt][r], acc[mt][nt][r]);
  }
  if constexpr (4 / GB == 1) {
    if (s1 & 1) {   // the last (even) step's zero-point term is still pending
#pragma unroll
      for (int t = 0; t < MT; ++t) zpa[t] = h ? 0.f : zpa[t];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mfma32f(zpa[mt], zpb[nt], acc[mt][nt]);
    }
  }

  // Epilogue.  A lane of a 32 x 32 MFMA tile holds 16 rows of one column, so
  // storing straight from the accumulators writes 2 bytes (or 4) per lane.
  // Where the tile fits in the LDS ring (free once every wave is past its
  // last step) it is staged there row-major and leaves in 16-byte chunks.
  constexpr int kEsz = 4;                                  // bytes per staged float32
  constexpr int kOutStride = BN * kEsz + 32;               // padded row: the lane halves' rows 4 apart hit other banks
  constexpr bool kStaged = BM * kOutStride <= S * kStage;
  // A K range of a split call leaves its float32 partial tile, without the
  // bias, in its own slice of the partial buffer.
  float* const part = p.part ? p.part + (int64_t)split * M * N : nullptr;
  void* const yout = part ? static_cast<void*>(part) : p.y;
  const int ybf = part ? 0 : p.y_bf16;
  const float* const bias = part ? nullptr : p.bias;
  const bool vec = part ? N % 4 == 0 : p.vec_out != 0;
  if (kStaged && vec) {
    __syncthreads();
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int n = n0 + brow[nt];
        const float b = bias && n < N ? bias[n] : 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 32 * MT * wm + 32 * mt + 8 * (r >> 2) + 4 * h + (r & 3);
          *reinterpret_cast<float*>(lds + row * kOutStride + brow[nt] * kEsz) = acc[mt][nt][r] + b;
        }
      }
    __syncthreads();
    // 16-byte output chunks: 8 bf16 or 4 float32 columns; N is a whole number
    // of chunks, so a chunk is wholly inside or wholly past the last column.
    const int ecols = ybf ? 8 : 4;
    const int cpr = BN / ecols;
    for (int c = tid; c < BM * cpr; c += 64 * kWaves) {
      const int row = c / cpr, col = (c - row * cpr) * ecols;
      const int m = m0 + row, n = n0 + col;
      if (m >= M || n >= N) continue;
      const float* src = reinterpret_cast<const float*>(lds + row * kOutStride + col * kEsz);
      if (ybf) {
        const f32x4_t lo = *reinterpret_cast<const f32x4_t*>(src);
        const f32x4_t hi = *reinterpret_cast<const f32x4_t*>(src + 4);
        u32x4_t o;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          o[e] = (uint32_t)f32_to_bf16_bits(lo[2 * e]) | ((uint32_t)f32_to_bf16_bits(lo[2 * e + 1]) << 16);
          o[e + 2] = (uint32_t)f32_to_bf16_bits(hi[2 * e]) | ((uint32_t)f32_to_bf16_bits(hi[2 * e + 1]) << 16);
        }
        *reinterpret_cast<u32x4_t*>(reinterpret_cast<uint16_t*>(yout) + (int64_t)m * N + n) = o;
      } else {
        *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(yout) + (int64_t)m * N + n) =
            *reinterpret_cast<const f32x4_t*>(src);
      }
    }
    return;
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = n0 + brow[nt];
      if (n >= N) continue;
      const float b = bias ? bias[n] : 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + 32 * MT * wm + 32 * mt + 8 * (r >> 2) + 4 * h + (r & 3);
        if (m < M) {
          const float v = acc[mt][nt][r] + b;
          if (ybf)
            reinterpret_cast<uint16_t*>(yout)[(int64_t)m * N + n] = f32_to_bf16_bits(v);
          else
            reinterpret_cast<float*>(yout)[(int64_t)m * N + n] = v;
        }
      }
    }
}

template <class Tl, int GB, int S>
size_t gemm_lds_bytes() {
  constexpr int NP = 4 / GB;
  return (size_t)S * (Tl::kABytes + Tl::kBBytes + NP * 1024 + NP * Tl::kSzParts * 1024) + kJunk;
}

template <class Tl, int GB, int S, int FMT>
int32_t launch_gemm_t(GemmParams gp, hipStream_t stream) {
  auto kern = gemm_kernel<Tl, GB, S, FMT>;
  const size_t lds = gemm_lds_bytes<Tl, GB, S>();
  static std::atomic<uint64_t> raised{0};   // per instantiation, one bit per device
  if (const int32_t st = raise_lds_limit(reinterpret_cast<const void*>(kern), (int)lds, raised); st != WOQ_OK)
    return st;
  gp.tiles_m = (gp.m + Tl::BM - 1) / Tl::BM;
  gp.tiles_n = (gp.n_cols + Tl::BN - 1) / Tl::BN;
  const int nsteps = (gp.k + kStepK - 1) / kStepK;
  const int splits = (nsteps + gp.sps - 1) / gp.sps;
  hipLaunchKernelGGL(kern, dim3((unsigned)(gp.tiles_m * gp.tiles_n * splits)), dim3(64 * Tl::kWaves), lds,
                     stream, gp);
  return hip_status(hipGetLastError());
}

// Stages in the LDS ring: three (two steps of loads ahead of the arithmetic)
// where they fit in one CU's LDS, else two.  Deeper rings measured slower on
// the narrow tiles: they cost workgroups per CU.
template <class Tl, int GB>
constexpr int gemm_stages() {
  constexpr int NP = 4 / GB;
  constexpr int stage = Tl::kABytes + Tl::kBBytes + NP * 1024 + NP * Tl::kSzParts * 1024;
  return 3 * stage + kJunk <= 160 * 1024 ? 3 : 2;
}

template <class Tl, int FMT>
int32_t launch_gemm_s(const GemmParams& gp, int gb, hipStream_t stream) {
  switch (gb) {
    case 1: return launch_gemm_t<Tl, 1, gemm_stages<Tl, 1>(), FMT>(gp, stream);
    case 2: return launch_gemm_t<Tl, 2, gemm_stages<Tl, 2>(), FMT>(gp, stream);
    case 4: return launch_gemm_t<Tl, 4, gemm_stages<Tl, 4>(), FMT>(gp, stream);
    default: return WOQ_EUNSUPPORTED;
  }
}

template <class Tl>
int32_t launch_gemm_gb(const GemmParams& gp, int gb, hipStream_t stream) {
  if (gp.mx) return gb == 1 ? launch_gemm_t<Tl, 1, gemm_stages<Tl, 1>(), kFmtMX>(gp, stream) : WOQ_EUNSUPPORTED;
  return gp.sym16 ? launch_gemm_s<Tl, kFmtS16>(gp, gb, stream) : launch_gemm_s<Tl, kFmtU4>(gp, gb, stream);
}

}  // namespace

int32_t launch_prep(const uint16_t* x, const int32_t* order, int32_t m, int32_t k, int32_t kpad,
                    int32_t group, int32_t permute, uint16_t* xg, float* xs, int64_t mpad,
                    hipStream_t stream) {
  const int32_t piece = group < kStepK ? group : kStepK;
  const int64_t total = mpad * (kpad / 8);
  if (total == 0) return WOQ_OK;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  const PrepArgs pa{x, order, m, k, kpad, permute, xg, xs, mpad};
  switch (piece / 8) {
    case 4: hipLaunchKernelGGL(prep_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, stream, pa); break;
    case 8: hipLaunchKernelGGL(prep_kernel<8>, dim3((unsigned)blocks), dim3(256), 0, stream, pa); break;
    case 16: hipLaunchKernelGGL(prep_kernel<16>, dim3((unsigned)blocks), dim3(256), 0, stream, pa); break;
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

size_t gemm_sz_bytes(int64_t n, int64_t k, int32_t group) {
  const int64_t npad = (n + kNPad - 1) / kNPad * kNPad;
  return (size_t)(k / group) * (size_t)npad * 8;
}

namespace {

int32_t launch_gemm_tiles(const LinearArgs& a, const LinearPlan& pl, const GemmParams& gp, hipStream_t stream) {
  // Tile by the number of activation rows: small M takes narrow tiles so the
  // grid still covers the chip.
  switch (pl.bm) {
    case 32: return launch_gemm_gb<Tile<1, 2, 1, 1>>(gp, pl.gb, stream);    // 32 x 64
    case 64: return launch_gemm_gb<Tile<2, 2, 1, 1>>(gp, pl.gb, stream);    // 64 x 64
    case 128:
      if (pl.bn == 64) return launch_gemm_gb<Tile<2, 2, 2, 1>>(gp, pl.gb, stream);   // 128 x 64
      if (pl.bn == 128) return launch_gemm_gb<Tile<2, 2, 2, 2>>(gp, pl.gb, stream);  // 128 x 128
      if (pl.tail_n > 0) {
        // columns before the tail in 128 x 256 tiles, the tail in 64 x 256
        GemmParams head = gp, tail = gp;
        head.n_cols = (int32_t)(a.n - pl.tail_n);
        tail.n_base = head.n_cols;
        tail.n_cols = (int32_t)pl.tail_n;
        const int32_t st = launch_gemm_gb<Tile<2, 4, 2, 2>>(head, pl.gb, stream);
        if (st != WOQ_OK) return st;
        return launch_gemm_gb<Tile<2, 4, 1, 2>>(tail, pl.gb, stream);                // 64 x 256
      }
      return launch_gemm_gb<Tile<2, 4, 2, 2>>(gp, pl.gb, stream);                    // 128 x 256
    default: return WOQ_EUNSUPPORTED;
  }
}

}  // namespace

namespace {

SzArgs sz_args(const LinearArgs& a, int32_t ngroups, int32_t npad, void* sz_ws) {
  return SzArgs{a.mx ? static_cast<const void*>(a.scale8)
                     : a.sym16 && !a.row_scale ? static_cast<const void*>(a.scale16)
                                               : static_cast<const void*>(a.scale),
                a.zero, a.n, ngroups, npad, a.mx ? kFmtMX : a.sym16 ? kFmtS16 : kFmtU4, a.row_scale, a.zp4,
                static_cast<f32x2_t*>(sz_ws)};
}

}  // namespace

int32_t launch_gemm_prep(const LinearArgs& a, const int32_t* order, uint16_t* xg, float* xs, void* sz_ws,
                         hipStream_t stream) {
  const int32_t ngroups = a.k / a.group;
  const int32_t npad = (a.n + kNPad - 1) / kNPad * kNPad;
  const int32_t piece = a.group < kStepK ? a.group : kStepK;
  const int64_t ptotal = a.mpad * (a.kpad / 8);
  const int64_t stotal = (int64_t)ngroups * npad;
  const int64_t pblocks = std::min<int64_t>((ptotal + 255) / 256, 65536);
  const int64_t sblocks = std::min<int64_t>((stotal + 255) / 256, 65536);
  if (pblocks + sblocks == 0) return WOQ_OK;
  // MXFP4 weights decode in natural input order and need no piece sums
  const PrepArgs pa{a.x, order, a.m, a.k, a.kpad, a.mx ? 0 : 1, xg, a.mx ? nullptr : xs, a.mpad};
  const SzArgs sa = sz_args(a, ngroups, npad, sz_ws);
  const dim3 grid((unsigned)(pblocks + sblocks)), block(256);
  switch (piece / 8) {
    case 4: hipLaunchKernelGGL(prep_sz_kernel<4>, grid, block, 0, stream, pa, sa, (int32_t)pblocks); break;
    case 8: hipLaunchKernelGGL(prep_sz_kernel<8>, grid, block, 0, stream, pa, sa, (int32_t)pblocks); break;
    case 16: hipLaunchKernelGGL(prep_sz_kernel<16>, grid, block, 0, stream, pa, sa, (int32_t)pblocks); break;
    default: return WOQ_EUNSUPPORTED;
  }
  return hip_status(hipGetLastError());
}

int32_t launch_gemm(const LinearArgs& a, const LinearPlan& pl, void* sz_ws, hipStream_t stream) {
  const int32_t ngroups = a.k / a.group;
  const int32_t npad = (a.n + kNPad - 1) / kNPad * kNPad;
  const int32_t piece = a.group < kStepK ? a.group : kStepK;
  const GemmParams gp{a.x, a.packed, a.xs, static_cast<const f32x2_t*>(sz_ws), a.bias, a.y,
                      a.m, a.n, a.k, a.kpad, a.group, a.y_bf16, a.mpad, npad, ngroups, a.k / piece,
                      0, 0, 0, a.n, a.prepared,
                      (reinterpret_cast<uintptr_t>(a.y) % 16 == 0 && a.n % (a.y_bf16 ? 8 : 4) == 0) ? 1 : 0,
                      a.sym16, a.mx, pl.splits > 1 ? pl.sps : (a.k + kStepK - 1) / kStepK,
                      pl.splits > 1 ? a.part : nullptr};
  const int32_t st = launch_gemm_tiles(a, pl, gp, stream);
  if (st != WOQ_OK || pl.splits <= 1) return st;
  return launch_splitk_reduce(a.part, pl.splits, a.m, a.n, a.bias, a.y_bf16, a.y, stream);
}

int32_t launch_splitk_reduce(const float* part, int32_t splits, int32_t m, int32_t n, const float* bias,
                             int32_t y_bf16, void* y, hipStream_t stream) {
  const int64_t total = (int64_t)m * n;
  const bool vec = n % 4 == 0 && aligned(part, 16) && aligned(y, y_bf16 ? 8 : 16) && (!bias || aligned(bias, 16));
  int64_t blocks = ((vec ? total / 4 : total) + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (vec)
    hipLaunchKernelGGL(splitk_reduce4_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, part, splits, m, n,
                       bias, y_bf16, y);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, part, splits, m, n,
                       bias, y_bf16, y);
  return hip_status(hipGetLastError());
}

}  // namespace woq
