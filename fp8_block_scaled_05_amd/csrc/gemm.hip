// Block-scaled FP8 GEMM (dense and grouped) for gfx950.
//
// Method: codingmall.com knowledge-base article on FP8 precision in
// DeepSeek-V3 training, section "Ökad ackumuleringsprecision": the matrix
// cores accumulate FP8 products with limited precision, so partial results
// are promoted into FP32 registers at fixed intervals.  With the 1x128 /
// 128x128 scaling of "Finkornig kvantisering" the scales are constant over
// each 128-deep K block, so the interval is one K block:
//     acc[m,n] += (sa[m,kb] * sb[n,kb]) * P_kb[m,n]
// where P_kb is the product of the E4M3 codes over the block.
//
// The same limitation exists on gfx950.  Its FP8 matrix instructions
// (v_mfma_*_f8f6f4 and v_mfma_*_fp8_fp8) add products in groups of 8
// consecutive K, keeping only the bits down to 2^-13 of the group's largest
// product and truncating the rest; the groups are then combined in FP32.
// That is about 14 significant bits - short of the 2e-5 * sum|a*b| accuracy
// asked of the GEMM on realistic data.  The f16 and bf16 matrix instructions
// accumulate exact products in FP32, and every E4M3 value is exact in f16.
// Two kernels therefore share everything but the block product:
//
//  * FP8BS_ACCUM_FP32 (default): E4M3 tiles are loaded from HBM (1 byte per
//    element), widened to f16 while being staged into LDS (one
//    v_cvt_scalef32_pk_f16_fp8 per two codes, exact), and multiplied with
//    v_mfma_f32_32x32x16_f16, eight per 128-deep block, chained in FP32.
//  * FP8BS_ACCUM_FP8_MFMA: one v_mfma_f32_16x16x128_f8f6f4 per 16x16 output
//    sub-tile and K block, straight from E4M3 tiles in LDS; twice the peak
//    rate, with the accumulation described above.
//
// Common design (one workgroup = 256 threads = 4 waves, output tile 128 x 128,
// each wave a 64 x 64 quadrant):
//  * the next K block's global loads are in flight while the current block
//    is multiplied; LDS is double-buffered, one barrier per block;
//  * the promotion is one FP32 FMA per output element per K block; the
//    scale product sa*sb is formed once per row (block128 B scales) or per
//    element (per-row B scales of the weight-gradient GEMM);
//  * workgroups are renumbered so that each XCD (which has its own L2) gets
//    a contiguous range of tiles, walked in groups of 8 M tiles so that a
//    range shares A rows and B rows in that L2;
//  * rows beyond M (or beyond a group's end) and columns beyond N are
//    loaded as zeros and never stored.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device.hpp"
#include "fp8bs.h"
#include "status.hpp"

namespace fp8bs {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kBK = 128;
constexpr int kGroupM = 8;           // tile-walk group height (in M tiles)
constexpr int kThreads = 256;
constexpr int kPitch8 = 144;         // LDS row pitch of an E4M3 tile, bytes
constexpr int kPitch16 = 136;        // LDS row pitch of an f16 tile, halves (272 bytes)

struct GemmArgs {
  const uint8_t* a;
  const float* a_scale;
  const uint8_t* b;
  const float* b_scale;
  void* y;
  const int32_t* off;      // grouped: [G+1] row offsets (device)
  int64_t lda, ldb, ldy;
  int64_t b_group_stride;  // grouped: bytes between experts' B
  int64_t bs_group_stride; // grouped: floats between experts' B scales
  int32_t M, N, KB;
  int32_t tiles_m, tiles_n;  // tiles_m: real (dense) or virtual upper bound (grouped)
  int32_t G;
};

// Workgroup id -> (M tile, N tile).
__device__ __forceinline__ void tile_of(uint32_t wg, uint32_t n_wg, int tiles_m, int tiles_n,
                                        int& tm, int& tn) {
  if ((n_wg & 7u) == 0) wg = (wg & 7u) * (n_wg >> 3) + (wg >> 3);   // XCD-contiguous ranges
  const uint32_t per_group = uint32_t(kGroupM) * tiles_n;
  const uint32_t g = wg / per_group;
  const uint32_t first_m = g * kGroupM;
  const uint32_t gm = min(uint32_t(tiles_m) - first_m, uint32_t(kGroupM));
  const uint32_t in_g = wg - g * per_group;
  tm = int(first_m + in_g % gm);
  tn = int(in_g / gm);
}

// The rows, B operand and scales one workgroup works on.
struct Tile {
  int64_t row0, row_end, n0;
  const uint8_t* bmat;
  const float* bscale;
};

// Returns false when a grouped workgroup has no tile (uniform across the
// workgroup, before any barrier).
template <bool kGrouped>
__device__ __forceinline__ bool locate_tile(const GemmArgs& args, Tile& tile) {
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, args.tiles_m, args.tiles_n, tm, tn);
  tile.bmat = args.b;
  tile.bscale = args.b_scale;
  tile.n0 = int64_t(tn) * kBN;
  if constexpr (kGrouped) {
    // Find the group holding virtual M tile `tm`; offsets are clamped into
    // [0, M] and a decreasing pair counts as an empty group.
    int vm = tm, g = 0;
    int64_t lo = 0, hi = 0;
    bool found = false;
    for (; g < args.G; ++g) {
      lo = max(int64_t(0), min(int64_t(args.off[g]), int64_t(args.M)));
      hi = max(int64_t(0), min(int64_t(args.off[g + 1]), int64_t(args.M)));
      if (hi < lo) hi = lo;
      const int cnt = int((hi - lo + kBM - 1) / kBM);
      if (vm < cnt) { found = true; break; }
      vm -= cnt;
    }
    if (!found) return false;
    tile.row0 = lo + int64_t(vm) * kBM;
    tile.row_end = hi;
    tile.bmat += int64_t(g) * args.b_group_stride;
    tile.bscale += int64_t(g) * args.bs_group_stride;
  } else {
    tile.row0 = int64_t(tm) * kBM;
    tile.row_end = args.M;
  }
  return true;
}

// Global -> register staging of one K block: thread t holds 16-byte chunks
// (rows (t/8) + 32p, bytes 16*(t%8)..) of the A and B tiles, plus one scale:
// threads 0..127 the A scale of row t, threads 128.. the B scale(s).
template <bool kRowScale>
struct BlockLoad {
  uint4 ra[4], rb[4];
  float rs;

  __device__ __forceinline__ void load(const GemmArgs& args, const Tile& tile, int kb) {
    const int t = threadIdx.x;
    const int cc = (t & 7) * 16;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = (t >> 3) + 32 * p;
      const int64_t ar = tile.row0 + r;
      ra[p] = ar < tile.row_end
                  ? *reinterpret_cast<const uint4*>(args.a + ar * args.lda + int64_t(kb) * kBK + cc)
                  : make_uint4(0, 0, 0, 0);
      const int64_t br = tile.n0 + r;
      rb[p] = br < args.N
                  ? *reinterpret_cast<const uint4*>(tile.bmat + br * args.ldb + int64_t(kb) * kBK + cc)
                  : make_uint4(0, 0, 0, 0);
    }
    rs = 0.0f;
    if (t < kBM) {
      const int64_t ar = tile.row0 + t;
      if (ar < tile.row_end) rs = args.a_scale[ar * args.KB + kb];
    } else if constexpr (kRowScale) {
      const int64_t br = tile.n0 + (t - kBM);
      if (br < args.N) rs = tile.bscale[br * args.KB + kb];
    } else {
      if (t == kBM) rs = tile.bscale[(tile.n0 / 128) * args.KB + kb];
    }
  }

  __device__ __forceinline__ void store_scales(float* sA, float* sB) const {
    const int t = threadIdx.x;
    if (t < kBM) sA[t] = rs;
    else if (kRowScale || t == kBM) sB[t - kBM] = rs;
  }
};

// 16 E4M3 codes -> 16 f16 values (exact: every E4M3 value is an f16 value).
__device__ __forceinline__ void widen16(const uint4& c, uint4& lo, uint4& hi) {
  const h2 h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c.x, 1.0f, false);
  const h2 h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c.x, 1.0f, true);
  const h2 h2_ = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c.y, 1.0f, false);
  const h2 h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c.y, 1.0f, true);
  const h2 h4 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c.z, 1.0f, false);
  const h2 h5 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c.z, 1.0f, true);
  const h2 h6 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c.w, 1.0f, false);
  const h2 h7 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c.w, 1.0f, true);
  lo = make_uint4(__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1),
                  __builtin_bit_cast(uint32_t, h2_), __builtin_bit_cast(uint32_t, h3));
  hi = make_uint4(__builtin_bit_cast(uint32_t, h4), __builtin_bit_cast(uint32_t, h5),
                  __builtin_bit_cast(uint32_t, h6), __builtin_bit_cast(uint32_t, h7));
}

template <bool kBf16Out>
__device__ __forceinline__ void store_out(const GemmArgs& args, int64_t row, int64_t col, float v) {
  if constexpr (kBf16Out)
    reinterpret_cast<uint16_t*>(args.y)[row * args.ldy + col] = static_cast<uint16_t>(f32_to_bf16_rne(v));
  else
    reinterpret_cast<float*>(args.y)[row * args.ldy + col] = v;
}

// ---------------------------------------------------------------------------
// FP32-accumulating kernel: f16 tiles in LDS, 32x32x16 f16 MFMA.
// Each wave owns 2 x 2 sub-tiles of 32 x 32; lane l of a sub-tile holds
// column l%32 and rows 8*(r/4) + 4*(l/32) + r%4 for its 16 registers r.
template <bool kRowScale, bool kBf16Out, bool kGrouped>
__global__ __launch_bounds__(kThreads) void gemm_f32acc_kernel(const GemmArgs args) {
  __shared__ __attribute__((aligned(16))) _Float16 As[2][kBM * kPitch16];
  __shared__ __attribute__((aligned(16))) _Float16 Bs[2][kBN * kPitch16];
  __shared__ __attribute__((aligned(16))) float sA[2][kBM];
  __shared__ __attribute__((aligned(16))) float sB[2][kRowScale ? kBN : 4];

  Tile tile;
  if (!locate_tile<kGrouped>(args, tile)) return;
  const int KB = args.KB;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave & 1;
  const int wn = wave >> 1;

  BlockLoad<kRowScale> ld;
  auto stage = [&](int buf) {
    const int cc = (t & 7) * 16;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = (t >> 3) + 32 * p;
      uint4 lo, hi;
      widen16(ld.ra[p], lo, hi);
      uint4* da = reinterpret_cast<uint4*>(&As[buf][r * kPitch16 + cc]);
      da[0] = lo;
      da[1] = hi;
      widen16(ld.rb[p], lo, hi);
      uint4* db = reinterpret_cast<uint4*>(&Bs[buf][r * kPitch16 + cc]);
      db[0] = lo;
      db[1] = hi;
    }
    ld.store_scales(sA[buf], sB[buf]);
  };

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  ld.load(args, tile, 0);
  stage(0);
  __syncthreads();

  const int frow = lane & 31;
  const int fk = (lane >> 5) * 8;
  for (int kb = 0; kb < KB; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < KB) ld.load(args, tile, kb + 1);

    v16f p[2][2];
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      h8 af[2], bf[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        af[mi] = *reinterpret_cast<const h8*>(&As[buf][(wm * 64 + mi * 32 + frow) * kPitch16 + s * 16 + fk]);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        bf[ni] = *reinterpret_cast<const h8*>(&Bs[buf][(wn * 64 + ni * 32 + frow) * kPitch16 + s * 16 + fk]);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          if (s == 0) {
            const v16f z = {};
            p[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[mi], bf[ni], z, 0, 0, 0);
          } else {
            p[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[mi], bf[ni], p[mi][ni], 0, 0, 0);
          }
        }
    }

    // Promotion: rows of register r are 8*(r/4) + 4*(lane/32) + r%4.
    float sa[2][16];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 s4 = *reinterpret_cast<const float4*>(&sA[buf][wm * 64 + mi * 32 + 8 * q + 4 * (lane >> 5)]);
        sa[mi][4 * q + 0] = s4.x;
        sa[mi][4 * q + 1] = s4.y;
        sa[mi][4 * q + 2] = s4.z;
        sa[mi][4 * q + 3] = s4.w;
      }
    if constexpr (!kRowScale) {
      const float sb = sB[buf][0];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) sa[mi][r] *= sb;
    }
    float sbc[2] = {1.0f, 1.0f};
    if constexpr (kRowScale) {
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) sbc[ni] = sB[buf][wn * 64 + ni * 32 + frow];
    }
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float c = kRowScale ? sa[mi][r] * sbc[ni] : sa[mi][r];
          acc[mi][ni][r] = __builtin_fmaf(p[mi][ni][r], c, acc[mi][ni][r]);
        }

    if (kb + 1 < KB) stage(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = tile.row0 + wm * 64 + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (row >= tile.row_end) continue;
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int64_t col = tile.n0 + wn * 64 + ni * 32 + frow;
        if (col < args.N) store_out<kBf16Out>(args, row, col, acc[mi][ni][r]);
      }
    }
}

// ---------------------------------------------------------------------------
// FP8-MFMA kernel: E4M3 tiles in LDS (144-byte rows: 16 lanes reading 16
// consecutive rows hit 16 distinct 4-bank groups), one 16x16x128 MFMA per
// sub-tile and K block.  Each wave owns 4 x 4 sub-tiles of 16 x 16; lane l
// holds column l%16 and rows 4*(l/16) + i.
__device__ __forceinline__ v4f mfma_fp8_16x16x128(const v8i& a, const v8i& b) {
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  // Format selectors 0/0 = E4M3 for both operands; zero scale operands make
  // the compiler emit the plain (unscaled) v_mfma_f32_16x16x128_f8f6f4.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

template <bool kRowScale, bool kBf16Out, bool kGrouped>
__global__ __launch_bounds__(kThreads) void gemm_fp8mfma_kernel(const GemmArgs args) {
  __shared__ __attribute__((aligned(16))) uint8_t As[2][kBM * kPitch8];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][kBN * kPitch8];
  __shared__ __attribute__((aligned(16))) float sA[2][kBM];
  __shared__ __attribute__((aligned(16))) float sB[2][kRowScale ? kBN : 4];

  Tile tile;
  if (!locate_tile<kGrouped>(args, tile)) return;
  const int KB = args.KB;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave & 1;
  const int wn = wave >> 1;

  BlockLoad<kRowScale> ld;
  auto stage = [&](int buf) {
    const int cc = (t & 7) * 16;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = (t >> 3) + 32 * p;
      *reinterpret_cast<uint4*>(&As[buf][r * kPitch8 + cc]) = ld.ra[p];
      *reinterpret_cast<uint4*>(&Bs[buf][r * kPitch8 + cc]) = ld.rb[p];
    }
    ld.store_scales(sA[buf], sB[buf]);
  };

  float acc[4][4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[i][j][k] = 0.0f;

  ld.load(args, tile, 0);
  stage(0);
  __syncthreads();

  const int frag_row = lane & 15;
  const int frag_k = (lane >> 4) * 32;
  for (int kb = 0; kb < KB; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < KB) ld.load(args, tile, kb + 1);

    v8i af[4], bf[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const uint8_t* p = &As[buf][(wm * 64 + mi * 16 + frag_row) * kPitch8 + frag_k];
      const uint4 lo = *reinterpret_cast<const uint4*>(p);
      const uint4 hi = *reinterpret_cast<const uint4*>(p + 16);
      af[mi] = v8i{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
    }
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const uint8_t* p = &Bs[buf][(wn * 64 + ni * 16 + frag_row) * kPitch8 + frag_k];
      const uint4 lo = *reinterpret_cast<const uint4*>(p);
      const uint4 hi = *reinterpret_cast<const uint4*>(p + 16);
      bf[ni] = v8i{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
    }
    float sa[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const float4 s4 = *reinterpret_cast<const float4*>(&sA[buf][wm * 64 + mi * 16 + 4 * (lane >> 4)]);
      sa[mi][0] = s4.x; sa[mi][1] = s4.y; sa[mi][2] = s4.z; sa[mi][3] = s4.w;
    }
    if constexpr (!kRowScale) {
      const float sb = sB[buf][0];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int i = 0; i < 4; ++i) sa[mi][i] *= sb;
    }
    float sbc[4] = {1.0f, 1.0f, 1.0f, 1.0f};
    if constexpr (kRowScale) {
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) sbc[ni] = sB[buf][wn * 64 + ni * 16 + frag_row];
    }

    v4f p[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) p[mi][ni] = mfma_fp8_16x16x128(af[mi], bf[ni]);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float c = kRowScale ? sa[mi][i] * sbc[ni] : sa[mi][i];
          acc[mi][ni][i] = __builtin_fmaf(p[mi][ni][i], c, acc[mi][ni][i]);
        }

    if (kb + 1 < KB) stage(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = tile.row0 + wm * 64 + mi * 16 + 4 * (lane >> 4) + i;
      if (row >= tile.row_end) continue;
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int64_t col = tile.n0 + wn * 64 + ni * 16 + frag_row;
        if (col < args.N) store_out<kBf16Out>(args, row, col, acc[mi][ni][i]);
      }
    }
}

// ---------------------------------------------------------------------------
#define FP8BS_DEFINE_LAUNCH(NAME)                                                                   \
  template <bool kGrouped>                                                                         \
  void launch_##NAME(const GemmArgs& args, bool row_scale, bool bf16_out, uint32_t n_wg,           \
                     hipStream_t stream) {                                                         \
    const dim3 grid(n_wg), block(kThreads);                                                        \
    if (row_scale) {                                                                               \
      if (bf16_out)                                                                                \
        hipLaunchKernelGGL((NAME<true, true, kGrouped>), grid, block, 0, stream, args);            \
      else                                                                                         \
        hipLaunchKernelGGL((NAME<true, false, kGrouped>), grid, block, 0, stream, args);           \
    } else {                                                                                       \
      if (bf16_out)                                                                                \
        hipLaunchKernelGGL((NAME<false, true, kGrouped>), grid, block, 0, stream, args);           \
      else                                                                                         \
        hipLaunchKernelGGL((NAME<false, false, kGrouped>), grid, block, 0, stream, args);          \
    }                                                                                              \
  }

FP8BS_DEFINE_LAUNCH(gemm_f32acc_kernel)
FP8BS_DEFINE_LAUNCH(gemm_fp8mfma_kernel)
#undef FP8BS_DEFINE_LAUNCH

template <bool kGrouped>
fp8bs_status launch(const GemmArgs& args, int32_t accum, bool row_scale, bool bf16_out,
                    uint32_t n_wg, hipStream_t stream) {
  if (accum == FP8BS_ACCUM_FP8_MFMA)
    launch_gemm_fp8mfma_kernel<kGrouped>(args, row_scale, bf16_out, n_wg, stream);
  else
    launch_gemm_f32acc_kernel<kGrouped>(args, row_scale, bf16_out, n_wg, stream);
  return check_launch(kGrouped ? "fp8_blockscaled_grouped_gemm" : "fp8_blockscaled_gemm");
}

bool valid_accum(int32_t accum) { return accum == FP8BS_ACCUM_FP32 || accum == FP8BS_ACCUM_FP8_MFMA; }

}  // namespace
}  // namespace fp8bs

using namespace fp8bs;

extern "C" fp8bs_status fp8_blockscaled_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a,
                                             int64_t lda, const float* a_scale, const uint8_t* b,
                                             int64_t ldb, const float* b_scale, int32_t b_kind,
                                             void* y, int32_t y_dtype, int64_t ldy, int32_t accum,
                                             hipStream_t stream) {
  const char* fn = "fp8_blockscaled_gemm";
  if (M < 0 || N < 0 || K < 0) return fail(FP8BS_ERR_INVALID_ARG, "%s: negative size", fn);
  if (b_kind != FP8BS_BSCALE_BLOCK128 && b_kind != FP8BS_BSCALE_ROW)
    return fail(FP8BS_ERR_INVALID_ARG, "%s: unknown b_kind %d", fn, b_kind);
  if (!valid_dtype(y_dtype)) return fail(FP8BS_ERR_INVALID_ARG, "%s: unknown y_dtype %d", fn, y_dtype);
  if (!valid_accum(accum)) return fail(FP8BS_ERR_INVALID_ARG, "%s: unknown accum %d", fn, accum);
  if (K % 128 || K < 128) return fail(FP8BS_ERR_SHAPE, "%s: K=%lld must be a positive multiple of 128", fn, (long long)K);
  if (b_kind == FP8BS_BSCALE_BLOCK128 && N % 128)
    return fail(FP8BS_ERR_SHAPE, "%s: block128 B scales need N %% 128 == 0 (N=%lld)", fn, (long long)N);
  if (N % 16) return fail(FP8BS_ERR_SHAPE, "%s: N=%lld must be a multiple of 16", fn, (long long)N);
  if (M == 0 || N == 0) return FP8BS_OK;
  if (!a || !b || !a_scale || !b_scale || !y) return fail(FP8BS_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (lda < K || ldb < K || ldy < N) return fail(FP8BS_ERR_INVALID_ARG, "%s: pitch smaller than the row", fn);
  if (!aligned16(a) || !aligned16(b) || !aligned16(y) || lda % 16 || ldb % 16 ||
      (ldy * elem_size(y_dtype)) % 16)
    return fail(FP8BS_ERR_ALIGNMENT, "%s: operands and row pitches must be 16-byte aligned", fn);
  if (!aligned4(a_scale) || !aligned4(b_scale)) return fail(FP8BS_ERR_ALIGNMENT, "%s: scales must be 4-byte aligned", fn);
  if (M > 0x7fffffff || N > 0x7fffffff || K / 128 > 0x7fffffff)
    return fail(FP8BS_ERR_INVALID_ARG, "%s: dimension too large", fn);

  GemmArgs args{};
  args.a = a; args.a_scale = a_scale; args.b = b; args.b_scale = b_scale; args.y = y;
  args.off = nullptr;
  args.lda = lda; args.ldb = ldb; args.ldy = ldy;
  args.M = int32_t(M); args.N = int32_t(N); args.KB = int32_t(K / 128);
  args.tiles_m = int32_t((M + kBM - 1) / kBM);
  args.tiles_n = int32_t((N + kBN - 1) / kBN);
  args.G = 1;
  const int64_t n_wg = int64_t(args.tiles_m) * args.tiles_n;
  if (n_wg > 0x7fffffff) return fail(FP8BS_ERR_INVALID_ARG, "%s: too many tiles", fn);
  return launch<false>(args, accum, b_kind == FP8BS_BSCALE_ROW, y_dtype == FP8BS_BF16,
                       uint32_t(n_wg), stream);
}

extern "C" fp8bs_status fp8_blockscaled_grouped_gemm(int64_t M_total, int64_t N, int64_t K, int32_t G,
                                                     const int32_t* off, const uint8_t* a,
                                                     const float* a_scale, const uint8_t* b,
                                                     const float* b_scale, void* y, int32_t y_dtype,
                                                     int32_t accum, hipStream_t stream) {
  const char* fn = "fp8_blockscaled_grouped_gemm";
  if (M_total < 0 || N < 0 || K < 0) return fail(FP8BS_ERR_INVALID_ARG, "%s: negative size", fn);
  if (G < 1 || G > 1024) return fail(FP8BS_ERR_INVALID_ARG, "%s: G=%d outside 1..1024", fn, G);
  if (!valid_dtype(y_dtype)) return fail(FP8BS_ERR_INVALID_ARG, "%s: unknown y_dtype %d", fn, y_dtype);
  if (!valid_accum(accum)) return fail(FP8BS_ERR_INVALID_ARG, "%s: unknown accum %d", fn, accum);
  if (K % 128 || K < 128) return fail(FP8BS_ERR_SHAPE, "%s: K=%lld must be a positive multiple of 128", fn, (long long)K);
  if (N % 128) return fail(FP8BS_ERR_SHAPE, "%s: N=%lld must be a multiple of 128", fn, (long long)N);
  if (M_total == 0 || N == 0) return FP8BS_OK;
  if (!off || !a || !a_scale || !b || !b_scale || !y) return fail(FP8BS_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (!aligned16(a) || !aligned16(b) || !aligned16(y))
    return fail(FP8BS_ERR_ALIGNMENT, "%s: operands must be 16-byte aligned", fn);
  if (!aligned4(a_scale) || !aligned4(b_scale) || !aligned4(off))
    return fail(FP8BS_ERR_ALIGNMENT, "%s: scales and offsets must be 4-byte aligned", fn);
  if (M_total > 0x7fffffff) return fail(FP8BS_ERR_INVALID_ARG, "%s: M_total too large", fn);

  GemmArgs args{};
  args.a = a; args.a_scale = a_scale; args.b = b; args.b_scale = b_scale; args.y = y;
  args.off = off;
  args.lda = K; args.ldb = K; args.ldy = N;
  args.b_group_stride = N * K;
  args.bs_group_stride = (N / 128) * (K / 128);
  args.M = int32_t(M_total); args.N = int32_t(N); args.KB = int32_t(K / 128);
  args.tiles_m = int32_t((M_total + kBM - 1) / kBM + G);   // upper bound on sum_g ceil(m_g/128)
  args.tiles_n = int32_t(N / kBN);
  args.G = G;
  const int64_t n_wg = int64_t(args.tiles_m) * args.tiles_n;
  if (n_wg > 0x7fffffff) return fail(FP8BS_ERR_INVALID_ARG, "%s: too many tiles", fn);
  return launch<true>(args, accum, false, y_dtype == FP8BS_BF16, uint32_t(n_wg), stream);
}
