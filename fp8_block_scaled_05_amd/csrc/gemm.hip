// Block-scaled FP8 GEMM (dense and grouped) for gfx950.
//
// Method: codingmall.com knowledge-base article on FP8 precision in
// DeepSeek-V3 training, section "Ökad ackumuleringsprecision": partial sums
// of the FP8 GEMM are promoted into FP32 registers at fixed intervals; with
// the 1x128 / 128x128 scaling of "Finkornig kvantisering" the scales are
// constant over each 128-deep K block, so the interval is one K block:
//     acc[m,n] += (sa[m,kb] * sb[n,kb]) * P_kb[m,n]
// where P_kb is the FP8 product over the block, accumulated in FP32 by the
// matrix cores.
//
// Design (one workgroup = 256 threads = 4 waves, output tile 128 x 128):
//  * one v_mfma_f32_16x16x128_f8f6f4 covers exactly one 128-deep K block of
//    a 16x16 output sub-tile, so P_kb comes out of a single instruction with
//    a zero accumulator and the promotion is one FP32 FMA per output element
//    per K block (the scale product sa*sb is formed once per row);
//  * each wave owns a 64x64 quadrant = 4x4 MFMA sub-tiles;
//  * A and B K-block tiles (128 rows x 128 bytes) are staged in LDS with a
//    144-byte row pitch (16 lanes reading 16 consecutive rows hit 16 distinct
//    4-bank groups), double-buffered: the next block's global loads are in
//    flight while the current one is multiplied, one barrier per block;
//  * workgroups are renumbered so that each XCD (which has its own L2) gets a
//    contiguous range of tiles, and tiles are walked in groups of 8 M-tiles
//    so that a range shares A rows and B rows in that L2.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device.hpp"
#include "fp8bs.h"
#include "status.hpp"

namespace fp8bs {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kBK = 128;
constexpr int kPitch = 144;          // LDS row pitch of an operand tile, bytes
constexpr int kGroupM = 8;           // tile-walk group height (in M tiles)
constexpr int kThreads = 256;

struct GemmArgs {
  const uint8_t* a;
  const float* a_scale;
  const uint8_t* b;
  const float* b_scale;
  void* y;
  const int32_t* off;      // grouped: [G+1] row offsets (device)
  int64_t lda, ldb, ldy;
  int64_t b_group_stride;  // grouped: elements between experts' B
  int64_t bs_group_stride; // grouped: floats between experts' B scales
  int32_t M, N, KB;
  int32_t tiles_m, tiles_n;  // tiles_m: real (dense) or virtual upper bound (grouped)
  int32_t G;
};

__device__ __forceinline__ v4f mfma_fp8_16x16x128(const v8i& a, const v8i& b) {
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  // Format selectors 0/0 = E4M3 for both operands; zero scale operands make
  // the compiler emit the plain (unscaled) v_mfma_f32_16x16x128_f8f6f4.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

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

template <bool kRowScale, bool kBf16Out, bool kGrouped>
__global__ __launch_bounds__(kThreads) void blockscaled_gemm_kernel(const GemmArgs args) {
  __shared__ __attribute__((aligned(16))) uint8_t As[2][kBM * kPitch];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][kBN * kPitch];
  __shared__ __attribute__((aligned(16))) float sA[2][kBM];
  __shared__ __attribute__((aligned(16))) float sB[2][kRowScale ? kBN : 4];

  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, args.tiles_m, args.tiles_n, tm, tn);

  // Row range [row0, row_end) of this tile and the B operand it multiplies.
  int64_t row0, row_end;
  const uint8_t* bmat = args.b;
  const float* bscale = args.b_scale;
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
    if (!found) return;                     // uniform across the workgroup
    row0 = lo + int64_t(vm) * kBM;
    row_end = hi;
    bmat += int64_t(g) * args.b_group_stride;
    bscale += int64_t(g) * args.bs_group_stride;
  } else {
    row0 = int64_t(tm) * kBM;
    row_end = args.M;
  }
  const int64_t n0 = int64_t(tn) * kBN;
  const int KB = args.KB;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave & 1;          // quadrant row
  const int wn = wave >> 1;         // quadrant column

  // Global -> register staging of one K block.
  uint4 ra[4], rb[4];
  float rs = 0.0f;
  auto load_block = [&](int kb) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = (t >> 3) + 32 * p;
      const int cc = (t & 7) * 16;
      const int64_t ar = row0 + r;
      ra[p] = ar < row_end
                  ? *reinterpret_cast<const uint4*>(args.a + ar * args.lda + int64_t(kb) * kBK + cc)
                  : make_uint4(0, 0, 0, 0);
      const int64_t br = n0 + r;
      rb[p] = br < args.N
                  ? *reinterpret_cast<const uint4*>(bmat + br * args.ldb + int64_t(kb) * kBK + cc)
                  : make_uint4(0, 0, 0, 0);
    }
    if (t < kBM) {
      const int64_t ar = row0 + t;
      rs = ar < row_end ? args.a_scale[ar * KB + kb] : 0.0f;
    } else if constexpr (kRowScale) {
      const int64_t br = n0 + (t - kBM);
      rs = br < args.N ? bscale[br * KB + kb] : 0.0f;
    } else {
      if (t == kBM) rs = bscale[(n0 / 128) * KB + kb];
    }
  };
  auto store_block = [&](int buf) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = (t >> 3) + 32 * p;
      const int cc = (t & 7) * 16;
      *reinterpret_cast<uint4*>(&As[buf][r * kPitch + cc]) = ra[p];
      *reinterpret_cast<uint4*>(&Bs[buf][r * kPitch + cc]) = rb[p];
    }
    if (t < kBM) sA[buf][t] = rs;
    else if (kRowScale || t == kBM) sB[buf][t - kBM] = rs;
  };

  float acc[4][4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[i][j][k] = 0.0f;

  load_block(0);
  store_block(0);
  __syncthreads();

  const int frag_row = lane & 15;
  const int frag_k = (lane >> 4) * 32;
  for (int kb = 0; kb < KB; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < KB) load_block(kb + 1);

    v8i af[4], bf[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const uint8_t* p = &As[buf][(wm * 64 + mi * 16 + frag_row) * kPitch + frag_k];
      const uint4 lo = *reinterpret_cast<const uint4*>(p);
      const uint4 hi = *reinterpret_cast<const uint4*>(p + 16);
      af[mi] = v8i{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
    }
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const uint8_t* p = &Bs[buf][(wn * 64 + ni * 16 + frag_row) * kPitch + frag_k];
      const uint4 lo = *reinterpret_cast<const uint4*>(p);
      const uint4 hi = *reinterpret_cast<const uint4*>(p + 16);
      bf[ni] = v8i{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
    }
    // Output rows of this lane in sub-tile mi: 4*(lane/16) + i.
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
    float sbc[4];
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

    if (kb + 1 < KB) store_block(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: lane holds column (lane % 16) and rows 4*(lane/16)+i of each sub-tile.
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = row0 + wm * 64 + mi * 16 + 4 * (lane >> 4) + i;
      if (row >= row_end) continue;
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int64_t col = n0 + wn * 64 + ni * 16 + frag_row;
        if (col >= args.N) continue;
        if constexpr (kBf16Out) {
          reinterpret_cast<uint16_t*>(args.y)[row * args.ldy + col] =
              static_cast<uint16_t>(f32_to_bf16_rne(acc[mi][ni][i]));
        } else {
          reinterpret_cast<float*>(args.y)[row * args.ldy + col] = acc[mi][ni][i];
        }
      }
    }
}

template <bool kGrouped>
fp8bs_status launch(const GemmArgs& args, bool row_scale, bool bf16_out, uint32_t n_wg,
                    hipStream_t stream) {
  const dim3 grid(n_wg), block(kThreads);
  if (row_scale) {
    if (bf16_out)
      hipLaunchKernelGGL((blockscaled_gemm_kernel<true, true, kGrouped>), grid, block, 0, stream, args);
    else
      hipLaunchKernelGGL((blockscaled_gemm_kernel<true, false, kGrouped>), grid, block, 0, stream, args);
  } else {
    if (bf16_out)
      hipLaunchKernelGGL((blockscaled_gemm_kernel<false, true, kGrouped>), grid, block, 0, stream, args);
    else
      hipLaunchKernelGGL((blockscaled_gemm_kernel<false, false, kGrouped>), grid, block, 0, stream, args);
  }
  return check_launch(kGrouped ? "fp8_blockscaled_grouped_gemm" : "fp8_blockscaled_gemm");
}

}  // namespace
}  // namespace fp8bs

using namespace fp8bs;

extern "C" fp8bs_status fp8_blockscaled_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a,
                                             int64_t lda, const float* a_scale, const uint8_t* b,
                                             int64_t ldb, const float* b_scale, int32_t b_kind,
                                             void* y, int32_t y_dtype, int64_t ldy,
                                             hipStream_t stream) {
  const char* fn = "fp8_blockscaled_gemm";
  if (M < 0 || N < 0 || K < 0) return fail(FP8BS_ERR_INVALID_ARG, "%s: negative size", fn);
  if (b_kind != FP8BS_BSCALE_BLOCK128 && b_kind != FP8BS_BSCALE_ROW)
    return fail(FP8BS_ERR_INVALID_ARG, "%s: unknown b_kind %d", fn, b_kind);
  if (!valid_dtype(y_dtype)) return fail(FP8BS_ERR_INVALID_ARG, "%s: unknown y_dtype %d", fn, y_dtype);
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
  return launch<false>(args, b_kind == FP8BS_BSCALE_ROW, y_dtype == FP8BS_BF16, uint32_t(n_wg), stream);
}

extern "C" fp8bs_status fp8_blockscaled_grouped_gemm(int64_t M_total, int64_t N, int64_t K, int32_t G,
                                                     const int32_t* off, const uint8_t* a,
                                                     const float* a_scale, const uint8_t* b,
                                                     const float* b_scale, void* y, int32_t y_dtype,
                                                     hipStream_t stream) {
  const char* fn = "fp8_blockscaled_grouped_gemm";
  if (M_total < 0 || N < 0 || K < 0) return fail(FP8BS_ERR_INVALID_ARG, "%s: negative size", fn);
  if (G < 1 || G > 1024) return fail(FP8BS_ERR_INVALID_ARG, "%s: G=%d outside 1..1024", fn, G);
  if (!valid_dtype(y_dtype)) return fail(FP8BS_ERR_INVALID_ARG, "%s: unknown y_dtype %d", fn, y_dtype);
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
  return launch<true>(args, false, y_dtype == FP8BS_BF16, uint32_t(n_wg), stream);
}
