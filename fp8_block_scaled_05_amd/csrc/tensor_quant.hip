// Per-tensor FP8 quantization for gfx950: the prior-art scalings that the
// fine-grained tiles are measured against.
//
// Current scaling with a margin: HolySheep AI (zh) FP8 article, troubleshooting
// entry on FP8 overflow, SafeFP8Quantizer.safe_quantize: one amax over the whole
// tensor, widened by (1 + margin), scale = that / 448, a scale below 1e-6
// replaced by 1, codes = E4M3 of x / scale.  Delayed scaling: the same
// article's FP8Config (amax history of 1024, margin 0, on Transformer Engine),
// read as: the scale comes from the largest amax of earlier calls, codes
// saturate, and this call's amax then enters the front of the history.
// E5M2 (max 57344) is the hybrid recipe's gradient format (German HolySheep
// article; codingmall "Unified E4M3 Format" says DeepSeek-V3 dropped it).
//
// The scale follows the page's arithmetic: the amax comes out of the tensor
// as a Python float and the margin, the product and the division by the
// format maximum are Python (binary64) floats, as is the "scale < 1e-6"
// test.  Here: binary64 (1 + margin), binary64 amax * that, binary64 division
// by the format maximum, the guard in binary64, then one rounding to float32,
// the precision in which the scale is stored and x / s is taken (correctly
// rounded).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "device.hpp"
#include "fp8bs.h"
#include "status.hpp"

namespace fp8bs {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kE5M2Max = 57344.0f;
constexpr double kTensorGuard = 1e-6;   // the page's "scale too small" threshold (binary64)
constexpr int kMaxHistory = 4096;

template <bool kE5M2>
__device__ __forceinline__ float fmt_max() { return kE5M2 ? kE5M2Max : kE4M3Max; }

// widen = 1 + margin in binary64.  Every step is an IEEE binary64 operation
// (correctly rounded); the result is rounded once to float32.
__device__ __forceinline__ float tensor_scale_dev(float amax, double widen, double fmax) {
  const double wide = double(amax) * widen;
  const double s = wide / fmax;
  return s < kTensorGuard ? 1.0f : float(s);
}

// Eight consecutive inputs of one row.
template <bool kBf16>
__device__ __forceinline__ void load8t(const void* p, float (&v)[8]) {
  if constexpr (kBf16) {
    const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x); v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
    v[4] = bf16_lo(u.z); v[5] = bf16_hi(u.z); v[6] = bf16_lo(u.w); v[7] = bf16_hi(u.w);
  } else {
    const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + 1);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// Four values (already clamped to the format's range) -> four codes.
template <bool kE5M2>
__device__ __forceinline__ uint32_t pack4(float v0, float v1, float v2, float v3) {
  if constexpr (kE5M2) {
    int w = __builtin_amdgcn_cvt_pk_bf8_f32(v0, v1, 0, false);
    return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_bf8_f32(v2, v3, w, true));
  } else {
    return pack4_e4m3(v0, v1, v2, v3);
  }
}

// Block-wide max of non-negative values; every thread gets the result.
__device__ __forceinline__ float block_max(float m, float* red) {
  m = wave_max(m);
  __syncthreads();                       // red may still be read from an earlier call
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < int(blockDim.x >> 6); ++w) r = fmaxf(r, red[w]);
  return r;
}

// Folds a non-negative float into *dst as a maximum: for non-negative IEEE
// values the unsigned bit patterns have the same order (a vector memory
// atomic).  Atomics on one address serialize in L2, so a workgroup whose
// value cannot raise the maximum already there skips it: the value read
// may be stale, which only costs an unneeded atomic, and the maximum only
// grows, so skipping never loses the result.
__device__ __forceinline__ void atomic_max_nonneg(float* dst, float v) {
  const unsigned int seen = __hip_atomic_load(reinterpret_cast<unsigned int*>(dst), __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
  if (__float_as_uint(v) > seen) atomicMax(reinterpret_cast<unsigned int*>(dst), __float_as_uint(v));
}

__global__ __launch_bounds__(64) void fill_kernel(float* p, float v) {
  if (threadIdx.x == 0) p[0] = v;
}

// Chunk c (8 elements) is row c / (cols / 8), columns 8 (c % (cols / 8)) ...
// Each thread takes kU chunks per pass of its grid-stride loop (chunks
// kTT u + t of a kTT kU block), all loads issued before their use.
constexpr int kTU = 4;
// Two workgroups of 1024 threads per CU (at most 64 registers per thread):
// at most 512 amax atomics per call, and 32 waves x 4 chunks of loads in
// flight per CU.  The grid is balanced so that every pass of the
// grid-stride loop is full but the last by less than one workgroup's share
// (a grid of 512 over 3.5 passes' worth of chunks would leave the last pass
// half idle).
constexpr int kTT = 1024;
constexpr int kTGrid = 512;

template <bool kBf16>
__device__ __forceinline__ const char* chunk_ptr(const void* x, int64_t ld_x, FastDiv per_row, uint32_t c,
                                                 uint32_t& row, uint32_t& col) {
  row = per_row.div(c);
  col = (c - row * per_row.d) * 8u;
  return static_cast<const char*>(x) + (int64_t(row) * ld_x + col) * (kBf16 ? 2 : 4);
}

template <bool kBf16>
__global__ __launch_bounds__(kTT) void tensor_amax_kernel(const void* __restrict__ x, int64_t ld_x,
                                                          uint32_t n_chunks, FastDiv per_row,
                                                          float* __restrict__ amax) {
  __shared__ float red[kTT / 64];
  float m = 0.0f;
  for (uint32_t base = blockIdx.x * kTT * kTU; base < n_chunks; base += gridDim.x * kTT * kTU) {
    float v[kTU][8];
#pragma unroll
    for (int u = 0; u < kTU; ++u) {
      uint32_t c = base + kTT * u + threadIdx.x, row, col;
      c = c < n_chunks ? c : n_chunks - 1;        // repeats a chunk: harmless for a maximum
      load8t<kBf16>(chunk_ptr<kBf16>(x, ld_x, per_row, c, row, col), v[u]);
    }
#pragma unroll
    for (int u = 0; u < kTU; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[u][i]));
  }
  m = block_max(m, red);
  if (threadIdx.x == 0) atomic_max_nonneg(amax, m);
}

// kDelayed: the scale comes from max(history[0 .. hist_len)) and this call's
// amax is accumulated into *amax_out; otherwise from *src (the amax of x).
// Quotients: with current scaling |x / s| <= 448 and Markstein's correction
// of x * fl32(1/s) (see div_bf16_by_scale) is the correctly rounded quotient
// wherever the code is not zero.  A stale delayed scale can make x / s
// exceed the format's range, even overflow float32, where the correction
// breaks down (x * r = inf gives NaN); there the code saturates whatever
// the exact quotient is, so when |x * r| > 2 * max (then |x / s| > max too)
// the kernel takes +-max directly and the correction everywhere else.  The
// codes equal those of the IEEE quotient clamped to +-max.
template <bool kBf16, bool kE5M2, bool kDelayed>
__global__ __launch_bounds__(kTT) void tensor_quant_kernel(const void* __restrict__ x, int64_t ld_x,
                                                           uint32_t n_chunks, FastDiv per_row,
                                                           const float* __restrict__ src, int hist_len,
                                                           double widen, uint8_t* __restrict__ q,
                                                           int64_t ld_q, float* __restrict__ scale_out,
                                                           float* __restrict__ amax_out) {
  __shared__ float red[kTT / 64];
  constexpr float kMax = kE5M2 ? kE5M2Max : kE4M3Max;
  float ref;
  if constexpr (kDelayed) {
    float h = 0.0f;
    for (int i = threadIdx.x; i < hist_len; i += kTT) h = fmaxf(h, src[i]);
    ref = block_max(h, red);
  } else {
    ref = src[0];
  }
  const float s = tensor_scale_dev(ref, widen, double(fmt_max<kE5M2>()));
  const float r = 1.0f / s;
  if (blockIdx.x == 0 && threadIdx.x == 0) scale_out[0] = s;
  float m = 0.0f;
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  for (uint32_t base = blockIdx.x * kTT * kTU; base < n_chunks; base += gridDim.x * kTT * kTU) {
    float v[kTU][8];
    uint32_t row[kTU], col[kTU];
#pragma unroll
    for (int u = 0; u < kTU; ++u) {
      uint32_t c = base + kTT * u + threadIdx.x;
      c = c < n_chunks ? c : n_chunks - 1;
      load8t<kBf16>(chunk_ptr<kBf16>(x, ld_x, per_row, c, row[u], col[u]), v[u]);
    }
#pragma unroll
    for (int u = 0; u < kTU; ++u) {
      if (base + kTT * u + threadIdx.x >= n_chunks) break;
      float w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (kDelayed) {
          m = fmaxf(m, fabsf(v[u][i]));
          const float q0 = v[u][i] * r;
          w[i] = fabsf(q0) > 2.0f * kMax ? __builtin_copysignf(kMax, v[u][i])
                                         : fminf(fmaxf(div_bf16_by_scale(v[u][i], s, r), -kMax), kMax);
        } else {
          w[i] = fminf(fmaxf(div_bf16_by_scale(v[u][i], s, r), -kMax), kMax);
        }
      }
      __builtin_nontemporal_store(u32x2{pack4<kE5M2>(w[0], w[1], w[2], w[3]), pack4<kE5M2>(w[4], w[5], w[6], w[7])},
                                  reinterpret_cast<u32x2*>(q + int64_t(row[u]) * ld_q + col[u]));
    }
  }
  if constexpr (kDelayed) {
    m = block_max(m, red);
    if (threadIdx.x == 0) atomic_max_nonneg(amax_out, m);
  }
}

// history <- [amax, history[0 .. len-2]] (one workgroup).
__global__ __launch_bounds__(1024) void history_roll_kernel(float* __restrict__ hist, int len,
                                                            const float* __restrict__ amax) {
  constexpr int kPer = kMaxHistory / 1024;
  float old[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int i = threadIdx.x + 1024 * k;
    old[k] = i < len ? hist[i] : 0.0f;
  }
  const float a = amax[0];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int i = threadIdx.x + 1024 * k;
    if (i + 1 < len) hist[i + 1] = old[k];
  }
  if (threadIdx.x == 0) hist[0] = a;
}

}  // namespace
}  // namespace fp8bs

using namespace fp8bs;

extern "C" fp8bs_status fp8_quant_tensor(const void* x, int32_t x_dtype, int64_t rows, int64_t cols,
                                         int64_t ld_x, int32_t format, double margin, float* history,
                                         int32_t history_len, uint8_t* q, int64_t ld_q, float* scale,
                                         float* amax, hipStream_t stream) {
  const char* fn = "fp8_quant_tensor";
  if (!valid_dtype(x_dtype)) return fail(FP8BS_ERR_INVALID_ARG, "%s: unknown x_dtype %d", fn, x_dtype);
  if (format != FP8BS_FMT_E4M3 && format != FP8BS_FMT_E5M2)
    return fail(FP8BS_ERR_INVALID_ARG, "%s: unknown format %d", fn, format);
  if (!(margin >= 0.0) || !(margin <= 1e6))
    return fail(FP8BS_ERR_INVALID_ARG, "%s: margin must be in [0, 1e6]", fn);
  if (history && (history_len < 1 || history_len > kMaxHistory))
    return fail(FP8BS_ERR_INVALID_ARG, "%s: history_len %d outside 1..%d", fn, history_len, kMaxHistory);
  if (rows < 0 || cols < 0) return fail(FP8BS_ERR_INVALID_ARG, "%s: negative size", fn);
  if (cols % 8) return fail(FP8BS_ERR_SHAPE, "%s: cols %lld not a multiple of 8", fn, (long long)cols);
  if (rows == 0 || cols == 0) return FP8BS_OK;
  if (!x || !q || !scale || !amax) return fail(FP8BS_ERR_INVALID_ARG, "%s: null pointer", fn);
  const int elt = elem_size(x_dtype);
  if (ld_x < cols || ld_q < cols) return fail(FP8BS_ERR_INVALID_ARG, "%s: pitch smaller than the row", fn);
  if (!sane_matrix(rows, ld_x, elt) || !sane_matrix(rows, ld_q, 1))
    return fail(FP8BS_ERR_INVALID_ARG, "%s: sizes and pitches exceed any allocation", fn);
  if (!aligned16(x) || !aligned16(q) || (ld_x * elt) % 16 || ld_q % 16)
    return fail(FP8BS_ERR_ALIGNMENT, "%s: input, codes and row pitches must be 16-byte aligned", fn);
  if (!aligned4(scale) || !aligned4(amax) || (history && !aligned4(history)))
    return fail(FP8BS_ERR_ALIGNMENT, "%s: scale, amax and history must be 4-byte aligned", fn);
  const int64_t per_row = cols / 8;
  const int64_t n_chunks = rows * per_row;
  if (n_chunks > 0xf0000000LL) return fail(FP8BS_ERR_INVALID_ARG, "%s: more than 2^32 chunks", fn);
  const FastDiv div(static_cast<uint32_t>(per_row));
  const int64_t per_pass = int64_t(kTGrid) * kTT * kTU;
  const int64_t passes = (n_chunks + per_pass - 1) / per_pass;
  const uint32_t grid = static_cast<uint32_t>((n_chunks + passes * kTT * kTU - 1) / (passes * kTT * kTU));
  const double widen = 1.0 + margin;
  const bool bf16 = x_dtype == FP8BS_BF16, e5 = format == FP8BS_FMT_E5M2;

  begin_launch();
  hipLaunchKernelGGL(fill_kernel, dim3(1), dim3(64), 0, stream, amax, 0.0f);
#define FP8BS_Q(B, E, D, SRC, L)                                                                 \
  hipLaunchKernelGGL((tensor_quant_kernel<B, E, D>), dim3(grid), dim3(kTT), 0, stream, x, ld_x, \
                     static_cast<uint32_t>(n_chunks), div, SRC, L, widen, q, ld_q, scale, amax)
#define FP8BS_Q2(D, SRC, L)                                                                       \
  if (bf16) { if (e5) FP8BS_Q(true, true, D, SRC, L); else FP8BS_Q(true, false, D, SRC, L); }    \
  else { if (e5) FP8BS_Q(false, true, D, SRC, L); else FP8BS_Q(false, false, D, SRC, L); }
  if (!history) {
    if (bf16)
      hipLaunchKernelGGL((tensor_amax_kernel<true>), dim3(grid), dim3(kTT), 0, stream, x, ld_x,
                         static_cast<uint32_t>(n_chunks), div, amax);
    else
      hipLaunchKernelGGL((tensor_amax_kernel<false>), dim3(grid), dim3(kTT), 0, stream, x, ld_x,
                         static_cast<uint32_t>(n_chunks), div, amax);
    FP8BS_Q2(false, amax, 0)
  } else {
    FP8BS_Q2(true, history, history_len)
    hipLaunchKernelGGL(history_roll_kernel, dim3(1), dim3(1024), 0, stream, history, history_len, amax);
  }
#undef FP8BS_Q2
#undef FP8BS_Q
  return check_launch(fn);
}
