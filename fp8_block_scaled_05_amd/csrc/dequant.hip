// Dequantization of E4M3 codes with their FP32 tile scales, for gfx950.
//
// Method: HolySheep AI (zh) FP8 mixed-precision article, section 2.2
// (FP8BlockQuantizer.dequantize): every code's value is multiplied by the
// scale stored for its tile.  Here the product is formed in float32, the way
// that method returns it: y = fl32(e4m3(code) * s).  The code value has at
// most 4 significant bits and s 24, so this is one rounding of the exact
// product; the bf16 output rounds that float32 to nearest even.
//
// HBM-bound: each thread reads a few chunks of codes with their tiles'
// scales (all loads issued first) and writes 16 bytes of output per chunk.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device.hpp"
#include "fp8bs.h"
#include "status.hpp"

namespace fp8bs {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Four codes (one word, byte i = code i) times s.
__device__ __forceinline__ f32x4 dec4_scaled(uint32_t w, float s) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
  return f32x4{lo[0] * s, lo[1] * s, hi[0] * s, hi[1] * s};
}

#ifndef FP8BS_DEQ_U
#define FP8BS_DEQ_U 2
#endif
constexpr int kDeqU = FP8BS_DEQ_U;

// Each lane writes 16 bytes per chunk so that every store instruction of a
// wave covers one contiguous kilobyte: a chunk is kE = 16 / (output size)
// codes (8 for bf16, 4 for f32).  Chunk c is row c / (cols / kE), columns
// kE (c % (cols / kE)) .. + kE - 1.  Workgroup g takes chunks 256 kU g ..
// + 256 kU - 1, thread t the chunks 256 u + t of them, all loads issued
// before the first store.  kBlock: the scale grid is [rows/128, cols/128];
// otherwise [rows, cols/128].
template <bool kBlock, bool kBf16Out, int kU>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ q, int64_t ld_q,
                                                      const float* __restrict__ scale, int64_t kb,
                                                      uint32_t n_chunks, FastDiv per_row,
                                                      void* __restrict__ y, int64_t ldy) {
  constexpr int kE = kBf16Out ? 8 : 4;
  uint32_t w[kU][kE / 4];
  float s[kU];
  uint32_t row[kU], col[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    uint32_t c = (blockIdx.x * kU + u) * 256u + threadIdx.x;
    c = c < n_chunks ? c : n_chunks - 1;          // clamped lanes redo the last chunk's load
    row[u] = per_row.div(c);
    col[u] = (c - row[u] * per_row.d) * kE;
    const uint8_t* src = q + int64_t(row[u]) * ld_q + col[u];
    if constexpr (kE == 8) {
      const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(src));
      w[u][0] = v.x;
      w[u][kE / 4 - 1] = v.y;
    } else {
      w[u][0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(src));
    }
    const int64_t srow = kBlock ? int64_t(row[u] >> 7) : int64_t(row[u]);
    s[u] = scale[srow * kb + (col[u] >> 7)];
  }
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    if ((blockIdx.x * kU + u) * 256u + threadIdx.x >= n_chunks) break;
    const f32x4 v0 = dec4_scaled(w[u][0], s[u]);
    if constexpr (kBf16Out) {
      const f32x4 v1 = dec4_scaled(w[u][kE / 4 - 1], s[u]);
      auto pk = [](float a, float b) { return f32_to_bf16_rne(a) | (f32_to_bf16_rne(b) << 16); };
      u32x4* dst = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(y) + int64_t(row[u]) * ldy + col[u]);
      __builtin_nontemporal_store(u32x4{pk(v0.x, v0.y), pk(v0.z, v0.w), pk(v1.x, v1.y), pk(v1.z, v1.w)}, dst);
    } else {
      f32x4* dst = reinterpret_cast<f32x4*>(static_cast<float*>(y) + int64_t(row[u]) * ldy + col[u]);
      __builtin_nontemporal_store(v0, dst);
    }
  }
}

}  // namespace
}  // namespace fp8bs

using namespace fp8bs;

extern "C" fp8bs_status fp8_dequant(const uint8_t* q, int64_t rows, int64_t cols, int64_t ld_q,
                                    const float* scale, int32_t tiling, void* y, int32_t y_dtype,
                                    int64_t ldy, hipStream_t stream) {
  const char* fn = "fp8_dequant";
  if (tiling == FP8BS_TILE_128x1_T)
    return fail(FP8BS_ERR_INVALID_ARG,
                "%s: a 128x1_T result is the 1x128 tiling of x^T; pass it with FP8BS_TILE_1x128", fn);
  if (tiling != FP8BS_TILE_1x128 && tiling != FP8BS_TILE_128x128)
    return fail(FP8BS_ERR_INVALID_ARG, "%s: unknown tiling %d", fn, tiling);
  if (!valid_dtype(y_dtype)) return fail(FP8BS_ERR_INVALID_ARG, "%s: unknown y_dtype %d", fn, y_dtype);
  if (rows < 0 || cols < 0) return fail(FP8BS_ERR_INVALID_ARG, "%s: negative size", fn);
  if (cols % 128) return fail(FP8BS_ERR_SHAPE, "%s: cols %lld not a multiple of 128", fn, (long long)cols);
  if (tiling == FP8BS_TILE_128x128 && rows % 128)
    return fail(FP8BS_ERR_SHAPE, "%s: 128x128 scales need rows %% 128 == 0 (rows %lld)", fn, (long long)rows);
  if (rows == 0 || cols == 0) return FP8BS_OK;
  if (!q || !scale || !y) return fail(FP8BS_ERR_INVALID_ARG, "%s: null pointer", fn);
  const int elt = elem_size(y_dtype);
  if (ld_q < cols || ldy < cols) return fail(FP8BS_ERR_INVALID_ARG, "%s: pitch smaller than the row", fn);
  if (!sane_matrix(rows, ld_q, 1) || !sane_matrix(rows, ldy, elt))
    return fail(FP8BS_ERR_INVALID_ARG, "%s: sizes and pitches exceed any allocation", fn);
  if (!aligned16(q) || !aligned16(y) || ld_q % 16 || (ldy * elt) % 16)
    return fail(FP8BS_ERR_ALIGNMENT, "%s: codes, output and row pitches must be 16-byte aligned", fn);
  if (!aligned4(scale)) return fail(FP8BS_ERR_ALIGNMENT, "%s: scale must be 4-byte aligned", fn);
  const int64_t per_row = cols / (y_dtype == FP8BS_BF16 ? 8 : 4);
  const int64_t n_chunks = rows * per_row;
  if (n_chunks > 0xfffff000LL || per_row > 0xffffffffLL)
    return fail(FP8BS_ERR_INVALID_ARG, "%s: more than 2^32 chunks of codes", fn);
  const dim3 grid(static_cast<uint32_t>((n_chunks + 256 * kDeqU - 1) / (256 * kDeqU)));
  const FastDiv div(static_cast<uint32_t>(per_row));
  const int64_t kb = cols / 128;
  const bool blk = tiling == FP8BS_TILE_128x128;
  const bool bf16 = y_dtype == FP8BS_BF16;
  begin_launch();
#define FP8BS_L(B, O) hipLaunchKernelGGL((dequant_kernel<B, O, kDeqU>), grid, dim3(256), 0, stream, q, ld_q, scale, kb, \
                                         static_cast<uint32_t>(n_chunks), div, y, ldy)
  if (blk) { if (bf16) FP8BS_L(true, true); else FP8BS_L(true, false); }
  else { if (bf16) FP8BS_L(false, true); else FP8BS_L(false, false); }
#undef FP8BS_L
  return check_launch(fn);
}
