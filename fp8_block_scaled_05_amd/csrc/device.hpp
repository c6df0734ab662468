// Device helpers shared by the gfx950 kernels: bf16 widening, 16-lane
// reductions, the exact quotient x/s and the packed E4M3 encode.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace fp8bs {

// Largest E4M3 (OCP E4M3FN) magnitude; the tile scale is amax / 448.
constexpr float kE4M3Max = 448.0f;
// Scales not above float32(1e-10) are replaced by 1 (the quantizer's
// divide-by-zero guard).
constexpr float kScaleGuard = 1e-10f;

// bf16 -> f32 is exact: the bf16 bits are the high half of the f32 bits.
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// max over the 16 lanes of a DPP row (lanes 16r..16r+15): rotate-and-max by
// 8, 4, 2, 1 leaves every lane of the row holding the row maximum.
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<0x128>(v));  // row_ror:8
  v = fmaxf(v, dpp_f<0x124>(v));  // row_ror:4
  v = fmaxf(v, dpp_f<0x122>(v));  // row_ror:2
  v = fmaxf(v, dpp_f<0x121>(v));  // row_ror:1
  return v;
}
// max over groups of 8 consecutive lanes (xor butterfly within the group).
__device__ __forceinline__ float group8_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 4, 8));
  v = fmaxf(v, __shfl_xor(v, 2, 8));
  v = fmaxf(v, __shfl_xor(v, 1, 8));
  return v;
}
// max over the whole wave (64 lanes).
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

// Tile scale: fl32(amax / 448), replaced by 1 when not above fl32(1e-10).
// The division is IEEE binary32 (hipcc's default correctly rounded divide).
__device__ __forceinline__ float tile_scale(float amax) {
  float s = amax / kE4M3Max;
  return (s > kScaleGuard) ? s : 1.0f;
}

// fl32(x / s) for a bf16-valued x, given r = fl32(1 / s): Markstein's
// quotient correction (P. Markstein, "Computation of elementary functions on
// the IBM RISC System/6000 processor", IBM J. Res. Dev. 34(1), 1990):
//   q0 = x*r;  e = q0*s - x (exact, fused);  q = q0 - e*r (fused).
// The remainder is taken with its sign flipped so that x = -0 keeps its sign.
// Checked exhaustively against IEEE division for every bf16 x and every
// scale a bf16 tile can produce: the E4M3 code of q always equals that of
// x/s (quotients can differ only below 2^-80, far under E4M3's smallest step,
// and never in sign).
__device__ __forceinline__ float div_bf16_by_scale(float x, float s, float r) {
  float q0 = x * r;
  float e = __builtin_fmaf(q0, s, -x);
  return __builtin_fmaf(-e, r, q0);
}

// Four floats -> four E4M3 codes (byte i = code of v_i), round to nearest
// even.  The gfx950 converter writes two codes per call into the low or the
// high half-word.  Inputs here never exceed 448 by more than an fp32 ulp, so
// saturation and overflow handling are never exercised.
__device__ __forceinline__ uint32_t pack4_e4m3(float v0, float v1, float v2, float v3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, w, true);
  return static_cast<uint32_t>(w);
}

// f32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Unsigned 32-bit division by a runtime constant (Granlund & Montgomery,
// "Division by invariant integers using multiplication", PLDI 1994):
// q = (umulhi(n, m) + n) >> s with s = ceil(log2 d), m = floor(2^32 (2^s - d) / d) + 1.
struct FastDiv {
  uint32_t d, m, s;
  __host__ __device__ FastDiv() : d(1), m(0), s(0) {}
  __host__ explicit FastDiv(uint32_t div) : d(div) {
    s = 0;
    while ((uint64_t(1) << s) < div) ++s;
    m = static_cast<uint32_t>(((uint64_t(1) << 32) * ((uint64_t(1) << s) - div)) / div + 1);
  }
  __device__ __forceinline__ uint32_t div(uint32_t n) const {
    uint64_t hi = __umulhi(n, m);
    return static_cast<uint32_t>((hi + n) >> s);
  }
};

}  // namespace fp8bs
