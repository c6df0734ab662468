// Online fine-grained E4M3 quantization kernels for gfx950.
//
// Method: codingmall.com knowledge-base article on FP8 precision in
// DeepSeek-V3 training, sections "Finkornig kvantisering" (1x128 activation
// tiles, 128x128 weight blocks, each with its own scale) and
// "Online-kvantisering" (the scale comes from the tile's current values);
// HolySheep AI (zh) FP8 mixed-precision article, section 2.2
// (FP8BlockQuantizer.quantize: scale = amax/448, guarded to 1 when not above
// 1e-10; codes = E4M3 of x/scale; the FP32 scale is returned).
//
// All three kernels are HBM-bound streaming kernels: every input byte is read
// once with 16-byte loads, every code written once with 8- or 16-byte
// stores.  Each 128-element tile's amax is reduced across the lanes that hold
// it (a 16-lane DPP row for 1x128), the scale and its reciprocal are formed
// once per tile (without a division sequence for bf16 inputs), and x/s is
// evaluated with a 3-instruction exact quotient for bf16 inputs (IEEE
// division for f32 inputs).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device.hpp"
#include "fp8bs.h"
#include "status.hpp"

namespace fp8bs {
namespace {

// ---------------------------------------------------------------------------
// 8 consecutive input elements starting at p (16-byte aligned) as floats.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <bool kBf16>
__device__ __forceinline__ void load8(const void* p, float (&v)[8]) {
  if constexpr (kBf16) {
    const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x);
    v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
    v[4] = bf16_lo(u.z); v[5] = bf16_hi(u.z);
    v[6] = bf16_lo(u.w); v[7] = bf16_hi(u.w);
  } else {
    const f32x4* f = reinterpret_cast<const f32x4*>(p);
    const f32x4 a = __builtin_nontemporal_load(f);
    const f32x4 b = __builtin_nontemporal_load(f + 1);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <bool kBf16>
__device__ __forceinline__ float quotient(float x, float s, float r) {
  if constexpr (kBf16) return div_bf16_by_scale(x, s, r);
  else return x / s;
}

// The scale s = fl32(amax / 448) (with the guard) and r, close to 1 / s, of
// a tile whose amax is a bf16 value, without IEEE division sequences:
//  - amax / 448 = (amax / 7) / 64.  The quotient by 7 is Markstein's
//    correction of amax * fl32(1/7), which returns fl32(amax / 7) for every
//    bf16 amax whose scale passes the guard (checked against exact rational
//    arithmetic for all of them; every smaller amax still gives a value at
//    or below the guard), and the division by 64 is exact there.
//  - r is the hardware reciprocal refined by one Newton-Raphson step.  It
//    only feeds the quotient correction of div_bf16_by_scale, whose result
//    is checked against fl32(x / s) for every pair of bf16 values x and
//    amax.
__device__ __forceinline__ void scale_recip_bf16(float amax, float& s, float& r) {
  constexpr float kInv7 = 0x1.24924ap-3f;   // fl32(1/7)
  const float q0 = amax * kInv7;
  const float q1 = __builtin_fmaf(__builtin_fmaf(-q0, 7.0f, amax), kInv7, q0);
  const float sc = q1 * 0x1p-6f;
  s = sc > kScaleGuard ? sc : 1.0f;
  const float r0 = __builtin_amdgcn_rcpf(s);
  r = __builtin_fmaf(__builtin_fmaf(-s, r0, 1.0f), r0, r0);
}

// Scale and reciprocal of a tile: the division-free form above for bf16
// inputs, IEEE division for float32 inputs (whose quotient is an IEEE
// division too, so r is not used there).
template <bool kBf16>
__device__ __forceinline__ void tile_scale_recip(float amax, float& s, float& r) {
  if constexpr (kBf16) {
    scale_recip_bf16(amax, s, r);
  } else {
    s = tile_scale(amax);
    r = 1.0f / s;
  }
}

template <bool kBf16>
__device__ __forceinline__ uint2 encode8(const float (&v)[8], float s, float r) {
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = quotient<kBf16>(v[i], s, r);
  return make_uint2(pack4_e4m3(q[0], q[1], q[2], q[3]), pack4_e4m3(q[4], q[5], q[6], q[7]));
}

__device__ __forceinline__ float absmax8(const float (&v)[8]) {
  float m0 = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fabsf(v[2]));
  float m1 = fmaxf(fmaxf(fabsf(v[3]), fabsf(v[4])), fabsf(v[5]));
  float m2 = fmaxf(fabsf(v[6]), fabsf(v[7]));
  return fmaxf(fmaxf(m0, m1), m2);
}

// ---------------------------------------------------------------------------
// 1x128 tiles.  A 16-lane DPP row owns one tile (8 elements per lane); a wave
// handles 4 consecutive tiles per step and kU steps, all loads issued before
// the first use.  Tile t is row t / KB, column block t % KB, and its scale
// sits at scale[t] (the scale array is dense [rows, KB]).
#ifndef FP8BS_ACT_U
#define FP8BS_ACT_U 2
#endif
#ifndef FP8BS_NT_STORE
#define FP8BS_NT_STORE 1
#endif
constexpr int kActU = FP8BS_ACT_U;

// Code stores cover whole cache lines per wave and are not read again here,
// so they stream past the caches (nontemporal).  Scale stores are 16 bytes
// per wave and step; they stay ordinary stores so that L2 merges them into
// whole lines before they reach memory.  The 128x128 and dual-orientation
// quantizers store their codes as ordinary stores when they fit well inside
// the 256 MB Infinity Cache (kNT false): the GEMM that follows then finds
// them there, and those kernels themselves ran faster that way at those
// sizes (the 1x128 kernel did not).
template <bool kNT = true>
__device__ __forceinline__ void store_codes8(uint8_t* dst, uint2 c) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  if (kNT && FP8BS_NT_STORE) __builtin_nontemporal_store(u32x2{c.x, c.y}, reinterpret_cast<u32x2*>(dst));
  else *reinterpret_cast<uint2*>(dst) = c;
}
__device__ __forceinline__ void store_scale(float* dst, float s) { *dst = s; }

template <bool kBf16, int kU>
__global__ __launch_bounds__(256) void quant_1x128_kernel(const void* __restrict__ x, int64_t ld_x,
                                                          uint32_t n_tiles, FastDiv per_row,
                                                          uint8_t* __restrict__ q, int64_t ld_q,
                                                          float* __restrict__ scale) {
  constexpr int kElt = kBf16 ? 2 : 4;
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t sub = lane & 15u;
  const uint32_t slot = lane >> 4;
  const uint32_t wave = blockIdx.x * 4u + (threadIdx.x >> 6);
  const uint32_t base = wave * (4u * kU);

  float v[kU][8];
  uint32_t tile[kU], row[kU], kb[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    uint32_t t = base + 4u * u + slot;
    tile[u] = t;
    t = t < n_tiles ? t : n_tiles - 1;          // clamp: every lane stays active
    row[u] = per_row.div(t);
    kb[u] = t - row[u] * per_row.d;
    const char* p = static_cast<const char*>(x) +
                    (int64_t(row[u]) * ld_x + int64_t(kb[u]) * 128 + sub * 8) * kElt;
    load8<kBf16>(p, v[u]);
  }
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    float s, r;
    tile_scale_recip<kBf16>(row16_max(absmax8(v[u])), s, r);
    const uint2 codes = encode8<kBf16>(v[u], s, r);
    if (tile[u] < n_tiles) {
      uint8_t* dst = q + int64_t(row[u]) * ld_q + int64_t(kb[u]) * 128 + sub * 8;
      store_codes8(dst, codes);
      if (sub == 0) store_scale(&scale[tile[u]], s);
    }
  }
}

// ---------------------------------------------------------------------------
// 128x1 tiles with transposed output.  A workgroup takes a 128-row x 64-column
// block of x, stages it in LDS as float32 (row pitch 66 floats), then thread
// (column pair cp, 16-row group j) reads its 2 x 16 values, the 8 row groups
// of a column reduce their amax (4 inside the wave, 2 waves through LDS), and
// each thread writes 16 codes per column: 16 contiguous bytes of the
// transposed output row.
constexpr int kTPitch = 66;

template <bool kBf16>
__global__ __launch_bounds__(256) void quant_128x1_t_kernel(const void* __restrict__ x, int64_t ld_x,
                                                            int64_t rows, int64_t cols,
                                                            uint8_t* __restrict__ q, int64_t ld_q,
                                                            float* __restrict__ scale) {
  __shared__ float tile[128 * kTPitch];
  __shared__ float part[2][64];
  constexpr int kElt = kBf16 ? 2 : 4;
  const int64_t c0 = int64_t(blockIdx.x) * 64;
  const int64_t r0 = int64_t(blockIdx.y) * 128;
  const char* xb = static_cast<const char*>(x);

  // Phase 1: 128 rows x 64 columns as 8-element chunks, 8 chunks per row.
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int chunk = threadIdx.x + 256 * p;
    const int r = chunk >> 3;
    const int cc = (chunk & 7) * 8;
    float v[8];
    const int64_t col = c0 + cc;
    const char* src = xb + ((r0 + r) * ld_x + col) * kElt;
    if (col + 8 <= cols) {
      load8<kBf16>(src, v);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float f = 0.0f;
        if (col + i < cols) {
          if constexpr (kBf16)
            f = __uint_as_float(uint32_t(reinterpret_cast<const uint16_t*>(src)[i]) << 16);
          else
            f = reinterpret_cast<const float*>(src)[i];
        }
        v[i] = f;
      }
    }
    float2* dst = reinterpret_cast<float2*>(&tile[r * kTPitch + cc]);
    dst[0] = make_float2(v[0], v[1]);
    dst[1] = make_float2(v[2], v[3]);
    dst[2] = make_float2(v[4], v[5]);
    dst[3] = make_float2(v[6], v[7]);
  }
  __syncthreads();

  // Phase 2.
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int cp = (lane & 15) + 16 * (w & 1);
  const int j = (lane >> 4) + 4 * (w >> 1);
  float a[16], b[16];
  float m0 = 0.0f, m1 = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float2 t = *reinterpret_cast<const float2*>(&tile[(16 * j + i) * kTPitch + 2 * cp]);
    a[i] = t.x;
    b[i] = t.y;
    m0 = fmaxf(m0, fabsf(t.x));
    m1 = fmaxf(m1, fabsf(t.y));
  }
  m0 = fmaxf(m0, __shfl_xor(m0, 16));
  m0 = fmaxf(m0, __shfl_xor(m0, 32));
  m1 = fmaxf(m1, __shfl_xor(m1, 16));
  m1 = fmaxf(m1, __shfl_xor(m1, 32));
  if ((lane >> 4) == 0) {
    part[w >> 1][2 * cp] = m0;
    part[w >> 1][2 * cp + 1] = m1;
  }
  __syncthreads();
  m0 = fmaxf(part[0][2 * cp], part[1][2 * cp]);
  m1 = fmaxf(part[0][2 * cp + 1], part[1][2 * cp + 1]);

  const int64_t kbt = rows / 128;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t col = c0 + 2 * cp + h;
    const float* val = h ? b : a;
    float s, r;
    tile_scale_recip<kBf16>(h ? m1 : m0, s, r);
    float qv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) qv[i] = quotient<kBf16>(val[i], s, r);
    if (col < cols) {
      uint4 out;
      out.x = pack4_e4m3(qv[0], qv[1], qv[2], qv[3]);
      out.y = pack4_e4m3(qv[4], qv[5], qv[6], qv[7]);
      out.z = pack4_e4m3(qv[8], qv[9], qv[10], qv[11]);
      out.w = pack4_e4m3(qv[12], qv[13], qv[14], qv[15]);
      *reinterpret_cast<uint4*>(q + col * ld_q + r0 + 16 * j) = out;
      if (j == 0) scale[col * kbt + blockIdx.y] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// 128x128 blocks.  One workgroup of kThreads (default 256) threads per
// block: thread t holds columns 8*(t%16)..+8 of rows t/16 + (kThreads/16) p,
// i.e. 2048/kThreads rows of 8 values in registers.  Block amax: per-thread max,
// wave max, then the waves through LDS.  With the transposed copy requested,
// the codes go through LDS (row pitch 132 bytes) and each of the first 256
// threads transposes one 8x8 byte sub-block with byte permutes, writing
// 8-byte pieces of the transposed rows.
constexpr int kCPitch = 132;  // bytes
#ifndef FP8BS_W_THREADS
#define FP8BS_W_THREADS 256
#endif
#ifndef FP8BS_CACHED_CODE_BYTES
#define FP8BS_CACHED_CODE_BYTES (192ll << 20)
#endif
#ifndef FP8BS_W_GRID
#define FP8BS_W_GRID 65536
#endif
#ifndef FP8BS_DUAL_THREADS
#define FP8BS_DUAL_THREADS 256
#endif
#ifndef FP8BS_DUAL_GRID
#define FP8BS_DUAL_GRID 65536
#endif
#ifndef FP8BS_T_VIA_BLOCKS
#define FP8BS_T_VIA_BLOCKS 1
#endif

__device__ __forceinline__ void transpose4x4_bytes(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3,
                                                   uint32_t& o0, uint32_t& o1, uint32_t& o2,
                                                   uint32_t& o3) {
  // v_perm_b32(a, b, sel): selector byte values 0..3 pick bytes of b, 4..7 bytes of a.
  const uint32_t t01l = __builtin_amdgcn_perm(w1, w0, 0x05010400u);
  const uint32_t t01h = __builtin_amdgcn_perm(w1, w0, 0x07030602u);
  const uint32_t t23l = __builtin_amdgcn_perm(w3, w2, 0x05010400u);
  const uint32_t t23h = __builtin_amdgcn_perm(w3, w2, 0x07030602u);
  o0 = __builtin_amdgcn_perm(t23l, t01l, 0x05040100u);
  o1 = __builtin_amdgcn_perm(t23l, t01l, 0x07060302u);
  o2 = __builtin_amdgcn_perm(t23h, t01h, 0x05040100u);
  o3 = __builtin_amdgcn_perm(t23h, t01h, 0x07060302u);
}

// Raw input of one 128x128 block held by one thread: its rows of 8 elements
// as 16-byte (bf16) or 2 x 16-byte (f32) loads.
template <bool kBf16, int kRows>
struct RawRows {
  u32x4 d[kRows][kBf16 ? 1 : 2];
};

template <bool kBf16, int kRows, int kRowStep>
__device__ __forceinline__ void load_rows(RawRows<kBf16, kRows>& raw, const void* w, int64_t ld_w,
                                          int64_t r0, int64_t c0, int rbase, int cc) {
  constexpr int kElt = kBf16 ? 2 : 4;
#pragma unroll
  for (int p = 0; p < kRows; ++p) {
    const u32x4* src = reinterpret_cast<const u32x4*>(
        static_cast<const char*>(w) + ((r0 + rbase + kRowStep * p) * ld_w + c0 + cc) * kElt);
    raw.d[p][0] = __builtin_nontemporal_load(src);
    if constexpr (!kBf16) raw.d[p][1] = __builtin_nontemporal_load(src + 1);
  }
}

template <bool kBf16>
__device__ __forceinline__ void unpack8(const u32x4 (&d)[kBf16 ? 1 : 2], float (&v)[8]) {
  if constexpr (kBf16) {
    v[0] = bf16_lo(d[0].x); v[1] = bf16_hi(d[0].x);
    v[2] = bf16_lo(d[0].y); v[3] = bf16_hi(d[0].y);
    v[4] = bf16_lo(d[0].z); v[5] = bf16_hi(d[0].z);
    v[6] = bf16_lo(d[0].w); v[7] = bf16_hi(d[0].w);
  } else {
    v[0] = __uint_as_float(d[0].x); v[1] = __uint_as_float(d[0].y);
    v[2] = __uint_as_float(d[0].z); v[3] = __uint_as_float(d[0].w);
    v[4] = __uint_as_float(d[1].x); v[5] = __uint_as_float(d[1].y);
    v[6] = __uint_as_float(d[1].z); v[7] = __uint_as_float(d[1].w);
  }
}

// Workgroup g handles blocks g, g + gridDim.x, ... (block b = row block
// b / col_blocks, column block b % col_blocks).  kPersist (grids smaller
// than the block count): it reads block i + 1 into registers while block i
// is reduced, encoded and stored, so that loads and stores of different
// blocks overlap.  Otherwise each workgroup takes one block and holds no
// second buffer, which leaves registers for more workgroups per CU.
template <bool kBf16, bool kTrans, int kThreads, bool kNT, bool kPersist>
__global__ __launch_bounds__(kThreads) void quant_128x128_kernel(const void* __restrict__ w, int64_t ld_w,
                                                                 int64_t rows, int64_t cols,
                                                                 uint8_t* __restrict__ q, int64_t ld_q,
                                                                 float* __restrict__ scale,
                                                                 uint8_t* __restrict__ q_t, int64_t ld_qt) {
  constexpr int kWaves = kThreads / 64;
  constexpr int kRowStep = kThreads / 16;
  constexpr int kRows = 128 / kRowStep;
  __shared__ float red[kWaves];
  __shared__ uint32_t ct[kTrans ? 128 * kCPitch / 4 : 1];
  const int t = threadIdx.x;
  const int cc = (t & 15) * 8;
  const int rbase = t >> 4;
  const uint32_t col_blocks = uint32_t(cols / 128);
  const uint32_t n_blocks = uint32_t(rows / 128) * col_blocks;

  RawRows<kBf16, kRows> cur, nxt;
  uint32_t blk = blockIdx.x;
  if (blk >= n_blocks) return;
  load_rows<kBf16, kRows, kRowStep>(cur, w, ld_w, int64_t(blk / col_blocks) * 128,
                                    int64_t(blk % col_blocks) * 128, rbase, cc);
  for (; blk < n_blocks; blk += gridDim.x) {
    const uint32_t bi = blk / col_blocks, bj = blk % col_blocks;
    const int64_t r0 = int64_t(bi) * 128, c0 = int64_t(bj) * 128;
    const uint32_t nb = blk + gridDim.x;
    if constexpr (kPersist) {
      if (nb < n_blocks)
        load_rows<kBf16, kRows, kRowStep>(nxt, w, ld_w, int64_t(nb / col_blocks) * 128,
                                          int64_t(nb % col_blocks) * 128, rbase, cc);
    }

    float v[kRows][8];
#pragma unroll
    for (int p = 0; p < kRows; ++p) unpack8<kBf16>(cur.d[p], v[p]);
    float m = 0.0f;
#pragma unroll
    for (int p = 0; p < kRows; ++p) m = fmaxf(m, absmax8(v[p]));
    m = wave_max(m);
    if ((t & 63) == 0) red[t >> 6] = m;
    __syncthreads();
    m = red[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) m = fmaxf(m, red[i]);
    float s, r;
    tile_scale_recip<kBf16>(m, s, r);

#pragma unroll
    for (int p = 0; p < kRows; ++p) {
      const uint2 codes = encode8<kBf16>(v[p], s, r);
      const int rr = rbase + kRowStep * p;
      store_codes8<kNT>(q + (r0 + rr) * ld_q + c0 + cc, codes);
      if constexpr (kTrans) {
        ct[(rr * kCPitch + cc) / 4] = codes.x;
        ct[(rr * kCPitch + cc) / 4 + 1] = codes.y;
      }
    }
    if (t == 0) scale[bi * col_blocks + bj] = s;
    __syncthreads();   // red (and ct) are reused by the next block
    if constexpr (kTrans) {
      if (t < 256) {
        const int lane = t & 63;
        const int a = (lane & 7) | ((lane >> 5) << 3);        // row octet 0..15
        const int b = ((lane >> 3) & 3) | ((t >> 6) << 2);    // column octet 0..15
        uint32_t lo[8], hi[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int idx = ((8 * a + i) * kCPitch + 8 * b) / 4;
          lo[i] = ct[idx];
          hi[i] = ct[idx + 1];
        }
        uint32_t col_lo[8], col_hi[8];   // column j: rows 0-3 in col_lo[j], rows 4-7 in col_hi[j]
        transpose4x4_bytes(lo[0], lo[1], lo[2], lo[3], col_lo[0], col_lo[1], col_lo[2], col_lo[3]);
        transpose4x4_bytes(lo[4], lo[5], lo[6], lo[7], col_hi[0], col_hi[1], col_hi[2], col_hi[3]);
        transpose4x4_bytes(hi[0], hi[1], hi[2], hi[3], col_lo[4], col_lo[5], col_lo[6], col_lo[7]);
        transpose4x4_bytes(hi[4], hi[5], hi[6], hi[7], col_hi[4], col_hi[5], col_hi[6], col_hi[7]);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
          store_codes8<kNT>(q_t + (c0 + 8 * b + jj) * ld_qt + r0 + 8 * a, make_uint2(col_lo[jj], col_hi[jj]));
      }
      __syncthreads();   // ct is rewritten by the next block
    }
    if constexpr (kPersist) cur = nxt; else break;
  }
}


// ---------------------------------------------------------------------------
// Both activation tilings of one tensor from a single read of it: 1x128 tiles
// along the rows (codes q [rows, cols], scales [rows, cols/128]) and 128x1
// tiles along the columns, written transposed (codes q_t = codes of x^T
// [cols, rows], scales [cols, rows/128]).  A workgroup of kThreads threads
// takes one 128x128 block of x at a time (block b: row block b / col_blocks,
// column block b % col_blocks) and holds it as the 128x128 kernel does:
// thread t owns columns 8 (t % 16) .. + 7 of rows t / 16 + (kThreads / 16) p.
//  - 1x128 tiles: the 16 lanes of a DPP row hold one row of the block, which
//    is one tile; row16_max gives its amax and the codes are stored straight
//    from registers.
//  - 128x1 tiles: each thread takes the maxima of its 8 columns over its
//    rows, then over the four 16-lane groups of its wave (xor 16, 32) and
//    over the waves through LDS.  The first 128 threads turn the column
//    maxima into scales; every thread encodes its values with its columns'
//    scales into an LDS byte tile, and 8x8 byte transposes turn that into
//    whole 128-byte rows of q_t.
// With kPersist (a grid smaller than the block count), the next block's
// input is loaded into registers while the current one is processed;
// otherwise each workgroup takes one block and holds no second buffer.
// Three barriers per block; the LDS buffers written after each one were last
// read before the previous one.
// kRowOut false: only the 128x1 output (the 128x1_T tiling of
// fp8_quant_act_1x128 when cols is a multiple of 128).
template <bool kBf16, int kThreads, bool kRowOut, bool kNT, bool kPersist>
__global__ __launch_bounds__(kThreads) void quant_dual_kernel(const void* __restrict__ x, int64_t ld_x,
                                                              int64_t rows, int64_t cols,
                                                              uint8_t* __restrict__ q, int64_t ld_q,
                                                              float* __restrict__ scale,
                                                              uint8_t* __restrict__ q_t, int64_t ld_qt,
                                                              float* __restrict__ scale_t) {
  constexpr int kWaves = kThreads / 64;
  constexpr int kRowStep = kThreads / 16;
  constexpr int kRows = 128 / kRowStep;
  static_assert(kThreads >= 256 && kThreads % 256 == 0 && kRows >= 1, "block layout");
  __shared__ __align__(16) float cmax[kWaves][128];
  __shared__ float csc[2][128];                 // column scales and their reciprocals
  __shared__ uint32_t ct[128 * kCPitch / 4];    // 128x1 codes, [row][column] bytes
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int cc = (t & 15) * 8;
  const int rbase = t >> 4;
  const uint32_t col_blocks = uint32_t(cols / 128);
  const uint32_t n_blocks = uint32_t(rows / 128) * col_blocks;
  const int64_t row_kb = cols / 128;   // scale columns of the 1x128 tiling
  const int64_t col_kb = rows / 128;   // scale columns of the 128x1 tiling

  RawRows<kBf16, kRows> cur, nxt;
  uint32_t blk = blockIdx.x;
  if (blk >= n_blocks) return;
  load_rows<kBf16, kRows, kRowStep>(cur, x, ld_x, int64_t(blk / col_blocks) * 128,
                                    int64_t(blk % col_blocks) * 128, rbase, cc);
  for (; blk < n_blocks; blk += gridDim.x) {
    const uint32_t bi = blk / col_blocks, bj = blk % col_blocks;
    const int64_t r0 = int64_t(bi) * 128, c0 = int64_t(bj) * 128;
    const uint32_t nb = blk + gridDim.x;
    if constexpr (kPersist) {
      if (nb < n_blocks)
        load_rows<kBf16, kRows, kRowStep>(nxt, x, ld_x, int64_t(nb / col_blocks) * 128,
                                          int64_t(nb % col_blocks) * 128, rbase, cc);
    }
    float v[kRows][8];
#pragma unroll
    for (int p = 0; p < kRows; ++p) unpack8<kBf16>(cur.d[p], v[p]);

    // 1x128 tiles.
    if constexpr (kRowOut) {
#pragma unroll
      for (int p = 0; p < kRows; ++p) {
        float s, r;
        tile_scale_recip<kBf16>(row16_max(absmax8(v[p])), s, r);
        const int64_t row = r0 + rbase + kRowStep * p;
        store_codes8<kNT>(q + row * ld_q + c0 + cc, encode8<kBf16>(v[p], s, r));
        if ((t & 15) == 0) store_scale(&scale[row * row_kb + bj], s);
      }
    }

    // 128x1 tiles: column maxima.
    float cm[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float m = fabsf(v[0][i]);
#pragma unroll
      for (int p = 1; p < kRows; ++p) m = fmaxf(m, fabsf(v[p][i]));
      m = fmaxf(m, __shfl_xor(m, 16));
      cm[i] = fmaxf(m, __shfl_xor(m, 32));
    }
    if (lane < 16) {
      float4* dst = reinterpret_cast<float4*>(&cmax[wave][cc]);
      dst[0] = make_float4(cm[0], cm[1], cm[2], cm[3]);
      dst[1] = make_float4(cm[4], cm[5], cm[6], cm[7]);
    }
    __syncthreads();
    if (t < 128) {
      float m = cmax[0][t];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) m = fmaxf(m, cmax[w][t]);
      float s, r;
      tile_scale_recip<kBf16>(m, s, r);
      csc[0][t] = s;
      csc[1][t] = r;
      store_scale(&scale_t[(c0 + t) * col_kb + bi], s);
    }
    __syncthreads();

    // 128x1 codes into the LDS byte tile.
    float cs[8], cr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      cs[i] = csc[0][cc + i];
      cr[i] = csc[1][cc + i];
    }
#pragma unroll
    for (int p = 0; p < kRows; ++p) {
      float qv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) qv[i] = quotient<kBf16>(v[p][i], cs[i], cr[i]);
      const int rr = rbase + kRowStep * p;
      ct[(rr * kCPitch + cc) / 4] = pack4_e4m3(qv[0], qv[1], qv[2], qv[3]);
      ct[(rr * kCPitch + cc) / 4 + 1] = pack4_e4m3(qv[4], qv[5], qv[6], qv[7]);
    }
    __syncthreads();

    // Transposed store: thread u < 256 takes the 8x8 byte sub-block (row
    // octet a, column octet b); lanes 0-7 and 32-39 of a wave cover the 16
    // row octets of one column octet, so every store instruction writes
    // whole 128-byte rows of q_t.
    if (t < 256) {
      const int a = (lane & 7) | ((lane >> 5) << 3);
      const int b = ((lane >> 3) & 3) | ((t >> 6) << 2);
      uint32_t lo[8], hi[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int idx = ((8 * a + i) * kCPitch + 8 * b) / 4;
        lo[i] = ct[idx];
        hi[i] = ct[idx + 1];
      }
      uint32_t col_lo[8], col_hi[8];
      transpose4x4_bytes(lo[0], lo[1], lo[2], lo[3], col_lo[0], col_lo[1], col_lo[2], col_lo[3]);
      transpose4x4_bytes(lo[4], lo[5], lo[6], lo[7], col_hi[0], col_hi[1], col_hi[2], col_hi[3]);
      transpose4x4_bytes(hi[0], hi[1], hi[2], hi[3], col_lo[4], col_lo[5], col_lo[6], col_lo[7]);
      transpose4x4_bytes(hi[4], hi[5], hi[6], hi[7], col_hi[4], col_hi[5], col_hi[6], col_hi[7]);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
        store_codes8<kNT>(q_t + (c0 + 8 * b + jj) * ld_qt + r0 + 8 * a, make_uint2(col_lo[jj], col_hi[jj]));
    }
    if constexpr (kPersist) cur = nxt; else break;
  }
}

// ---------------------------------------------------------------------------
// Several quantization jobs in one launch (fp8_quant_batch): each job is a
// 1x128 activation quantization or a 128x128 weight quantization, computed
// exactly as its single call does (bit-identical outputs).  The launch grid
// is the concatenation of the jobs' workgroups; a workgroup finds its job
// from the jobs' first workgroup indices (uniform per workgroup) and runs
// that job's code: 32 1x128 tiles (4 waves x 4 tiles x kBatchU steps) or
// one 128x128 block (thread t holds columns 8 (t % 16) .. + 7 of rows
// t / 16 + 16 p, p < 8).  One launch pays one fill and drain of the machine
// for all the jobs; the host puts the 128x128 jobs first, so that their
// heavier workgroups start first instead of trailing.
constexpr int kMaxBatchJobs = 8;
// 1x128 steps per wave.  At the lower occupancy of this kernel, four steps
// keep more loads in flight than the single kernel's two: X [4096, 7168]
// 1x128 + W [2048, 7168] 128x128 took 23.2 us with 3 or 4 steps, 23.8 us
// with 2, 24.4 with 6 and 25.0 with 8 (alternated on one MI355X).
#ifndef FP8BS_BATCH_U
#define FP8BS_BATCH_U 4
#endif
constexpr int kBatchU = FP8BS_BATCH_U;

enum BatchKind : int32_t {
  kAct1x128Bf16 = 0, kAct1x128F32 = 1,
  kW128Bf16 = 2, kW128Bf16NT = 3, kW128F32 = 4, kW128F32NT = 5
};

struct BatchJob {
  const void* x;
  uint8_t* q;
  float* scale;
  int64_t ld_x, ld_q;
  uint32_t n_units;      // 1x128: tiles; 128x128: blocks
  uint32_t col_blocks;   // 128-column blocks per row (128x128)
  FastDiv per_row;       // 1x128: tiles per row
  uint32_t first_wg;
  int32_t kind;
};

struct BatchArgs {
  BatchJob job[kMaxBatchJobs];
  int32_t n;
};

// 1x128 tiles base .. of one job for global wave `wave` (the body of
// quant_1x128_kernel).
template <bool kBf16, int kU>
__device__ __forceinline__ void act_tiles(const BatchJob& jb, uint32_t wave) {
  constexpr int kElt = kBf16 ? 2 : 4;
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t sub = lane & 15u;
  const uint32_t slot = lane >> 4;
  const uint32_t base = wave * (4u * kU);
  const uint32_t n_tiles = jb.n_units;
  float v[kU][8];
  uint32_t tile[kU], row[kU], kb[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    uint32_t t = base + 4u * u + slot;
    tile[u] = t;
    t = t < n_tiles ? t : n_tiles - 1;          // clamp: every lane stays active
    row[u] = jb.per_row.div(t);
    kb[u] = t - row[u] * jb.per_row.d;
    const char* p = static_cast<const char*>(jb.x) +
                    (int64_t(row[u]) * jb.ld_x + int64_t(kb[u]) * 128 + sub * 8) * kElt;
    load8<kBf16>(p, v[u]);
  }
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    float s, r;
    tile_scale_recip<kBf16>(row16_max(absmax8(v[u])), s, r);
    const uint2 codes = encode8<kBf16>(v[u], s, r);
    if (tile[u] < n_tiles) {
      store_codes8(jb.q + int64_t(row[u]) * jb.ld_q + int64_t(kb[u]) * 128 + sub * 8, codes);
      if (sub == 0) store_scale(&jb.scale[tile[u]], s);
    }
  }
}

// One 128x128 block of one job (the body of quant_128x128_kernel without
// the transposed copy), 256 threads.
template <bool kBf16, bool kNT>
__device__ __forceinline__ void w_block(const BatchJob& jb, uint32_t blk, float* red) {
  constexpr int kRowStep = 16, kRows = 8;
  const int t = threadIdx.x;
  const int cc = (t & 15) * 8;
  const int rbase = t >> 4;
  const uint32_t bi = blk / jb.col_blocks, bj = blk - bi * jb.col_blocks;
  const int64_t r0 = int64_t(bi) * 128, c0 = int64_t(bj) * 128;
  RawRows<kBf16, kRows> raw;
  load_rows<kBf16, kRows, kRowStep>(raw, jb.x, jb.ld_x, r0, c0, rbase, cc);
  // The raw input stays in registers; it is widened to float32 once for the
  // maximum and again for the codes (cheaper than holding 64 floats).
  float m = 0.0f;
#pragma unroll
  for (int p = 0; p < kRows; ++p) {
    float v[8];
    unpack8<kBf16>(raw.d[p], v);
    m = fmaxf(m, absmax8(v));
  }
  m = wave_max(m);
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float s, r;
  tile_scale_recip<kBf16>(m, s, r);
#pragma unroll
  for (int p = 0; p < kRows; ++p) {
    float v[8];
    unpack8<kBf16>(raw.d[p], v);
    store_codes8<kNT>(jb.q + (r0 + rbase + kRowStep * p) * jb.ld_q + c0 + cc, encode8<kBf16>(v, s, r));
  }
  if (t == 0) jb.scale[blk] = s;
}

// kF32: the batch holds float32 inputs (their code paths need more
// registers, so batches of bf16 inputs get a variant without them).  The
// occupancy floors (6 and 5 waves per SIMD) are the highest at which each
// variant compiles without spills: the 1x128 jobs keep many loads in flight.
#ifndef FP8BS_BATCH_OCC
#define FP8BS_BATCH_OCC 6
#endif
template <bool kF32>
__global__ __launch_bounds__(256, kF32 ? 5 : FP8BS_BATCH_OCC) void quant_batch_kernel(const BatchArgs args) {
  __shared__ float red[4];
  const uint32_t wg = blockIdx.x;
  int j = 0;
  while (j + 1 < args.n && wg >= args.job[j + 1].first_wg) ++j;
  const BatchJob& jb = args.job[j];
  const uint32_t local = wg - jb.first_wg;
  const uint32_t wave = local * 4u + (threadIdx.x >> 6);
  if constexpr (kF32) {
    switch (jb.kind) {
      case kAct1x128Bf16: act_tiles<true, kBatchU>(jb, wave); break;
      case kAct1x128F32: act_tiles<false, kBatchU>(jb, wave); break;
      case kW128Bf16: w_block<true, false>(jb, local, red); break;
      case kW128Bf16NT: w_block<true, true>(jb, local, red); break;
      case kW128F32: w_block<false, false>(jb, local, red); break;
      default: w_block<false, true>(jb, local, red); break;
    }
  } else {
    switch (jb.kind) {
      case kAct1x128Bf16: act_tiles<true, kBatchU>(jb, wave); break;
      case kW128Bf16: w_block<true, false>(jb, local, red); break;
      default: w_block<true, true>(jb, local, red); break;
    }
  }
}

fp8bs_status check_matrix(const void* p, int64_t rows, int64_t ld, int64_t cols, int elt, const char* name) {
  if (ld < cols) return fail(FP8BS_ERR_INVALID_ARG, "%s: pitch %lld < columns %lld", name, (long long)ld, (long long)cols);
  if (!sane_matrix(rows, ld, elt))
    return fail(FP8BS_ERR_INVALID_ARG, "%s: %lld rows of pitch %lld exceed any allocation", name, (long long)rows, (long long)ld);
  if (!aligned16(p) || (ld * elt) % 16 != 0)
    return fail(FP8BS_ERR_ALIGNMENT, "%s: pointer and row pitch must be 16-byte aligned", name);
  return FP8BS_OK;
}

}  // namespace
}  // namespace fp8bs

using namespace fp8bs;

extern "C" fp8bs_status fp8_quant_act_1x128(const void* x, int32_t x_dtype, int64_t rows, int64_t cols,
                                            int64_t ld_x, int32_t tiling, uint8_t* q, int64_t ld_q,
                                            float* scale, hipStream_t stream) {
  const char* fn = "fp8_quant_act_1x128";
  if (!valid_dtype(x_dtype)) return fail(FP8BS_ERR_INVALID_ARG, "%s: unknown x_dtype %d", fn, x_dtype);
  if (tiling != FP8BS_TILE_1x128 && tiling != FP8BS_TILE_128x1_T)
    return fail(FP8BS_ERR_INVALID_ARG, "%s: unknown tiling %d", fn, tiling);
  if (rows < 0 || cols < 0) return fail(FP8BS_ERR_INVALID_ARG, "%s: negative size", fn);
  const bool t128x1 = tiling == FP8BS_TILE_128x1_T;
  if (!t128x1 && cols % 128) return fail(FP8BS_ERR_SHAPE, "%s: cols %lld not a multiple of 128", fn, (long long)cols);
  if (t128x1 && rows % 128) return fail(FP8BS_ERR_SHAPE, "%s: 128x1 tiling needs rows %% 128 == 0 (rows %lld)", fn, (long long)rows);
  if (rows == 0 || cols == 0) return FP8BS_OK;
  if (!x || !q || !scale) return fail(FP8BS_ERR_INVALID_ARG, "%s: null pointer", fn);
  const int elt = elem_size(x_dtype);
  fp8bs_status st = check_matrix(x, rows, ld_x, cols, elt, "x");
  if (st != FP8BS_OK) return st;
  st = check_matrix(q, t128x1 ? cols : rows, ld_q, t128x1 ? rows : cols, 1, "q");
  if (st != FP8BS_OK) return st;
  if (!aligned4(scale)) return fail(FP8BS_ERR_ALIGNMENT, "%s: scale must be 4-byte aligned", fn);

  const bool bf16 = x_dtype == FP8BS_BF16;
  begin_launch();
  if (!t128x1) {
    const int64_t kb = cols / 128;
    const int64_t n_tiles = rows * kb;
    if (n_tiles > (int64_t(1) << 31)) return fail(FP8BS_ERR_INVALID_ARG, "%s: more than 2^31 tiles", fn);
    const int64_t tiles_per_block = 4 * 4 * kActU;   // 4 waves x 4 tiles x kActU steps
    const dim3 grid(static_cast<uint32_t>((n_tiles + tiles_per_block - 1) / tiles_per_block));
    const FastDiv per_row(static_cast<uint32_t>(kb));
    if (bf16)
      hipLaunchKernelGGL((quant_1x128_kernel<true, kActU>), grid, dim3(256), 0, stream, x, ld_x,
                         static_cast<uint32_t>(n_tiles), per_row, q, ld_q, scale);
    else
      hipLaunchKernelGGL((quant_1x128_kernel<false, kActU>), grid, dim3(256), 0, stream, x, ld_x,
                         static_cast<uint32_t>(n_tiles), per_row, q, ld_q, scale);
  } else if (cols % 128 == 0 && FP8BS_T_VIA_BLOCKS) {
    // Whole 128x128 blocks: the dual kernel without its row output.
    const int64_t n_blocks = (rows / 128) * (cols / 128);
    if (n_blocks > 0x7fffffff) return fail(FP8BS_ERR_INVALID_ARG, "%s: too many blocks", fn);
    const int64_t per_wg = (n_blocks + FP8BS_DUAL_GRID - 1) / FP8BS_DUAL_GRID;
    const dim3 grid(static_cast<uint32_t>((n_blocks + per_wg - 1) / per_wg));
    constexpr int kT = FP8BS_DUAL_THREADS;
    const bool cached = rows * cols <= int64_t(FP8BS_CACHED_CODE_BYTES);
#define FP8BS_TLP(B, NT, P) hipLaunchKernelGGL((quant_dual_kernel<B, kT, false, NT, P>), grid, dim3(kT), 0, stream, \
                                               x, ld_x, rows, cols, nullptr, int64_t(0), nullptr, q, ld_q, scale)
#define FP8BS_TL(B, NT) do { if (per_wg > 1) FP8BS_TLP(B, NT, true); else FP8BS_TLP(B, NT, false); } while (0)
    if (bf16) { if (cached) FP8BS_TL(true, false); else FP8BS_TL(true, true); }
    else { if (cached) FP8BS_TL(false, false); else FP8BS_TL(false, true); }
#undef FP8BS_TL
#undef FP8BS_TLP
  } else {
    if ((cols + 63) / 64 > 0x7fffffff || rows / 128 > 65535)
      return fail(FP8BS_ERR_INVALID_ARG, "%s: too many tiles for the launch grid", fn);
    const dim3 grid(static_cast<uint32_t>((cols + 63) / 64), static_cast<uint32_t>(rows / 128));
    if (bf16)
      hipLaunchKernelGGL((quant_128x1_t_kernel<true>), grid, dim3(256), 0, stream, x, ld_x, rows, cols, q, ld_q, scale);
    else
      hipLaunchKernelGGL((quant_128x1_t_kernel<false>), grid, dim3(256), 0, stream, x, ld_x, rows, cols, q, ld_q, scale);
  }
  return check_launch(fn);
}

extern "C" fp8bs_status fp8_quant_w_128x128(const void* w, int32_t w_dtype, int64_t rows, int64_t cols,
                                            int64_t ld_w, uint8_t* q, int64_t ld_q, float* scale,
                                            uint8_t* q_t, int64_t ld_qt, hipStream_t stream) {
  const char* fn = "fp8_quant_w_128x128";
  if (!valid_dtype(w_dtype)) return fail(FP8BS_ERR_INVALID_ARG, "%s: unknown w_dtype %d", fn, w_dtype);
  if (rows < 0 || cols < 0) return fail(FP8BS_ERR_INVALID_ARG, "%s: negative size", fn);
  if (rows % 128 || cols % 128)
    return fail(FP8BS_ERR_SHAPE, "%s: rows %lld and cols %lld must be multiples of 128", fn, (long long)rows, (long long)cols);
  if (rows == 0 || cols == 0) return FP8BS_OK;
  if (!w || !q || !scale) return fail(FP8BS_ERR_INVALID_ARG, "%s: null pointer", fn);
  fp8bs_status st = check_matrix(w, rows, ld_w, cols, elem_size(w_dtype), "w");
  if (st != FP8BS_OK) return st;
  st = check_matrix(q, rows, ld_q, cols, 1, "q");
  if (st != FP8BS_OK) return st;
  if (q_t) {
    st = check_matrix(q_t, cols, ld_qt, rows, 1, "q_t");
    if (st != FP8BS_OK) return st;
  }
  if (!aligned4(scale)) return fail(FP8BS_ERR_ALIGNMENT, "%s: scale must be 4-byte aligned", fn);
  // One block per workgroup up to FP8BS_W_GRID blocks; beyond that each
  // workgroup takes ceil(blocks / FP8BS_W_GRID) blocks in turn.
  const int64_t n_blocks = (rows / 128) * (cols / 128);
  if (n_blocks > 0x7fffffff) return fail(FP8BS_ERR_INVALID_ARG, "%s: too many blocks", fn);
  const int64_t per_wg = (n_blocks + FP8BS_W_GRID - 1) / FP8BS_W_GRID;
  const dim3 grid(static_cast<uint32_t>((n_blocks + per_wg - 1) / per_wg));
  const bool bf16 = w_dtype == FP8BS_BF16;
  constexpr int kT = FP8BS_W_THREADS;
  // Codes (and their transposed copy) up to FP8BS_CACHED_CODE_BYTES are written
  // with ordinary stores, larger outputs stream past the caches.
  const bool cached = rows * cols * (q_t ? 2 : 1) <= int64_t(FP8BS_CACHED_CODE_BYTES);
  begin_launch();
#define FP8BS_WLP(B, T, NT, P) hipLaunchKernelGGL((quant_128x128_kernel<B, T, kT, NT, P>), grid, dim3(kT), 0, \
                                                  stream, w, ld_w, rows, cols, q, ld_q, scale, q_t, ld_qt)
#define FP8BS_WL(B, T, NT) do { if (per_wg > 1) FP8BS_WLP(B, T, NT, true); else FP8BS_WLP(B, T, NT, false); } while (0)
#define FP8BS_WL2(B, T) if (cached) FP8BS_WL(B, T, false); else FP8BS_WL(B, T, true);
  if (bf16 && q_t) { FP8BS_WL2(true, true) }
  else if (bf16) { FP8BS_WL2(true, false) }
  else if (q_t) { FP8BS_WL2(false, true) }
  else { FP8BS_WL2(false, false) }
#undef FP8BS_WL2
#undef FP8BS_WL
#undef FP8BS_WLP
  return check_launch(fn);
}

extern "C" fp8bs_status fp8_quant_act_dual(const void* x, int32_t x_dtype, int64_t rows, int64_t cols,
                                           int64_t ld_x, uint8_t* q, int64_t ld_q, float* scale,
                                           uint8_t* q_t, int64_t ld_qt, float* scale_t,
                                           hipStream_t stream) {
  const char* fn = "fp8_quant_act_dual";
  if (!valid_dtype(x_dtype)) return fail(FP8BS_ERR_INVALID_ARG, "%s: unknown x_dtype %d", fn, x_dtype);
  if (rows < 0 || cols < 0) return fail(FP8BS_ERR_INVALID_ARG, "%s: negative size", fn);
  if (rows % 128 || cols % 128)
    return fail(FP8BS_ERR_SHAPE, "%s: rows %lld and cols %lld must be multiples of 128", fn, (long long)rows, (long long)cols);
  if (rows == 0 || cols == 0) return FP8BS_OK;
  if (!x || !q || !scale || !q_t || !scale_t) return fail(FP8BS_ERR_INVALID_ARG, "%s: null pointer", fn);
  fp8bs_status st = check_matrix(x, rows, ld_x, cols, elem_size(x_dtype), "x");
  if (st != FP8BS_OK) return st;
  st = check_matrix(q, rows, ld_q, cols, 1, "q");
  if (st != FP8BS_OK) return st;
  st = check_matrix(q_t, cols, ld_qt, rows, 1, "q_t");
  if (st != FP8BS_OK) return st;
  if (!aligned4(scale) || !aligned4(scale_t))
    return fail(FP8BS_ERR_ALIGNMENT, "%s: scales must be 4-byte aligned", fn);
  const int64_t n_blocks = (rows / 128) * (cols / 128);
  if (n_blocks > 0x7fffffff) return fail(FP8BS_ERR_INVALID_ARG, "%s: too many blocks", fn);
  const int64_t per_wg = (n_blocks + FP8BS_DUAL_GRID - 1) / FP8BS_DUAL_GRID;
  const dim3 grid(static_cast<uint32_t>((n_blocks + per_wg - 1) / per_wg));
  constexpr int kT = FP8BS_DUAL_THREADS;
  const bool cached = 2 * rows * cols <= int64_t(FP8BS_CACHED_CODE_BYTES);
  begin_launch();
#define FP8BS_DLP(B, NT, P) hipLaunchKernelGGL((quant_dual_kernel<B, kT, true, NT, P>), grid, dim3(kT), 0, stream, \
                                               x, ld_x, rows, cols, q, ld_q, scale, q_t, ld_qt, scale_t)
#define FP8BS_DL(B, NT) do { if (per_wg > 1) FP8BS_DLP(B, NT, true); else FP8BS_DLP(B, NT, false); } while (0)
  if (x_dtype == FP8BS_BF16) { if (cached) FP8BS_DL(true, false); else FP8BS_DL(true, true); }
  else { if (cached) FP8BS_DL(false, false); else FP8BS_DL(false, true); }
#undef FP8BS_DL
#undef FP8BS_DLP
  return check_launch(fn);
}

extern "C" fp8bs_status fp8_quant_batch(const fp8bs_quant_job* jobs, int32_t n_jobs, hipStream_t stream) {
  const char* fn = "fp8_quant_batch";
  static_assert(FP8BS_MAX_QUANT_JOBS == kMaxBatchJobs, "job capacity");
  if (n_jobs < 0 || n_jobs > FP8BS_MAX_QUANT_JOBS)
    return fail(FP8BS_ERR_INVALID_ARG, "%s: n_jobs=%d outside 0..%d", fn, n_jobs, FP8BS_MAX_QUANT_JOBS);
  if (n_jobs > 0 && !jobs) return fail(FP8BS_ERR_INVALID_ARG, "%s: null job array", fn);
  // Validate every job before anything is launched, exactly as the single
  // calls validate their arguments.
  for (int32_t i = 0; i < n_jobs; ++i) {
    const fp8bs_quant_job& jb = jobs[i];
    if (!valid_dtype(jb.x_dtype)) return fail(FP8BS_ERR_INVALID_ARG, "%s: job %d: unknown x_dtype %d", fn, i, jb.x_dtype);
    if (jb.tiling != FP8BS_TILE_1x128 && jb.tiling != FP8BS_TILE_128x128)
      return fail(FP8BS_ERR_INVALID_ARG, "%s: job %d: tiling %d is not 1x128 or 128x128", fn, i, jb.tiling);
    if (jb.rows < 0 || jb.cols < 0) return fail(FP8BS_ERR_INVALID_ARG, "%s: job %d: negative size", fn, i);
    if (jb.cols % 128 || (jb.tiling == FP8BS_TILE_128x128 && jb.rows % 128))
      return fail(FP8BS_ERR_SHAPE, "%s: job %d: rows %lld / cols %lld not whole tiles", fn, i,
                  (long long)jb.rows, (long long)jb.cols);
    if (jb.rows == 0 || jb.cols == 0) continue;
    if (!jb.x || !jb.q || !jb.scale) return fail(FP8BS_ERR_INVALID_ARG, "%s: job %d: null pointer", fn, i);
    fp8bs_status st = check_matrix(jb.x, jb.rows, jb.ld_x, jb.cols, elem_size(jb.x_dtype), "x");
    if (st != FP8BS_OK) return fail(st, "%s: job %d: %s", fn, i, fp8bs_last_error());
    st = check_matrix(jb.q, jb.rows, jb.ld_q, jb.cols, 1, "q");
    if (st != FP8BS_OK) return fail(st, "%s: job %d: %s", fn, i, fp8bs_last_error());
    if (!aligned4(jb.scale)) return fail(FP8BS_ERR_ALIGNMENT, "%s: job %d: scale must be 4-byte aligned", fn, i);
    const int64_t units = jb.tiling == FP8BS_TILE_1x128 ? jb.rows * (jb.cols / 128)
                                                       : (jb.rows / 128) * (jb.cols / 128);
    if (units > 0x7fffffffLL) return fail(FP8BS_ERR_INVALID_ARG, "%s: job %d: more than 2^31 tiles", fn, i);
  }
  // 128x128 jobs first (heavier workgroups start first), then 1x128 jobs.
  BatchArgs args{};
  int64_t total = 0;
  for (int pass = 0; pass < 2; ++pass) {
    for (int32_t i = 0; i < n_jobs; ++i) {
      const fp8bs_quant_job& jb = jobs[i];
      const bool w = jb.tiling == FP8BS_TILE_128x128;
      if (w != (pass == 0) || jb.rows == 0 || jb.cols == 0) continue;
      BatchJob& d = args.job[args.n++];
      d.x = jb.x; d.q = jb.q; d.scale = jb.scale; d.ld_x = jb.ld_x; d.ld_q = jb.ld_q;
      d.first_wg = uint32_t(total);
      const bool bf16 = jb.x_dtype == FP8BS_BF16;
      if (w) {
        d.n_units = uint32_t((jb.rows / 128) * (jb.cols / 128));
        d.col_blocks = uint32_t(jb.cols / 128);
        const bool nt = jb.rows * jb.cols > int64_t(FP8BS_CACHED_CODE_BYTES);
        d.kind = bf16 ? (nt ? kW128Bf16NT : kW128Bf16) : (nt ? kW128F32NT : kW128F32);
        total += d.n_units;
      } else {
        d.n_units = uint32_t(jb.rows * (jb.cols / 128));
        d.per_row = FastDiv(uint32_t(jb.cols / 128));
        d.kind = bf16 ? kAct1x128Bf16 : kAct1x128F32;
        total += (int64_t(d.n_units) + 4 * 4 * kBatchU - 1) / (4 * 4 * kBatchU);
      }
      if (total > 0x7fffffffLL) return fail(FP8BS_ERR_INVALID_ARG, "%s: more than 2^31 workgroups", fn);
    }
  }
  if (total == 0) return FP8BS_OK;
  bool any_f32 = false;
  for (int i = 0; i < args.n; ++i)
    any_f32 |= args.job[i].kind == kAct1x128F32 || args.job[i].kind == kW128F32 || args.job[i].kind == kW128F32NT;
  begin_launch();
  if (any_f32)
    hipLaunchKernelGGL(quant_batch_kernel<true>, dim3(uint32_t(total)), dim3(256), 0, stream, args);
  else
    hipLaunchKernelGGL(quant_batch_kernel<false>, dim3(uint32_t(total)), dim3(256), 0, stream, args);
  return check_launch(fn);
}
