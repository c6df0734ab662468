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
// (v_mfma_*_f8f6f4) add products in groups of 8 consecutive K, keeping only
// the bits down to 2^-13 of the group's largest product (each smaller product
// is cut toward zero); the groups are then combined in FP32.  That is about
// 14 significant bits - short of the 2e-5 * sum|a*b| accuracy asked of the
// GEMM on realistic data.  The 16-bit matrix instructions accumulate exact
// products in FP32, and every E4M3 value is exact in bf16 (and in f16).  One
// kernel template serves both block products:
//
//  * The exact path (fp8_blockscaled_gemm, the grouped GEMM and the
//    E4M3-output GEMM): E4M3 tiles go from HBM to LDS unchanged (1 byte
//    per element); each wave widens the 8-byte K slices it feeds to the
//    matrix core into bf16 in registers (v_cvt_scalef32_pk_bf16_fp8, two
//    codes per instruction, exact) and multiplies them with
//    v_mfma_f32_32x32x16_bf16, eight chained per 128-deep block.  On
//    E4M3-valued operands it returns bit for bit what the f16 instruction
//    does; its narrower multipliers draw less power, and sustained matrix
//    work on this chip is power-limited, so it runs at a higher clock.
//  * fp8_blockscaled_gemm_fp8mma: two v_mfma_f32_32x32x64_f8f6f4 per 32x32
//    output and K block, straight from the E4M3 bytes; twice the peak rate,
//    with the accumulation described above (outside the accuracy contract).
//
// Structure (dense 256 x 128 output tile, 8 waves of 64 x 64):
//  * A three-stage LDS ring.  Each stage holds one K block of the A and B
//    tiles (128 bytes per row), filled by 16-byte direct global->LDS buffer
//    loads issued two blocks ahead; the scales follow in groups of four K
//    blocks, double-buffered.  Buffer
//    addressing returns zeros for rows past the end of A (or of a group) and
//    past N, so tails need no branches.  Each stage lives in its own LDS
//    object so the compiler can track which loads a read depends on.
//  * Rows are stored 128 bytes apart with the 16-byte chunks XOR-swizzled by
//    (row & 7) ^ ((row >> 3) & 1): the matrix-core reads (16 consecutive
//    rows, one chunk) hit distinct banks with 32 or 64 banks.
//  * The B tile is the matrix instruction's first operand and the A tile
//    its second, so a lane's accumulators share one output row (m) per 32-row
//    subtile and the promotion needs one sa*sb product per subtile.
//  * Promotion: one FP32 FMA per output element per K block (two with the
//    per-row B scales of the weight-gradient GEMM).  With block-128 B
//    scales, two blocks in three are promoted during the next block's
//    matrix work instead of after it (see the main loop).
//  * Workgroups are renumbered so that each XCD (own L2) works on a compact
//    block of output tiles (4 M tiles x 8 N tiles for the 256 x 128 case).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "device.hpp"
#include "fp8bs.h"
#include "status.hpp"

namespace fp8bs {

namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Direct global->LDS buffer loads: lane i's 16 (or 4) bytes at
// voffset + soffset of the buffer land at LDS byte lds_addr + 16 i (4 i).
// Offsets outside the buffer read as zero.  Issued from inline asm so the
// compiler does not track them; the kernel orders them explicitly with
// s_waitcnt vmcnt + s_barrier before any wave reads the stage they fill.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t lds_addr, int voffset, int soffset) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds_addr), "v"(voffset), "s"(rsrc), "s"(soffset) : "memory");
}
__device__ __forceinline__ void dma4(i32x4 rsrc, uint32_t lds_addr, int voffset, int soffset) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(lds_addr), "v"(voffset), "s"(rsrc), "s"(soffset) : "memory");
}

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 w2 __attribute__((ext_vector_type(2)));
typedef __bf16 w8 __attribute__((ext_vector_type(8)));

// Buffer resource for `bytes` bytes at `base` (raw, stride 0).
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r.x = static_cast<int32_t>(static_cast<uint32_t>(a));
  r.y = static_cast<int32_t>(static_cast<uint32_t>(a >> 32) & 0xffffu);
  r.z = static_cast<int32_t>(bytes > 0xffffffffull ? 0xffffffffu : static_cast<uint32_t>(bytes));
  r.w = 0x00020000;
  return r;
}

// 32-bit LDS address of a __shared__ object.
template <typename T>
__device__ __forceinline__ uint32_t lds_addr(const T* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) T*)(p)));
}

// Wait until at most N of this wave's vector-memory operations are
// outstanding and all its LDS/scalar reads are done, then barrier.  The asm
// clobber keeps the compiler from moving memory operations across it.
template <int N>
__device__ __forceinline__ void wait_and_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
  asm volatile("s_barrier" ::: "memory");
}

struct GemmArgs {
  const uint8_t* a;
  const float* a_scale;
  const uint8_t* b;
  const float* b_scale;
  void* y;
  float* y_scale;           // E4M3 output: [M, N/128] scales of its 1x128 tiles
  const int32_t* off;       // grouped: [G+1] row offsets (device)
  int64_t lda, ldb, ldy;
  int64_t b_group_stride;   // grouped: bytes between experts' B
  int64_t bs_group_stride;  // grouped: floats between experts' B scales
  int32_t M, N, KB;
  int32_t tiles_m, tiles_n;  // tiles_m: real (dense) or an upper bound (grouped)
  int32_t G;
};

template <int BM_, int BN_, int WM_, int WN_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int kWaves = WM * WN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
  static constexpr int SM = TM / 32, SN = TN / 32;  // 32 x 32 subtiles per wave
  static constexpr int kGroupM = 4;                 // tile-walk group height (M tiles)
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32x32 subtiles");
  static_assert((BM / 8) % kWaves == 0 && (BN / 8) % kWaves == 0, "tile loads must split evenly");
  // Scale loads: one 64-lane load covers 16 rows x 4 K blocks.
  static constexpr int kScaleLoadsA = BM / 16 / kWaves, kScaleLoadsB = BN / 16 / kWaves;
  static_assert((BM / 16) % kWaves == 0 && (BN / 16) % kWaves == 0, "scale loads must split evenly");
};

// One K block of the A and B tiles.
template <int BM, int BN>
struct alignas(16) Stage {
  uint8_t a[BM * 128];
  uint8_t b[BN * 128];
};

// Scales of four consecutive K blocks.  A scales: [row][kb % 4]; a 64-lane
// load fills 16 rows x 4 blocks (16 cache lines), where loading one block
// per step would touch one line per row.  Per-row B scales: [column / 16]
// [kb % 4][column % 16], so that the four consecutive columns a lane needs
// for one K block are 16 contiguous bytes (one LDS read); the same 64-lane
// load fills one such [4][16] piece.  Two groups alternate.
template <int BM, int BN, bool kRowScale>
struct alignas(16) ScaleGroup {
  float sa[BM][4];
  float sb[kRowScale ? BN / 16 : 1][4][kRowScale ? 16 : 1];
};

// 16-byte chunk swizzle of a 128-byte LDS row.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// Byte offset of logical 16-byte chunk `chunk` of LDS row `row`.
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * 128 + ((chunk ^ swz(row)) << 4); }

__device__ __forceinline__ uint4 lds_read16(const uint8_t* base, int off) {
  return *reinterpret_cast<const uint4*>(base + off);
}

// Workgroup id -> (M tile, N tile).  The hardware hands workgroup i to XCD
// i % 8; renumber so each XCD gets a contiguous range of the tile walk, and
// walk kGroupM M tiles at a time so a range shares A and B rows in its L2.
template <int kGroupM>
__device__ __forceinline__ void tile_of(uint32_t wg, uint32_t n_wg, int tiles_m, int tiles_n,
                                        int& tm, int& tn) {
  const uint32_t q = n_wg >> 3, r = n_wg & 7u;
  const uint32_t x = wg & 7u;
  wg = x * q + min(x, r) + (wg >> 3);
  const uint32_t per_group = uint32_t(kGroupM) * uint32_t(tiles_n);
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
template <class C, bool kGrouped>
__device__ __forceinline__ bool locate_tile(const GemmArgs& args, Tile& tile) {
  int tm, tn;
  tile_of<C::kGroupM>(blockIdx.x, gridDim.x, args.tiles_m, args.tiles_n, tm, tn);
  tile.bmat = args.b;
  tile.bscale = args.b_scale;
  tile.n0 = int64_t(tn) * C::BN;
  if constexpr (kGrouped) {
    // Find the group holding virtual M tile `tm`.  Offsets are clamped into
    // [0, M], and each group starts no earlier than the previous one ends (a
    // group whose end lies before that is empty), so the groups' row ranges
    // never overlap whatever the table holds; for a valid table this changes
    // nothing.  With c_g the clamped offsets and P_g = max(0, c_0 .. c_g),
    // group g owns rows [P_g, P_g+1).  Every wave searches 64 groups per
    // step, one per lane: a prefix maximum of c gives the ranges, a prefix
    // sum of their tile counts the first group whose tiles reach past `tm`.
    // (A search one group at a time took 1.99 ms instead of 1.58 ms for a
    // GEMM of 256 experts, and 7.7 ms instead of 2.5 ms for 1024.)
    const int lane = threadIdx.x & 63;
    int vm = tm;          // tiles still to skip
    int run = 0;          // P at the start of this step
    int gsel = -1, lo_s = 0, hi_s = 0, vm_s = 0;
    for (int g0 = 0; g0 < args.G && gsel < 0; g0 += 64) {
      const int g = g0 + lane;
      const bool real = g < args.G;
      const int cg = real ? min(max(args.off[g], 0), args.M) : 0;
      const int cn = real ? min(max(args.off[g + 1], 0), args.M) : 0;
      int pm = cg;        // max(c_g0 .. c_g)
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int t = __shfl_up(pm, d);
        if (lane >= d) pm = max(pm, t);
      }
      const int lo_g = max(run, pm);
      const int hi_g = max(lo_g, cn);
      const int cnt = real ? (hi_g - lo_g + C::BM - 1) / C::BM : 0;
      int ps = cnt;       // tiles of groups g0 .. g
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int t = __shfl_up(ps, d);
        if (lane >= d) ps += t;
      }
      const uint64_t hit = __ballot(vm < ps);
      if (hit) {
        const int l = __builtin_ctzll(hit);
        gsel = g0 + l;
        lo_s = __shfl(lo_g, l);
        hi_s = __shfl(hi_g, l);
        vm_s = vm - (__shfl(ps, l) - __shfl(cnt, l));
      } else {
        vm -= __shfl(ps, 63);
        run = __shfl(hi_g, 63);
      }
    }
    const int g = __builtin_amdgcn_readfirstlane(gsel);
    if (g < 0) return false;
    tile.row0 = int64_t(__builtin_amdgcn_readfirstlane(lo_s)) + int64_t(__builtin_amdgcn_readfirstlane(vm_s)) * C::BM;
    tile.row_end = __builtin_amdgcn_readfirstlane(hi_s);
    tile.bmat += int64_t(g) * args.b_group_stride;
    tile.bscale += int64_t(g) * args.bs_group_stride;
  } else {
    tile.row0 = int64_t(tm) * C::BM;
    tile.row_end = args.M;
  }
  return true;
}

// Output element types of the GEMM.
enum OutKind : int { kOutF32 = 0, kOutBf16 = 1, kOutE4M3 = 2 };

// 16 bytes from LDS to global memory with a nontemporal store.  The GEMM's
// output is written once and not read again by the kernel; streaming it
// keeps it from displacing the operand tiles that the XCD's L2 is serving
// to the other workgroups.
__device__ __forceinline__ void store16_nt(uint8_t* dst, const uint8_t* src) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(src), reinterpret_cast<u32x4*>(dst));
}

// Makes x live in registers here: values feeding it must be computed first.
__device__ __forceinline__ void keep_in_vgprs(v16f& x) { asm volatile("" : "+v"(x)); }

// 8 E4M3 codes (two words) -> 8 bf16 values (exact).
__device__ __forceinline__ w8 widen8(uint32_t w0, uint32_t w1) {
  const w2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const w2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const w2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const w2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return w8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// ---------------------------------------------------------------------------
template <class C, bool kWiden, bool kRowScale, int kOut, bool kGrouped>
__global__ __launch_bounds__(C::kThreads, 1) void gemm_kernel(const GemmArgs args) {
  using St = Stage<C::BM, C::BN>;
  using Sg = ScaleGroup<C::BM, C::BN, kRowScale>;
  __shared__ St st0, st1, st2;
  __shared__ Sg sg[2];
  constexpr int SM = C::SM, SN = C::SN, NW = C::kWaves;

  Tile tile;
  if (!locate_tile<C, kGrouped>(args, tile)) return;
  const int KB = args.KB;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Wave w runs on SIMD w % 4.  Consecutive waves take the WN column slabs
  // of one row slab, so a row slab is spread over WN SIMDs (an expert's
  // tail tile with few rows then keeps several SIMDs busy).
  const int wm = wave / C::WN;
  const int wn = wave % C::WN;
  const int r32 = lane & 31;
  const int hk = lane >> 5;

  const int64_t rows = min(tile.row_end - tile.row0, int64_t(C::BM));
  const int64_t cols = min(int64_t(args.N) - tile.n0, int64_t(C::BN));
  // block128: this tile's row of B scales, read with scalar loads (the
  // constant address space tells the compiler nothing writes it).
  const __attribute__((address_space(4))) float* sb_blk =
      (const __attribute__((address_space(4))) float*)(tile.bscale + (tile.n0 / 128) * KB);

  // Buffer descriptors and per-lane offsets.  The hardware range check of a
  // raw buffer load covers the VGPR offset only, not the SGPR offset, so
  // every row-dependent part of an address is in the descriptor base or the
  // VGPR offset.  Load v of a wave covers rows 8 (v * NW + wave) .. + 7 of the
  // tile, lane i taking row + i / 8 and the logical chunk that lands at
  // physical chunk i % 8.  Each v has its own descriptor whose base is the
  // first row of its row group (8 v NW) and whose size counts only the rows
  // that exist from there on, so one VGPR offset per operand (lane row times
  // pitch plus chunk) serves every v: the swizzle of those rows does not
  // depend on v (NW is even).  The SGPR offset holds only the K block's
  // kb * 128 < K <= pitch, which stays inside any row that passes the check;
  // rows that do not exist read as zero.
  constexpr int LA = C::BM / 8 / NW, LB = C::BN / 8 / NW;
  constexpr int kLoadsPerStage = LA + LB;   // tile loads per wave and stage
  static_assert(NW % 2 == 0, "the swizzle argument needs an even wave count");
  const int lrow = 8 * wave + (lane >> 3);
  const int chunk = ((lane & 7) ^ swz(lrow)) << 4;
  const int voff_a = lrow * int(args.lda) + chunk;
  const int voff_b = lrow * int(args.ldb) + chunk;
  i32x4 rs_a[LA], rs_b[LB];
#pragma unroll
  for (int v = 0; v < LA; ++v) {
    const int64_t r = int64_t(8 * v * NW);
    rs_a[v] = make_rsrc(args.a + (tile.row0 + r) * args.lda, uint64_t(max(rows - r, int64_t(0))) * args.lda);
  }
#pragma unroll
  for (int v = 0; v < LB; ++v) {
    const int64_t r = int64_t(8 * v * NW);
    rs_b[v] = make_rsrc(tile.bmat + (tile.n0 + r) * args.ldb, uint64_t(max(cols - r, int64_t(0))) * args.ldb);
  }
  // Scale-group loads: load u of this wave covers rows 16 (u * NW + wave) +
  // lane / 4 and K block 4 g + lane % 4 of the A scales (B scale columns
  // 16 (u * NW + wave) + lane % 16 and K block 4 g + lane / 16, in the
  // layout of ScaleGroup), again with a descriptor per u that starts at its
  // row group.  The group's K blocks go in the VGPR offset: a lane whose K
  // block is past the last one reads the next row's first scales (unused)
  // or, on the last row, zero.
  constexpr int SUA = C::kScaleLoadsA, SUB = kRowScale ? C::kScaleLoadsB : 1;
  const int voff_s = ((16 * wave + (lane >> 2)) * KB + (lane & 3)) * 4;
  const int voff_sb = ((16 * wave + (lane & 15)) * KB + (lane >> 4)) * 4;
  i32x4 rs_sa[SUA], rs_sb[SUB];
#pragma unroll
  for (int u = 0; u < SUA; ++u) {
    const int64_t r = int64_t(16 * u * NW);
    rs_sa[u] = make_rsrc(args.a_scale + (tile.row0 + r) * KB, uint64_t(max(rows - r, int64_t(0))) * KB * 4);
  }
  if constexpr (kRowScale) {
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      const int64_t r = int64_t(16 * u * NW);
      rs_sb[u] = make_rsrc(tile.bscale + (tile.n0 + r) * KB, uint64_t(max(cols - r, int64_t(0))) * KB * 4);
    }
  }

  auto load_stage = [&](St& s, int kb) {
#pragma unroll
    for (int v = 0; v < LA; ++v)
      dma16(rs_a[v], lds_addr(&s.a[(v * NW + wave) * 1024]), voff_a, kb * 128);
#pragma unroll
    for (int v = 0; v < LB; ++v)
      dma16(rs_b[v], lds_addr(&s.b[(v * NW + wave) * 1024]), voff_b, kb * 128);
  };
  // Scales of K blocks 4 g .. 4 g + 3 into sg[g & 1].
  auto load_scales = [&](int g) {
    Sg& d = sg[g & 1];
    const int vo = voff_s + g * 16;
#pragma unroll
    for (int u = 0; u < SUA; ++u)
      dma4(rs_sa[u], lds_addr(&d.sa[16 * (u * NW + wave)][0]), vo, 0);
    if constexpr (kRowScale) {
#pragma unroll
      for (int u = 0; u < SUB; ++u)
        dma4(rs_sb[u], lds_addr(&d.sb[u * NW + wave][0][0]), voff_sb + g * 16, 0);
    }
  };

  v16f acc[SM][SN];
#pragma unroll
  for (int i = 0; i < SM; ++i)
#pragma unroll
    for (int j = 0; j < SN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int arow0 = wm * C::TM + r32;
  const int brow0 = wn * C::TN + r32;
  // LDS offsets of this lane's four 16-byte chunks (4 hk + q) of its first A
  // and B rows; the rows 32 i further on have the same swizzle (it depends on
  // row % 16 only), so they are these offsets plus 4096 i.
  int a_off[4], b_off[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    a_off[q] = lds_off(arow0, 4 * hk + q);
    b_off[q] = lds_off(brow0, 4 * hk + q);
  }

  // Block partials P_kb of the wave's subtiles.  On the bf16 path with
  // block-128 B scales (kLag), a block may be left pending in one of two
  // buffers and promoted during the next block's first two operand slices,
  // two subtiles per slice, so its FMAs issue between that block's matrix
  // instructions rather than in one run after the barrier, where both waves
  // of a SIMD would reach them together and leave the matrix core idle.
  // (Finishing before the slice after the barrier keeps the kernel within
  // the register budget without spills.)  Which blocks are deferred is
  // fixed per unrolled step (see the main loops).  Otherwise (FP8 path,
  // per-row B scales) p[0] holds every block and is promoted at the end of
  // its step.  (Deferring per-row promotions the same way measured no
  // faster.)  Either way each accumulator receives the same FMAs in the same
  // order.
  constexpr bool kLag = kWiden && !kRowScale;
  v16f p[2][SM][SN];
  float cl[SM];   // kLag: sa * sb of the pending block
  if constexpr (kLag) {
#pragma unroll
    for (int i = 0; i < SM; ++i) {
      cl[i] = 0.0f;   // nothing is pending before block 0: acc += 0 * 0
#pragma unroll
      for (int j = 0; j < SN; ++j) p[1][i][j] = v16f{};
    }
  }
  auto promote = [&](auto par_c, int i, int j, float c) {
    constexpr int par = decltype(par_c)::value;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][j][r] = __builtin_fmaf(p[par][i][j][r], c, acc[i][j][r]);
  };
  // Per-row B scales: column slab j of a block from p[par], with A scales
  // ca and B scales sbr.  The slab's 16 accumulators per lane are 16
  // columns, each with its own B scale and product sa * sb.
  auto promote_row = [&](auto par_c, int j, const float (&ca)[SM], const float (&sbr)[SN][16]) {
    constexpr int par = decltype(par_c)::value;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
#pragma unroll
      for (int i = 0; i < SM; ++i)
        acc[i][j][r] = __builtin_fmaf(p[par][i][j][r], ca[i] * sbr[j][r], acc[i][j][r]);
    }
  };
  // kLag: the pending block's subtiles s = i * SN + j with s / 2 == q.  The
  // empty asm makes the updated accumulators live at this point, so the
  // compiler cannot sink these FMAs into a later run.
  static_assert(!kLag || SM * SN <= 4, "the pending block is promoted in slices 0 and 1");
  auto promote_lagged = [&](auto par_c, int q) {
    constexpr int prev = decltype(par_c)::value ^ 1;
#pragma unroll
    for (int s = 0; s < SM * SN; ++s)
      if (s / 2 == q) {
        promote(std::integral_constant<int, prev>{}, s / SN, s % SN, cl[s / SN]);
        keep_in_vgprs(acc[s / SN][s % SN]);
      }
  };

  // Operand fragments, carried across steps.  bf16 path: raw E4M3 slices of
  // 16 bytes per row (two 16-deep k-steps), slice q in buffer q & 1.  FP8
  // path: 32-byte slices (one 64-deep matrix instruction), slice qq in
  // buffer qq.  Slice 0 of the next block is read into buffer 0 right after
  // the barrier that makes that block visible, while the current block's
  // last slice is multiplied.
  uint4 ra[2][SM], rb[2][SN];
  v8i fa8[2][SM], fb8[2][SN];
  auto read_slice = [&](const St& s, int q, int buf) {
#pragma unroll
    for (int i = 0; i < SM; ++i) ra[buf][i] = lds_read16(s.a, a_off[q] + 4096 * i);
#pragma unroll
    for (int j = 0; j < SN; ++j) rb[buf][j] = lds_read16(s.b, b_off[q] + 4096 * j);
  };
  auto read_slice8 = [&](const St& s, int qq, int buf) {
#pragma unroll
    for (int i = 0; i < SM; ++i) {
      const uint4 lo = lds_read16(s.a, a_off[2 * qq] + 4096 * i);
      const uint4 hi = lds_read16(s.a, a_off[2 * qq + 1] + 4096 * i);
      fa8[buf][i] = v8i{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
    }
#pragma unroll
    for (int j = 0; j < SN; ++j) {
      const uint4 lo = lds_read16(s.b, b_off[2 * qq] + 4096 * j);
      const uint4 hi = lds_read16(s.b, b_off[2 * qq + 1] + 4096 * j);
      fb8[buf][j] = v8i{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
    }
  };
  // bf16 path: widen slice q and run its two k-steps.
  auto mma_slice = [&](auto par_c, int q, int buf) {
    constexpr int par = decltype(par_c)::value;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      w8 fa[SM], fb[SN];
#pragma unroll
      for (int i = 0; i < SM; ++i)
        fa[i] = t ? widen8(ra[buf][i].z, ra[buf][i].w) : widen8(ra[buf][i].x, ra[buf][i].y);
#pragma unroll
      for (int j = 0; j < SN; ++j)
        fb[j] = t ? widen8(rb[buf][j].z, rb[buf][j].w) : widen8(rb[buf][j].x, rb[buf][j].y);
#pragma unroll
      for (int i = 0; i < SM; ++i)
#pragma unroll
        for (int j = 0; j < SN; ++j) {
          if (q == 0 && t == 0) {
            const v16f z = {};   // a new block's partial starts from zero
            p[par][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], z, 0, 0, 0);
          } else {
            p[par][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], p[par][i][j], 0, 0, 0);
          }
        }
    }
  };
  // FP8 path: one 64-deep instruction per subtile.  Format selectors 0/0 =
  // E4M3 for both operands; zero scale operands give the plain instruction.
  auto mma_slice8 = [&](int qq) {
#pragma unroll
    for (int i = 0; i < SM; ++i)
#pragma unroll
      for (int j = 0; j < SN; ++j) {
        if (qq == 0) {
          p[0][i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb8[0][j], fa8[0][i], v16f{}, 0, 0, 0, 0, 0, 0);
        } else {
          p[0][i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb8[1][j], fa8[1][i], p[0][i][j], 0, 0, 0, 0, 0, 0);
        }
      }
  };

  // One K block from stage s.  mode 0: last block; 1: the next block's
  // loads are complete except those of the block after it (issued at the
  // start of this step); 2: the next block's loads are the last ones.  Every
  // read of stage s is issued before the barrier, which is what lets the
  // next step refill it.  The scales are read after it: their group buffer
  // is refilled only two steps later.
  // The lag arguments are std::integral_constant (p[] is indexed
  // statically) and matter only with kLag: par_c, the buffer this block
  // accumulates into; in_c, promote the pending block of the other buffer
  // during this one; keep_c, leave this block pending (else it is promoted
  // at the end of the step).
  auto step = [&](auto par_c, auto in_c, auto keep_c, const St& s, const St& nxt, int kb, float sbv,
                  int mode) {
    using Par = std::integral_constant<int, kLag ? decltype(par_c)::value : 0>;
    constexpr bool kIn = kLag && decltype(in_c)::value;
    constexpr bool kKeep = kLag && decltype(keep_c)::value;
    const Sg& scl = sg[(kb >> 2) & 1];
    // Per-row B scales of the lane's 16 columns per slab, read before the
    // matrix work so that their latency is hidden by it (four 16-byte reads
    // per slab; reading them one by one at the promotion made the weight-
    // gradient GEMM 5-6% slower).  The scale group is visible from the start
    // of the step on.
    float sbr[SN][16];
    if constexpr (kRowScale) {
#pragma unroll
      for (int j = 0; j < SN; ++j)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int c = wn * C::TN + 32 * j + 8 * rq + 4 * hk;
          const float4 v4 = *reinterpret_cast<const float4*>(&scl.sb[c >> 4][kb & 3][c & 15]);
          sbr[j][4 * rq] = v4.x;
          sbr[j][4 * rq + 1] = v4.y;
          sbr[j][4 * rq + 2] = v4.z;
          sbr[j][4 * rq + 3] = v4.w;
        }
    }
    // The scheduling fences keep the compiler from hoisting later slices'
    // reads and widening ahead of the current slice's matrix work, which
    // would raise register pressure past the two-waves-per-SIMD budget.
    if constexpr (kWiden) {
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        read_slice(s, q + 1, (q + 1) & 1);
        mma_slice(Par{}, q, q & 1);
        if constexpr (kIn) promote_lagged(Par{}, q);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      read_slice8(s, 1, 1);
      mma_slice8(0);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (mode == 1) wait_and_barrier<kLoadsPerStage>();
    else if (mode == 2) wait_and_barrier<0>();
    if (mode != 0) {
      if constexpr (kWiden) read_slice(nxt, 0, 0);
      else read_slice8(nxt, 0, 0);
    }
    if constexpr (kWiden) {
      mma_slice(Par{}, 3, 1);
      if constexpr (kIn) promote_lagged(Par{}, 3);
    } else {
      mma_slice8(1);
    }
    __builtin_amdgcn_sched_barrier(0);

    // Promotion.  Accumulator r of subtile (i, j) is output row
    // m = arow0 + 32 i and column n = wn*TN + 32 j + 8 (r/4) + 4 hk + r%4.
    float ca[SM];
#pragma unroll
    for (int i = 0; i < SM; ++i) ca[i] = scl.sa[arow0 + 32 * i][kb & 3];
    if constexpr (kKeep) {
      // This block waits in p[Par]; the next step (or the end of the loop)
      // promotes it with these products.
#pragma unroll
      for (int i = 0; i < SM; ++i) cl[i] = ca[i] * sbv;
    } else if constexpr (!kRowScale) {
#pragma unroll
      for (int i = 0; i < SM; ++i) {
        const float c = ca[i] * sbv;
#pragma unroll
        for (int j = 0; j < SN; ++j) {
          promote(Par{}, i, j, c);
          keep_in_vgprs(acc[i][j]);
        }
      }
    } else {
      // Per-row B scales, one column slab at a time; the empty asm keeps the
      // compiler from sinking these FMAs into the next step, which would hold
      // the slab's B scales across it and spill.
#pragma unroll
      for (int j = 0; j < SN; ++j) {
        promote_row(Par{}, j, ca, sbr);
#pragma unroll
        for (int i = 0; i < SM; ++i) keep_in_vgprs(acc[i][j]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // A grouped wave with no rows of its expert (see below) skips the matrix
  // work but still takes every barrier, the epilogue's included.
  bool idle = false;
  if constexpr (kGrouped) {
    // A wave whose TM-row slab lies entirely past its group's last row (in
    // an expert's tail tile) has nothing to multiply.  It issues its share
    // of the stage and scale loads and takes the same barriers, with the
    // same waits, as the main loop below, then goes on to the epilogue,
    // whose barriers it takes too; its rows are not stored.
    if (int64_t(wm) * C::TM >= rows) {
      load_scales(0);
      load_stage(st0, 0);
      if (KB > 1) {
        load_stage(st1, 1);
        wait_and_barrier<kLoadsPerStage>();
      } else {
        wait_and_barrier<0>();
      }
      for (int kb = 0; kb < KB; ++kb) {
        if ((kb & 3) == 1 && kb + 3 < KB) load_scales((kb >> 2) + 1);
        if (kb + 2 < KB) load_stage(kb % 3 == 0 ? st2 : (kb % 3 == 1 ? st0 : st1), kb + 2);
        if (kb + 2 < KB) wait_and_barrier<kLoadsPerStage>();
        else if (kb + 1 < KB) wait_and_barrier<0>();
      }
      idle = true;
    }
  }
  if (!idle) {
  // Prologue: scales of K blocks 0..3 and K blocks 0 and 1 in flight,
  // block 0 visible, its slice 0 read.
  load_scales(0);
  load_stage(st0, 0);
  if (KB > 1) {
    load_stage(st1, 1);
    wait_and_barrier<kLoadsPerStage>();
  } else {
    wait_and_barrier<0>();
  }
  if constexpr (kWiden) read_slice(st0, 0, 0);
  else read_slice8(st0, 0, 0);

  // Stage ring: block kb is in stage kb % 3; block kb + 2 is loaded while kb
  // is multiplied; the barrier inside step kb makes block kb + 1 visible and,
  // since every read of stage kb % 3 precedes it, lets step kb + 1 refill
  // that stage with block kb + 3.  The steady-state loop issues its loads
  // unconditionally (three blocks per iteration, every one with kb + 2 < KB);
  // the last (up to four) blocks run in a tail with the conditions spelled
  // out.  Scale group g + 1 (blocks 4 g + 4 ..) is loaded at step 4 g + 1,
  // ahead of that step's tile loads, so the barrier inside step 4 g + 1
  // already covers it; its buffer held group g - 1, last read in step
  // 4 g - 1, which every wave has finished once it passes the barrier of
  // step 4 g.
#define FP8BS_STEP_FULL(KIND, CUR, NXT, FUT, KBV)                          \
  {                                                                       \
    const int kb_ = (KBV);                                                \
    if ((kb_ & 3) == 1 && kb_ + 3 < KB) load_scales((kb_ >> 2) + 1);      \
    load_stage(FUT, kb_ + 2);                                             \
    const float sbv_ = kRowScale ? 1.0f : sb_blk[kb_];                    \
    step(KIND##_PAR{}, KIND##_IN{}, KIND##_KEEP{}, CUR, NXT, kb_, sbv_, 1);  \
  }
#define FP8BS_STEP_TAIL(KIND, CUR, NXT, FUT, KBV)                          \
  if ((KBV) < KB) {                                                       \
    const int kb_ = (KBV);                                                \
    if ((kb_ & 3) == 1 && kb_ + 3 < KB) load_scales((kb_ >> 2) + 1);      \
    if (kb_ + 2 < KB) load_stage(FUT, kb_ + 2);                           \
    const float sbv_ = kRowScale ? 1.0f : sb_blk[kb_];                    \
    step(KIND##_PAR{}, KIND##_IN{}, KIND##_KEEP{}, CUR, NXT, kb_, sbv_,   \
         kb_ + 1 >= KB ? 0 : (kb_ + 2 < KB ? 1 : 2));                      \
  }
  // With kLag, blocks 3 j, 3 j + 1, 3 j + 2 are steps of kinds A, B, C:
  // A accumulates into p[0] and stays pending; B promotes it while
  // accumulating into p[1], which stays pending; C promotes that while
  // accumulating into p[0] and promotes its own block at its end.  So no
  // block is pending across iterations, and two promotions in three overlap
  // matrix work.  (Alternating all blocks would need a six-block loop,
  // whose code the compiler cannot fit in the register budget.)
  using A_PAR = std::integral_constant<int, 0>;
  using A_IN = std::false_type;
  using A_KEEP = std::true_type;
  using B_PAR = std::integral_constant<int, 1>;
  using B_IN = std::true_type;
  using B_KEEP = std::true_type;
  using C_PAR = std::integral_constant<int, 0>;
  using C_IN = std::true_type;
  using C_KEEP = std::false_type;
  int kb = 0;
  for (; kb + 4 < KB; kb += 3) {
    FP8BS_STEP_FULL(A, st0, st1, st2, kb)
    FP8BS_STEP_FULL(B, st1, st2, st0, kb + 1)
    FP8BS_STEP_FULL(C, st2, st0, st1, kb + 2)
  }
  FP8BS_STEP_TAIL(A, st0, st1, st2, kb)
  FP8BS_STEP_TAIL(B, st1, st2, st0, kb + 1)
  FP8BS_STEP_TAIL(C, st2, st0, st1, kb + 2)
  FP8BS_STEP_TAIL(A, st0, st1, st2, kb + 3)
#undef FP8BS_STEP_FULL
#undef FP8BS_STEP_TAIL
  }  // !idle

  // kLag: the last block, K block KB - 1, may still be pending: in p[0]
  // after an A step and in p[1] after a B step.
  if constexpr (kLag) {
    const int last = idle ? -1 : (KB - 1) % 3;
#pragma unroll
    for (int i = 0; i < SM; ++i)
#pragma unroll
      for (int j = 0; j < SN; ++j) {
        if (last == 1) promote(std::integral_constant<int, 1>{}, i, j, cl[i]);
        else if (last == 0) promote(std::integral_constant<int, 0>{}, i, j, cl[i]);
      }
  }

  if constexpr (kOut == kOutE4M3) {
    // Output quantized in 1x128 tiles: the N tile is 128 wide, so each of its
    // rows is one whole tile.  Row amax over this lane's 32 values, the
    // partner lane (lane ^ 32) and the other wave column (through LDS); then
    // s = fl32(amax/448) with the 1e-10 guard and codes of fl32(y/s), the
    // same operations as the 1x128 quantizer on a float32 input.  Codes go
    // through an LDS tile (the first stage buffer, free after the main loop;
    // row pitch 144 bytes) and leave as whole 128-byte rows.
    static_assert(C::BN == 128, "one 1x128 output tile per row of the N tile");
    constexpr int kPitch = 144;
    static_assert(C::BM * kPitch <= int(sizeof(St)), "code tile fits the stage buffer");
    __shared__ float rmax[C::WN][C::BM];
    uint8_t* ct = reinterpret_cast<uint8_t*>(&st0);
    __syncthreads();   // every wave is past its last read of the stages
    float m[SM];
#pragma unroll
    for (int i = 0; i < SM; ++i) {
      float v = 0.0f;
#pragma unroll
      for (int j = 0; j < SN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) v = fmaxf(v, fabsf(acc[i][j][r]));
      v = fmaxf(v, __shfl_xor(v, 32));
      m[i] = v;
    }
    if (hk == 0) {
#pragma unroll
      for (int i = 0; i < SM; ++i) rmax[wn][arow0 + 32 * i] = m[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < SM; ++i) {
      const int rl = arow0 + 32 * i;
      float amax = rmax[0][rl];
#pragma unroll
      for (int w = 1; w < C::WN; ++w) amax = fmaxf(amax, rmax[w][rl]);
      const float sc = tile_scale(amax);
#pragma unroll
      for (int j = 0; j < SN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int cl = wn * C::TN + 32 * j + 8 * g + 4 * hk;
          *reinterpret_cast<uint32_t*>(ct + rl * kPitch + cl) =
              pack4_e4m3(acc[i][j][4 * g] / sc, acc[i][j][4 * g + 1] / sc, acc[i][j][4 * g + 2] / sc,
                         acc[i][j][4 * g + 3] / sc);
        }
      const int64_t row = tile.row0 + rl;
      if (wn == 0 && hk == 0 && row < tile.row_end)
        args.y_scale[row * (args.N / 128) + tile.n0 / 128] = sc;
    }
    __syncthreads();
    uint8_t* yq = static_cast<uint8_t*>(args.y);
#pragma unroll
    for (int c = threadIdx.x; c < C::BM * 8; c += C::kThreads) {
      const int rl = c >> 3, ch = c & 7;
      const int64_t row = tile.row0 + rl;
      if (row < tile.row_end) store16_nt(yq + row * args.ldy + tile.n0 + 16 * ch, ct + rl * kPitch + 16 * ch);
    }
  } else {
    // Epilogue through LDS.  A lane's accumulators hold four consecutive
    // columns of 32 different rows per register group, so direct stores
    // would scatter each instruction over 32 rows.  Instead each wave writes
    // its converted values row-major into LDS (rows [0, BM/2) in the first
    // stage buffer, the rest in the second; row pitch = the round's columns
    // plus 16 bytes), and the workgroup then stores whole rows with 16-byte
    // chunks, consecutive threads on consecutive addresses.  bf16 output
    // takes the whole tile in one round; f32 output one wave column (TN
    // columns) per round.  Every tile of this configuration is one wave of
    // workgroups on the chip, so these stores are not hidden behind other
    // tiles' matrix work: whole-line (and nontemporal) writes keep them
    // short.
    constexpr int kElt = kOut == kOutBf16 ? 2 : 4;
    constexpr int kRounds = kOut == kOutBf16 ? 1 : C::WN;
    constexpr int kCols = C::BN / kRounds;            // columns per round
    constexpr int kPitch = kCols * kElt + 16;         // LDS row pitch (bytes)
    constexpr int kHalf = C::BM / 2;
    static_assert(kHalf * kPitch <= int(sizeof(St)), "half the output tile fits a stage buffer");
    static_assert(C::TM <= kHalf && kHalf % C::TM == 0, "a wave's rows lie in one half");
    constexpr int kChunks = kCols * kElt / 16;        // 16-byte chunks per row and round
    uint8_t* const lo_half = reinterpret_cast<uint8_t*>(&st0);
    uint8_t* const hi_half = reinterpret_cast<uint8_t*>(&st1);
    __syncthreads();   // every wave is past its last read of the stages
#pragma unroll
    for (int rd = 0; rd < kRounds; ++rd) {
      if (kRounds == 1 || wn == rd) {
        const int c0 = kRounds == 1 ? wn * C::TN : 0;   // the wave's first column in this round
#pragma unroll
        for (int i = 0; i < SM; ++i) {
          const int rl = arow0 + 32 * i;
          uint8_t* rowp = (rl < kHalf ? lo_half : hi_half) + (rl % kHalf) * kPitch;
#pragma unroll
          for (int j = 0; j < SN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int cl = c0 + 32 * j + 8 * g + 4 * hk;
              const float v0 = acc[i][j][4 * g], v1 = acc[i][j][4 * g + 1];
              const float v2 = acc[i][j][4 * g + 2], v3 = acc[i][j][4 * g + 3];
              if constexpr (kOut == kOutBf16) {
                *reinterpret_cast<uint2*>(rowp + cl * 2) =
                    make_uint2(f32_to_bf16_rne(v0) | (f32_to_bf16_rne(v1) << 16),
                               f32_to_bf16_rne(v2) | (f32_to_bf16_rne(v3) << 16));
              } else {
                *reinterpret_cast<float4*>(rowp + cl * 4) = make_float4(v0, v1, v2, v3);
              }
            }
        }
      }
      __syncthreads();
      const int64_t col0 = tile.n0 + (kRounds == 1 ? 0 : rd * kCols);
      uint8_t* ybase = static_cast<uint8_t*>(args.y);
#pragma unroll 4
      for (int c = threadIdx.x; c < C::BM * kChunks; c += C::kThreads) {
        const int rl = c / kChunks, ch = c % kChunks;
        const int64_t row = tile.row0 + rl;
        const int64_t col = col0 + ch * (16 / kElt);
        if (row < tile.row_end && col < args.N)
          store16_nt(ybase + (row * args.ldy + col) * kElt, (rl < kHalf ? lo_half : hi_half) + (rl % kHalf) * kPitch + ch * 16);
      }
      if (rd + 1 < kRounds) __syncthreads();   // the next round rewrites the buffers
    }
  }
}

// ---------------------------------------------------------------------------
using CfgLarge = TileCfg<256, 128, 4, 2>;   // 256 x 128 tile, 8 waves of 64 x 64
using CfgSmall = TileCfg<128, 128, 2, 2>;   // 128 x 128 tile, 4 waves of 64 x 64

// Launches the kernel variant for one tile configuration; `out` is an
// OutKind.  Only the variants the entry points can reach are instantiated:
// E4M3 output exists for the dense exact path only.
template <class C, bool kWiden, bool kRowScale, bool kGrouped>
void launch_cfg(const GemmArgs& args, int out, uint32_t n_wg, hipStream_t stream) {
  const dim3 grid(n_wg), block(C::kThreads);
  if (out == kOutBf16) {
    hipLaunchKernelGGL((gemm_kernel<C, kWiden, kRowScale, kOutBf16, kGrouped>), grid, block, 0, stream, args);
  } else if (out == kOutF32) {
    hipLaunchKernelGGL((gemm_kernel<C, kWiden, kRowScale, kOutF32, kGrouped>), grid, block, 0, stream, args);
  } else if constexpr (kWiden && !kGrouped) {
    hipLaunchKernelGGL((gemm_kernel<C, kWiden, kRowScale, kOutE4M3, kGrouped>), grid, block, 0, stream, args);
  }
}

// Tile size: the large tile when it still gives at least one workgroup per
// CU, otherwise the small one.
constexpr int64_t kNumCU = 256;

}  // namespace
}  // namespace fp8bs

using namespace fp8bs;

namespace fp8bs {
namespace {

// Shared by the dense entry points.  `out` is an OutKind; for kOutE4M3, y
// holds the codes (pitch ldy bytes) and y_scale the [M, N/128] scales.
// `widen`: the exact path (E4M3 widened to bf16, bf16 matrix instructions);
// otherwise the FP8 matrix instructions.
fp8bs_status dense_gemm(const char* fn, int64_t M, int64_t N, int64_t K, const uint8_t* a,
                        int64_t lda, const float* a_scale, const uint8_t* b, int64_t ldb,
                        const float* b_scale, int32_t b_kind, void* y, int out, int64_t ldy,
                        float* y_scale, bool widen, hipStream_t stream) {
  if (M < 0 || N < 0 || K < 0) return fail(FP8BS_ERR_INVALID_ARG, "%s: negative size", fn);
  if (b_kind != FP8BS_BSCALE_BLOCK128 && b_kind != FP8BS_BSCALE_ROW)
    return fail(FP8BS_ERR_INVALID_ARG, "%s: unknown b_kind %d", fn, b_kind);
  if (K % 128 || K < 128) return fail(FP8BS_ERR_SHAPE, "%s: K=%lld must be a positive multiple of 128", fn, (long long)K);
  if (b_kind == FP8BS_BSCALE_BLOCK128 && N % 128)
    return fail(FP8BS_ERR_SHAPE, "%s: block128 B scales need N %% 128 == 0 (N=%lld)", fn, (long long)N);
  if (out == kOutE4M3 && N % 128)
    return fail(FP8BS_ERR_SHAPE, "%s: 1x128 output tiles need N %% 128 == 0 (N=%lld)", fn, (long long)N);
  if (N % 16) return fail(FP8BS_ERR_SHAPE, "%s: N=%lld must be a multiple of 16", fn, (long long)N);
  if (M == 0 || N == 0) return FP8BS_OK;
  if (!a || !b || !a_scale || !b_scale || !y || (out == kOutE4M3 && !y_scale))
    return fail(FP8BS_ERR_INVALID_ARG, "%s: null pointer", fn);
  const int64_t y_elt = out == kOutF32 ? 4 : (out == kOutBf16 ? 2 : 1);
  if (lda < K || ldb < K || ldy < N) return fail(FP8BS_ERR_INVALID_ARG, "%s: pitch smaller than the row", fn);
  if (!aligned16(a) || !aligned16(b) || !aligned16(y) || lda % 16 || ldb % 16 || (ldy * y_elt) % 16)
    return fail(FP8BS_ERR_ALIGNMENT, "%s: operands and row pitches must be 16-byte aligned", fn);
  if (!aligned4(a_scale) || !aligned4(b_scale) || (y_scale && !aligned4(y_scale)))
    return fail(FP8BS_ERR_ALIGNMENT, "%s: scales must be 4-byte aligned", fn);
  if (M > 0x7fffffff || N > 0x7fffffff)
    return fail(FP8BS_ERR_INVALID_ARG, "%s: dimension too large", fn);
  if (!sane_matrix(M, ldy, int(y_elt)) || !sane_matrix(M, lda, 1) || !sane_matrix(N, ldb, 1))
    return fail(FP8BS_ERR_INVALID_ARG, "%s: sizes and pitches exceed any allocation", fn);
  // Offsets inside one tile are 32-bit: 256 rows of codes or scales.
  if (lda > (int64_t(1) << 22) || ldb > (int64_t(1) << 22) || K / 128 * 256 * 4 > 0x7fffffff)
    return fail(FP8BS_ERR_INVALID_ARG, "%s: row pitch too large", fn);

  GemmArgs args{};
  args.a = a; args.a_scale = a_scale; args.b = b; args.b_scale = b_scale; args.y = y;
  args.y_scale = y_scale;
  args.off = nullptr;
  args.lda = lda; args.ldb = ldb; args.ldy = ldy;
  args.M = int32_t(M); args.N = int32_t(N); args.KB = int32_t(K / 128);
  args.G = 1;
  const bool row = b_kind == FP8BS_BSCALE_ROW;
  const int64_t tiles_large = ((M + 255) / 256) * ((N + 127) / 128);
  // The 256 x 128 tile when it gives at least one workgroup per CU, else
  // the 128 x 128 tile.
  const int bm = tiles_large >= kNumCU ? 256 : 128;
  args.tiles_m = int32_t((M + bm - 1) / bm);
  args.tiles_n = int32_t((N + 127) / 128);
  const int64_t n_wg = int64_t(args.tiles_m) * args.tiles_n;
  if (n_wg > 0x7fffffff) return fail(FP8BS_ERR_INVALID_ARG, "%s: too many tiles", fn);
  begin_launch();
#define FP8BS_DENSE(W)                                                                         \
  if (tiles_large >= kNumCU) {                                                                 \
    if (row) launch_cfg<CfgLarge, W, true, false>(args, out, uint32_t(n_wg), stream);           \
    else launch_cfg<CfgLarge, W, false, false>(args, out, uint32_t(n_wg), stream);             \
  } else {                                                                                     \
    if (row) launch_cfg<CfgSmall, W, true, false>(args, out, uint32_t(n_wg), stream);          \
    else launch_cfg<CfgSmall, W, false, false>(args, out, uint32_t(n_wg), stream);             \
  }
  if (widen) { FP8BS_DENSE(true) } else { FP8BS_DENSE(false) }
#undef FP8BS_DENSE
  return check_launch(fn);
}

}  // namespace
}  // namespace fp8bs

extern "C" fp8bs_status fp8_blockscaled_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a,
                                             int64_t lda, const float* a_scale, const uint8_t* b,
                                             int64_t ldb, const float* b_scale, int32_t b_kind,
                                             void* y, int32_t y_dtype, int64_t ldy, hipStream_t stream) {
  const char* fn = "fp8_blockscaled_gemm";
  if (!valid_dtype(y_dtype)) return fail(FP8BS_ERR_INVALID_ARG, "%s: unknown y_dtype %d", fn, y_dtype);
  return dense_gemm(fn, M, N, K, a, lda, a_scale, b, ldb, b_scale, b_kind, y,
                    y_dtype == FP8BS_BF16 ? kOutBf16 : kOutF32, ldy, nullptr, true, stream);
}

extern "C" fp8bs_status fp8_blockscaled_gemm_fp8mma(int64_t M, int64_t N, int64_t K, const uint8_t* a,
                                                    int64_t lda, const float* a_scale, const uint8_t* b,
                                                    int64_t ldb, const float* b_scale, int32_t b_kind,
                                                    void* y, int32_t y_dtype, int64_t ldy,
                                                    hipStream_t stream) {
  const char* fn = "fp8_blockscaled_gemm_fp8mma";
  if (!valid_dtype(y_dtype)) return fail(FP8BS_ERR_INVALID_ARG, "%s: unknown y_dtype %d", fn, y_dtype);
  return dense_gemm(fn, M, N, K, a, lda, a_scale, b, ldb, b_scale, b_kind, y,
                    y_dtype == FP8BS_BF16 ? kOutBf16 : kOutF32, ldy, nullptr, false, stream);
}

extern "C" fp8bs_status fp8_blockscaled_gemm_quant(int64_t M, int64_t N, int64_t K, const uint8_t* a,
                                                   int64_t lda, const float* a_scale, const uint8_t* b,
                                                   int64_t ldb, const float* b_scale, int32_t b_kind,
                                                   uint8_t* yq, int64_t ldyq, float* y_scale,
                                                   hipStream_t stream) {
  return dense_gemm("fp8_blockscaled_gemm_quant", M, N, K, a, lda, a_scale, b, ldb, b_scale, b_kind,
                    yq, kOutE4M3, ldyq, y_scale, true, stream);
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
  if (M_total > 0x7fffffff || N > 0x7fffffff) return fail(FP8BS_ERR_INVALID_ARG, "%s: size too large", fn);
  if (!sane_matrix(M_total, N, elem_size(y_dtype)) || !sane_matrix(M_total, K, 1) ||
      !sane_matrix(int64_t(G) * N, K, 1))
    return fail(FP8BS_ERR_INVALID_ARG, "%s: sizes exceed any allocation", fn);
  if (K > (int64_t(1) << 22)) return fail(FP8BS_ERR_INVALID_ARG, "%s: K too large", fn);

  GemmArgs args{};
  args.a = a; args.a_scale = a_scale; args.b = b; args.b_scale = b_scale; args.y = y;
  args.off = off;
  args.lda = K; args.ldb = K; args.ldy = N;
  args.b_group_stride = N * K;
  args.bs_group_stride = (N / 128) * (K / 128);
  args.M = int32_t(M_total); args.N = int32_t(N); args.KB = int32_t(K / 128);
  args.G = G;
  const int out = y_dtype == FP8BS_BF16 ? kOutBf16 : kOutF32;
  // Upper bound on sum_g ceil(m_g / BM): ceil(M_total / BM) + G.
  const int64_t tiles_large = ((M_total + 255) / 256 + G) * (N / 128);
  const bool large = tiles_large >= 2 * kNumCU;
  const int bm = large ? 256 : 128;
  args.tiles_m = int32_t((M_total + bm - 1) / bm + G);
  args.tiles_n = int32_t(N / 128);
  const int64_t n_wg = int64_t(args.tiles_m) * args.tiles_n;
  if (n_wg > 0x7fffffff) return fail(FP8BS_ERR_INVALID_ARG, "%s: too many tiles", fn);
  begin_launch();
  if (large) launch_cfg<CfgLarge, true, false, true>(args, out, uint32_t(n_wg), stream);
  else launch_cfg<CfgSmall, true, false, true>(args, out, uint32_t(n_wg), stream);
  return check_launch(fn);
}
