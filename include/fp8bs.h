/*
 * fp8bs.h - fine-grained FP8 (E4M3) block-scaled quantization and GEMM on
 * AMD MI355X (gfx950).  C ABI of libfp8bs.so.
 *
 * The method (sources cited per call below):
 *  - codingmall.com knowledge-base article on the role of FP8 precision in
 *    DeepSeek-V3 training, section "Finkornig kvantisering": activations are
 *    scaled per 1x128 tile and weights per 128x128 block; section
 *    "Online-kvantisering": each scale comes from its own tile's current
 *    values; section "Ökad ackumuleringsprecision": GEMM partial sums are
 *    promoted into FP32 at fixed intervals; section "Unified E4M3 Format":
 *    E4M3 for every GEMM operand, forward and backward.
 *  - HolySheep AI (zh) article on FP8 mixed-precision training at
 *    DeepSeek-671B scale, section "2.2 细粒度量化实现" (fine-grained
 *    quantization implementation), class FP8BlockQuantizer: per tile,
 *    scale = amax / 448 (a scale not above 1e-10 becomes 1), codes = E4M3 of
 *    x / scale, the FP32 scale is returned beside the codes, and
 *    dequantization multiplies by it.
 *
 * Conventions shared by every call:
 *  - All data pointers are DEVICE pointers owned by the caller.  The library
 *    allocates nothing, keeps no state between calls, never synchronizes and
 *    enqueues its work on `stream` (0 = the null stream).
 *  - Matrices are row-major.  `ld_*` is the row pitch in ELEMENTS.  E4M3
 *    codes are uint8 (OCP E4M3FN: bias 7, max 448 = 0x7E, no infinity,
 *    S.1111.111 = NaN).  Scales are float32 and dense (row pitch = number of
 *    scale columns).
 *  - Validation is synchronous.  Every status other than FP8BS_ERR_HIP comes
 *    from it, and then nothing is enqueued and no output byte is written;
 *    fp8bs_last_error() gives the reason.  FP8BS_ERR_HIP means the HIP
 *    runtime refused a launch of this call (any HIP error left over from an
 *    earlier call on the thread is cleared before the first launch); in a
 *    call that enqueues several kernels the earlier ones may then already
 *    be enqueued.  Device-side faults surface at the caller's next
 *    synchronization.
 *  - Zero rows (or M = 0) is a no-op that returns FP8BS_OK.
 *  - Alignment: every code/input/output pointer 16-byte aligned and every
 *    row pitch a multiple of 16 bytes; scale pointers 4-byte aligned.
 *  - Quantization rounds to nearest (ties to even) and saturates at +-448; it
 *    never reports a range error.  Inputs must be finite: a NaN or infinity
 *    gives unspecified codes and scale for the tiles that hold it, and
 *    leaves every other tile as it would be without it.
 *  - Tiled dimensions must be whole multiples of 128 (FP8BS_ERR_SHAPE);
 *    partial tail tiles are rejected, not dropped.
 *  - Thread-safe: the only global state is the thread-local error text.
 */
#ifndef FP8BS_H
#define FP8BS_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fp8bs_status {
  FP8BS_OK = 0,
  FP8BS_ERR_INVALID_ARG = 1,   /* null pointer, negative size, pitch too small, bad enum */
  FP8BS_ERR_SHAPE = 2,         /* a tiled dimension is not a multiple of 128, or K < 128 */
  FP8BS_ERR_ALIGNMENT = 3,     /* pointer or pitch not aligned as required */
  FP8BS_ERR_UNSUPPORTED = 4,   /* valid enum values in a combination not provided */
  FP8BS_ERR_HIP = 5            /* the HIP runtime refused the launch */
} fp8bs_status;

typedef enum fp8bs_dtype { FP8BS_BF16 = 0, FP8BS_F32 = 1 } fp8bs_dtype;

typedef enum fp8bs_act_tiling {
  FP8BS_TILE_1x128 = 0,        /* 128 consecutive elements of a row */
  FP8BS_TILE_128x1_T = 1,      /* 128 consecutive rows of a column; codes written transposed */
  FP8BS_TILE_128x128 = 2       /* 128x128 blocks (weights); accepted by fp8_dequant */
} fp8bs_act_tiling;

typedef enum fp8bs_format {
  FP8BS_FMT_E4M3 = 0,          /* OCP E4M3FN, max 448 */
  FP8BS_FMT_E5M2 = 1           /* OCP E5M2, max 57344 (per-tensor baselines only) */
} fp8bs_format;

typedef enum fp8bs_bscale_kind {
  FP8BS_BSCALE_BLOCK128 = 0,   /* b_scale[N/128][K/128]: one scale per 128x128 block of B */
  FP8BS_BSCALE_ROW = 1         /* b_scale[N][K/128]: one scale per row of B and 128-K block */
} fp8bs_bscale_kind;

/*
 * Online activation quantization (codingmall "Finkornig kvantisering" /
 * "Online-kvantisering"; HolySheep (zh) section 2.2, FP8BlockQuantizer).
 *
 * x:       [rows, cols] of x_dtype (bf16 or f32), pitch ld_x >= cols.
 * tiling = FP8BS_TILE_1x128: needs cols % 128 == 0.
 *     q     [rows, cols] uint8, pitch ld_q >= cols;
 *     scale [rows, cols/128] float32.
 * tiling = FP8BS_TILE_128x1_T (operands of the weight-gradient GEMM, whose
 *   contraction runs over rows/tokens): needs rows % 128 == 0.
 *     q     [cols, rows] uint8 = codes of x^T, pitch ld_q >= rows;
 *     scale [cols, rows/128] float32.
 * Per tile: s = fl32(amax/448), s = 1 if not s > fl32(1e-10);
 * code = E4M3_RNE_SAT(fl32(x/s)).  Codes and scales are bit-exact with that
 * definition.
 */
fp8bs_status fp8_quant_act_1x128(const void* x, int32_t x_dtype, int64_t rows, int64_t cols,
                                 int64_t ld_x, int32_t tiling, uint8_t* q, int64_t ld_q,
                                 float* scale, hipStream_t stream);

/*
 * Weight quantization in 128x128 blocks (codingmall "Finkornig
 * kvantisering"; HolySheep (zh) section 2.2 rule applied per block).
 *
 * w:       [rows, cols] of w_dtype, pitch ld_w >= cols; rows % 128 == 0 and
 *          cols % 128 == 0.
 * q:       [rows, cols] uint8, pitch ld_q >= cols.
 * scale:   [rows/128, cols/128] float32.
 * q_t:     optional (may be NULL): the same codes transposed, [cols, rows],
 *          pitch ld_qt >= rows (the B operand of the data-gradient GEMM).
 *          A block's scale does not depend on its orientation, so the scale
 *          grid of q_t is scale transposed ([cols/128, rows/128]): a view of
 *          scale, not a separate output.
 */
fp8bs_status fp8_quant_w_128x128(const void* w, int32_t w_dtype, int64_t rows, int64_t cols,
                                 int64_t ld_w, uint8_t* q, int64_t ld_q, float* scale,
                                 uint8_t* q_t, int64_t ld_qt, hipStream_t stream);

/*
 * Several quantization jobs in one launch: each job is what
 * fp8_quant_act_1x128 computes with FP8BS_TILE_1x128, or what
 * fp8_quant_w_128x128 computes without the transposed copy, with the same
 * arguments (codingmall "Finkornig kvantisering": 1x128 activation tiles and
 * 128x128 weight blocks, each with its own scale; HolySheep (zh) section 2.2
 * rule per tile).  Outputs are bit-identical to the single calls.  One launch
 * pays the machine's fill and drain once for all jobs: a linear layer's
 * activations and weight, or the separate weights of several experts.
 *
 * jobs:    HOST array of n_jobs descriptors, read during the call only.
 *   x, x_dtype, rows, cols, ld_x: the input, as for the single calls;
 *   tiling:  FP8BS_TILE_1x128 (needs cols % 128 == 0) or FP8BS_TILE_128x128
 *            (needs rows % 128 == 0 and cols % 128 == 0);
 *   q, ld_q: codes [rows, cols];
 *   scale:   [rows, cols/128] (1x128) or [rows/128, cols/128] (128x128).
 * n_jobs:  0 .. FP8BS_MAX_QUANT_JOBS.  Jobs with zero rows or columns are
 *          skipped.  The outputs of different jobs must not overlap.
 * Every job is validated before anything is enqueued; the error text names
 * the failing job.
 */
#define FP8BS_MAX_QUANT_JOBS 8
typedef struct fp8bs_quant_job {
  const void* x;
  int32_t x_dtype;
  int32_t tiling;
  int64_t rows;
  int64_t cols;
  int64_t ld_x;
  uint8_t* q;
  int64_t ld_q;
  float* scale;
} fp8bs_quant_job;

fp8bs_status fp8_quant_batch(const fp8bs_quant_job* jobs, int32_t n_jobs, hipStream_t stream);

/*
 * Both activation tilings of one tensor in a single pass over it: what
 * fp8_quant_act_1x128 writes with FP8BS_TILE_1x128 and with
 * FP8BS_TILE_128x1_T, from one read of x.  The backward pass needs both for
 * the same tensor (codingmall "Unified E4M3 Format": the data-gradient GEMM
 * contracts the output gradient over its columns, the weight-gradient GEMM
 * over its rows/tokens; "Finkornig kvantisering" fixes the 1x128 tiles).
 *
 * x:       [rows, cols] of x_dtype, pitch ld_x >= cols; rows % 128 == 0 and
 *          cols % 128 == 0.
 * q:       [rows, cols] uint8, pitch ld_q >= cols (1x128 tiles along rows);
 * scale:   [rows, cols/128] float32.
 * q_t:     [cols, rows] uint8, pitch ld_qt >= rows: codes of x^T (128x1
 *          tiles of x, i.e. 1x128 tiles of x^T);
 * scale_t: [cols, rows/128] float32.
 * Every output is required (non-NULL) and must not overlap another.  Codes
 * and scales are bit-identical to the two single-tiling calls.
 */
fp8bs_status fp8_quant_act_dual(const void* x, int32_t x_dtype, int64_t rows, int64_t cols,
                                int64_t ld_x, uint8_t* q, int64_t ld_q, float* scale,
                                uint8_t* q_t, int64_t ld_qt, float* scale_t,
                                hipStream_t stream);

/*
 * Dequantization (HolySheep (zh) section 2.2, FP8BlockQuantizer.dequantize:
 * each code's value times its tile's stored scale):
 *   y[r,c] = fl32(e4m3(q[r,c]) * s),  bf16 output: that float32 rounded to
 *   nearest even.  The product is exact before its one float32 rounding.
 *
 * q:       [rows, cols] uint8 codes, pitch ld_q >= cols; cols % 128 == 0.
 * scale:   tiling FP8BS_TILE_1x128:   [rows, cols/128] float32;
 *          tiling FP8BS_TILE_128x128: [rows/128, cols/128] (rows % 128 == 0).
 *          (The output of the 128x1_T tiling is the 1x128 tiling of x^T:
 *          pass it as FP8BS_TILE_1x128 to get x^T back.)
 * y:       [rows, cols] of y_dtype, pitch ldy >= cols.
 * NaN codes (S.1111.111) give NaN.
 */
fp8bs_status fp8_dequant(const uint8_t* q, int64_t rows, int64_t cols, int64_t ld_q,
                         const float* scale, int32_t tiling, void* y, int32_t y_dtype,
                         int64_t ldy, hipStream_t stream);

/*
 * Per-tensor quantization: the prior-art scalings that the fine-grained
 * tiles are compared with (one scale for the whole tensor).
 *
 * Current scaling (history == NULL), HolySheep (zh) troubleshooting entry
 * on FP8 overflow, SafeFP8Quantizer.safe_quantize, whose scale arithmetic
 * is on Python (binary64) floats:
 *   amax = max|x|;  d = rn64(rn64(amax * rn64(1 + margin)) / fmt_max);
 *   s = 1 if d < 1e-6 (binary64), else s = fl32(d);
 *   code = SAT(RNE(fl32(x / s))).
 *   Two passes over x (amax, then the codes).
 * Delayed scaling (history != NULL), HolySheep (zh) FP8Config
 *   (amax_history_len 1024, margin 0): the same formula with amax replaced
 *   by max(history[0 .. history_len)), the amaxes of earlier calls; codes
 *   saturate at the format maximum (a stale scale can be too small); then
 *   history becomes [max|x|, history[0 .. history_len-2]].  One pass.
 *
 * format:  fp8bs_format.  E5M2 is the hybrid recipe's gradient format
 *          (German HolySheep article); DeepSeek-V3 uses E4M3 throughout
 *          (codingmall "Unified E4M3 Format").
 * x:       [rows, cols] of x_dtype, pitch ld_x >= cols; cols % 8 == 0.
 * q:       [rows, cols] uint8 codes, pitch ld_q >= cols.
 * scale:   DEVICE float[1]: the dequantizing scale s used.
 * amax:    DEVICE float[1]: max|x| of this call (also the reduction's
 *          accumulator).
 * history: DEVICE float[history_len] (1..4096) or NULL; updated in place.
 * margin:  binary64 in [0, 1e6] (the page's margin is a Python float, e.g.
 *          0.1 or 0.15).  Zero rows or columns: nothing is written (the
 *          history is unchanged).  Inputs must be finite.
 */
fp8bs_status fp8_quant_tensor(const void* x, int32_t x_dtype, int64_t rows, int64_t cols,
                              int64_t ld_x, int32_t format, double margin, float* history,
                              int32_t history_len, uint8_t* q, int64_t ld_q, float* scale,
                              float* amax, hipStream_t stream);

/*
 * Block-scaled FP8 GEMM with FP32 promotion per 128-deep K block
 * (codingmall "Ökad ackumuleringsprecision"):
 *   y[m,n] = sum_kb  a_scale[m,kb] * bs(n,kb) * P_kb[m,n],
 *   P_kb[m,n] = sum_{k in block kb} e4m3(a[m,k]) * e4m3(b[n,k])
 * where P_kb comes from the matrix cores and the promotion is an FP32
 * multiply-add per K block.  Each product of two E4M3 values is exact and
 * the 128 products of a K block are summed in FP32: the codes are widened
 * to bf16 (exactly) inside the kernel and multiplied on the bf16 matrix
 * cores.
 *
 * a:       [M, K] codes, pitch lda >= K;  a_scale [M, K/128] float32.
 * b:       [N, K] codes, pitch ldb >= K (y = A . B^T).
 * b_scale: BLOCK128: [N/128, K/128] (needs N % 128 == 0);
 *          ROW:      [N, K/128].
 * y:       [M, N] of y_dtype (f32, or bf16 rounded to nearest even), pitch
 *          ldy >= N.
 * K % 128 == 0 and K >= 128; N % 16 == 0.  M may be any count >= 0.
 * Accuracy: |y - exact| <= 2e-5 * sum_k |a_k b_k| (+ half a bf16 ulp for
 * bf16 output), where a_k, b_k are the dequantized operands.
 */
fp8bs_status fp8_blockscaled_gemm(int64_t M, int64_t N, int64_t K,
                                  const uint8_t* a, int64_t lda, const float* a_scale,
                                  const uint8_t* b, int64_t ldb, const float* b_scale,
                                  int32_t b_kind, void* y, int32_t y_dtype, int64_t ldy,
                                  hipStream_t stream);

/*
 * NOT COVERED BY THE ACCURACY CONTRACT: fp8_blockscaled_gemm computed with
 * the gfx950 FP8 matrix instructions, at twice their peak rate, for
 * comparison.  Same arguments, layouts and errors as fp8_blockscaled_gemm.
 * These instructions add products in groups of 8 consecutive K and keep only
 * the bits down to 2^-13 of each group's largest product (truncating the
 * rest) before combining the groups in FP32: an error of up to about
 * 7 * 2^-13 of the largest product per group of 8, which exceeds
 * 2e-5 * sum_k |a_k b_k| when one product dominates its group (as the
 * activations' outliers make it).  This is the limited matrix-core
 * accumulation that codingmall "Ökad ackumuleringsprecision" describes, here
 * inside every instruction, so promoting more often cannot remove it.
 */
fp8bs_status fp8_blockscaled_gemm_fp8mma(int64_t M, int64_t N, int64_t K,
                                         const uint8_t* a, int64_t lda, const float* a_scale,
                                         const uint8_t* b, int64_t ldb, const float* b_scale,
                                         int32_t b_kind, void* y, int32_t y_dtype, int64_t ldy,
                                         hipStream_t stream);

/*
 * The block-scaled GEMM with its output quantized in 1x128 tiles inside the
 * GEMM's epilogue: the online quantization of the next GEMM's activations
 * done by their producer (codingmall "Online-kvantisering": each tile's
 * scale comes from its current values; "Finkornig kvantisering": 1x128
 * activation tiles).  Every 128-wide output tile of a row is whole inside
 * one workgroup, so no extra pass over y is needed.
 *
 * Same operands and accuracy as fp8_blockscaled_gemm; N % 128 == 0.
 * The float32 result y[m,n] (the value fp8_blockscaled_gemm would store
 * with FP8BS_F32) is quantized exactly as fp8_quant_act_1x128 quantizes a
 * float32 input:
 *   yq:      [M, N] uint8 codes, pitch ldyq >= N (16-byte aligned);
 *   y_scale: [M, N/128] float32, s = fl32(amax/448) (1 if not above
 *            fl32(1e-10)), codes = E4M3_RNE_SAT(fl32(y/s)).
 */
fp8bs_status fp8_blockscaled_gemm_quant(int64_t M, int64_t N, int64_t K,
                                        const uint8_t* a, int64_t lda, const float* a_scale,
                                        const uint8_t* b, int64_t ldb, const float* b_scale,
                                        int32_t b_kind, uint8_t* yq, int64_t ldyq,
                                        float* y_scale, hipStream_t stream);

/*
 * Grouped (mixture-of-experts) block-scaled GEMM: group g owns rows
 * [off[g], off[g+1]) of a and y and has its own weight b[g]
 * (HolySheep (zh) MoE module: each expert multiplies its own tokens).
 *
 * off:     DEVICE int32 [G+1], off[0] = 0, nondecreasing, off[G] = M_total.
 *          Not read on the host.  The kernel reads group g's rows as
 *          [lo_g, hi_g) with lo_g = max(clamp(off[g]), hi_{g-1}) and
 *          hi_g = max(clamp(off[g+1]), lo_g), clamp() into [0, M_total]
 *          (hi_{-1} = 0).  For a valid table that is [off[g], off[g+1]); for
 *          any other table the ranges are still disjoint and inside a, so the
 *          result is deterministic, no access goes out of bounds, and rows
 *          covered by no range are not written.
 * a:       [M_total, K] codes (dense, pitch K);  a_scale [M_total, K/128].
 * b:       [G, N, K] codes (dense);  b_scale [G, N/128, K/128] (BLOCK128).
 * y:       [M_total, N] of y_dtype (dense, pitch N).  Rows of empty groups
 *          are not written.
 * Accuracy as for fp8_blockscaled_gemm, per group.
 * N % 128 == 0, K % 128 == 0, K >= 128, 1 <= G <= 1024.
 */
fp8bs_status fp8_blockscaled_grouped_gemm(int64_t M_total, int64_t N, int64_t K, int32_t G,
                                          const int32_t* off, const uint8_t* a,
                                          const float* a_scale, const uint8_t* b,
                                          const float* b_scale, void* y, int32_t y_dtype,
                                          hipStream_t stream);

/* Text of the last non-OK status returned on this thread ("" if none). */
const char* fp8bs_last_error(void);

/* Library version string. */
const char* fp8bs_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8BS_H */
