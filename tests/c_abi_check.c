/* Plain C user of the library: includes fp8bs.h as C, links libfp8bs.so and
 * exercises argument validation, which returns before any GPU work (so this
 * runs without a GPU).  Exit status 0 means every check held. */
#include <stdio.h>
#include <string.h>

#include "fp8bs.h"

static int failures = 0;

static void expect(const char* what, fp8bs_status got, fp8bs_status want) {
  if (got != want) {
    fprintf(stderr, "%s: status %d, expected %d (%s)\n", what, (int)got, (int)want, fp8bs_last_error());
    ++failures;
  }
}

int main(void) {
  const void* fake = (const void*)(uintptr_t)0x10000; /* never dereferenced */
  expect("empty activation", fp8_quant_act_1x128(NULL, FP8BS_BF16, 0, 256, 256, FP8BS_TILE_1x128, NULL, 256, NULL, 0), FP8BS_OK);
  expect("negative rows", fp8_quant_act_1x128(fake, FP8BS_BF16, -1, 256, 256, FP8BS_TILE_1x128, (uint8_t*)fake, 256, (float*)fake, 0), FP8BS_ERR_INVALID_ARG);
  if (strstr(fp8bs_last_error(), "negative") == NULL) {
    fprintf(stderr, "last error text: '%s'\n", fp8bs_last_error());
    ++failures;
  }
  expect("ragged weight", fp8_quant_w_128x128(fake, FP8BS_BF16, 200, 256, 256, (uint8_t*)fake, 256, (float*)fake, NULL, 0, 0), FP8BS_ERR_SHAPE);
  expect("gemm K", fp8_blockscaled_gemm(4, 256, 100, (const uint8_t*)fake, 112, (const float*)fake, (const uint8_t*)fake, 112,
                                        (const float*)fake, FP8BS_BSCALE_BLOCK128, (void*)fake, FP8BS_F32, 256,
                                        0), FP8BS_ERR_SHAPE);
  expect("gemm_fp8mma kind", fp8_blockscaled_gemm_fp8mma(4, 256, 256, (const uint8_t*)fake, 256, (const float*)fake,
                                                         (const uint8_t*)fake, 256, (const float*)fake, 7, (void*)fake,
                                                         FP8BS_F32, 256, 0), FP8BS_ERR_INVALID_ARG);
  expect("gemm_quant N", fp8_blockscaled_gemm_quant(4, 144, 256, (const uint8_t*)fake, 256, (const float*)fake, (const uint8_t*)fake, 256,
                                                    (const float*)fake, FP8BS_BSCALE_ROW, (uint8_t*)fake, 144, (float*)fake,
                                                    0), FP8BS_ERR_SHAPE);
  expect("grouped G", fp8_blockscaled_grouped_gemm(256, 256, 256, 0, (const int32_t*)fake, (const uint8_t*)fake, (const float*)fake,
                                                   (const uint8_t*)fake, (const float*)fake, (void*)fake, FP8BS_BF16,
                                                   0), FP8BS_ERR_INVALID_ARG);
  {
    fp8bs_quant_job jobs[2];
    memset(jobs, 0, sizeof jobs);
    jobs[0].x = fake; jobs[0].x_dtype = FP8BS_BF16; jobs[0].tiling = FP8BS_TILE_1x128;
    jobs[0].rows = 4; jobs[0].cols = 256; jobs[0].ld_x = 256; jobs[0].q = (uint8_t*)fake; jobs[0].ld_q = 256;
    jobs[0].scale = (float*)fake;
    jobs[1] = jobs[0];
    jobs[1].tiling = FP8BS_TILE_128x128; /* rows 4: not whole blocks */
    expect("batch shape", fp8_quant_batch(jobs, 2, 0), FP8BS_ERR_SHAPE);
    if (sizeof(fp8bs_quant_job) != 64) {
      fprintf(stderr, "sizeof(fp8bs_quant_job) = %d\n", (int)sizeof(fp8bs_quant_job));
      ++failures;
    }
  }
  expect("dual alignment", fp8_quant_act_dual((const char*)fake + 8, FP8BS_BF16, 128, 128, 128, (uint8_t*)fake, 128, (float*)fake,
                                              (uint8_t*)fake, 128, (float*)fake, 0), FP8BS_ERR_ALIGNMENT);
  expect("dequant tiling", fp8_dequant((const uint8_t*)fake, 4, 128, 128, (const float*)fake, FP8BS_TILE_128x1_T, (void*)fake,
                                       FP8BS_F32, 128, 0), FP8BS_ERR_INVALID_ARG);
  expect("tensor format", fp8_quant_tensor(fake, FP8BS_BF16, 4, 64, 64, 7, 0.15, NULL, 0, (uint8_t*)fake, 64, (float*)fake,
                                           (float*)fake, 0), FP8BS_ERR_INVALID_ARG);
  if (strstr(fp8bs_version(), "gfx950") == NULL) {
    fprintf(stderr, "version: '%s'\n", fp8bs_version());
    ++failures;
  }
  printf("c_abi_check: %d failure(s)\n", failures);
  return failures == 0 ? 0 : 1;
}
