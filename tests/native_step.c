/* A plain C caller of the library on the GPU, with HIP memory and a HIP
 * stream of its own (no PyTorch): the linear step, i.e. one fp8_quant_batch
 * launch for X (1x128 tiles) and W (128x128 blocks), then
 * fp8_blockscaled_gemm with float32 output.
 *
 *   native_step M N K x.bin w.bin out_prefix
 *
 * x.bin holds M*K bf16 bit patterns (uint16, row-major), w.bin N*K.  Writes
 * out_prefix.qa (M*K codes), .sa (M*K/128 float32), .qb (N*K codes), .sb
 * (N/128*K/128 float32) and .y (M*N float32).  Exit status 0 on success; a
 * library or HIP error is printed with the library's message. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fp8bs.h"

#define HIP_OK(call)                                                          \
  do {                                                                        \
    hipError_t e_ = (call);                                                   \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));              \
      return 1;                                                               \
    }                                                                         \
  } while (0)

#define FP8BS_OK_OR_FAIL(call)                                                \
  do {                                                                        \
    fp8bs_status s_ = (call);                                                 \
    if (s_ != FP8BS_OK) {                                                     \
      fprintf(stderr, "%s: status %d: %s\n", #call, (int)s_, fp8bs_last_error()); \
      return 1;                                                               \
    }                                                                         \
  } while (0)

static void* read_file(const char* path, size_t bytes) {
  FILE* f = fopen(path, "rb");
  if (!f) return NULL;
  void* p = malloc(bytes ? bytes : 1);
  if (p && fread(p, 1, bytes, f) != bytes) {
    free(p);
    p = NULL;
  }
  fclose(f);
  return p;
}

static int write_file(const char* prefix, const char* ext, const void* data, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s.%s", prefix, ext);
  FILE* f = fopen(path, "wb");
  if (!f) return 1;
  size_t n = fwrite(data, 1, bytes, f);
  fclose(f);
  return n != bytes;
}

int main(int argc, char** argv) {
  if (argc != 7) {
    fprintf(stderr, "usage: %s M N K x.bin w.bin out_prefix\n", argv[0]);
    return 2;
  }
  const int64_t M = atoll(argv[1]), N = atoll(argv[2]), K = atoll(argv[3]);
  if (M <= 0 || N <= 0 || K <= 0 || K % 128 || N % 128) {
    fprintf(stderr, "need M, N, K > 0 with N and K multiples of 128\n");
    return 2;
  }
  const size_t nx = (size_t)(M * K), nw = (size_t)(N * K), ny = (size_t)(M * N);
  const size_t nsa = (size_t)(M * (K / 128)), nsb = (size_t)((N / 128) * (K / 128));
  uint16_t* hx = (uint16_t*)read_file(argv[4], nx * 2);
  uint16_t* hw = (uint16_t*)read_file(argv[5], nw * 2);
  if (!hx || !hw) {
    fprintf(stderr, "cannot read the inputs\n");
    return 2;
  }

  void *dx, *dw, *dqa, *dsa, *dqb, *dsb, *dy;
  HIP_OK(hipMalloc(&dx, nx * 2));
  HIP_OK(hipMalloc(&dw, nw * 2));
  HIP_OK(hipMalloc(&dqa, nx));
  HIP_OK(hipMalloc(&dsa, nsa * 4));
  HIP_OK(hipMalloc(&dqb, nw));
  HIP_OK(hipMalloc(&dsb, nsb * 4));
  HIP_OK(hipMalloc(&dy, ny * 4));
  HIP_OK(hipMemcpy(dx, hx, nx * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dw, hw, nw * 2, hipMemcpyHostToDevice));
  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));

  fp8bs_quant_job jobs[2];
  memset(jobs, 0, sizeof jobs);
  jobs[0].x = dx; jobs[0].x_dtype = FP8BS_BF16; jobs[0].tiling = FP8BS_TILE_1x128;
  jobs[0].rows = M; jobs[0].cols = K; jobs[0].ld_x = K;
  jobs[0].q = (uint8_t*)dqa; jobs[0].ld_q = K; jobs[0].scale = (float*)dsa;
  jobs[1].x = dw; jobs[1].x_dtype = FP8BS_BF16; jobs[1].tiling = FP8BS_TILE_128x128;
  jobs[1].rows = N; jobs[1].cols = K; jobs[1].ld_x = K;
  jobs[1].q = (uint8_t*)dqb; jobs[1].ld_q = K; jobs[1].scale = (float*)dsb;
  FP8BS_OK_OR_FAIL(fp8_quant_batch(jobs, 2, stream));
  FP8BS_OK_OR_FAIL(fp8_blockscaled_gemm(M, N, K, (const uint8_t*)dqa, K, (const float*)dsa, (const uint8_t*)dqb, K,
                                        (const float*)dsb, FP8BS_BSCALE_BLOCK128, dy, FP8BS_F32, N, stream));
  HIP_OK(hipStreamSynchronize(stream));

  size_t most = ny * 4;
  if (nx > most) most = nx;
  if (nw > most) most = nw;
  if (nsa * 4 > most) most = nsa * 4;
  if (nsb * 4 > most) most = nsb * 4;
  void* out = malloc(most);
  if (!out) return 1;
  int bad = 0;
  HIP_OK(hipMemcpy(out, dqa, nx, hipMemcpyDeviceToHost));
  bad |= write_file(argv[6], "qa", out, nx);
  HIP_OK(hipMemcpy(out, dsa, nsa * 4, hipMemcpyDeviceToHost));
  bad |= write_file(argv[6], "sa", out, nsa * 4);
  HIP_OK(hipMemcpy(out, dqb, nw, hipMemcpyDeviceToHost));
  bad |= write_file(argv[6], "qb", out, nw);
  HIP_OK(hipMemcpy(out, dsb, nsb * 4, hipMemcpyDeviceToHost));
  bad |= write_file(argv[6], "sb", out, nsb * 4);
  HIP_OK(hipMemcpy(out, dy, ny * 4, hipMemcpyDeviceToHost));
  bad |= write_file(argv[6], "y", out, ny * 4);
  if (bad) {
    fprintf(stderr, "cannot write the outputs\n");
    return 1;
  }
  HIP_OK(hipStreamDestroy(stream));
  HIP_OK(hipFree(dx)); HIP_OK(hipFree(dw)); HIP_OK(hipFree(dqa)); HIP_OK(hipFree(dsa));
  HIP_OK(hipFree(dqb)); HIP_OK(hipFree(dsb)); HIP_OK(hipFree(dy));
  free(out); free(hx); free(hw);
  printf("native step %lld x %lld x %lld ok\n", (long long)M, (long long)N, (long long)K);
  return 0;
}
