/* A plain C caller of the library on the GPU, with HIP memory and a HIP
 * stream of its own (no PyTorch).  Inputs and outputs go through files of
 * raw little-endian values; out_prefix.<name> receives each output.
 *
 *   native_step step M N K x.bin w.bin out_prefix
 *     The linear step: one fp8_quant_batch launch for X [M, K] (1x128 tiles)
 *     and W [N, K] (128x128 blocks), then fp8_blockscaled_gemm into float32.
 *     Writes .qa (M*K codes), .sa (M*K/128 float32), .qb (N*K codes), .sb
 *     (N/128*K/128 float32) and .y (M*N float32).
 *
 *   native_step moe G N K off.bin x.bin w.bin out_prefix
 *     The grouped step: off.bin holds G+1 int32 row offsets (off[G] = M),
 *     X [M, K] is quantized 1x128 by fp8_quant_act_1x128, the G expert
 *     weights [G*N, K] by one fp8_quant_w_128x128 call, then
 *     fp8_blockscaled_grouped_gemm into float32.  Same outputs as "step".
 *
 *   native_step dual R C x.bin out_prefix
 *     fp8_quant_act_dual on X [R, C]: .q (R*C codes), .s (R*C/128 float32),
 *     .qt (C*R codes of the transposed tiling), .st (C*R/128 float32).
 *
 * x.bin and w.bin hold bf16 bit patterns (uint16, row-major).  Exit status 0
 * on success, 1 on a library or HIP error (printed with the library's
 * message), 2 on bad usage or unreadable inputs. */
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

/* Copies `bytes` of device memory to out_prefix.ext. */
static int save(const char* prefix, const char* ext, const void* dev, size_t bytes) {
  void* host = malloc(bytes ? bytes : 1);
  if (!host) return 1;
  if (hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost) != hipSuccess) {
    free(host);
    return 1;
  }
  char path[4096];
  snprintf(path, sizeof path, "%s.%s", prefix, ext);
  FILE* f = fopen(path, "wb");
  size_t n = f ? fwrite(host, 1, bytes, f) : 0;
  if (f) fclose(f);
  free(host);
  return n != bytes;
}

/* A device buffer holding `bytes` of the file at `path` (NULL if unreadable). */
static void* upload(const char* path, size_t bytes) {
  void* host = read_file(path, bytes);
  if (!host) return NULL;
  void* dev = NULL;
  if (hipMalloc(&dev, bytes ? bytes : 1) != hipSuccess ||
      hipMemcpy(dev, host, bytes, hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(dev);
    dev = NULL;
  }
  free(host);
  return dev;
}

static int run_step(int64_t M, int64_t N, int64_t K, const char* xf, const char* wf, const char* pre) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 128 || N % 128) {
    fprintf(stderr, "need M, N, K > 0 with N and K multiples of 128\n");
    return 2;
  }
  const size_t nx = (size_t)(M * K), nw = (size_t)(N * K), ny = (size_t)(M * N);
  const size_t nsa = (size_t)(M * (K / 128)), nsb = (size_t)((N / 128) * (K / 128));
  void* dx = upload(xf, nx * 2);
  void* dw = upload(wf, nw * 2);
  if (!dx || !dw) {
    fprintf(stderr, "cannot read the inputs\n");
    return 2;
  }
  void *dqa, *dsa, *dqb, *dsb, *dy;
  HIP_OK(hipMalloc(&dqa, nx));
  HIP_OK(hipMalloc(&dsa, nsa * 4));
  HIP_OK(hipMalloc(&dqb, nw));
  HIP_OK(hipMalloc(&dsb, nsb * 4));
  HIP_OK(hipMalloc(&dy, ny * 4));
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

  if (save(pre, "qa", dqa, nx) || save(pre, "sa", dsa, nsa * 4) || save(pre, "qb", dqb, nw) ||
      save(pre, "sb", dsb, nsb * 4) || save(pre, "y", dy, ny * 4)) {
    fprintf(stderr, "cannot write the outputs\n");
    return 1;
  }
  HIP_OK(hipStreamDestroy(stream));
  HIP_OK(hipFree(dx)); HIP_OK(hipFree(dw)); HIP_OK(hipFree(dqa)); HIP_OK(hipFree(dsa));
  HIP_OK(hipFree(dqb)); HIP_OK(hipFree(dsb)); HIP_OK(hipFree(dy));
  printf("native step %lld x %lld x %lld ok\n", (long long)M, (long long)N, (long long)K);
  return 0;
}

static int run_moe(int32_t G, int64_t N, int64_t K, const char* of, const char* xf, const char* wf,
                   const char* pre) {
  if (G < 1 || N <= 0 || K <= 0 || K % 128 || N % 128) {
    fprintf(stderr, "need G >= 1, N, K > 0 with N and K multiples of 128\n");
    return 2;
  }
  int32_t* off = (int32_t*)read_file(of, (size_t)(G + 1) * 4);
  if (!off) {
    fprintf(stderr, "cannot read the offsets\n");
    return 2;
  }
  const int64_t M = off[G];
  if (M <= 0) {
    fprintf(stderr, "need at least one row\n");
    return 2;
  }
  const size_t nx = (size_t)(M * K), nw = (size_t)(G * N * K), ny = (size_t)(M * N);
  const size_t nsa = (size_t)(M * (K / 128)), nsb = (size_t)(G * (N / 128) * (K / 128));
  void* dx = upload(xf, nx * 2);
  void* dw = upload(wf, nw * 2);
  void* doff = upload(of, (size_t)(G + 1) * 4);
  if (!dx || !dw || !doff) {
    fprintf(stderr, "cannot read the inputs\n");
    return 2;
  }
  void *dqa, *dsa, *dqb, *dsb, *dy;
  HIP_OK(hipMalloc(&dqa, nx));
  HIP_OK(hipMalloc(&dsa, nsa * 4));
  HIP_OK(hipMalloc(&dqb, nw));
  HIP_OK(hipMalloc(&dsb, nsb * 4));
  HIP_OK(hipMalloc(&dy, ny * 4));
  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  FP8BS_OK_OR_FAIL(fp8_quant_act_1x128(dx, FP8BS_BF16, M, K, K, FP8BS_TILE_1x128, (uint8_t*)dqa, K, (float*)dsa,
                                       stream));
  /* The G weights stacked as one [G*N, K] matrix: its 128x128 blocks are the
     experts' blocks, in the [G, N/128, K/128] scale layout. */
  FP8BS_OK_OR_FAIL(fp8_quant_w_128x128(dw, FP8BS_BF16, G * N, K, K, (uint8_t*)dqb, K, (float*)dsb, NULL, 0,
                                       stream));
  FP8BS_OK_OR_FAIL(fp8_blockscaled_grouped_gemm(M, N, K, G, (const int32_t*)doff, (const uint8_t*)dqa,
                                                (const float*)dsa, (const uint8_t*)dqb, (const float*)dsb, dy,
                                                FP8BS_F32, stream));
  HIP_OK(hipStreamSynchronize(stream));

  if (save(pre, "qa", dqa, nx) || save(pre, "sa", dsa, nsa * 4) || save(pre, "qb", dqb, nw) ||
      save(pre, "sb", dsb, nsb * 4) || save(pre, "y", dy, ny * 4)) {
    fprintf(stderr, "cannot write the outputs\n");
    return 1;
  }
  HIP_OK(hipStreamDestroy(stream));
  HIP_OK(hipFree(dx)); HIP_OK(hipFree(dw)); HIP_OK(hipFree(doff)); HIP_OK(hipFree(dqa)); HIP_OK(hipFree(dsa));
  HIP_OK(hipFree(dqb)); HIP_OK(hipFree(dsb)); HIP_OK(hipFree(dy));
  free(off);
  printf("native moe %d experts, %lld rows, N %lld, K %lld ok\n", (int)G, (long long)M, (long long)N, (long long)K);
  return 0;
}

static int run_dual(int64_t R, int64_t C, const char* xf, const char* pre) {
  if (R <= 0 || C <= 0 || R % 128 || C % 128) {
    fprintf(stderr, "need R, C > 0, multiples of 128\n");
    return 2;
  }
  const size_t n = (size_t)(R * C), ns = n / 128;
  void* dx = upload(xf, n * 2);
  if (!dx) {
    fprintf(stderr, "cannot read the input\n");
    return 2;
  }
  void *dq, *ds, *dqt, *dst;
  HIP_OK(hipMalloc(&dq, n));
  HIP_OK(hipMalloc(&ds, ns * 4));
  HIP_OK(hipMalloc(&dqt, n));
  HIP_OK(hipMalloc(&dst, ns * 4));
  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  FP8BS_OK_OR_FAIL(fp8_quant_act_dual(dx, FP8BS_BF16, R, C, C, (uint8_t*)dq, C, (float*)ds, (uint8_t*)dqt, R,
                                      (float*)dst, stream));
  HIP_OK(hipStreamSynchronize(stream));
  if (save(pre, "q", dq, n) || save(pre, "s", ds, ns * 4) || save(pre, "qt", dqt, n) || save(pre, "st", dst, ns * 4)) {
    fprintf(stderr, "cannot write the outputs\n");
    return 1;
  }
  HIP_OK(hipStreamDestroy(stream));
  HIP_OK(hipFree(dx)); HIP_OK(hipFree(dq)); HIP_OK(hipFree(ds)); HIP_OK(hipFree(dqt)); HIP_OK(hipFree(dst));
  printf("native dual %lld x %lld ok\n", (long long)R, (long long)C);
  return 0;
}

int main(int argc, char** argv) {
  if (argc == 8 && strcmp(argv[1], "step") == 0)
    return run_step(atoll(argv[2]), atoll(argv[3]), atoll(argv[4]), argv[5], argv[6], argv[7]);
  if (argc == 9 && strcmp(argv[1], "moe") == 0)
    return run_moe((int32_t)atoi(argv[2]), atoll(argv[3]), atoll(argv[4]), argv[5], argv[6], argv[7], argv[8]);
  if (argc == 6 && strcmp(argv[1], "dual") == 0)
    return run_dual(atoll(argv[2]), atoll(argv[3]), argv[4], argv[5]);
  fprintf(stderr,
          "usage: %s step M N K x.bin w.bin out_prefix\n"
          "       %s moe G N K off.bin x.bin w.bin out_prefix\n"
          "       %s dual R C x.bin out_prefix\n",
          argv[0], argv[0], argv[0]);
  return 2;
}
