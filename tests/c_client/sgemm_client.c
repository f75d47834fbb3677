/* A plain C99 consumer of the library's C ABI (include/fp32_gemm.h): no
 * Python, no torch.  Test infrastructure: it shows that the header is valid
 * C and that the shared library links and runs from C.
 *
 *   sgemm_client info
 *       device-free calls only: prints the configuration count, the plan
 *       sgemm_plan gives for a 4096^3 product with aligned pointers, and a
 *       status string.
 *   sgemm_client run M N K alpha beta A.bin B.bin C.bin out.bin
 *       reads row-major float32 A (M x K), B (K x N) and C (M x N) from
 *       files, copies them to the current HIP device (hipMalloc), computes
 *       C = alpha*A*B + beta*C with sgemm() on the null stream, and writes
 *       the result (M x N float32) to out.bin.
 *
 * Exit status: 0 on success, 2 on a library error (its status is printed),
 * 3 on a HIP or file error, 1 on bad usage.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fp32_gemm.h"

static float* read_floats(const char* path, size_t n) {
  float* p = (float*)malloc(n * sizeof(float) + 1);
  FILE* f = fopen(path, "rb");
  if (p == NULL || f == NULL || fread(p, sizeof(float), n, f) != n) {
    if (f != NULL) fclose(f);
    free(p);
    return NULL;
  }
  fclose(f);
  return p;
}

static int info(void) {
  sgemm_config_t cfg;
  sgemm_plan_t plan;
  const int n = sgemm_num_configs();
  if (n <= 0 || sgemm_config_info(0, &cfg) != SGEMM_OK) return 2;
  /* Never dereferenced: sgemm_plan only inspects alignment and extents. */
  const float* a = (const float*)(uintptr_t)(1ull << 40);
  const float* b = (const float*)(uintptr_t)(2ull << 40);
  const float* c = (const float*)(uintptr_t)(4ull << 40);
  const int rc = sgemm_plan(4096, 4096, 4096, a, 4096, b, 4096, c, 4096, -1, &plan);
  printf("configs %d\n", n);
  printf("plan %d cfg %d vector %d grid %lld block %d\n", rc, (int)plan.cfg_id,
         (int)plan.vector_variant, (long long)plan.grid, (int)plan.block);
  printf("status -6 %s\n", sgemm_status_string(-6));
  return rc == SGEMM_OK ? 0 : 2;
}

static int run(char** argv) {
  const int64_t M = atoll(argv[0]), N = atoll(argv[1]), K = atoll(argv[2]);
  const float alpha = (float)atof(argv[3]), beta = (float)atof(argv[4]);
  if (M <= 0 || N <= 0 || K <= 0) return 1;
  const size_t na = (size_t)(M * K), nb = (size_t)(K * N), nc = (size_t)(M * N);
  float* A = read_floats(argv[5], na);
  float* B = read_floats(argv[6], nb);
  float* C = read_floats(argv[7], nc);
  float *dA = NULL, *dB = NULL, *dC = NULL;
  int status = 3;
  if (A == NULL || B == NULL || C == NULL) goto done;
  if (hipMalloc((void**)&dA, na * sizeof(float)) != hipSuccess ||
      hipMalloc((void**)&dB, nb * sizeof(float)) != hipSuccess ||
      hipMalloc((void**)&dC, nc * sizeof(float)) != hipSuccess)
    goto done;
  if (hipMemcpy(dA, A, na * sizeof(float), hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(dB, B, nb * sizeof(float), hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(dC, C, nc * sizeof(float), hipMemcpyHostToDevice) != hipSuccess)
    goto done;
  {
    const int rc = sgemm(M, N, K, alpha, dA, K, dB, N, beta, dC, N);
    if (rc != SGEMM_OK) {
      printf("sgemm: %d %s\n", rc, sgemm_status_string(rc));
      status = 2;
      goto done;
    }
  }
  if (hipDeviceSynchronize() != hipSuccess ||
      hipMemcpy(C, dC, nc * sizeof(float), hipMemcpyDeviceToHost) != hipSuccess)
    goto done;
  {
    FILE* f = fopen(argv[8], "wb");
    if (f == NULL) goto done;
    const size_t w = fwrite(C, sizeof(float), nc, f);
    fclose(f);
    if (w != nc) goto done;
  }
  status = 0;
done:
  if (dA != NULL) (void)hipFree(dA);
  if (dB != NULL) (void)hipFree(dB);
  if (dC != NULL) (void)hipFree(dC);
  free(A);
  free(B);
  free(C);
  return status;
}

int main(int argc, char** argv) {
  if (argc == 2 && strcmp(argv[1], "info") == 0) return info();
  if (argc == 11 && strcmp(argv[1], "run") == 0) return run(argv + 2);
  fprintf(stderr, "usage: sgemm_client info | run M N K alpha beta A.bin B.bin C.bin out.bin\n");
  return 1;
}
