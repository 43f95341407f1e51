/*
 * Plain C client of the library: the whole call sequence with nothing but
 * include/psgd.h, libpsgd.so and the HIP runtime (no Python, no PyTorch).
 *
 * A two-tensor set -- a 300 x 200 matrix of exact rank 2 and a 7-element bias
 * vector -- compressed at rank 4 from a seeded Q: since P = M Q has rank 2,
 * P_hat spans the column space of M (its two dependent columns are zero) and
 * the reconstruction P_hat Q^T = P_hat P_hat^T M returns M itself ([N152]
 * Method; exact recovery of a matrix of rank <= r).  The program checks
 * M_hat = M and E = M - M_hat = 0 to fp32 rounding, the bias passing through
 * exactly, and prints "c-abi smoke: ok" (exit status 0) or the failure.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "psgd.h"

#define HIP_OK(x)                                                          \
  do {                                                                     \
    hipError_t e_ = (x);                                                   \
    if (e_ != hipSuccess) {                                                \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 2;                                                            \
    }                                                                      \
  } while (0)

#define PSGD_OK(x)                                                         \
  do {                                                                     \
    psgd_status_t s_ = (x);                                                \
    if (s_ != PSGD_OK) {                                                   \
      fprintf(stderr, "psgd error %d at line %d: %s\n", (int)s_, __LINE__, psgd_last_error()); \
      return 3;                                                            \
    }                                                                      \
  } while (0)

int main(void) {
  enum { M = 300, N = 200, V = 7, RANK = 4 };
  const int64_t rows[2] = {M, V}, cols[2] = {N, 1};
  psgd_plan_t plan = NULL;
  PSGD_OK(psgd_plan_create(2, rows, cols, NULL, RANK, 0u, 0.f, &plan));
  psgd_plan_info_t info;
  PSGD_OK(psgd_plan_get_info(plan, &info));
  int32_t kind[2];
  int64_t off[2], poff[2], qoff[2];
  for (int t = 0; t < 2; ++t) PSGD_OK(psgd_plan_tensor(plan, t, &kind[t], &off[t], &poff[t], &qoff[t]));
  if (kind[0] != PSGD_KIND_COMPRESSED || kind[1] != PSGD_KIND_VECTOR) {
    fprintf(stderr, "unexpected tensor kinds %d %d\n", kind[0], kind[1]);
    return 4;
  }

  /* host gradients: M = u1 v1^T + 0.5 u2 v2^T, bias = 1..7 */
  float* g = (float*)calloc(info.flat_elems, sizeof(float));
  for (int i = 0; i < M; ++i)
    for (int j = 0; j < N; ++j)
      g[off[0] + (int64_t)i * N + j] =
          (float)(sin(0.01 * (i + 1)) * cos(0.02 * (j + 1)) + 0.5 * cos(0.03 * i) * sin(0.05 * j + 0.3));
  for (int k = 0; k < V; ++k) g[off[1] + k] = (float)(k + 1);

  float *grads, *err, *q, *p, *mhat;
  void* ws;
  const size_t fb = info.flat_elems * sizeof(float);
  HIP_OK(hipMalloc((void**)&grads, fb));
  HIP_OK(hipMalloc((void**)&err, fb));
  HIP_OK(hipMalloc((void**)&mhat, fb));
  HIP_OK(hipMalloc((void**)&q, info.q_elems * sizeof(float)));
  HIP_OK(hipMalloc((void**)&p, info.p_buffer_elems * sizeof(float)));
  HIP_OK(hipMalloc(&ws, info.workspace_bytes));
  HIP_OK(hipMemcpy(grads, g, fb, hipMemcpyHostToDevice));
  HIP_OK(hipMemset(err, 0, fb));
  HIP_OK(hipMemset(mhat, 0, fb));

  PSGD_OK(psgd_workspace_init(plan, ws, info.workspace_bytes, 0));
  PSGD_OK(psgd_init_q(plan, q, 2024u, ws, info.workspace_bytes, 0));
  PSGD_OK(psgd_compress(plan, grads, err, NULL, q, p, mhat, NULL, NULL, NULL, ws, info.workspace_bytes, 0));
  HIP_OK(hipDeviceSynchronize());

  float* mh = (float*)malloc(fb);
  float* e = (float*)malloc(fb);
  HIP_OK(hipMemcpy(mh, mhat, fb, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(e, err, fb, hipMemcpyDeviceToHost));
  double gmax = 0.0, dmax = 0.0, emax = 0.0;
  for (int64_t x = off[0]; x < off[0] + (int64_t)M * N; ++x) {
    gmax = fmax(gmax, fabs(g[x]));
    dmax = fmax(dmax, fabs((double)mh[x] - g[x]));
    emax = fmax(emax, fabs(e[x]));
  }
  int bias_ok = 1;
  for (int k = 0; k < V; ++k) bias_ok &= mh[off[1] + k] == g[off[1] + k];

  int ok = dmax <= 1e-5 * gmax && emax <= 1e-5 * gmax && bias_ok;
  printf("c-abi smoke: %s (max |M_hat - M| = %.3g, max |E| = %.3g, max |M| = %.3g, bias %s; %s)\n",
         ok ? "ok" : "FAILED", dmax, emax, gmax, bias_ok ? "exact" : "wrong", psgd_version());

  hipFree(grads);
  hipFree(err);
  hipFree(mhat);
  hipFree(q);
  hipFree(p);
  hipFree(ws);
  psgd_plan_destroy(plan);
  free(g);
  free(mh);
  free(e);
  return ok ? 0 : 1;
}
