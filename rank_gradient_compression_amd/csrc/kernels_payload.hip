// Payload quantiser of the transmitted factors to 8 bits (gfx950, wave64).
//
// Compound compression (glossary entry "PowerSGD", compound-compression
// paragraph: the factors PowerSGD produces can themselves be quantised) with
// the OCP FP8 E4M3 format and one power-of-two scale per factor column.  The
// kernel runs between a factor's formation and its aggregation hook; it is
// latency-bound (one read and one write of the factor columns).

#include <hip/hip_runtime.h>

#include "psgd_payload.h"
#include "psgd_tables.h"

namespace psgd {

// Payload quantiser to 8 bits: OCP FP8 E4M3 values (3 fraction bits,
// exponents -6..8, subnormals below 2^-6, largest finite value 448) times one
// power of two 2^k per factor column, k the smallest integer with
// max|column| <= 448 * 2^k.  Scaling by 2^-k, rounding the magnitude to a
// multiple of its spacing (2^(b-3) in the binade [2^b, 2^(b+1)), 2^-9 below
// 2^-6) with rintf (ties to even) and scaling back are each exact in fp32,
// so the stored value is exactly the transmitted code times 2^k.  Finite
// values only.
__device__ __forceinline__ float round_e4m3_scaled(float x, int k) {
  const float a = fabsf(ldexpf(x, -k));
  int e;
  (void)frexpf(a, &e);  // a = f 2^e with f in [0.5, 1): binade 2^(e-1)
  const int s = (a < 0x1p-6f ? -6 : e - 1) - 3;
  return copysignf(ldexpf(rintf(ldexpf(a, -s)), s + k), x);
}

// One workgroup per (descriptor first + blockIdx.x, column blockIdx.y): the
// column's largest magnitude, its exponent k, then every value rounded in
// place.  448 = 0.875 * 2^9, so with max = f 2^E (f in [0.5, 1)) the
// smallest sufficient k is E - 9 when f <= 0.875 and E - 8 otherwise.  Each
// thread keeps kFp8Unroll loads in flight (at clamped addresses, masked
// afterwards): one load at a time left a 32000-row column waiting out one
// memory latency per 256 rows.
constexpr int kFp8Unroll = 8;

__global__ __launch_bounds__(256) void k_round_fp8_cols(const OrthDesc* __restrict__ orth, int first,
                                                        float* __restrict__ base) {
  const OrthDesc d = orth[first + blockIdx.x];
  float* __restrict__ col = base + d.off + (int64_t)blockIdx.y * d.rows;
  const int rows = d.rows;
  constexpr int STEP = 256 * kFp8Unroll;
  float a = 0.f;
  for (int i0 = 0; i0 < rows; i0 += STEP) {
    float v[kFp8Unroll];
#pragma unroll
    for (int u = 0; u < kFp8Unroll; ++u) v[u] = col[min(i0 + 256 * u + (int)threadIdx.x, rows - 1)];
#pragma unroll
    for (int u = 0; u < kFp8Unroll; ++u)
      if (i0 + 256 * u + (int)threadIdx.x < rows) a = fmaxf(a, fabsf(v[u]));
  }
  for (int o = 32; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o));
  __shared__ float wmax[4];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = a;
  __syncthreads();
  const float amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  if (amax == 0.f) return;  // an all-zero column stays zero
  int E;
  const float f = frexpf(amax, &E);
  const int k = f <= 0.875f ? E - 9 : E - 8;
  for (int i0 = 0; i0 < rows; i0 += STEP) {
    float v[kFp8Unroll];
#pragma unroll
    for (int u = 0; u < kFp8Unroll; ++u) v[u] = col[min(i0 + 256 * u + (int)threadIdx.x, rows - 1)];
#pragma unroll
    for (int u = 0; u < kFp8Unroll; ++u) {
      const int i = i0 + 256 * u + (int)threadIdx.x;
      if (i < rows) col[i] = round_e4m3_scaled(v[u], k);
    }
  }
}

hipError_t launch_round_fp8_cols(const LaunchCtx& c, int first, float* base) {
  if (c.nmat == 0 || c.rank == 0) return hipSuccess;
  hipLaunchKernelGGL(k_round_fp8_cols, dim3((unsigned)c.nmat, (unsigned)c.rank), dim3(256), 0, c.stream, c.orth,
                     first, base);
  return hipGetLastError();
}

}  // namespace psgd
