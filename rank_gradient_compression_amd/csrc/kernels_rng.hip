// Seeded standard-normal start for the warm-start factors Q.
//
// The PowerSGD pages start each power iteration from the previous step's Q
// and leave the very first Q open; here it is i.i.d. N(0, 1), drawn from a
// counter-based generator keyed by (seed, tensor index) so that every worker
// using the same seed starts from the same Q whatever the launch shape.
//
// Generator: Philox-4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC'11, section 5).  Normals: the Box-Muller
// transform (Box and Muller, 1958) in fp64, rounded once to fp32.
// Element e = c*n + j of a tensor's packed column-major n x r Q is normal e
// of its stream: Philox block e/4 (counter (e/4, 0, 0, 0)); words 0,1 give
// the normals of e%4 = 0,1 and words 2,3 those of e%4 = 2,3.

#include <hip/hip_runtime.h>

#include "psgd_kernels.h"
#include "psgd_tables.h"

namespace psgd {

namespace {

constexpr uint64_t kPhiloxM0 = 0xD2E7470EE14C6C93ull;
constexpr uint64_t kPhiloxM1 = 0xCA5A826395121157ull;
constexpr uint64_t kPhiloxW0 = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kPhiloxW1 = 0xBB67AE8584CAA73Bull;

__device__ __forceinline__ void philox4x64_10(uint64_t (&x)[4], uint64_t k0, uint64_t k1) {
#pragma unroll
  for (int rnd = 0; rnd < 10; ++rnd) {
    if (rnd > 0) {
      k0 += kPhiloxW0;
      k1 += kPhiloxW1;
    }
    const uint64_t hi0 = __umul64hi(kPhiloxM0, x[0]), lo0 = kPhiloxM0 * x[0];
    const uint64_t hi1 = __umul64hi(kPhiloxM1, x[2]), lo1 = kPhiloxM1 * x[2];
    const uint64_t y0 = hi1 ^ x[1] ^ k0;
    const uint64_t y2 = hi0 ^ x[3] ^ k1;
    x[0] = y0;
    x[1] = lo1;
    x[2] = y2;
    x[3] = lo0;
  }
}

// Two words -> u1 in (0, 1], u2 in [0, 1) (53 bits each) -> two normals.
__device__ __forceinline__ void box_muller(uint64_t wa, uint64_t wb, float& z0, float& z1) {
  const double u1 = 1.0 - (double)(wa >> 11) * 0x1p-53;
  const double u2 = (double)(wb >> 11) * 0x1p-53;
  const double rad = sqrt(-2.0 * log(u1));
  const double ang = (2.0 * M_PI) * u2;
  z0 = (float)(rad * cos(ang));
  z1 = (float)(rad * sin(ang));
}

}  // namespace

__global__ __launch_bounds__(256) void k_init_q(const MatDesc* __restrict__ mats, int mat_base, int rank,
                                                float* __restrict__ Q, uint64_t seed) {
  const MatDesc& d = mats[mat_base + blockIdx.y];
  const int64_t count = (int64_t)d.n * rank;
  const int64_t nblk = (count + 3) / 4;
  float* out = Q + d.q_off;  // 64-element aligned: 4-element groups are 16-byte aligned
  for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < nblk; b += (int64_t)gridDim.x * 256) {
    uint64_t x[4] = {(uint64_t)b, 0ull, 0ull, 0ull};
    philox4x64_10(x, seed, (uint64_t)d.tensor);
    float z[4];
    box_muller(x[0], x[1], z[0], z[1]);
    box_muller(x[2], x[3], z[2], z[3]);
    const int64_t e = 4 * b;
    if (e + 4 <= count) {
      *reinterpret_cast<float4*>(out + e) = make_float4(z[0], z[1], z[2], z[3]);
    } else {
      for (int j = 0; j < 4; ++j)
        if (e + j < count) out[e + j] = z[j];
    }
  }
}

hipError_t launch_init_q(const LaunchCtx& c, float* Q, uint64_t seed, int64_t max_blocks) {
  if (c.nmat == 0) return hipSuccess;
  const int64_t gx = std::min<int64_t>(std::max<int64_t>((max_blocks + 255) / 256, 1), 64);
  for (int base = 0; base < c.nmat; base += 65535) {
    const int ny = std::min(c.nmat - base, 65535);
    hipLaunchKernelGGL(k_init_q, dim3((unsigned)gx, (unsigned)ny), dim3(256), 0, c.stream, c.mats, base, c.rank, Q,
                       seed);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace psgd
