// Measurement kernels: the plain copy that calibrates the byte counters and
// sets a bandwidth ceiling, and the streaming probe that moves the byte
// pattern of one pass of the step without its arithmetic.

#include <hip/hip_runtime.h>

#include "psgd_kernels.h"
#include "psgd_tables.h"

namespace psgd {

typedef float v4f_nt __attribute__((ext_vector_type(4)));

// 16-byte non-temporal accesses (the data streams through once); loads at a
// clamped, always valid index, so that they need no branch and all of a
// thread's loads can be in flight together.
__device__ __forceinline__ v4f_nt ld_stream(const float4* p, int64_t i, int64_t n4) {
  return __builtin_nontemporal_load(reinterpret_cast<const v4f_nt*>(p + (i < n4 ? i : n4 - 1)));
}

__device__ __forceinline__ void st_stream(float4* p, int64_t i, v4f_nt v) {
  __builtin_nontemporal_store(v, reinterpret_cast<v4f_nt*>(p + i));
}

// Plain 16-byte copy: the bandwidth ceiling and counter calibration.  Each
// thread moves kStreamUnroll vectors per grid step, all loads issued before
// the stores, on at most kCopyMaxBlocks workgroups (the grid-stride form
// copies 4 GiB at 5.7 TB/s, one run per workgroup at 5.2).
__global__ __launch_bounds__(256) void k_stream_copy(float4* __restrict__ dst, const float4* __restrict__ src,
                                                     int64_t n4) {
  constexpr int U = kStreamUnroll;
  const int64_t stride = (int64_t)gridDim.x * 256 * U;
  for (int64_t i0 = (int64_t)blockIdx.x * 256 * U + threadIdx.x; i0 < n4; i0 += stride) {
    v4f_nt x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = ld_stream(src, i0 + (int64_t)u * 256, n4);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + (int64_t)u * 256;
      if (i < n4) st_stream(dst, i, x[u]);
    }
  }
}

// Streaming-bandwidth probe: the byte pattern of a pass (NIN arrays read,
// NOUT written) without its arithmetic, out_j[i] = sum_k in_k[i] (zero with
// no input).  The arrays are viewed as rows of kProbeRowVec 16-byte vectors
// (a 4096-column fp32 matrix) and walked with the geometry of the streaming
// passes: a workgroup owns one tile of kRowsPerWG rows x one
// kRecSplitCols-column split (splits fastest, one tile per workgroup and no
// grid-stride loop: a capped grid that loops made the resident workgroups
// touch tiles far apart and cost 5-10% on patterns that read and write),
// each wavefront kWaveRows rows of it, one 16-byte access per lane and row
// (a 1 KB row segment per instruction), every load of the wavefront issued
// before its sums and stores, with non-temporal loads and stores.  With no
// output the sums are reduced per wavefront and added into
// sink[blockIdx.x % kProbeSinkFloats], so the loads are not dead.
constexpr int64_t kProbeRowVec = 1024;
constexpr int kProbeSplitVec = kRecSplitCols / 4;  // 16-byte vectors per row segment (one per lane)
static_assert(kProbeSplitVec == 64, "one vector per lane and row");

template <int NIN, int NOUT>
__global__ __launch_bounds__(kWGThreads) void k_stream_probe(ProbeArgs a) {
  constexpr int SPLITS = (int)(kProbeRowVec / kProbeSplitVec);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = blockIdx.x;
  const int64_t row0 = (t / SPLITS) * kRowsPerWG + (int64_t)wave * kWaveRows;
  const int64_t col = (t % SPLITS) * kProbeSplitVec + lane;
  v4f_nt x[NIN > 0 ? NIN : 1][kWaveRows];
#pragma unroll
  for (int k = 0; k < NIN; ++k)
#pragma unroll
    for (int rr = 0; rr < kWaveRows; ++rr) x[k][rr] = ld_stream(a.in[k], (row0 + rr) * kProbeRowVec + col, a.n4);
  float part = 0.f;
#pragma unroll
  for (int rr = 0; rr < kWaveRows; ++rr) {
    const int64_t i = (row0 + rr) * kProbeRowVec + col;
    v4f_nt v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < NIN; ++k) v += x[k][rr];
    if constexpr (NOUT == 0) {
      if (i < a.n4) part += (v[0] + v[1]) + (v[2] + v[3]);
    } else if (i < a.n4) {
#pragma unroll
      for (int j = 0; j < NOUT; ++j) st_stream(a.out[j], i, v);
    }
  }
  if constexpr (NOUT == 0) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
    if (lane == 0) atomicAdd(&a.sink[blockIdx.x % kProbeSinkFloats], part);
  }
}

hipError_t launch_stream_copy(float* dst, const float* src, size_t n, hipStream_t stream) {
  const int64_t n4 = (int64_t)(n / 4);
  if (n4 == 0) return hipSuccess;
  int64_t blocks = (n4 + 256 * kStreamUnroll - 1) / (256 * kStreamUnroll);
  if (blocks > kCopyMaxBlocks) blocks = kCopyMaxBlocks;
  hipLaunchKernelGGL(k_stream_copy, dim3((unsigned)blocks), dim3(256), 0, stream, reinterpret_cast<float4*>(dst),
                     reinterpret_cast<const float4*>(src), n4);
  return hipGetLastError();
}

hipError_t launch_stream_probe(const ProbeArgs& a, int nin, int nout, hipStream_t stream) {
  if (a.n4 == 0) return hipSuccess;
  const int64_t rows = (a.n4 + kProbeRowVec - 1) / kProbeRowVec;
  const int64_t blocks = (rows + kRowsPerWG - 1) / kRowsPerWG * (kProbeRowVec / kProbeSplitVec);
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  const dim3 g((unsigned)blocks), b(kWGThreads);
#define PSGD_PROBE(I, O) \
  if (nin == I && nout == O) hipLaunchKernelGGL((k_stream_probe<I, O>), g, b, 0, stream, a)
  PSGD_PROBE(0, 1); PSGD_PROBE(0, 2);
  PSGD_PROBE(1, 0); PSGD_PROBE(1, 1); PSGD_PROBE(1, 2);
  PSGD_PROBE(2, 0); PSGD_PROBE(2, 1); PSGD_PROBE(2, 2);
  PSGD_PROBE(3, 0); PSGD_PROBE(3, 1); PSGD_PROBE(3, 2);
#undef PSGD_PROBE
  return hipGetLastError();
}

}  // namespace psgd
