// Diagnostics of a compression step, outside the step itself: the share of
// each matrix's input that error feedback carries over, ||E|| / ||M||, and the
// overlap of the subspaces two steps' Q span (mean cosine of their principal
// angles).  Sums are fp64 and taken in a fixed order: repeatable bit for bit.

#include <hip/hip_runtime.h>

#include "psgd_kernels.h"
#include "psgd_tables.h"

namespace psgd {

// fp64 sum over a 256-thread workgroup, in a fixed order; the total is valid
// in thread 0.
__device__ __forceinline__ double block_sum(double v, double* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double t = 0.0;
  if (threadIdx.x == 0) t = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return t;
}

// ||E||^2 and ||M_hat + E||^2 of each compressed matrix (M = M_hat + E up to
// the rounding of the residual's subtraction): kStatsWGs workgroups per
// matrix, each striding over its elements with 16-byte loads where the
// matrix starts 16-byte aligned, writing its two partial sums into the
// matrix's Gram scratch.
__global__ __launch_bounds__(256) void k_sumsq_partial(const MatDesc* __restrict__ mats, const float* __restrict__ E,
                                                       const float* __restrict__ Mh, double* __restrict__ gram) {
  __shared__ double red[4];
  const int k = blockIdx.x / kStatsWGs, b = blockIdx.x % kStatsWGs;
  const MatDesc d = mats[k];
  const int64_t len = (int64_t)d.m * d.n;
  const float* e = E + d.off;
  const float* h = Mh + d.off;
  constexpr int64_t STRIDE = (int64_t)kStatsWGs * 256;
  double se = 0.0, sm = 0.0;
  int64_t done = 0;
  if ((d.off & 3) == 0) {
    const int64_t n4 = len / 4;
    const float4* e4 = reinterpret_cast<const float4*>(e);
    const float4* h4 = reinterpret_cast<const float4*>(h);
    for (int64_t i = (int64_t)b * 256 + threadIdx.x; i < n4; i += STRIDE) {
      const float4 ev = e4[i], hv = h4[i];
      const double m0 = (double)ev.x + hv.x, m1 = (double)ev.y + hv.y;
      const double m2 = (double)ev.z + hv.z, m3 = (double)ev.w + hv.w;
      se += ((double)ev.x * ev.x + (double)ev.y * ev.y) + ((double)ev.z * ev.z + (double)ev.w * ev.w);
      sm += (m0 * m0 + m1 * m1) + (m2 * m2 + m3 * m3);
    }
    done = 4 * n4;
  }
  for (int64_t i = done + (int64_t)b * 256 + threadIdx.x; i < len; i += STRIDE) {
    const double ev = e[i], mv = (double)e[i] + h[i];
    se += ev * ev;
    sm += mv * mv;
  }
  const double te = block_sum(se, red);
  const double tm = block_sum(sm, red);
  if (threadIdx.x == 0) {
    gram[d.gram_off + 2 * b] = te;
    gram[d.gram_off + 2 * b + 1] = tm;
  }
}

// The kStatsWGs partial sums of each matrix added in workgroup order.
__global__ __launch_bounds__(64) void k_sumsq_final(const MatDesc* __restrict__ mats, int nmat,
                                                    const double* __restrict__ gram, double* __restrict__ out) {
  const int k = blockIdx.x * 64 + threadIdx.x;
  if (k >= nmat) return;
  const double* part = gram + mats[k].gram_off;
  double se = 0.0, sm = 0.0;
  for (int b = 0; b < kStatsWGs; ++b) {
    se += part[2 * b];
    sm += part[2 * b + 1];
  }
  out[2 * k] = se;
  out[2 * k + 1] = sm;
}

// C_b = A_b^T B_b for one block of kGramRows rows of two factors laid out
// alike (the two orthonormalised Q copies), on the fp64 matrix core as in the
// Gram blocks of the orthonormalisation: all (RP/16)^2 16 x 16 tiles, dealt
// round-robin to the four wavefronts, summed over the block's rows in order.
typedef double v4d_diag __attribute__((ext_vector_type(4)));

template <int RP>
__global__ __launch_bounds__(256) void k_cross_partial(const OrthDesc* __restrict__ descs,
                                                       const int32_t* __restrict__ map, int first, int r,
                                                       const float* __restrict__ base_a,
                                                       const float* __restrict__ base_b, double* __restrict__ gram) {
  constexpr int LS = RP + 1;
  constexpr int NT = RP / 16;
  constexpr int NL = kGramRows * RP / 256;
  __shared__ float Al[kGramRows * LS];
  __shared__ float Bl[kGramRows * LS];
  const int idx = first + map[blockIdx.x];
  const OrthDesc o = descs[idx];
  const int local = blockIdx.x - o.wg0;
  const float* pa = base_a + o.off;
  const float* pb = base_b + o.off;
  const int r0 = local * kGramRows;
  float va[NL], vb[NL];
#pragma unroll
  for (int u = 0; u < NL; ++u) {
    const int e = threadIdx.x + 256 * u, i = e % kGramRows, t = e / kGramRows;
    const int64_t at = (int64_t)min(t, r - 1) * o.rows + min(r0 + i, o.rows - 1);
    va[u] = pa[at];
    vb[u] = pb[at];
  }
#pragma unroll
  for (int u = 0; u < NL; ++u) {
    const int e = threadIdx.x + 256 * u, i = e % kGramRows, t = e / kGramRows;
    const bool ok = t < r && r0 + i < o.rows;
    Al[i * LS + t] = ok ? va[u] : 0.f;
    Bl[i * LS + t] = ok ? vb[u] : 0.f;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, ls = lane >> 4;
  double* g = gram + o.gram_off + (int64_t)local * RP * RP;
  for (int u = wave; u < NT * NT; u += 4) {
    const int ta = u / NT, tb = u % NT;
    v4d_diag acc = v4d_diag{0.0, 0.0, 0.0, 0.0};
#pragma unroll 8
    for (int kk = 0; kk < kGramRows / 4; ++kk) {
      const int i = 4 * kk + ls;
      const double a = (double)Al[i * LS + 16 * ta + li];
      const double bv = (double)Bl[i * LS + 16 * tb + li];
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a, bv, acc, 0, 0, 0);
    }
    // acc[e] of lane (li, ls) is C_b[16 ta + 4 e + ls][16 tb + li]
#pragma unroll
    for (int e = 0; e < 4; ++e) g[(16 * ta + 4 * e + ls) * RP + 16 * tb + li] = acc[e];
  }
}

// Mean cosine of the principal angles, one workgroup per matrix: the
// cosines are the singular values of C = A_hat^T B_hat (summed into the
// matrix's T slot), i.e. the square roots of the eigenvalues of S = C^T C,
// found by cyclic Jacobi rotations on S in LDS.  Each round rotates RP / 2
// disjoint index pairs at once (round-robin pairing: index RP - 1 stays, the
// others move one place per round), all rows first and then all columns, so
// that the round equals the same rotations applied one after another; a
// sweep is RP - 1 rounds and meets every pair once, kJacobiSweeps sweeps.
// The mean is over the r columns (padding and zero columns add cosines of
// 0).
template <int RP>
__global__ __launch_bounds__(256) void k_overlap_final(const OrthDesc* __restrict__ descs, int first, int r,
                                                       const double* __restrict__ gram, double* __restrict__ out) {
  constexpr int NP = RP / 2;
  constexpr int LD = RP + 1;
  __shared__ double S[RP * LD];
  __shared__ double Cl[RP * RP];
  __shared__ double cs[NP], sn[NP];
  __shared__ int pp[NP], qq[NP];
  const OrthDesc o = descs[first + blockIdx.x];
  const double* c = gram + o.t_off;
  for (int e = threadIdx.x; e < RP * RP; e += 256) Cl[e] = c[e];
  __syncthreads();
  for (int e = threadIdx.x; e < RP * RP; e += 256) {
    const int i = e / RP, j = e % RP;
    double s = 0.0;
    for (int k = 0; k < RP; ++k) s = fma(Cl[k * RP + i], Cl[k * RP + j], s);
    S[i * LD + j] = s;
  }
  __syncthreads();
  for (int sweep = 0; sweep < kJacobiSweeps; ++sweep) {
    for (int round = 0; round < RP - 1; ++round) {
      if (threadIdx.x < NP) {
        const int t = threadIdx.x;
        int a, b;
        if (t == 0) {
          a = RP - 1;
          b = round;
        } else {
          a = (round + t) % (RP - 1);
          b = (round - t + RP - 1) % (RP - 1);
        }
        const int p = min(a, b), q = max(a, b);
        const double apq = S[p * LD + q];
        double cc = 1.0, ss = 0.0;
        if (apq != 0.0) {
          const double th = (S[q * LD + q] - S[p * LD + p]) / (2.0 * apq);
          const double tt = (th >= 0.0 ? 1.0 : -1.0) / (fabs(th) + sqrt(th * th + 1.0));
          cc = 1.0 / sqrt(tt * tt + 1.0);
          ss = tt * cc;
        }
        cs[t] = cc;
        sn[t] = ss;
        pp[t] = p;
        qq[t] = q;
      }
      __syncthreads();
      for (int e = threadIdx.x; e < NP * RP; e += 256) {  // rows p and q: S <- J^T S
        const int t = e / RP, j = e % RP;
        const int p = pp[t], q = qq[t];
        const double sp = S[p * LD + j], sq = S[q * LD + j];
        S[p * LD + j] = cs[t] * sp - sn[t] * sq;
        S[q * LD + j] = sn[t] * sp + cs[t] * sq;
      }
      __syncthreads();
      for (int e = threadIdx.x; e < NP * RP; e += 256) {  // columns p and q: S <- S J
        const int t = e / RP, i = e % RP;
        const int p = pp[t], q = qq[t];
        const double sp = S[i * LD + p], sq = S[i * LD + q];
        S[i * LD + p] = cs[t] * sp - sn[t] * sq;
        S[i * LD + q] = sn[t] * sp + cs[t] * sq;
      }
      __syncthreads();
    }
  }
  if (threadIdx.x == 0) {
    double tot = 0.0;
    for (int i = 0; i < RP; ++i) tot += sqrt(fmax(S[i * LD + i], 0.0));
    out[blockIdx.x] = tot / (double)r;
  }
}

hipError_t launch_sumsq(const LaunchCtx& c, const float* E, const float* Mh, double* out) {
  if (c.nmat == 0) return hipSuccess;
  hipLaunchKernelGGL(k_sumsq_partial, dim3(c.nmat * kStatsWGs), dim3(256), 0, c.stream, c.mats, E, Mh, c.gram);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_sumsq_final, dim3((c.nmat + 63) / 64), dim3(64), 0, c.stream, c.mats, c.nmat, c.gram, out);
  return hipGetLastError();
}

template <int RP>
static hipError_t overlap_rp(const LaunchCtx& c, int first, const float* a, const float* b, double* out) {
  hipLaunchKernelGGL((k_cross_partial<RP>), dim3(c.wg_gramq), dim3(256), 0, c.stream, c.orth, c.gramq_map, first,
                     c.rank, a, b, c.gram);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_gram_reduce(c, first, c.nmat);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_overlap_final<RP>), dim3(c.nmat), dim3(256), 0, c.stream, c.orth, first, c.rank, c.gram, out);
  return hipGetLastError();
}

hipError_t launch_overlap(const LaunchCtx& c, int first, const float* a, const float* b, double* out) {
  if (c.nmat == 0 || c.wg_gramq == 0) return hipSuccess;
  switch (c.rank_pad) {
    case 16: return overlap_rp<16>(c, first, a, b, out);
    case 32: return overlap_rp<32>(c, first, a, b, out);
    case 48: return overlap_rp<48>(c, first, a, b, out);
    case 64: return overlap_rp<64>(c, first, a, b, out);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace psgd
