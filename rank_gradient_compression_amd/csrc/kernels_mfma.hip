// Matrix-core kernels of the PowerSGD step for ranks 9..64 (gfx950, wave64).
//
// The anthology note on PowerSGD (note 152, "Limitations") points out that
// transformer language models may need ranks of 32 and more.  At such ranks
// each pass does 2r flops per element, which the vector units can no longer
// hide behind HBM traffic, so the three products run on the fp32 matrix
// cores: v_mfma_f32_16x16x4_f32, D(16x16) += A(16x4) B(4x16), with the rank
// padded to RP, a multiple of 16 (padding columns are zero).
//
// Operand layout of v_mfma_f32_16x16x4_f32 on a 64-lane wavefront:
//   A[i][k] is supplied by lane i + 16k, B[k][j] by lane j + 16k,
//   D[i][j] is returned in lane j + 16*(i/4), element i%4.
// The summation index k can be bound to any four columns (or rows) of M as
// long as A and B agree, which lets each lane feed the matrix core straight
// from its own 16-byte load of a row of M.
//
//   pass 1  P = M Q (with the EF-add and optional momentum), per 64-row tile
//           and column split; Q chunks are staged in LDS and shared by the
//           four wavefronts; split partials are summed in fixed order.
//   pass 2  Q = M^T P_hat per row block; P_hat rows staged in LDS.
//   pass 3  M_hat = P_hat Q^T computed transposed (M_hat^T = Q P_hat^T), so
//           that each lane holds four consecutive columns of one row and
//           the residual E = M - M_hat streams with 16-byte accesses.
// The orthonormalisation of P for these ranks is Gram-Schmidt carried out on
// the fp64 Gram matrix of P, spread over many workgroups (partial Gram
// blocks, a one-wavefront triangular solve per matrix, and P_hat = P T).

#include <hip/hip_runtime.h>

#include "psgd_kernels.h"
#include "psgd_tables.h"

namespace psgd {

typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4f mfma16x16x4(float a, float b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Four consecutive floats of a row from column `col` (zero past the row end).
__device__ __forceinline__ float4 ld4(const float* p, int col, int n, bool vec4) {
  if (vec4) return col < n ? *reinterpret_cast<const float4*>(p + col) : make_float4(0.f, 0.f, 0.f, 0.f);
  float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
  if (col < n) r.x = p[col];
  if (col + 1 < n) r.y = p[col + 1];
  if (col + 2 < n) r.z = p[col + 2];
  if (col + 3 < n) r.w = p[col + 3];
  return r;
}

__device__ __forceinline__ void st4(float* p, int col, int n, bool vec4, float4 v) {
  if (vec4) {
    if (col < n) *reinterpret_cast<float4*>(p + col) = v;
    return;
  }
  if (col < n) p[col] = v.x;
  if (col + 1 < n) p[col + 1] = v.y;
  if (col + 2 < n) p[col + 2] = v.z;
  if (col + 3 < n) p[col + 3] = v.w;
}

__device__ __forceinline__ int wg_of(const int32_t* map, int wg_base, int& idx) {
  const int wg = blockIdx.x + wg_base;
  idx = map[wg];
  return wg;
}

// ---------------------------------------------------------------------------
// Pass 1: P = M Q (MODE 0: M read as is; 1: M = G + E stored over E;
// 2: u = beta u + G, M = u + E)
// ---------------------------------------------------------------------------

template <int RP, int MODE>
__global__ __launch_bounds__(256) void k_mfma_p(const MatDesc* __restrict__ mats, const int32_t* __restrict__ map,
                                                int wg_base, int r, const float* __restrict__ G,
                                                float* __restrict__ E, float* __restrict__ U, float beta,
                                                const float* __restrict__ Q, float* __restrict__ P, int64_t p_fixed,
                                                float* __restrict__ ppart) {
  constexpr int QS = RP + 4;  // LDS row stride: conflict-free B-operand reads
  __shared__ float Qs[64 * QS];
  int mi;
  const int wg = wg_of(map, wg_base, mi);
  const MatDesc d = mats[mi];
  const int m = d.m, n = d.n;
  const bool vec4 = d.vec == 4;
  const int local = wg - d.wg_rows0;
  const int rb = local / d.s1, split = local - rb * d.s1;
  const int c_begin = split * d.s1_cols;
  const int c_end = min(n, c_begin + d.s1_cols);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 15, ls = lane >> 4;
  const int i0 = rb * kMfmaRows + wave * 16;
  const int row = i0 + li;
  const bool row_ok = row < m;
  const int64_t roff = d.off + (int64_t)min(row, m - 1) * n;
  const float* q = Q + d.q_off;

  v4f acc[RP / 16];
#pragma unroll
  for (int T = 0; T < RP / 16; ++T) acc[T] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int c0 = c_begin; c0 < c_end; c0 += 64) {
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * RP; e += 256) {
      const int c = e & 63, t = e >> 6;
      float v = 0.f;
      if (t < r && c0 + c < c_end) v = q[(int64_t)t * n + c0 + c];
      Qs[c * QS + t] = v;
    }
    __syncthreads();
    float4 x[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int col = c0 + 16 * qq + 4 * ls;
      const bool col_ok = col < c_end;
      if constexpr (MODE == 0) {
        x[qq] = ld4(E + roff, col_ok ? col : n, n, vec4);
      } else {
        const float4 g = ld4(G + roff, col_ok ? col : n, n, vec4);
        const float4 e = ld4(E + roff, col_ok ? col : n, n, vec4);
        float4 s;
        if constexpr (MODE == 2) {
          float4 u = ld4(U + roff, col_ok ? col : n, n, vec4);
          u.x = fmaf(beta, u.x, g.x);
          u.y = fmaf(beta, u.y, g.y);
          u.z = fmaf(beta, u.z, g.z);
          u.w = fmaf(beta, u.w, g.w);
          if (row_ok && col_ok) st4(U + roff, col, n, vec4, u);
          s = make_float4(u.x + e.x, u.y + e.y, u.z + e.z, u.w + e.w);
        } else {
          s = make_float4(g.x + e.x, g.y + e.y, g.z + e.z, g.w + e.w);
        }
        if (row_ok && col_ok) st4(E + roff, col, n, vec4, s);
        x[qq] = s;
      }
    }
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const float xv[4] = {x[qq].x, x[qq].y, x[qq].z, x[qq].w};
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float a = row_ok ? xv[v] : 0.f;
        const float* qrow = &Qs[(16 * qq + 4 * ls + v) * QS + li];
#pragma unroll
        for (int T = 0; T < RP / 16; ++T) acc[T] = mfma16x16x4(a, qrow[16 * T], acc[T]);
      }
    }
  }

  float* dst = d.s1 > 1 ? ppart + d.ppart_off + (int64_t)split * r * m : P + (p_fixed >= 0 ? p_fixed : d.p_off);
#pragma unroll
  for (int T = 0; T < RP / 16; ++T) {
    const int t = 16 * T + li;
    if (t < r) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rr = i0 + 4 * ls + e;
        if (rr < m) dst[(int64_t)t * m + rr] = acc[T][e];
      }
    }
  }
}

// Fixed-order sum of the column-split partials of pass 1.
__global__ __launch_bounds__(kRedCols) void k_psum(const MatDesc* __restrict__ mats, const int32_t* __restrict__ map,
                                                   int wg_base, int r, const float* __restrict__ ppart,
                                                   float* __restrict__ P, int64_t p_fixed) {
  int mi;
  const int wg = wg_of(map, wg_base, mi);
  const MatDesc d = mats[mi];
  const int64_t len = (int64_t)r * d.m;
  const int64_t idx = (int64_t)(wg - d.wg_pred0) * kRedCols + threadIdx.x;
  if (idx >= len) return;
  const float* src = ppart + d.ppart_off + idx;
  float s0 = 0.f, s1 = 0.f;
  int b = 0;
  for (; b + 2 <= d.s1; b += 2) {
    s0 += src[(int64_t)b * len];
    s1 += src[(int64_t)(b + 1) * len];
  }
  if (b < d.s1) s0 += src[(int64_t)b * len];
  P[(p_fixed >= 0 ? p_fixed : d.p_off) + idx] = s0 + s1;
}

// ---------------------------------------------------------------------------
// Pass 2: Q = M^T P_hat over one row block (partials when the matrix has
// several row blocks)
// ---------------------------------------------------------------------------

template <int RP>
__global__ __launch_bounds__(256) void k_mfma_qt(const MatDesc* __restrict__ mats, const int32_t* __restrict__ map,
                                                 int wg_base, int r, const float* __restrict__ M,
                                                 const float* __restrict__ Ph, int64_t ph_fixed,
                                                 float* __restrict__ Q, float* __restrict__ part) {
  constexpr int PS = RP == 16 ? 16 : 80;  // LDS row stride: conflict-free B-operand reads
  __shared__ float Ps[64 * PS];
  int mi;
  const int wg = wg_of(map, wg_base, mi);
  const MatDesc d = mats[mi];
  const int m = d.m, n = d.n;
  const bool vec4 = d.vec == 4;
  const int local = wg - d.wg_mtp0;
  const int rb = local / d.ncb, cb = local - rb * d.ncb;
  const int i0 = rb * d.rb_rows;
  const int i1 = min(m, i0 + d.rb_rows);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 15, ls = lane >> 4;
  const int j0 = cb * kMfmaCols + wave * 64;
  const int col = j0 + 4 * li;
  const float* ph = Ph + (ph_fixed >= 0 ? ph_fixed : d.p_off);

  v4f acc[4][RP / 16];
#pragma unroll
  for (int v = 0; v < 4; ++v)
#pragma unroll
    for (int T = 0; T < RP / 16; ++T) acc[v][T] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int ib = i0; ib < i1; ib += 64) {
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * RP; e += 256) {
      const int k = e & 63, t = e >> 6;
      float v = 0.f;
      if (t < r && ib + k < i1) v = ph[(int64_t)t * m + ib + k];
      Ps[k * PS + t] = v;
    }
    __syncthreads();
    float4 x[16];
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const int rrow = ib + 4 * kk + ls;
      x[kk] = rrow < i1 ? ld4(M + d.off + (int64_t)rrow * n, col, n, vec4) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const float xv[4] = {x[kk].x, x[kk].y, x[kk].z, x[kk].w};
      const float* prow = &Ps[(4 * kk + ls) * PS + li];
#pragma unroll
      for (int T = 0; T < RP / 16; ++T) {
        const float b = prow[16 * T];
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[v][T] = mfma16x16x4(xv[v], b, acc[v][T]);
      }
    }
  }

  float* out = d.nrb > 1 ? part + d.part_off + (int64_t)rb * r * n : Q + d.q_off;
#pragma unroll
  for (int T = 0; T < RP / 16; ++T) {
    const int t = 16 * T + li;
    if (t < r) {
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = j0 + 4 * (4 * ls + e) + v;
          if (c < n) out[(int64_t)t * n + c] = acc[v][T][e];
        }
    }
  }
}

// ---------------------------------------------------------------------------
// Pass 3: M_hat = P_hat Q^T (transposed on the matrix core); residual and/or
// decompression.  One wavefront: 64 rows (four 16-row tiles) and every fourth
// 16-column tile of the workgroup's column split.
// ---------------------------------------------------------------------------

template <int RP, bool READ_M, bool WRITE_E, bool WRITE_MHAT>
__global__ __launch_bounds__(256) void k_mfma_recon(const MatDesc* __restrict__ mats, const int32_t* __restrict__ map,
                                                    int wg_base, int r, float* __restrict__ E,
                                                    const float* __restrict__ Q, const float* __restrict__ Ph,
                                                    float* __restrict__ Mhat) {
  constexpr int KS = RP / 4;  // k-steps of 4 rank columns
  int mi;
  const int wg = wg_of(map, wg_base, mi);
  const MatDesc d = mats[mi];
  const int m = d.m, n = d.n;
  const bool vec4 = d.vec == 4;
  const int local = wg - d.wg_rows0;
  const int rb = local / d.s1, split = local - rb * d.s1;
  const int c_begin = split * d.s1_cols;
  const int c_end = min(n, c_begin + d.s1_cols);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 15, ls = lane >> 4;
  const int i0 = rb * kMfmaRows;
  const float* ph = Ph + d.p_off;
  const float* q = Q + d.q_off;

  // B operand: P_hat^T, lane (li, ls) holds P_hat[i0 + 16 rt + li][4 kk + ls]
  float bfr[4][KS];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int rr = i0 + 16 * rt + li, t = 4 * kk + ls;
      bfr[rt][kk] = (rr < m && t < r) ? ph[(int64_t)t * m + rr] : 0.f;
    }

  for (int j0 = c_begin + 16 * wave; j0 < c_end; j0 += 64) {
    // A operand: Q, lane (li, ls) holds Q[j0 + li][4 kk + ls]
    float afr[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int t = 4 * kk + ls, c = j0 + li;
      afr[kk] = (t < r && c < c_end) ? q[(int64_t)t * n + c] : 0.f;
    }
    const int col = j0 + 4 * ls;
    const bool col_ok = col < c_end;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) acc = mfma16x16x4(afr[kk], bfr[rt][kk], acc);
      const int rr = i0 + 16 * rt + li;
      if (rr < m && col_ok) {
        float* rowp = E + d.off + (int64_t)rr * n;
        const float4 mh = make_float4(acc[0], acc[1], acc[2], acc[3]);
        if constexpr (READ_M) {
          const float4 x = ld4(rowp, col, n, vec4);
          if constexpr (WRITE_E)
            st4(rowp, col, n, vec4, make_float4(x.x - mh.x, x.y - mh.y, x.z - mh.z, x.w - mh.w));
        }
        if constexpr (WRITE_MHAT) st4(Mhat + d.off + (int64_t)rr * n, col, n, vec4, mh);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Orthonormalisation: Gram-Schmidt carried out on the fp64 Gram matrix
// ---------------------------------------------------------------------------
//
// Gram-Schmidt on the columns of P (rows x r) in natural order with positive
// normalisation gives P_hat = P T, T upper triangular.  In exact arithmetic
// its coefficients are those of the Cholesky factor R of A = P^T P: the norm
// of column k after projection on the previous P_hat columns is R_kk, and
// R_kj = P_hat_k^T P_j.  A column whose norm after projection is at most
// 1e-4 of its norm before (sqrt(A_kk)), or whose norm is zero, is dependent:
// its P_hat column is zero and nothing is projected on it (row k of R is
// zero).  A is accumulated in fp64 from the fp32 P (each product exact), so
// the cancellation in R_kk^2 = A_kk - sum_j R_jk^2 is harmless at fp32 output
// precision and the threshold is decided reliably.  Four launches, all
// grouped over the matrices:
//   k_gram_partial  A_b = P_b^T P_b over blocks of kGramRows rows
//   k_gram_reduce   A = sum_b A_b in block order
//   k_gram_solve    R (right-looking Cholesky) and T = R^-1, one wavefront
//   k_apply_t       P_hat = P T row by row in fp64, rounded to fp32

// Descriptor of this workgroup: first + map[wg] over a grouped grid, or the
// single descriptor `first`.
__device__ __forceinline__ int orth_idx(const OrthDesc* descs, const int32_t* map, int first, int& local) {
  if (map) {
    const int idx = first + map[blockIdx.x];
    local = blockIdx.x - descs[idx].wg0;
    return idx;
  }
  local = blockIdx.x;
  return first;
}

constexpr int kGramChunk = 128;  // rows staged in LDS at a time

template <int RP>
__global__ __launch_bounds__(256) void k_gram_partial(const OrthDesc* __restrict__ descs, const int32_t* __restrict__ map,
                                                      int first, int r, const float* __restrict__ base,
                                                      double* __restrict__ gram) {
  constexpr int LS = RP + 1;
  constexpr int BF = RP / 16;  // each of the 16 x 16 threads owns a BF x BF block of A
  __shared__ float Pl[kGramChunk * LS];
  int local;
  const OrthDesc o = descs[orth_idx(descs, map, first, local)];
  const float* p = base + o.off;
  const int ta = threadIdx.x >> 4, tb = threadIdx.x & 15;
  double acc[BF][BF];
#pragma unroll
  for (int a = 0; a < BF; ++a)
#pragma unroll
    for (int b = 0; b < BF; ++b) acc[a][b] = 0.0;
  for (int r0 = local * kGramRows; r0 < min(o.rows, (local + 1) * kGramRows); r0 += kGramChunk) {
    __syncthreads();
    for (int e = threadIdx.x; e < kGramChunk * RP; e += 256) {
      const int i = e % kGramChunk, t = e / kGramChunk;
      Pl[i * LS + t] = (t < r && r0 + i < o.rows) ? p[(int64_t)t * o.rows + r0 + i] : 0.f;
    }
    __syncthreads();
    for (int i = 0; i < kGramChunk; ++i) {
      double xa[BF], xb[BF];
#pragma unroll
      for (int a = 0; a < BF; ++a) {
        xa[a] = (double)Pl[i * LS + ta * BF + a];
        xb[a] = (double)Pl[i * LS + tb * BF + a];
      }
#pragma unroll
      for (int a = 0; a < BF; ++a)
#pragma unroll
        for (int b = 0; b < BF; ++b) acc[a][b] = fma(xa[a], xb[b], acc[a][b]);
    }
  }
  double* g = gram + o.gram_off + (int64_t)local * RP * RP;
#pragma unroll
  for (int a = 0; a < BF; ++a)
#pragma unroll
    for (int b = 0; b < BF; ++b) g[(ta * BF + a) * RP + tb * BF + b] = acc[a][b];
}

// Fixed-order block sum: A (at t_off) = sum_b A_b.  Four running sums over
// interleaved blocks keep several loads in flight; they are combined in a
// fixed order, so the result is deterministic.
template <int RP>
__global__ __launch_bounds__(256) void k_gram_reduce(const OrthDesc* __restrict__ descs, int first,
                                                     double* __restrict__ gram) {
  constexpr int WPD = RP * RP / 256;  // workgroups per descriptor
  const OrthDesc o = descs[first + blockIdx.x / WPD];
  const int e = (blockIdx.x % WPD) * 256 + threadIdx.x;
  const double* g = gram + o.gram_off + e;
  double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
  int b = 0;
  for (; b + 4 <= o.ngb; b += 4) {
    s0 += g[(int64_t)b * RP * RP];
    s1 += g[(int64_t)(b + 1) * RP * RP];
    s2 += g[(int64_t)(b + 2) * RP * RP];
    s3 += g[(int64_t)(b + 3) * RP * RP];
  }
  for (; b < o.ngb; ++b) s0 += g[(int64_t)b * RP * RP];
  gram[o.t_off + e] = (s0 + s1) + (s2 + s3);
}

// One wavefront per factor: Cholesky of A with the dependence rule, then
// T = R^-1 (lane l computes row l of T, which depends on no other row).
template <int RP>
__global__ __launch_bounds__(64) void k_gram_solve(const OrthDesc* __restrict__ descs, int first, int r,
                                                   double* __restrict__ gram, float zero_rel) {
  constexpr int SS = RP + 1;
  __shared__ double S[RP * SS];   // Schur complement; row k becomes row k of R
  __shared__ double dg[RP];       // diagonal of A (norms before projection)
  __shared__ double rkk[RP];      // R_kk, 0 for dependent columns
  const OrthDesc o = descs[first + blockIdx.x];
  const int lane = threadIdx.x;
  double* a = gram + o.t_off;
  for (int e = lane; e < RP * RP; e += 64) S[(e / RP) * SS + e % RP] = a[e];
  __syncthreads();
  if (lane < RP) dg[lane] = S[lane * SS + lane];
  __syncthreads();
  for (int k = 0; k < r; ++k) {
    const double d = S[k * SS + k];
    const double nu0 = sqrt(dg[k]);
    const double nv = d > 0.0 ? sqrt(d) : 0.0;
    const bool zero = !(nu0 > 0.0) || nv <= (double)zero_rel * nu0;
    const double inv = zero ? 0.0 : 1.0 / nv;
    __syncthreads();
    if (lane > k && lane < r) S[k * SS + lane] *= inv;
    if (lane == 0) {
      rkk[k] = zero ? 0.0 : nv;
      S[k * SS + k] = zero ? 0.0 : nv;
    }
    __syncthreads();
    const int w = r - k - 1;
    for (int e = lane; e < w * w; e += 64) {
      const int i = k + 1 + e / w, j = k + 1 + e % w;
      if (i <= j) S[i * SS + j] = fma(-S[k * SS + i], S[k * SS + j], S[i * SS + j]);
    }
    __syncthreads();
  }
  // T = R^-1 on the non-dependent columns: T_lk = (delta_lk - sum_{l<=j<k}
  // T_lj R_jk) / R_kk, zero for dependent k.  Row l of T uses only row l.
  double* t = a;  // overwrite A with T
  if (lane < RP) {
    double trow[RP];
#pragma unroll
    for (int k = 0; k < RP; ++k) trow[k] = 0.0;
#pragma unroll
    for (int k = 0; k < RP; ++k) {
      if (k < r && k >= lane) {
        double s = k == lane ? 1.0 : 0.0;
#pragma unroll
        for (int j = 0; j < RP; ++j)
          if (j >= lane && j < k) s = fma(-trow[j], S[j * SS + k], s);
        trow[k] = rkk[k] > 0.0 ? s / rkk[k] : 0.0;
      }
    }
#pragma unroll
    for (int k = 0; k < RP; ++k) t[lane * RP + k] = trow[k];
  }
}

// P_hat = P T, rows in parallel, evaluated in fp64 and rounded to fp32.
// Column block k0..k0+15 of P_hat needs the columns a <= k0+15 of P, so the
// blocks are produced from the last to the first and each overwrites only
// columns no later block reads.
template <int RP>
__global__ __launch_bounds__(256) void k_apply_t(const OrthDesc* __restrict__ descs, const int32_t* __restrict__ map,
                                                 int first, int r, float* __restrict__ base,
                                                 const double* __restrict__ gram) {
  __shared__ double T[RP * RP];
  int local;
  const OrthDesc o = descs[orth_idx(descs, map, first, local)];
  const double* t = gram + o.t_off;
  for (int e = threadIdx.x; e < RP * RP; e += 256) T[e] = t[e];
  __syncthreads();
  const int i = local * kGramRows + threadIdx.x;
  if (i >= o.rows) return;
  float* p = base + o.off + i;
  const int64_t ld = o.rows;
  for (int k0 = (r - 1) / 16 * 16; k0 >= 0; k0 -= 16) {
    double s[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) s[c] = 0.0;
    const int amax = min(r, k0 + 16);
#pragma unroll 2
    for (int a = 0; a < amax; ++a) {
      const double xa = (double)p[a * ld];
      const double* trow = &T[a * RP + k0];
#pragma unroll
      for (int c = 0; c < 16; ++c) s[c] = fma(xa, trow[c], s[c]);
    }
#pragma unroll
    for (int c = 0; c < 16; ++c)
      if (k0 + c < r) p[(k0 + c) * ld] = (float)s[c];
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

#define PSGD_RP_SWITCH(RP_, CALL)                     \
  switch (RP_) {                                      \
    case 16: { constexpr int RPV = 16; return CALL; } \
    case 32: { constexpr int RPV = 32; return CALL; } \
    case 48: { constexpr int RPV = 48; return CALL; } \
    case 64: { constexpr int RPV = 64; return CALL; } \
    default: return hipErrorInvalidValue;             \
  }

template <int RP>
static hipError_t mfma_p_rp(const LaunchCtx& c, const GridRange& g, int mode, const float* G, float* E, float* U,
                            float beta, const float* Q, float* P, int64_t p_fixed) {
  if (g.count == 0) return hipSuccess;
  const dim3 gr(g.count), b(256);
  if (mode == 0)
    hipLaunchKernelGGL((k_mfma_p<RP, 0>), gr, b, 0, c.stream, c.mats, c.rows_map, g.base, c.rank, G, E, U, beta, Q,
                       P, p_fixed, c.ppart);
  else if (mode == 1)
    hipLaunchKernelGGL((k_mfma_p<RP, 1>), gr, b, 0, c.stream, c.mats, c.rows_map, g.base, c.rank, G, E, U, beta, Q,
                       P, p_fixed, c.ppart);
  else
    hipLaunchKernelGGL((k_mfma_p<RP, 2>), gr, b, 0, c.stream, c.mats, c.rows_map, g.base, c.rank, G, E, U, beta, Q,
                       P, p_fixed, c.ppart);
  return hipGetLastError();
}

hipError_t launch_mfma_p(const LaunchCtx& c, const GridRange& g, int mode, const float* G, float* E, float* U,
                         float beta, const float* Q, float* P, int64_t p_fixed) {
  PSGD_RP_SWITCH(c.rank_pad, mfma_p_rp<RPV>(c, g, mode, G, E, U, beta, Q, P, p_fixed));
}

hipError_t launch_psum(const LaunchCtx& c, const GridRange& g, float* P, int64_t p_fixed) {
  if (g.count == 0) return hipSuccess;
  hipLaunchKernelGGL(k_psum, dim3(g.count), dim3(kRedCols), 0, c.stream, c.mats, c.pred_map, g.base, c.rank, c.ppart,
                     P, p_fixed);
  return hipGetLastError();
}

template <int RP>
static hipError_t mfma_qt_rp(const LaunchCtx& c, const GridRange& g, const float* M, const float* Ph, int64_t ph_fixed,
                             float* Q) {
  if (g.count == 0) return hipSuccess;
  hipLaunchKernelGGL((k_mfma_qt<RP>), dim3(g.count), dim3(256), 0, c.stream, c.mats, c.mtp_map, g.base, c.rank, M, Ph,
                     ph_fixed, Q, c.part);
  return hipGetLastError();
}

hipError_t launch_mfma_qt(const LaunchCtx& c, const GridRange& g, const float* M, const float* Ph, int64_t ph_fixed,
                          float* Q) {
  PSGD_RP_SWITCH(c.rank_pad, mfma_qt_rp<RPV>(c, g, M, Ph, ph_fixed, Q));
}

template <int RP>
static hipError_t mfma_recon_rp(const LaunchCtx& c, float* E, const float* Q, const float* Ph, float* Mhat,
                                bool residual) {
  if (c.wg_rows == 0) return hipSuccess;
  const dim3 g(c.wg_rows), b(256);
  if (residual && Mhat)
    hipLaunchKernelGGL((k_mfma_recon<RP, true, true, true>), g, b, 0, c.stream, c.mats, c.rows_map, 0, c.rank, E, Q,
                       Ph, Mhat);
  else if (residual)
    hipLaunchKernelGGL((k_mfma_recon<RP, true, true, false>), g, b, 0, c.stream, c.mats, c.rows_map, 0, c.rank, E, Q,
                       Ph, Mhat);
  else
    hipLaunchKernelGGL((k_mfma_recon<RP, false, false, true>), g, b, 0, c.stream, c.mats, c.rows_map, 0, c.rank, E,
                       Q, Ph, Mhat);
  return hipGetLastError();
}

hipError_t launch_mfma_recon(const LaunchCtx& c, float* E, const float* Q, const float* Ph, float* Mhat,
                             bool residual) {
  PSGD_RP_SWITCH(c.rank_pad, mfma_recon_rp<RPV>(c, E, Q, Ph, Mhat, residual));
}

template <int RP>
static hipError_t gram_orth_rp(const LaunchCtx& c, int first, int count, const int32_t* map, int nblocks,
                               float* base) {
  if (nblocks == 0 || count == 0) return hipSuccess;
  hipLaunchKernelGGL((k_gram_partial<RP>), dim3(nblocks), dim3(256), 0, c.stream, c.orth, map, first, c.rank, base,
                     c.gram);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_gram_reduce<RP>), dim3(count * (RP * RP / 256)), dim3(256), 0, c.stream, c.orth, first,
                     c.gram);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_gram_solve<RP>), dim3(count), dim3(64), 0, c.stream, c.orth, first, c.rank, c.gram,
                     kZeroColumnRel);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_apply_t<RP>), dim3(nblocks), dim3(256), 0, c.stream, c.orth, map, first, c.rank, base, c.gram);
  return hipGetLastError();
}

hipError_t launch_gram_orth(const LaunchCtx& c, int first, int count, const int32_t* map, int nblocks,
                            float* base) {
  PSGD_RP_SWITCH(c.rank_pad, gram_orth_rp<RPV>(c, first, count, map, nblocks, base));
}

}  // namespace psgd
