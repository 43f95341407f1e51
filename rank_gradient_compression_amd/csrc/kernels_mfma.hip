// Matrix-core kernels of the PowerSGD step for ranks 9..64 and the
// orthonormalisation for every rank (gfx950, wave64).
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
// long as A and B agree, so that a lane's operands for four steps are one
// 16-byte read.
//
// Global memory is read and written row-contiguously (a wavefront moves 512
// bytes to 1 KB of one or two rows per instruction) and the tiles reach the
// matrix core through LDS; reading the operands from global memory in the
// matrix core's own layout (16 rows x 64 bytes per instruction) streamed
// markedly slower.
//
//   pass 1  P = M Q (with the EF-add and optional momentum): a workgroup
//           walks its 64-row tile of one column split in 128- or 64-column
//           chunks (M formed, stored back and staged in LDS with the chunk
//           of Q);
//           split partials are summed in fixed order.  With a deferred
//           residual each wavefront first forms its 16 rows of the previous
//           step's reconstruction in LDS from the staged Q chunk.
//   pass 2  Q = M^T P_hat: a workgroup walks 128 columns of a row block in
//           32-row chunks staged in LDS with the chunk's P_hat rows.
//   pass 3  M_hat = P_hat Q^T computed transposed (M_hat^T = Q P_hat^T) into
//           an LDS tile of 32 rows x 256 columns, then streamed out with E.
// The orthonormalisation (every rank) is Gram-Schmidt carried out on the
// fp64 Gram matrix of P: Gram blocks on the fp64 matrix core, a fixed-order
// reduction, a one-wavefront Cholesky per matrix, and P_hat = P R^-1 by
// substitution.

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

// Rows whose length and start allow 16-byte accesses (VEC4) load at a
// clamped, always valid column and zero the value when out of range: no
// branches, so every load of a step can be in flight at once.  Other rows
// take the guarded scalar path.
// Values past the row end are zeroed with a select between the loaded value
// and a zero rvalue, which the compiler can defer to the value's use (so the
// loads stay in flight together); a select between two struct lvalues
// (r = ok ? v : r) is lowered to a select of stack addresses, i.e. private
// scratch, and masking each component right after the load makes the
// compiler wait for that load there (k_mfma_qt<64> 72 -> 88 us).
template <bool VEC4>
__device__ __forceinline__ float4 ldq(const float* rowp, int col, bool ok, int col_safe, int n) {
  if constexpr (VEC4) {
    const float4 v = *reinterpret_cast<const float4*>(rowp + (ok ? col : col_safe));
    return ok ? v : make_float4(0.f, 0.f, 0.f, 0.f);
  } else {
    return ld4(rowp, ok ? col : n, n, false);
  }
}

// Streaming (non-temporal) variants for data used once per step: the M read
// and the M_hat write of the residual pass.
typedef float v4f_nt __attribute__((ext_vector_type(4)));

template <bool VEC4>
__device__ __forceinline__ float4 ldq_nt(const float* rowp, int col, bool ok, int col_safe, int n) {
  if constexpr (VEC4) {
    const v4f_nt v = __builtin_nontemporal_load(reinterpret_cast<const v4f_nt*>(rowp + (ok ? col : col_safe)));
    return ok ? make_float4(v[0], v[1], v[2], v[3]) : make_float4(0.f, 0.f, 0.f, 0.f);
  } else {
    return ld4(rowp, ok ? col : n, n, false);
  }
}

template <bool VEC4>
__device__ __forceinline__ void stq_nt(float* rowp, int col, int n, float4 v) {
  if constexpr (VEC4) {
    if (col < n) {
      const v4f_nt t = {v.x, v.y, v.z, v.w};
      __builtin_nontemporal_store(t, reinterpret_cast<v4f_nt*>(rowp + col));
    }
  } else {
    st4(rowp, col, n, false, v);
  }
}

// Four bfloat16 gradients widened to fp32 (same masking as ldq).
template <bool VEC4>
__device__ __forceinline__ float4 ldq_bf16(const uint16_t* rowp, int col, bool ok, int col_safe, int n) {
  float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
  if constexpr (VEC4) {
    const uint2 t = *reinterpret_cast<const uint2*>(rowp + (ok ? col : col_safe));
    const float4 v = make_float4(__uint_as_float(t.x << 16), __uint_as_float(t.x & 0xffff0000u),
                                 __uint_as_float(t.y << 16), __uint_as_float(t.y & 0xffff0000u));
    return ok ? v : make_float4(0.f, 0.f, 0.f, 0.f);
  } else {
    // clamped addresses (col_safe < n), values zeroed past the row end
    const int c = ok ? col : col_safe;
    const uint32_t a0 = rowp[min(c, n - 1)], a1 = rowp[min(c + 1, n - 1)];
    const uint32_t a2 = rowp[min(c + 2, n - 1)], a3 = rowp[min(c + 3, n - 1)];
    if (ok) {
      r.x = col < n ? __uint_as_float(a0 << 16) : 0.f;
      r.y = col + 1 < n ? __uint_as_float(a1 << 16) : 0.f;
      r.z = col + 2 < n ? __uint_as_float(a2 << 16) : 0.f;
      r.w = col + 3 < n ? __uint_as_float(a3 << 16) : 0.f;
    }
  }
  return r;
}

template <bool VEC4>
__device__ __forceinline__ void stq(float* rowp, int col, int n, float4 v) {
  st4(rowp, col, n, VEC4, v);
}

__device__ __forceinline__ int wg_of(const int32_t* map, int wg_base, int& idx) {
  const int wg = blockIdx.x + wg_base;
  idx = map[wg];
  return wg;
}

// ---------------------------------------------------------------------------
// Pass 1: P = M Q (MODE 0: M read as is; 1: M = G + E stored over E;
// 2: u = beta u + G, M = u + E; 3: M = G; 4: u = beta u + G, M = u --
// modes 3 and 4 without error feedback, M still stored over E; 5 and 6: as 1
// and 2 with a deferred residual, E = E_in - Pold Q^T formed here)
//
// With a deferred residual the reconstruction of a 16 x 16 tile is the same
// sequence of matrix-core steps as in the residual pass (A = Q, B = P_hat^T,
// summed over the rank in order), and its result layout -- lane (li, ls)
// holds row li, columns 4 ls .. 4 ls + 3 -- is the layout this pass loads M
// in, so E is formed bit for bit as the residual pass would have stored it.
// ---------------------------------------------------------------------------

// P = M Q with the EF-add of MODE 1..6 (or M as is, MODE 0: the refresh),
// staged: a workgroup owns the 64-row tile of its column split and walks the
// split in CH-column chunks.  Each wavefront loads 16 rows of a chunk with
// row-contiguous accesses (CH / 4 lanes x 16 bytes per row, 256 / CH rows
// per instruction) -- G, E and u as the mode needs --, forms M (and u) and
// stores it back over E the same way, and writes M into an LDS tile; the
// chunk's Q columns go to LDS once for the workgroup.  Each wavefront then
// accumulates its own 16 rows (every rank tile) on the matrix core from LDS.
// The next chunk's loads are issued before the current chunk's matrix
// products.  The summation index of matrix-core step v of a 16-column block
// is bound, for lane (li, ls), to column 4 ls + v, so that the lane's A and B
// operands are one 16-byte LDS read each per block.
//
// Accumulation: the matrix core sums one chunk's products in fp32, and each
// chunk's sums are then added into fp64 running sums (and the column-split
// partials are kept and summed in fp64).  A long fp32 accumulation loses
// digits to rounding at the size of the running sum, while P = M Q can be
// much smaller than that after cancellation: with a warm start, column k of
// Q lines up with the k-th right singular direction of M, so |P_k| ~ s_k^2
// against running sums of order s_1 s_k (s_k the singular values).  On
// spectra that fall off like k^-1.5 that cancellation costs fp32 most of its
// digits at ranks of 32 and more; summing short fp32 runs in fp64 keeps P
// accurate to about the fp32 rounding of its own entries.
//
// Columns per LDS chunk: 128 by default; 64 where the workgroups are
// limited by LDS and registers (the plain M Q of the refresh, ranks above
// 32), halving both so that more workgroups stay resident per compute unit.
constexpr int mq_chunk(int rp, int mode) { return (mode == 0 || rp > 32) ? 64 : 128; }

template <int RP, int MODE, bool VEC4, bool GBF16, int CH>
__device__ __forceinline__ void mfma_mq_body(const MatDesc& d, int wg, int r, const void* __restrict__ G,
                                             float* __restrict__ E, float* __restrict__ U, float beta,
                                             const float* __restrict__ Q, float* P, int64_t p_fixed,
                                             double* __restrict__ ppart, float* smem, const float* Pold) {
  static_assert(MODE >= 0 && MODE <= 6, "pass 1 modes");
  constexpr bool LOAD_G = MODE != 0;
  constexpr bool DEFERRED = MODE >= 5;
  constexpr bool LOAD_E = MODE <= 2 || DEFERRED;
  constexpr bool MOM = MODE == 2 || MODE == 4 || MODE == 6;
  constexpr int KS = RP / 4;
  static_assert(CH == 64 || CH == 128, "chunk width");
  constexpr int LDM = CH + 4;    // LDS row stride of the M chunk (floats)
  constexpr int LPR = CH / 4;    // lanes per row of a chunk
  constexpr int RPI = 64 / LPR;  // rows per wavefront load
  constexpr int NU = 16 / RPI;   // wavefront loads per chunk (16 rows)
  constexpr int QLD = CH + 4;                     // LDS stride of one rank's Q chunk
  constexpr int QPT = (RP * CH / 4 + 255) / 256;  // Q float4s a thread loads per chunk
  float* Ms = smem;                               // [64 rows][LDM]
  float* Qs = smem + kMfmaRows * LDM;             // [RP ranks][QLD]
  const int m = d.m, n = d.n;
  const int local = wg - d.wg_rows0;
  const int rb = local / d.s1, split = local - rb * d.s1;
  const int c_begin = split * d.s1_cols;
  const int c_end = min(n, c_begin + d.s1_cols);
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, ls = lane >> 4;
  const int i0 = rb * kMfmaRows;
  const float* q = Q + d.q_off;
  // row accesses: lane (hr = lane / LPR, lane % LPR) covers columns
  // 4 (lane % LPR) .. + 3 of rows RPI u + hr
  const int hr = lane / LPR, cl4 = 4 * (lane % LPR);

  v4f acc[RP / 16];        // this chunk's products (fp32, matrix core)
  double accd[RP / 16][4];  // running sums over the chunks (fp64)
#pragma unroll
  for (int T = 0; T < RP / 16; ++T) {
    acc[T] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) accd[T][e] = 0.0;
  }

  // Deferred residual: B operand P_hat_old^T of the wavefront's 16 rows, lane
  // (li, ls) holding Pold[row][4 kk + ls] (read before any P is written).
  float bfr[DEFERRED ? KS : 1];
  if constexpr (DEFERRED) {
    const int row = i0 + 16 * wave + li;
    const float* po = Pold + d.p_off;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int t = 4 * kk + ls;
      bfr[kk] = (row < m && t < r) ? po[(int64_t)t * m + row] : 0.f;
    }
  }

  float4 xg[NU], xe[LOAD_E ? NU : 1], xu[MOM ? NU : 1], qn[QPT];
  auto row_of = [&](int u) { return i0 + 16 * wave + RPI * u + hr; };
  auto load_chunk = [&](int c0) {
    const int col = c0 + cl4;
    const bool col_ok = col < c_end;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int row = row_of(u);
      const bool ok = row < m && col_ok;
      const int64_t ro = d.off + (int64_t)min(row, m - 1) * n;
      if constexpr (!LOAD_G) {
        xg[u] = ldq<VEC4>(E + ro, col, ok, c_begin, n);
      } else if constexpr (GBF16) {
        xg[u] = ldq_bf16<VEC4>(static_cast<const uint16_t*>(G) + ro, col, ok, c_begin, n);
      } else {
        xg[u] = ldq<VEC4>(static_cast<const float*>(G) + ro, col, ok, c_begin, n);
      }
      if constexpr (LOAD_E) xe[u] = ldq<VEC4>(E + ro, col, ok, c_begin, n);
      if constexpr (MOM) xu[u] = ldq<VEC4>(U + ro, col, ok, c_begin, n);
    }
#pragma unroll
    for (int u = 0; u < QPT; ++u) {
      const int e = threadIdx.x + 256 * u;  // float4 index within [RP][CH / 4]
      const int t = e / (CH / 4), c = c0 + 4 * (e % (CH / 4));
      qn[u] = (e < RP * CH / 4 && t < r) ? ldq<VEC4>(q + (int64_t)t * n, c, c < c_end, c_begin, n)
                                               : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto stage_q = [&]() {
#pragma unroll
    for (int u = 0; u < QPT; ++u) {
      const int e = threadIdx.x + 256 * u;
      if (e < RP * CH / 4)
        *reinterpret_cast<float4*>(&Qs[(e / (CH / 4)) * QLD + 4 * (e % (CH / 4))]) = qn[u];
    }
  };
  // Deferred residual: the previous step's reconstruction of the wavefront's
  // 16 rows x CH columns, M_hat^T = Q P_hat_old^T tile by tile (A = Q
  // from LDS, the same operands and rank order as the residual pass), into
  // the wavefront's own rows of Ms in the result layout (row li, columns
  // 4 ls .. 4 ls + 3).
  auto recon_tile = [&]() {
#pragma unroll
    for (int ct = 0; ct < CH / 16; ++ct) {
      v4f a4 = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) a4 = mfma16x16x4(Qs[(4 * kk + ls) * QLD + 16 * ct + li], bfr[kk], a4);
      *reinterpret_cast<float4*>(&Ms[(16 * wave + li) * LDM + 16 * ct + 4 * ls]) =
          make_float4(a4[0], a4[1], a4[2], a4[3]);
    }
  };
  // EF-add of the loaded chunk (E = E_in - M_hat_old first with a deferred
  // residual), M (and u) stored back, M into the wavefront's rows of Ms.
  auto ef_chunk = [&](int c0) {
    const int col = c0 + cl4;
    const bool col_ok = col < c_end;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int row = row_of(u);
      float* mrow = &Ms[(16 * wave + RPI * u + hr) * LDM + cl4];
      float4 s;
      if constexpr (MODE == 0) {
        s = xg[u];
      } else {
        const float4 g = xg[u];
        float4 e = LOAD_E ? xe[LOAD_E ? u : 0] : make_float4(0.f, 0.f, 0.f, 0.f);
        if constexpr (DEFERRED) {
          const float4 mh = *reinterpret_cast<const float4*>(mrow);
          e = make_float4(e.x - mh.x, e.y - mh.y, e.z - mh.z, e.w - mh.w);
        }
        if constexpr (MOM) {
          float4 uu = xu[MOM ? u : 0];
          uu.x = fmaf(beta, uu.x, g.x);
          uu.y = fmaf(beta, uu.y, g.y);
          uu.z = fmaf(beta, uu.z, g.z);
          uu.w = fmaf(beta, uu.w, g.w);
          if (row < m && col_ok) stq<VEC4>(U + d.off + (int64_t)row * n, col, n, uu);
          s = make_float4(uu.x + e.x, uu.y + e.y, uu.z + e.z, uu.w + e.w);
        } else {
          s = make_float4(g.x + e.x, g.y + e.y, g.z + e.z, g.w + e.w);
        }
        if (row < m && col_ok) stq<VEC4>(E + d.off + (int64_t)row * n, col, n, s);
      }
      *reinterpret_cast<float4*>(mrow) = s;
    }
  };

  // A wavefront reads only its own rows of Ms, so the barrier per chunk
  // guards the shared Q chunk (and the overwrite of both tiles).  In the
  // deferred modes a wavefront's own rows of Ms pass between its lanes three
  // times (reconstruction written, read back and overwritten with M by other
  // lanes, then read as A operands) with no workgroup barrier in between:
  // the LDS instructions of one wavefront complete in program order, and a
  // wave barrier between the phases keeps the compiler from moving an LDS
  // access of one phase past the other (it costs no instruction).
  load_chunk(c_begin);
  for (int c0 = c_begin; c0 < c_end; c0 += CH) {
    stage_q();
    if constexpr (DEFERRED) {
      __syncthreads();
      recon_tile();
      __builtin_amdgcn_wave_barrier();
      ef_chunk(c0);
      __builtin_amdgcn_wave_barrier();
    } else {
      ef_chunk(c0);
      __syncthreads();
    }
    if (c0 + CH < c_end) load_chunk(c0 + CH);
#pragma unroll
    for (int kb = 0; kb < CH / 16; ++kb) {
      const float4 a4 = *reinterpret_cast<const float4*>(&Ms[(16 * wave + li) * LDM + 16 * kb + 4 * ls]);
      float4 b4[RP / 16];
#pragma unroll
      for (int T = 0; T < RP / 16; ++T)
        b4[T] = *reinterpret_cast<const float4*>(&Qs[(16 * T + li) * QLD + 16 * kb + 4 * ls]);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float a = v == 0 ? a4.x : v == 1 ? a4.y : v == 2 ? a4.z : a4.w;
#pragma unroll
        for (int T = 0; T < RP / 16; ++T) {
          const float b = v == 0 ? b4[T].x : v == 1 ? b4[T].y : v == 2 ? b4[T].z : b4[T].w;
          acc[T] = mfma16x16x4(a, b, acc[T]);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int T = 0; T < RP / 16; ++T) {
#pragma unroll
      for (int e = 0; e < 4; ++e) accd[T][e] += (double)acc[T][e];
      acc[T] = v4f{0.f, 0.f, 0.f, 0.f};
    }
  }

  // accd[T][e] of lane (li, ls) is P[i0 + 16 wave + 4 ls + e][16 T + li]:
  // this split's fp64 partial, or P itself rounded to fp32.
  const int row = i0 + 16 * wave + 4 * ls;
  if (d.s1 > 1) {
    double* dst = ppart + d.ppart_off + (int64_t)split * r * m;
#pragma unroll
    for (int T = 0; T < RP / 16; ++T) {
      const int t = 16 * T + li;
      if (t < r) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (row + e < m) dst[(int64_t)t * m + row + e] = accd[T][e];
      }
    }
  } else {
    float* dst = P + (p_fixed >= 0 ? p_fixed : d.p_off);
    const bool out4 = (m & 3) == 0;
#pragma unroll
    for (int T = 0; T < RP / 16; ++T) {
      const int t = 16 * T + li;
      if (t < r)
        st4(dst + (int64_t)t * m, row, m, out4,
            make_float4((float)accd[T][0], (float)accd[T][1], (float)accd[T][2], (float)accd[T][3]));
    }
  }
}

// VEC4: every matrix of this launch has rows that allow 16-byte accesses (the
// plan puts them first in the grid), or none has.
template <int RP, int MODE, bool GBF16, bool VEC4>
__global__ __launch_bounds__(256) void k_mfma_p(const MatDesc* __restrict__ mats, const int32_t* __restrict__ map,
                                                int wg_base, int r, const void* __restrict__ G,
                                                float* __restrict__ E, float* __restrict__ U, float beta,
                                                const float* __restrict__ Q, float* P, int64_t p_fixed,
                                                double* __restrict__ ppart, const float* Pold) {
  constexpr int CH = mq_chunk(RP, MODE);
  __shared__ float smem[(kMfmaRows + RP) * (CH + 4)];
  int mi;
  const int wg = wg_of(map, wg_base, mi);
  const MatDesc d = mats[mi];
  mfma_mq_body<RP, MODE, VEC4, GBF16, CH>(d, wg, r, G, E, U, beta, Q, P, p_fixed, ppart, smem, Pold);
}

// Fixed-order sum of the column-split partials of pass 1 (fp32 partials of
// the vector path, fp64 ones of the matrix cores, summed in their own
// precision and rounded to fp32 once).
template <typename T>
__global__ __launch_bounds__(kRedCols) void k_psum(const MatDesc* __restrict__ mats, const int32_t* __restrict__ map,
                                                   int wg_base, int r, const T* __restrict__ ppart,
                                                   float* __restrict__ P, int64_t p_fixed) {
  int mi;
  const int wg = wg_of(map, wg_base, mi);
  const MatDesc d = mats[mi];
  const int64_t len = (int64_t)r * d.m;
  const int64_t idx = (int64_t)(wg - d.wg_pred0) * kRedCols + threadIdx.x;
  if (idx >= len) return;
  const T* src = ppart + d.ppart_off + idx;
  T s0 = 0, s1 = 0;
  int b = 0;
  for (; b + 2 <= d.s1; b += 2) {
    s0 += src[(int64_t)b * len];
    s1 += src[(int64_t)(b + 1) * len];
  }
  if (b < d.s1) s0 += src[(int64_t)b * len];
  P[(p_fixed >= 0 ? p_fixed : d.p_off) + idx] = (float)(s0 + s1);
}

// ---------------------------------------------------------------------------
// Pass 2: Q = M^T P_hat over one row block (partials when the matrix has
// several row blocks).
//
// A workgroup owns kMfmaCols (128) columns of one row block and walks it in
// kQtChunk-row chunks.  Each wavefront loads kQtChunk / 4 rows of a chunk
// with row-contiguous accesses (32 lanes x 16 bytes per row, two 512-byte
// row segments per instruction) into an LDS tile, and the chunk's P_hat rows
// go to LDS once for the workgroup; each wavefront then accumulates its 32
// columns (two 16-column tiles, every rank tile) on the matrix core from LDS.
// A 128-column tile rather than 256 doubles the workgroups of a row block and
// halves their LDS and load registers (about 3% on the refresh and on single
// large matrices).  The
// next chunk's loads are issued before the current chunk's matrix products.
// The summation index of matrix-core step v of a 16-row block is bound, for
// lane (li, ls), to row 4 ls + v, so that lane's B operands P_hat[4 ls ..
// 4 ls + 3][rank] are one 16-byte LDS read.  Each wavefront owns its columns:
// nothing is summed across wavefronts.
// ---------------------------------------------------------------------------

constexpr int kQtChunk = 32;              // rows per LDS chunk
constexpr int kQtLd = kMfmaCols + 4;      // LDS row stride of the M chunk (floats)
constexpr int kQtPld = kQtChunk + 4;      // LDS stride of one rank's P_hat rows (floats)
constexpr int kQtLpr = kMfmaCols / 4;      // lanes per row of a wavefront load
constexpr int kQtRpi = 64 / kQtLpr;        // rows per wavefront load
constexpr int kQtWc = kMfmaCols / 4;       // columns a wavefront owns
constexpr int kQtNct = kQtWc / 16;         // its 16-column tiles
static_assert(kMfmaCols == 128 || kMfmaCols == 256, "a wavefront load covers whole rows of the tile");

template <int RP, bool VEC4>
__device__ __forceinline__ void mfma_qt_body(const MatDesc& d, int wg, int r, const float* __restrict__ M,
                                             const float* __restrict__ Ph, int64_t ph_fixed, float* __restrict__ Q,
                                             float* __restrict__ part, float* Ms, float* Ps) {
  constexpr int RPW = kQtChunk / 4;                        // rows a wavefront loads per chunk
  constexpr int NL = RPW / kQtRpi;                         // its load instructions per chunk
  constexpr int PPT = (RP * kQtChunk + 255) / 256;         // P_hat values a thread loads per chunk
  const int m = d.m, n = d.n;
  const int local = wg - d.wg_mtp0;
  const int rb = local / d.ncb, cb = local - rb * d.ncb;
  const int i0 = rb * d.rb_rows;
  const int i1 = min(m, i0 + d.rb_rows);
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, ls = lane >> 4;
  const int cbase = cb * kMfmaCols;
  const int hr = lane / kQtLpr;                      // the lane's row within a load
  const int scol = cbase + 4 * (lane % kQtLpr);  // the lane's four columns in the row loads
  const bool scol_ok = scol < n;
  const float* ph = Ph + (ph_fixed >= 0 ? ph_fixed : d.p_off);

  v4f acc[kQtNct][RP / 16];
#pragma unroll
  for (int ct = 0; ct < kQtNct; ++ct)
#pragma unroll
    for (int T = 0; T < RP / 16; ++T) acc[ct][T] = v4f{0.f, 0.f, 0.f, 0.f};

  float4 xn[NL];
  float pn[PPT];
  auto load_chunk = [&](int ib) {
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int row = ib + RPW * wave + kQtRpi * u + hr;
      xn[u] = row < i1 ? ldq<VEC4>(M + d.off + (int64_t)row * n, scol, scol_ok, cbase, n)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int e = threadIdx.x + 256 * u;
      const int t = e / kQtChunk, rr = e % kQtChunk;
      pn[u] = (e < RP * kQtChunk && t < r && ib + rr < i1) ? ph[(int64_t)t * m + ib + rr] : 0.f;
    }
  };
  auto store_chunk = [&]() {
#pragma unroll
    for (int u = 0; u < NL; ++u)
      *reinterpret_cast<float4*>(&Ms[(RPW * wave + kQtRpi * u + hr) * kQtLd + 4 * (lane % kQtLpr)]) = xn[u];
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int e = threadIdx.x + 256 * u;
      if (e < RP * kQtChunk) Ps[(e / kQtChunk) * kQtPld + e % kQtChunk] = pn[u];
    }
  };

  if (i0 < i1) load_chunk(i0);
  for (int ib = i0; ib < i1; ib += kQtChunk) {
    store_chunk();
    __syncthreads();
    if (ib + kQtChunk < i1) load_chunk(ib + kQtChunk);
#pragma unroll
    for (int kb = 0; kb < kQtChunk / 16; ++kb) {
      float4 pb[RP / 16];
#pragma unroll
      for (int T = 0; T < RP / 16; ++T)
        pb[T] = *reinterpret_cast<const float4*>(&Ps[(16 * T + li) * kQtPld + 16 * kb + 4 * ls]);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float* mrow = &Ms[(16 * kb + 4 * ls + v) * kQtLd + kQtWc * wave + li];
#pragma unroll
        for (int ct = 0; ct < kQtNct; ++ct) {
          const float a = mrow[16 * ct];
#pragma unroll
          for (int T = 0; T < RP / 16; ++T) {
            const float b = v == 0 ? pb[T].x : v == 1 ? pb[T].y : v == 2 ? pb[T].z : pb[T].w;
            acc[ct][T] = mfma16x16x4(a, b, acc[ct][T]);
          }
        }
      }
    }
    __syncthreads();
  }

  // acc[ct][T][e] of lane (li, ls) is Q[cbase + kQtWc wave + 16 ct + 4 ls + e][16 T + li].
  float* out = d.nrb > 1 ? part + d.part_off + (int64_t)rb * r * n : Q + d.q_off;
  const bool out4 = (n & 3) == 0;
#pragma unroll
  for (int T = 0; T < RP / 16; ++T) {
    const int t = 16 * T + li;
    if (t < r) {
#pragma unroll
      for (int ct = 0; ct < kQtNct; ++ct)
        st4(out + (int64_t)t * n, cbase + kQtWc * wave + 16 * ct + 4 * ls, n, out4,
            make_float4(acc[ct][T][0], acc[ct][T][1], acc[ct][T][2], acc[ct][T][3]));
    }
  }
}

template <int RP>
__global__ __launch_bounds__(256) void k_mfma_qt(const MatDesc* __restrict__ mats, const int32_t* __restrict__ map,
                                                 int wg_base, int r, const float* __restrict__ M,
                                                 const float* __restrict__ Ph, int64_t ph_fixed,
                                                 float* __restrict__ Q, float* __restrict__ part) {
  __shared__ float Ms[kQtChunk * kQtLd];
  __shared__ float Ps[RP * kQtPld];
  int mi;
  const int wg = wg_of(map, wg_base, mi);
  const MatDesc d = mats[mi];
  if (d.vec == 4)
    mfma_qt_body<RP, true>(d, wg, r, M, Ph, ph_fixed, Q, part, Ms, Ps);
  else
    mfma_qt_body<RP, false>(d, wg, r, M, Ph, ph_fixed, Q, part, Ms, Ps);
}

// ---------------------------------------------------------------------------
// Pass 3: M_hat = P_hat Q^T (transposed on the matrix core); residual and/or
// decompression.  A workgroup owns kRecRows rows x one kRecCols-column split.
// Phase 1: the 16 x 16 tiles of M_hat^T = Q P_hat^T on the matrix core (a
// wavefront takes four adjacent column tiles of both row tiles), each written
// to LDS in its result layout (lane = one row, four consecutive columns).
// Phase 2: each wavefront streams kWaveRows rows of the tile with
// row-contiguous accesses -- 64 lanes x 16 bytes, one 1 KB row segment per
// instruction -- reading M, writing E and M_hat (and the SGD state), as the
// vector-ALU residual pass does.  A tile is summed over the rank in the same
// matrix-core step order as the deferred-residual form of pass 1.
// ---------------------------------------------------------------------------

constexpr int kRecRows = kRowsPerWG;  // rows of a workgroup tile (two 16-row tiles)
constexpr int kRecLd = kRecSplitCols + 4;  // LDS row stride (floats)
static_assert(kRecRows == 32 && kRecSplitCols == 256, "tile shape of the matrix-core residual pass");

template <int RP, bool RESID, bool WRITE_MHAT, bool SGD, bool VEC4>
__device__ __forceinline__ void mfma_recon_body(const MatDesc& d, int wg, int r, float* __restrict__ E,
                                                const float* __restrict__ Q, const float* __restrict__ Ph,
                                                float* __restrict__ Mhat, const SgdArgs& sg, float* tile) {
  constexpr int KS = RP / 4;  // k-steps of 4 rank columns
  const int m = d.m, n = d.n;
  const int local = wg - d.wg_rec0;
  const int rb = local / d.s3, split = local - rb * d.s3;
  const int c_begin = split * d.s3_cols;
  const int c_end = min(n, c_begin + d.s3_cols);
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, ls = lane >> 4;
  const int i0 = rb * kRecRows;
  const float* ph = Ph + d.p_off;
  const float* q = Q + d.q_off;

  // Phase 1.  B operand: P_hat^T, lane (li, ls) holds P_hat[i0 + 16 rt + li][4 kk + ls];
  // A operand: Q, lane (li, ls) holds Q[column j0 + li][4 kk + ls].
  float bfr[2][KS];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int rr = i0 + 16 * rt + li, t = 4 * kk + ls;
      bfr[rt][kk] = (rr < m && t < r) ? ph[(int64_t)t * m + rr] : 0.f;
    }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int ct = 4 * wave + u;
    const int j0 = c_begin + 16 * ct;
    if (j0 < c_end) {  // wavefront-uniform
      float afr[KS];
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const int t = 4 * kk + ls, c = j0 + li;
        afr[kk] = (t < r && c < c_end) ? q[(int64_t)t * n + c] : 0.f;
      }
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) acc = mfma16x16x4(afr[kk], bfr[rt][kk], acc);
        *reinterpret_cast<float4*>(&tile[(16 * rt + li) * kRecLd + 16 * ct + 4 * ls]) =
            make_float4(acc[0], acc[1], acc[2], acc[3]);
      }
    }
  }
  __syncthreads();

  // Phase 2: rows i0 + kWaveRows * wave + rr, columns c_begin + 4 lane .. + 3.
  const int row_base = i0 + kWaveRows * wave;
  const int nrows = min(kWaveRows, m - row_base);
  if (nrows <= 0) return;
  const int cl = 4 * lane, col = c_begin + cl;
  const bool col_ok = col < c_end;
  float4 x[kWaveRows], xx[kWaveRows], xb[kWaveRows];
#pragma unroll
  for (int rr = 0; rr < kWaveRows; ++rr) {
    const int64_t ro = d.off + (int64_t)(row_base + min(rr, nrows - 1)) * n;
    if constexpr (RESID) x[rr] = ldq_nt<VEC4>(E + ro, col, col_ok, c_begin, n);
    if constexpr (SGD) {
      xx[rr] = ldq<VEC4>(sg.x + ro, col, col_ok, c_begin, n);
      xb[rr] = ldq<VEC4>(sg.m + ro, col, col_ok, c_begin, n);
    }
  }
#pragma unroll
  for (int rr = 0; rr < kWaveRows; ++rr) {
    if (rr < nrows && col_ok) {
      const int64_t ro = d.off + (int64_t)(row_base + rr) * n;
      const float4 mh = *reinterpret_cast<const float4*>(&tile[(kWaveRows * wave + rr) * kRecLd + cl]);
      if constexpr (RESID) {
        const float4 xm = x[rr];
        stq_nt<VEC4>(E + ro, col, n, make_float4(xm.x - mh.x, xm.y - mh.y, xm.z - mh.z, xm.w - mh.w));
      }
      if constexpr (WRITE_MHAT) stq_nt<VEC4>(Mhat + ro, col, n, mh);
      if constexpr (SGD) {
        float4 mm = xb[rr], xp = xx[rr];
        mm.x = fmaf(sg.mu, mm.x, mh.x);
        mm.y = fmaf(sg.mu, mm.y, mh.y);
        mm.z = fmaf(sg.mu, mm.z, mh.z);
        mm.w = fmaf(sg.mu, mm.w, mh.w);
        if (sg.nesterov) {
          xp.x = fmaf(-sg.lr, fmaf(sg.mu, mm.x, mh.x), xp.x);
          xp.y = fmaf(-sg.lr, fmaf(sg.mu, mm.y, mh.y), xp.y);
          xp.z = fmaf(-sg.lr, fmaf(sg.mu, mm.z, mh.z), xp.z);
          xp.w = fmaf(-sg.lr, fmaf(sg.mu, mm.w, mh.w), xp.w);
        } else {
          xp.x = fmaf(-sg.lr, mm.x, xp.x);
          xp.y = fmaf(-sg.lr, mm.y, xp.y);
          xp.z = fmaf(-sg.lr, mm.z, xp.z);
          xp.w = fmaf(-sg.lr, mm.w, xp.w);
        }
        stq<VEC4>(sg.m + ro, col, n, mm);
        stq<VEC4>(sg.x + ro, col, n, xp);
      }
    }
  }
}

template <int RP, bool RESID, bool WRITE_MHAT, bool SGD>
__global__ __launch_bounds__(256) void k_mfma_recon(const MatDesc* __restrict__ mats, const int32_t* __restrict__ map,
                                                    int wg_base, int r, float* __restrict__ E,
                                                    const float* __restrict__ Q, const float* __restrict__ Ph,
                                                    float* __restrict__ Mhat, SgdArgs sg) {
  __shared__ float tile[kRecRows * kRecLd];
  int mi;
  const int wg = wg_of(map, wg_base, mi);
  const MatDesc d = mats[mi];
  if (d.vec == 4)
    mfma_recon_body<RP, RESID, WRITE_MHAT, SGD, true>(d, wg, r, E, Q, Ph, Mhat, sg, tile);
  else
    mfma_recon_body<RP, RESID, WRITE_MHAT, SGD, false>(d, wg, r, E, Q, Ph, Mhat, sg, tile);
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
//   k_gram_partial  A_b = P_b^T P_b over blocks of kGramRows rows (the
//                   upper block triangle; A is symmetric)
//   k_gram_reduce   A = sum_b A_b in block order
//   k_gram_solve    R by right-looking Cholesky with the dependence rule
//   k_apply_t       P_hat rows by forward substitution, x R = p, in fp64
//                   registers, rounded to fp32

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

constexpr int kGramChunk = kGramRows;  // rows staged in LDS at a time

// A_b = P_b^T P_b for one block of kGramRows rows on the fp64 matrix core
// (v_mfma_f64_16x16x4f64; each fp32 product is exact in fp64).  The block is
// staged in LDS; the 16 x 16 tiles (ta, tb) of A_b with ta <= tb (A is
// symmetric: the Cholesky reads the lower block triangle from the upper) are
// dealt round-robin to the four wavefronts, each summing its tiles over the
// block's rows in order, four rows per matrix-core step.
typedef double v4d __attribute__((ext_vector_type(4)));

template <int RP>
__global__ __launch_bounds__(256) void k_gram_partial(const OrthDesc* __restrict__ descs, const int32_t* __restrict__ map,
                                                      int first, int r, const float* __restrict__ base,
                                                      double* __restrict__ gram) {
  constexpr int LS = RP + 1;
  constexpr int NT = RP / 16;
  __shared__ float Pl[kGramChunk * LS];
  int local;
  const OrthDesc o = descs[orth_idx(descs, map, first, local)];
  const float* p = base + o.off;
  const int r0 = local * kGramRows;
  // Every load at a clamped, valid address and the value zeroed when out of
  // range: no branches, so all of a thread's loads are in flight together.
  constexpr int NL = kGramChunk * RP / 256;
  float v[NL];
#pragma unroll
  for (int u = 0; u < NL; ++u) {
    const int e = threadIdx.x + 256 * u, i = e % kGramChunk, t = e / kGramChunk;
    v[u] = p[(int64_t)min(t, r - 1) * o.rows + min(r0 + i, o.rows - 1)];
  }
#pragma unroll
  for (int u = 0; u < NL; ++u) {
    const int e = threadIdx.x + 256 * u, i = e % kGramChunk, t = e / kGramChunk;
    Pl[i * LS + t] = (t < r && r0 + i < o.rows) ? v[u] : 0.f;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, ls = lane >> 4;
  double* g = gram + o.gram_off + (int64_t)local * RP * RP;
  constexpr int NUT = NT * (NT + 1) / 2;  // upper tiles, row by row
  for (int u = wave; u < NUT; u += 4) {
    int ta = 0, rem = u;  // tile row ta holds NT - ta tiles
#pragma unroll
    for (int a = 0; a < NT - 1; ++a) {
      if (ta == a && rem >= NT - a) {
        rem -= NT - a;
        ta = a + 1;
      }
    }
    const int tb = ta + rem;
    v4d acc = v4d{0.0, 0.0, 0.0, 0.0};
#pragma unroll 8
    for (int kk = 0; kk < kGramChunk / 4; ++kk) {
      const int i = 4 * kk + ls;
      const double a = (double)Pl[i * LS + 16 * ta + li];
      const double b = (double)Pl[i * LS + 16 * tb + li];
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc, 0, 0, 0);
    }
    // fp64 result layout: acc[e] of lane (li, ls) is A_b[16 ta + 4 e + ls][16 tb + li]
#pragma unroll
    for (int e = 0; e < 4; ++e) g[(16 * ta + 4 * e + ls) * RP + 16 * tb + li] = acc[e];
  }
}

// Fixed-order block sum: A (at t_off) = sum_b A_b.  A workgroup covers 256
// entries of one factor's A with kGramRedGroups groups of 256 threads: group
// g sums the blocks b = g, g + kGramRedGroups, ... in eight running sums (so
// that eight loads are in flight), and the group totals are added in
// group order through LDS.  The order is fixed: deterministic.
constexpr int kGramRedGroups = 4;

template <int RP>
__global__ __launch_bounds__(256 * kGramRedGroups) void k_gram_reduce(const OrthDesc* __restrict__ descs, int first,
                                                                      double* __restrict__ gram) {
  constexpr int WPD = RP * RP / 256;  // workgroups per descriptor
  constexpr int NG = kGramRedGroups;
  constexpr int64_t BS = (int64_t)RP * RP;  // doubles per block partial
  __shared__ double tot[NG][256];
  const OrthDesc o = descs[first + blockIdx.x / WPD];
  const int grp = threadIdx.x >> 8, t = threadIdx.x & 255;
  const int e = (blockIdx.x % WPD) * 256 + t;
  const double* g = gram + o.gram_off + e;
  double s[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
  int b = grp;
  for (; b + 7 * NG < o.ngb; b += 8 * NG) {
#pragma unroll
    for (int u = 0; u < 8; ++u) s[u] += g[(b + u * NG) * BS];
  }
  for (; b < o.ngb; b += NG) s[0] += g[b * BS];
  tot[grp][t] = ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
  __syncthreads();
  if (grp == 0) {
    double a = tot[0][t];
#pragma unroll
    for (int u = 1; u < NG; ++u) a += tot[u][t];
    gram[o.t_off + e] = a;
  }
}

__device__ __forceinline__ double readlane_f64(double v, int l) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(b & 0xffffffffull), l);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(b >> 32), l);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// 1 / sqrt(d) for a positive normal d: the hardware estimate refined by two
// Newton steps y <- y + y (1 - d y^2) / 2, each of which roughly doubles the
// number of correct bits, to within a few units in the last place of fp64.
__device__ __forceinline__ double rsqrt_nr(double d) {
  double y = __builtin_amdgcn_rsq(d);
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const double e = fma(-d * y, y, 1.0);
    y = fma(0.5 * y, e, y);
  }
  return y;
}

// One wavefront per factor: right-looking Cholesky of A with the dependence
// rule.  Lane j keeps column j of the (symmetric) Schur complement S in fp64
// registers.  At step k the pivot S_kk comes from lane k's registers
// (readlane), every lane publishes S_kj through LDS and reads the row S_k.
// back as broadcasts, and updates S_ij -= S_ki (S_kj / S_kk) for i > k; only
// the reciprocal square root of S_kk is on the step-to-step path.  Row k of R
// is S_k. / sqrt(S_kk), zero for a dependent column: sqrt(S_kk) <= 1e-4 of the
// norm before projection sqrt(A_kk), tested squared.  A single wavefront
// needs no barrier: its LDS accesses complete in program order.  The upper
// triangle of the factor's A slot (diagonal included) is overwritten with R,
// row by row (A is read first).
// With zcount non-null, zcount[blockIdx.x] receives the number of columns
// the dependence rule set to zero.
template <int RP>
__global__ __launch_bounds__(64) void k_gram_solve(const OrthDesc* __restrict__ descs, int first, int r,
                                                   double* __restrict__ gram, float zero_rel,
                                                   int32_t* __restrict__ zcount) {
  __shared__ double rowbuf[RP];
  __shared__ double Rl[RP * RP];  // the factor, until it is written out
  const OrthDesc o = descs[first + blockIdx.x];
  const int j = threadIdx.x;
  const bool own = j < RP;
  double* a = gram + o.t_off;
  // A's lower block triangle is read from the upper one (only its 16 x 16
  // tiles with ta <= tb are accumulated); every load at a valid address, the
  // value selected afterwards
  const int jc = min(j, RP - 1);
  double sc[RP];
#pragma unroll
  for (int i = 0; i < RP; ++i) {
    const double v = a[(i >> 4) <= (jc >> 4) ? i * RP + jc : jc * RP + i];
    sc[i] = own ? v : 0.0;
  }
  const double dv = a[jc * RP + jc];
  const double dgj = own ? dv : 0.0;  // A_jj: squared norm before projection
  const double zr2 = (double)zero_rel * (double)zero_rel;
  int nzero = 0;  // wavefront-uniform
  // Fully unrolled so that sc[] stays in registers; steps k >= r are skipped
  // by a uniform branch.  No global store inside the steps: a pending store
  // would be waited for at every step.
#pragma unroll
  for (int k = 0; k < RP; ++k) {
    if (k < r) {
      if (own) rowbuf[j] = sc[k];
      // the whole row S_k. read back before the pivot arithmetic, so that the
      // LDS latency overlaps it
      double rk[RP];
#pragma unroll
      for (int i = k + 1; i < RP; ++i) rk[i] = rowbuf[i];
      const double d = readlane_f64(sc[k], k);
      const double dg = readlane_f64(dgj, k);
      const bool zero = !(dg > 0.0) || !(d > 0.0) || d <= zr2 * dg;
      nzero += zero ? 1 : 0;
      const double y = zero ? 0.0 : rsqrt_nr(d);  // 1 / sqrt(S_kk)
      const double c = sc[k] * (y * y);            // S_kj / S_kk
      if (own && j >= k && j < r) Rl[k * RP + j] = j == k ? d * y : sc[k] * y;
#pragma unroll
      for (int i = k + 1; i < RP; ++i) sc[i] = fma(-rk[i], c, sc[i]);
    }
  }
  // write-out: slot[kr RP + jc] = R_{kr jc} for kr <= jc < r
#pragma unroll
  for (int u = 0; u < RP * RP / 64; ++u) {
    const int e = j + 64 * u, kr = e / RP, jc = e % RP;
    if (kr <= jc && jc < r) a[e] = Rl[e];
  }
  if (zcount && j == 0) zcount[blockIdx.x] = nzero;
}

// P_hat = P R^-1, one row per thread: x R = p by forward substitution in
// right-looking order.  Step k takes x_k = b_k / R_kk (b starts as p; x_k = 0
// for a dependent column) and removes its share from the later right-hand
// sides, b_i -= x_k R_ki for i > k, with row k of R: only x_k and the next
// b_{k+1} are on the step-to-step path, and row k's coefficients, the same
// for every thread, are LDS broadcasts that do not depend on x.  The steps
// run in groups of four without branches so that the reads of later steps
// can be issued early (steps k >= r inside the last group are harmless:
// 1 / R_kk is set to 0 there, and their b_i are never stored).  x is kept in
// fp64 registers and rounded to fp32 when stored in place.  The row's p
// values are all loaded up front (clamped addresses, no branches).
template <int RP>
__global__ __launch_bounds__(kGramRows) void k_apply_t(const OrthDesc* __restrict__ descs,
                                                       const int32_t* __restrict__ map, int first, int r,
                                                       float* __restrict__ base, const double* __restrict__ gram) {
  constexpr int NS = RP * RP / kGramRows;
  static_assert(NS * kGramRows == RP * RP, "whole slot per thread");
  static_assert(RP % 4 == 0, "groups of four steps");
  __shared__ double Rr[RP * RP];  // Rr[k RP + i] = R_ki
  __shared__ double rinv[RP];
  int local;
  const OrthDesc o = descs[orth_idx(descs, map, first, local)];
  const double* rs = gram + o.t_off;
  const int i = local * kGramRows + threadIdx.x;
  float* p = base + o.off + min(i, o.rows - 1);
  const int64_t ld = o.rows;
  float pv[RP];
#pragma unroll
  for (int k = 0; k < RP; ++k) pv[k] = p[(int64_t)min(k, r - 1) * ld];
  double sv[NS];
#pragma unroll
  for (int u = 0; u < NS; ++u) sv[u] = rs[threadIdx.x + u * kGramRows];
  const double dk = rs[min((int)threadIdx.x, RP - 1) * (RP + 1)];
#pragma unroll
  for (int u = 0; u < NS; ++u) Rr[threadIdx.x + u * kGramRows] = sv[u];
  if (threadIdx.x < RP) rinv[threadIdx.x] = ((int)threadIdx.x < r && dk > 0.0) ? 1.0 / dk : 0.0;
  __syncthreads();
  if (i >= o.rows) return;
  double b[RP];
#pragma unroll
  for (int k = 0; k < RP; ++k) b[k] = (double)pv[k];
  // row k + 1 of R is read while step k runs (software pipelining by hand)
  double rc[RP], rn[RP];
#pragma unroll
  for (int q = 1; q < RP; ++q) rc[q] = Rr[q];
#pragma unroll
  for (int k = 0; k < RP; ++k) {
    if ((k & 3) == 0 && k >= r) break;
    if (k + 1 < RP) {
#pragma unroll
      for (int q = k + 2; q < RP; ++q) rn[q] = Rr[(k + 1) * RP + q];
    }
    const double xk = b[k] * rinv[k];
    b[k] = xk;
#pragma unroll
    for (int q = k + 1; q < RP; ++q) b[q] = fma(-xk, rc[q], b[q]);
#pragma unroll
    for (int q = k + 2; q < RP; ++q) rc[q] = rn[q];
  }
#pragma unroll
  for (int k = 0; k < RP; ++k)
    if (k < r) p[k * ld] = (float)b[k];
}

// Blocked form of the same Cholesky for RP >= 32: 16-row block rows, each
// factored by one wavefront over all of its remaining columns, then a
// rank-16 update of the trailing tiles on the fp64 matrix core by all four
// wavefronts.  Within block row B (rows 16 B .. 16 B + 15), lane j of
// wavefront 0 keeps column 16 B + j of the Schur complement S restricted to
// the block row's 16 rows, and step k runs as in the one-wavefront form
// (pivot, dependence rule, row k of R, update of the later rows of the
// block row), so a step updates at most 15 entries per lane instead of up
// to RP - 1.  The contribution of the block row's 16 rows of R to the later
// rows, S_CD -= R_BC^T R_BD over the upper trailing tiles (C <= D), is then
// one 16 x 16 x 16 product per tile (the negated R_BC^T as A operand).  The
// arithmetic is that of the right-looking factorisation; only the order in
// which each later entry of S receives the 16 terms of one block row
// differs (summed on the matrix core, then subtracted).  S holds A's upper
// 16 x 16 tiles (the diagonal ones whole), which is all the updates and the
// block rows read.  A is read whole before the first step, so the rows of R
// are written over it block row by block row.  Block rows from r on are
// skipped; inside the last one, steps k >= r find zero pivots (A is zero
// there) and leave their rows of R zero.
template <int RP>
__global__ __launch_bounds__(256) void k_gram_solve_blk(const OrthDesc* __restrict__ descs, int first, int r,
                                                        double* __restrict__ gram, float zero_rel,
                                                        int32_t* __restrict__ zcount) {
  static_assert(RP % 16 == 0 && RP >= 32 && RP <= 64, "16-row block rows, one lane per column");
  constexpr int NB = RP / 16;
  __shared__ double S[RP * RP];
  __shared__ double Rb[16 * RP];  // the block row's rows of R (zero until a step writes one)
  __shared__ double dgl[RP];      // A_kk: squared norms before projection
  __shared__ double rowbuf[64];
  const OrthDesc o = descs[first + blockIdx.x];
  double* a = gram + o.t_off;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, ls = lane >> 4;
#pragma unroll
  for (int u = 0; u < RP * RP / 256; ++u) {
    const int e = tid + 256 * u, i = e / RP, j = e % RP;
    const double v = a[e];  // every entry of the slot is a valid address
    S[e] = (i >> 4) <= (j >> 4) ? v : 0.0;
    if (i == j) dgl[i] = v;
  }
  __syncthreads();
  const double zr2 = (double)zero_rel * (double)zero_rel;
  int nzero = 0;  // counted by wavefront 0 (uniform there)
  for (int B = 0; B < NB && 16 * B < r; ++B) {
    if (wave == 0) {
      const int ncol = RP - 16 * B;
      const bool own = lane < ncol;
      const int col = 16 * B + min(lane, ncol - 1);
      const double dgv = dgl[16 * B + min(lane, 15)];  // lane k < 16: A_kk of the block row's step k
      double sc[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sc[i] = S[(16 * B + i) * RP + col];
        if (lane < RP) Rb[i * RP + lane] = 0.0;
      }
      // Steps past r need no guard (a uniform branch per step would cost
      // register copies at every join): A's rows and columns from r on are
      // zero (P's padding), so there the pivot and A_kk are zero, the
      // dependence rule applies, and the step changes nothing.  The pivot
      // arithmetic runs without a branch and the rule selects its result.
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int kk = 16 * B + k;
        // row k of the block row's Schur complement (S_ki = S_ik for the
        // later rows i) through LDS, read back before the pivot arithmetic
        rowbuf[lane] = sc[k];  // lanes past the last column repeat it; only entries < 16 are read
        double rk[16];
#pragma unroll
        for (int i = k + 1; i < 16; ++i) rk[i] = rowbuf[i];
        const double d = readlane_f64(sc[k], k);
        const double dg = readlane_f64(dgv, k);
        const bool zero = !(dg > 0.0) || !(d > 0.0) || d <= zr2 * dg;
        nzero += (zero && kk < r) ? 1 : 0;
        const double yn = rsqrt_nr(d);
        const double y = zero ? 0.0 : yn;
        const double c = sc[k] * (y * y);
        if (own && lane >= k) Rb[k * RP + col] = lane == k ? d * y : sc[k] * y;
#pragma unroll
        for (int i = k + 1; i < 16; ++i) sc[i] = fma(-rk[i], c, sc[i]);
      }
    }
    __syncthreads();
    // the block row's rows of R into the slot (kr <= jc < r) ...
#pragma unroll
    for (int u = 0; u < RP / 16; ++u) {
      const int e = tid + 256 * u, kr = 16 * B + e / RP, jc = e % RP;
      if (kr <= jc && jc < r) a[kr * RP + jc] = Rb[e];
    }
    // ... and their contribution to the later rows
    const int nt = NB - 1 - B;
    for (int u = wave; u < nt * (nt + 1) / 2; u += 4) {
      int C = B + 1, rem = u;  // tile row C holds NB - C tiles
      while (rem >= NB - C) {
        rem -= NB - C;
        ++C;
      }
      const int D = C + rem;
      // acc[e] of lane (li, ls) is S[16 C + 4 e + ls][16 D + li]
      v4d acc;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = S[(16 * C + 4 * e + ls) * RP + 16 * D + li];
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) {
        const int row = 4 * kq + ls;
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(-Rb[row * RP + 16 * C + li], Rb[row * RP + 16 * D + li], acc, 0,
                                                   0, 0);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) S[(16 * C + 4 * e + ls) * RP + 16 * D + li] = acc[e];
    }
    __syncthreads();
  }
  if (zcount && tid == 0) zcount[blockIdx.x] = nzero;
}

// x from lane G of each group of four lanes (a quad permutation on the
// data-parallel-primitive path; both halves of the double).
template <int G>
__device__ __forceinline__ double quad_bcast(double v) {
  constexpr int ctrl = G * 0x55;  // quad_perm [G, G, G, G]
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(b & 0xffffffffll), ctrl, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), ctrl, 0xf, 0xf, false);
  return __longlong_as_double(((long long)hi << 32) | (long long)(unsigned)lo);
}

__device__ __forceinline__ double quad_bcast_k(double v, int g) {
  switch (g) {
    case 0: return quad_bcast<0>(v);
    case 1: return quad_bcast<1>(v);
    case 2: return quad_bcast<2>(v);
    default: return quad_bcast<3>(v);
  }
}

// P_hat = P R^-1 with four lanes per row: the forward substitution x R = p
// of the one-lane form (step k: x_k = b_k / R_kk, zero for a dependent
// column, then b_q -= x_k R_kq for q > k, in the order k = 0, 1, ...), with
// the columns dealt to the lanes of a quad cyclically (lane g keeps b_q for
// q = 4 j + g).  The owner of column k forms x_k and hands it to the other
// three lanes with a quad permutation; each lane then updates only its own
// columns, reading R_kq from an LDS copy laid out by lane (Rg[g][k][j] =
// R_{k, 4 j + g}).  Every b_q receives the same operations in the same
// order as in the one-lane form: the result is the same, bit for bit, with
// a quarter of the per-lane work and four times the lanes.
template <int RP>
__global__ __launch_bounds__(4 * kGramRows) void k_apply_q4(const OrthDesc* __restrict__ descs,
                                                            const int32_t* __restrict__ map, int first, int r,
                                                            float* __restrict__ base, const double* __restrict__ gram) {
  constexpr int NJ = RP / 4;
  constexpr int NT = 4 * kGramRows;
  // one table per lane of the quad, each 16 bytes past a multiple of 256:
  // the four lanes' 16-byte reads of a step fall in different banks
  constexpr int TS = RP * NJ + 2;
  __shared__ double Rg[4 * TS];
  __shared__ double rinv[RP];
  int local;
  const OrthDesc o = descs[orth_idx(descs, map, first, local)];
  const double* rs = gram + o.t_off;
  const int tid = threadIdx.x, g = tid & 3;
  const int i = local * kGramRows + (tid >> 2);
  float* p = base + o.off + min(i, o.rows - 1);
  const int64_t ld = o.rows;
  float pv[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) pv[j] = p[(int64_t)min(4 * j + g, r - 1) * ld];
  // R staged by lane: entries with q <= k or q >= r are zero (never used)
#pragma unroll
  for (int u = 0; u < (RP * RP + NT - 1) / NT; ++u) {
    const int e = tid + NT * u;
    if (e < RP * RP) {
      const int k = e / RP, q = e % RP;
      const double v = rs[e];
      Rg[(q & 3) * TS + k * NJ + (q >> 2)] = (q > k && q < r) ? v : 0.0;
      if (q == k) rinv[k] = (k < r && v > 0.0) ? 1.0 / v : 0.0;
    }
  }
  __syncthreads();
  if (i >= o.rows) return;
  double b[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) b[j] = (double)pv[j];
  const double* rg = Rg + g * TS;
  // Steps in groups of four (one column per lane of the quad), a group
  // skipped by a uniform branch once 4 G >= r; inside the last group, steps
  // k >= r have 1 / R_kk = 0 and zero rows of R, so they change nothing that
  // is stored.  A break instead of the branch keeps the loop rolled, with b
  // indexed at run time.  Step k + 1's coefficients are read during step k.
  double rc[NJ], rn[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) rc[j] = rg[j];
#pragma unroll
  for (int G = 0; G < NJ; ++G) {
    if (4 * G < r) {
#pragma unroll
      for (int gk = 0; gk < 4; ++gk) {
        const int k = 4 * G + gk;
        if (k + 1 < RP) {
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            if (j >= ((k + 1) >> 2)) rn[j] = rg[(k + 1) * NJ + j];
        }
        const double xk = quad_bcast_k(b[G] * rinv[k], gk);
        const double own = fma(-xk, rc[G], b[G]);  // zero coefficient for q <= k
        b[G] = g == gk ? xk : (g > gk ? own : b[G]);
#pragma unroll
        for (int j = 0; j < NJ; ++j)  // constant trip count: unrolled before the outer loops
          if (j > G) b[j] = fma(-xk, rc[j], b[j]);
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          if (j >= ((k + 1) >> 2)) rc[j] = rn[j];
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    if (4 * j + g < r) p[(int64_t)(4 * j + g) * ld] = (float)b[j];
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

// One launch per access-width part of the grid range g (the plan puts the
// 16-byte-row matrices first, in [0, wg_rows_v4)).
template <int RP, int MODE, bool GBF16>
static hipError_t mfma_p_launch(const LaunchCtx& c, const GridRange& g, const void* G, float* E, float* U, float beta,
                                const float* Q, float* P, int64_t p_fixed) {
  const int split = min(max(c.wg_rows_v4, g.base), g.base + g.count);
  const float* pold = MODE >= 5 ? c.p_prev : nullptr;
  double* pp = static_cast<double*>(c.ppart);
  if (split > g.base)
    hipLaunchKernelGGL((k_mfma_p<RP, MODE, GBF16, true>), dim3(split - g.base), dim3(256), 0, c.stream, c.mats,
                       c.rows_map, g.base, c.rank, G, E, U, beta, Q, P, p_fixed, pp, pold);
  if (g.base + g.count > split)
    hipLaunchKernelGGL((k_mfma_p<RP, MODE, GBF16, false>), dim3(g.base + g.count - split), dim3(256), 0, c.stream,
                       c.mats, c.rows_map, split, c.rank, G, E, U, beta, Q, P, p_fixed, pp, pold);
  return hipGetLastError();
}

template <int RP, bool GBF16>
static hipError_t mfma_p_rpg(const LaunchCtx& c, const GridRange& g, int mode, const void* G, float* E, float* U,
                             float beta, const float* Q, float* P, int64_t p_fixed) {
  switch (mode) {
    case 1: return mfma_p_launch<RP, 1, GBF16>(c, g, G, E, U, beta, Q, P, p_fixed);
    case 2: return mfma_p_launch<RP, 2, GBF16>(c, g, G, E, U, beta, Q, P, p_fixed);
    case 3: return mfma_p_launch<RP, 3, GBF16>(c, g, G, E, U, beta, Q, P, p_fixed);
    case 4: return mfma_p_launch<RP, 4, GBF16>(c, g, G, E, U, beta, Q, P, p_fixed);
    case 5: return mfma_p_launch<RP, 5, GBF16>(c, g, G, E, U, beta, Q, P, p_fixed);
    case 6: return mfma_p_launch<RP, 6, GBF16>(c, g, G, E, U, beta, Q, P, p_fixed);
    default: return hipErrorInvalidValue;
  }
}

template <int RP>
static hipError_t mfma_p_rp(const LaunchCtx& c, const GridRange& g, int mode, const void* G, float* E, float* U,
                            float beta, const float* Q, float* P, int64_t p_fixed) {
  if (g.count == 0) return hipSuccess;
  if (mode == 0)  // M read from E: no gradient involved
    return mfma_p_launch<RP, 0, false>(c, g, G, E, U, beta, Q, P, p_fixed);
  return c.g_bf16 ? mfma_p_rpg<RP, true>(c, g, mode, G, E, U, beta, Q, P, p_fixed)
                  : mfma_p_rpg<RP, false>(c, g, mode, G, E, U, beta, Q, P, p_fixed);
}

hipError_t launch_mfma_p(const LaunchCtx& c, const GridRange& g, int mode, const void* G, float* E, float* U,
                         float beta, const float* Q, float* P, int64_t p_fixed) {
  PSGD_RP_SWITCH(c.rank_pad, mfma_p_rp<RPV>(c, g, mode, G, E, U, beta, Q, P, p_fixed));
}

hipError_t launch_psum(const LaunchCtx& c, const GridRange& g, float* P, int64_t p_fixed) {
  if (g.count == 0) return hipSuccess;
  if (c.mfma)
    hipLaunchKernelGGL(k_psum<double>, dim3(g.count), dim3(kRedCols), 0, c.stream, c.mats, c.pred_map, g.base, c.rank,
                       static_cast<const double*>(c.ppart), P, p_fixed);
  else
    hipLaunchKernelGGL(k_psum<float>, dim3(g.count), dim3(kRedCols), 0, c.stream, c.mats, c.pred_map, g.base, c.rank,
                       static_cast<const float*>(c.ppart), P, p_fixed);
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
                                bool residual, const SgdArgs& sg) {
  if (c.wg_rec == 0) return hipSuccess;
  const dim3 g(c.wg_rec), b(256);
  const bool mh = Mhat != nullptr, sgd = sg.x != nullptr;
#define PSGD_MRECON(RS, MH, SG)                                                                             \
  hipLaunchKernelGGL((k_mfma_recon<RP, RS, MH, SG>), g, b, 0, c.stream, c.mats, c.rec_map, 0, c.rank, E, Q, Ph, \
                     Mhat, sg)
  if (residual) {
    if (mh && sgd) PSGD_MRECON(true, true, true);
    else if (mh) PSGD_MRECON(true, true, false);
    else if (sgd) PSGD_MRECON(true, false, true);
    else PSGD_MRECON(true, false, false);
  } else {
    if (mh && sgd) PSGD_MRECON(false, true, true);
    else if (mh) PSGD_MRECON(false, true, false);
    else if (sgd) PSGD_MRECON(false, false, true);
    else return hipSuccess;
  }
#undef PSGD_MRECON
  return hipGetLastError();
}

hipError_t launch_mfma_recon(const LaunchCtx& c, float* E, const float* Q, const float* Ph, float* Mhat,
                             bool residual, const SgdArgs& sg) {
  PSGD_RP_SWITCH(c.rank_pad, mfma_recon_rp<RPV>(c, E, Q, Ph, Mhat, residual, sg));
}

template <int RP>
static hipError_t gram_orth_rp(const LaunchCtx& c, int first, int count, const int32_t* map, int nblocks,
                               float* base, int32_t* zcount) {
  if (nblocks == 0 || count == 0) return hipSuccess;
  hipLaunchKernelGGL((k_gram_partial<RP>), dim3(nblocks), dim3(256), 0, c.stream, c.orth, map, first, c.rank, base,
                     c.gram);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_gram_reduce<RP>), dim3(count * (RP * RP / 256)), dim3(256 * kGramRedGroups), 0, c.stream,
                     c.orth, first, c.gram);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (RP >= 32)
    hipLaunchKernelGGL((k_gram_solve_blk<RP>), dim3(count), dim3(256), 0, c.stream, c.orth, first, c.rank, c.gram,
                       kZeroColumnRel, zcount);
  else
    hipLaunchKernelGGL((k_gram_solve<RP>), dim3(count), dim3(64), 0, c.stream, c.orth, first, c.rank, c.gram,
                       kZeroColumnRel, zcount);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (RP >= 32)
    hipLaunchKernelGGL((k_apply_q4<RP>), dim3(nblocks), dim3(4 * kGramRows), 0, c.stream, c.orth, map, first, c.rank,
                       base, c.gram);
  else
    hipLaunchKernelGGL((k_apply_t<RP>), dim3(nblocks), dim3(kGramRows), 0, c.stream, c.orth, map, first, c.rank, base,
                       c.gram);
  return hipGetLastError();
}

template <int RP>
static hipError_t gram_reduce_rp(const LaunchCtx& c, int first, int count) {
  if (count == 0) return hipSuccess;
  hipLaunchKernelGGL((k_gram_reduce<RP>), dim3(count * (RP * RP / 256)), dim3(256 * kGramRedGroups), 0, c.stream,
                     c.orth, first, c.gram);
  return hipGetLastError();
}

hipError_t launch_gram_reduce(const LaunchCtx& c, int first, int count) {
  PSGD_RP_SWITCH(c.rank_pad, gram_reduce_rp<RPV>(c, first, count));
}

hipError_t launch_gram_orth(const LaunchCtx& c, int first, int count, const int32_t* map, int nblocks,
                            float* base, int32_t* zcount) {
  PSGD_RP_SWITCH(c.rank_pad, gram_orth_rp<RPV>(c, first, count, map, nblocks, base, zcount));
}

}  // namespace psgd
