// Streaming kernels of the PowerSGD step for ranks up to 8 (gfx950, wave64);
// the orthonormalisation for every rank is in kernels_mfma.hip.
//
// One PowerSGD step per gradient matrix, as the "Method" section of the
// anthology note on PowerSGD (note 152) describes it: P = M Q with the
// previous step's Q, aggregate P, orthogonalise P, Q = M^T P_hat, aggregate Q;
// with error feedback (glossary entry "PowerSGD", error-feedback paragraph)
// M = G + E before the products and E = M - P_hat Q^T after them.
//
// The work is bound by HBM traffic at these ranks (about 2r+1 flops per
// 4-byte element per pass), so the kernels are organised around streaming
// each gradient-sized array once per pass with 16-byte accesses:
//   pass 1  read G, E (and u)  -> write M over E (and u), P = M Q      12 B/el
//   pass 2  read M             -> Q = M^T P_hat (partials per row block) 4 B/el
//   pass 3  read M             -> write E = M - P_hat Q^T (and M_hat)  8 B/el
// Matrices of the whole model share one launch per pass; a per-workgroup
// table maps each workgroup to its matrix.

#include <hip/hip_runtime.h>

#include "psgd_flat.h"
#include "psgd_kernels.h"
#include "psgd_tables.h"

namespace psgd {

// ---------------------------------------------------------------------------
// Vector access helpers (VEC = 4, 2 or 1 consecutive floats)
// ---------------------------------------------------------------------------

template <int VEC>
struct Vec {
  float v[VEC];
};

template <int VEC>
__device__ __forceinline__ Vec<VEC> ldv(const float* p) {
  Vec<VEC> r;
  if constexpr (VEC == 4) {
    const float4 t = *reinterpret_cast<const float4*>(p);
    r.v[0] = t.x; r.v[1] = t.y; r.v[2] = t.z; r.v[3] = t.w;
  } else if constexpr (VEC == 2) {
    const float2 t = *reinterpret_cast<const float2*>(p);
    r.v[0] = t.x; r.v[1] = t.y;
  } else {
    r.v[0] = *p;
  }
  return r;
}

template <int VEC>
__device__ __forceinline__ void stv(float* p, const Vec<VEC>& a) {
  if constexpr (VEC == 4) {
    *reinterpret_cast<float4*>(p) = make_float4(a.v[0], a.v[1], a.v[2], a.v[3]);
  } else if constexpr (VEC == 2) {
    *reinterpret_cast<float2*>(p) = make_float2(a.v[0], a.v[1]);
  } else {
    *p = a.v[0];
  }
}

// Non-temporal (streaming) variants: the nt bit on the access tells the
// caches the line will not be reused soon.  Measured on the grouped 7B-shaped
// set: streaming loads of G and of M in the residual pass and streaming
// stores of M_hat and E there shave a few percent off a step (E is read
// again only by the next step).  In pass 1, streaming loads of E and a
// streaming store of M pay together with 256-column splits (14.8 -> 13.4 ms
// with both) and cost with 1024-column ones.
typedef float v4f_nt __attribute__((ext_vector_type(4)));
typedef float v2f_nt __attribute__((ext_vector_type(2)));
typedef uint32_t v2u_nt __attribute__((ext_vector_type(2)));

template <int VEC>
__device__ __forceinline__ void stv_nt(float* p, const Vec<VEC>& a) {
  if constexpr (VEC == 4) {
    v4f_nt t = {a.v[0], a.v[1], a.v[2], a.v[3]};
    __builtin_nontemporal_store(t, reinterpret_cast<v4f_nt*>(p));
  } else if constexpr (VEC == 2) {
    v2f_nt t = {a.v[0], a.v[1]};
    __builtin_nontemporal_store(t, reinterpret_cast<v2f_nt*>(p));
  } else {
    __builtin_nontemporal_store(a.v[0], p);
  }
}

template <int VEC>
__device__ __forceinline__ Vec<VEC> ldv_nt(const float* p) {
  Vec<VEC> r;
  if constexpr (VEC == 4) {
    const v4f_nt t = __builtin_nontemporal_load(reinterpret_cast<const v4f_nt*>(p));
    r.v[0] = t[0]; r.v[1] = t[1]; r.v[2] = t[2]; r.v[3] = t[3];
  } else if constexpr (VEC == 2) {
    const v2f_nt t = __builtin_nontemporal_load(reinterpret_cast<const v2f_nt*>(p));
    r.v[0] = t[0]; r.v[1] = t[1];
  } else {
    r.v[0] = __builtin_nontemporal_load(p);
  }
  return r;
}

// Loads and stores of the arrays a pass streams through (E, M, u), with the
// non-temporal hint when NT: for sets far larger than the caches, where no
// pass finds the previous one's lines anyway.
template <int VEC, bool NT>
__device__ __forceinline__ Vec<VEC> ldv_s(const float* p) {
  if constexpr (NT) return ldv_nt<VEC>(p);
  else return ldv<VEC>(p);
}

template <int VEC, bool NT>
__device__ __forceinline__ void stv_s(float* p, const Vec<VEC>& a) {
  if constexpr (NT) stv_nt<VEC>(p, a);
  else stv<VEC>(p, a);
}

// Gradient loads: fp32, or bfloat16 widened exactly to fp32 (the upper 16
// bits of the fp32 pattern).  Both are read once per step: streaming hint.
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

template <int VEC, bool BF16>
__device__ __forceinline__ Vec<VEC> ldg(const void* G, unsigned idx) {
  if constexpr (!BF16) {
    return ldv_nt<VEC>(static_cast<const float*>(G) + idx);
  } else {
    const uint16_t* p = static_cast<const uint16_t*>(G) + idx;
    Vec<VEC> r;
    if constexpr (VEC == 4) {
      const v2u_nt t = __builtin_nontemporal_load(reinterpret_cast<const v2u_nt*>(p));
      r.v[0] = bf16_to_f32(t[0] & 0xffffu);
      r.v[1] = bf16_to_f32(t[0] >> 16);
      r.v[2] = bf16_to_f32(t[1] & 0xffffu);
      r.v[3] = bf16_to_f32(t[1] >> 16);
    } else if constexpr (VEC == 2) {
      const uint32_t t = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
      r.v[0] = bf16_to_f32(t & 0xffffu);
      r.v[1] = bf16_to_f32(t >> 16);
    } else {
      r.v[0] = bf16_to_f32(*p);
    }
    return r;
  }
}

// Element j of a row whose base pointer is wavefront-uniform, addressed by a
// 32-bit byte offset (the scalar-base + vector-offset form of the memory
// instructions; rows are shorter than 2^30 elements).
__device__ __forceinline__ const float* at_row(const float* rowp, unsigned j) {
  return reinterpret_cast<const float*>(reinterpret_cast<const char*>(rowp) + (j << 2));
}
__device__ __forceinline__ float* at_row(float* rowp, unsigned j) {
  return reinterpret_cast<float*>(reinterpret_cast<char*>(rowp) + (j << 2));
}
__device__ __forceinline__ const void* at_row_g(const void* rowp, unsigned j, bool bf16) {
  return static_cast<const char*>(rowp) + (bf16 ? (j << 1) : (j << 2));
}

// Sum of NV per-lane values over the 64 lanes of a wavefront, transposed: on
// return lane l holds the total of value (l >> (6 - log2 NV)).  Each butterfly
// step halves the values a lane carries, so the cost is about NV shuffles
// instead of 6 NV.
template <int NV>
__device__ __forceinline__ float wave_transpose_sum(float (&v)[NV], int lane) {
  static_assert(NV >= 1 && NV <= 64 && (NV & (NV - 1)) == 0, "NV must be a power of two <= 64");
  constexpr int LOG = NV >= 64 ? 6 : NV >= 32 ? 5 : NV >= 16 ? 4 : NV >= 8 ? 3 : NV >= 4 ? 2 : NV >= 2 ? 1 : 0;
#pragma unroll
  for (int s = 0; s < LOG; ++s) {
    const int bit = 5 - s;
    const int half = NV >> (s + 1);
    // lane-dependent exchange written as bit operations on the two values:
    // a select between v[i] and v[i + half] is turned by the compiler into a
    // load through a lane-dependent index, which keeps v an indexable array
    // (compare-and-select chains over all of it, or private scratch)
    const uint32_t up = 0u - ((uint32_t)(lane >> bit) & 1u);
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const uint32_t a = __float_as_uint(v[i]), b = __float_as_uint(v[i + half]);
      const float send = __uint_as_float((a & up) | (b & ~up));
      const float keep = __uint_as_float((b & up) | (a & ~up));
      v[i] = keep + __shfl_xor(send, 1 << bit);
    }
  }
  float x = v[0];
#pragma unroll
  for (int bit = 5 - LOG; bit >= 0; --bit) x += __shfl_xor(x, 1 << bit);
  return x;
}

constexpr int pow2_at_least(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// ---------------------------------------------------------------------------
// Pass-through tensors
// ---------------------------------------------------------------------------

// One pass-through workgroup (kPassChunk elements of one tensor): the value
// (u = beta u + G first with momentum) copied into the P buffer after the
// factors, where the P aggregation carries it.
template <bool MOM, bool GBF16>
__device__ __forceinline__ void pass_pack_wg(const PassDesc* __restrict__ pass, const int32_t* __restrict__ map,
                                             int wg, const void* __restrict__ G, float* __restrict__ U, float beta,
                                             float* __restrict__ Pbuf) {
  const PassDesc pd = pass[map[wg]];
  const int64_t c0 = (int64_t)(wg - pd.wg0) * kPassChunk;
  const int64_t c1 = c0 + kPassChunk < pd.len ? c0 + kPassChunk : pd.len;
  for (int64_t i = c0 + threadIdx.x; i < c1; i += 256) {
    float x;
    if constexpr (GBF16)
      x = bf16_to_f32(static_cast<const uint16_t*>(G)[pd.off + i]);
    else
      x = static_cast<const float*>(G)[pd.off + i];
    if constexpr (MOM) {
      x = fmaf(beta, U[pd.off + i], x);
      U[pd.off + i] = x;
    }
    Pbuf[pd.p_off + i] = x;
  }
}

// Aggregated pass-through values back to flat buffers: into `out` (if
// non-null) and/or as the update of the fused SGD step.
template <bool SGD>
__device__ __forceinline__ void pass_unpack_wg(const PassDesc* __restrict__ pass, const int32_t* __restrict__ map,
                                               int wg, const float* __restrict__ Pbuf, float* __restrict__ out,
                                               const SgdArgs& sg) {
  const PassDesc pd = pass[map[wg]];
  const int64_t c0 = (int64_t)(wg - pd.wg0) * kPassChunk;
  const int64_t c1 = c0 + kPassChunk < pd.len ? c0 + kPassChunk : pd.len;
  for (int64_t i = c0 + threadIdx.x; i < c1; i += 256) {
    const float v = Pbuf[pd.p_off + i];
    if (out) out[pd.off + i] = v;
    if constexpr (SGD) {
      const float mm = fmaf(sg.mu, sg.m[pd.off + i], v);
      sg.m[pd.off + i] = mm;
      const float dir = sg.nesterov ? fmaf(sg.mu, mm, v) : mm;
      sg.x[pd.off + i] = fmaf(-sg.lr, dir, sg.x[pd.off + i]);
    }
  }
}

// ---------------------------------------------------------------------------
// Pass 1: EF-add (+ momentum) and P = M Q
// ---------------------------------------------------------------------------

// One wavefront: rows [row0, row0 + kWaveRows) of matrix d, columns
// [c0, c1) (all of them, or one column split).  Each lane keeps its VEC x R
// slice of Q in registers for the current column step and reuses it across
// the wavefront's rows.  The row sums of P go to pdst (column k of m floats
// from there): P itself, or this split's partial.
// Row `rr` of P_hat Q^T at the lane's VEC columns: the reconstruction of the
// residual pass, in one fixed summation order.  The leading product is kept a
// separately rounded multiply (no contraction into a later subtraction), so
// every kernel that forms M - P_hat Q^T rounds the same way.
template <int R, int VEC>
__device__ __forceinline__ Vec<VEC> recon_row(const float (&ph)[R], const Vec<VEC> (&qv)[R]) {
#pragma clang fp contract(off)
  Vec<VEC> mh;
#pragma unroll
  for (int c = 0; c < VEC; ++c) {
    float s = ph[0] * qv[0].v[c];
#pragma unroll
    for (int k = 1; k < R; ++k) s = fmaf(ph[k], qv[k].v[c], s);
    mh.v[c] = s;
  }
  return mh;
}

// The kWaveRows x R row sums of a pass-1 wavefront into pdst (column k of m
// floats), at most 32 values per transposed butterfly (a 64-value one does
// not stay in registers: it spilled to scratch).  BASE, the first value of
// this piece, is a template parameter so that every index into acc is a
// compile-time constant (a run-time index into a register array is lowered
// to a compare-and-select over all of its elements).
template <int R, int BASE>
__device__ __forceinline__ void row_sums(const float (&acc)[kWaveRows][R], int lane, int nrows, int m, int row0,
                                         float* pdst) {
  constexpr int NALL = kWaveRows * R;
  constexpr int NV = pow2_at_least(NALL < 32 ? NALL : 32);
  constexpr int SHIFT = NV >= 32 ? 1 : NV >= 16 ? 2 : NV >= 8 ? 3 : NV >= 4 ? 4 : NV >= 2 ? 5 : 6;
  float vals[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) vals[i] = BASE + i < NALL ? acc[(BASE + i) / R][(BASE + i) % R] : 0.f;
  const float tot = wave_transpose_sum<NV>(vals, lane);
  const int vi = BASE + (lane >> SHIFT);
  if ((lane & ((1 << SHIFT) - 1)) == 0 && vi < NALL) {
    const int rr = vi / R, k = vi % R;
    if (rr < nrows) pdst[(int64_t)k * m + row0 + rr] = tot;
  }
  if constexpr (BASE + NV < NALL) row_sums<R, BASE + NV>(acc, lane, nrows, m, row0, pdst);
}

// MODE 0: M read from E (plain M Q); 1: M = G + E; 2: u = beta u + G,
// M = u + E; 3: M = G (no error feedback); 4: u = beta u + G, M = u.
// Deferred residual: E holds the previous step's M and Pold / Q its P_hat and
// Q, so E = M_prev - P_hat Q^T is formed here on the fly; 5: M = G + E,
// 6: u = beta u + G, M = u + E.  Modes 1..6 store M over E.  Pold may be P
// itself: each wavefront reads its rows of Pold before writing them in P.
template <int R, int VEC, int MODE, bool GBF16, bool NT>
__device__ __forceinline__ void ef_p_wave(const MatDesc& d, int row0, int c0, int c1, int lane,
                                          const void* __restrict__ G, float* __restrict__ E, float* __restrict__ U,
                                          float beta, const float* __restrict__ Q, float* pdst, const float* Pold) {
  constexpr bool MOM = MODE == 2 || MODE == 4 || MODE == 6;
  constexpr bool LOAD_E = MODE <= 2 || MODE >= 5;
  constexpr bool DEFERRED = MODE >= 5;
  const int m = d.m, n = d.n;
  const int nrows = min(kWaveRows, m - row0);
  float acc[kWaveRows][R];
#pragma unroll
  for (int rr = 0; rr < kWaveRows; ++rr)
#pragma unroll
    for (int k = 0; k < R; ++k) acc[rr][k] = 0.f;
  float ph[kWaveRows][R];
  if constexpr (DEFERRED) {
#pragma unroll
    for (int rr = 0; rr < kWaveRows; ++rr)
#pragma unroll
      for (int k = 0; k < R; ++k) ph[rr][k] = Pold[d.p_off + (int64_t)k * m + row0 + min(rr, nrows - 1)];
  }

  // Row and Q-column base pointers are wavefront-uniform (scalar
  // registers) and the lane's column is a 32-bit unsigned offset from them,
  // so every access takes the scalar-base + vector-offset form (no 64-bit
  // address per lane and row).  Rows past the matrix repeat its last row for
  // the loads; their stores are skipped.
  const float* qcol[R];
#pragma unroll
  for (int k = 0; k < R; ++k) qcol[k] = Q + d.q_off + (int64_t)k * n;
  float* erow[kWaveRows];
  const void* grow[kWaveRows];
  float* urow[kWaveRows];
#pragma unroll
  for (int rr = 0; rr < kWaveRows; ++rr) {
    const int64_t ro = d.off + (int64_t)(row0 + min(rr, nrows - 1)) * n;
    erow[rr] = E + ro;
    grow[rr] = GBF16 ? static_cast<const void*>(static_cast<const uint16_t*>(G) + ro)
                     : static_cast<const void*>(static_cast<const float*>(G) + ro);
    urow[rr] = U + ro;
  }
  for (unsigned j = (unsigned)(c0 + lane * VEC); j < (unsigned)c1; j += 64 * VEC) {
    Vec<VEC> qv[R];
#pragma unroll
    for (int k = 0; k < R; ++k) qv[k] = ldv<VEC>(at_row(qcol[k], j));
    Vec<VEC> g[kWaveRows], e[kWaveRows];
#pragma unroll
    for (int rr = 0; rr < kWaveRows; ++rr) {
      if constexpr (MODE != 0) g[rr] = ldg<VEC, GBF16>(at_row_g(grow[rr], j, GBF16), 0u);
      if constexpr (LOAD_E) e[rr] = ldv_s<VEC, NT>(at_row(erow[rr], j));
    }
    Vec<VEC> u[kWaveRows];
    if constexpr (MOM) {
#pragma unroll
      for (int rr = 0; rr < kWaveRows; ++rr) u[rr] = ldv_s<VEC, NT>(at_row(urow[rr], j));
    }
#pragma unroll
    for (int rr = 0; rr < kWaveRows; ++rr) {
      if (rr < nrows) {
        Vec<VEC> mv;
        if constexpr (DEFERRED) {
          const Vec<VEC> mh = recon_row<R, VEC>(ph[rr], qv);
#pragma unroll
          for (int c = 0; c < VEC; ++c) e[rr].v[c] = e[rr].v[c] - mh.v[c];
        }
        if constexpr (MODE == 0) {
          mv = e[rr];
        } else if constexpr (MOM) {
#pragma unroll
          for (int c = 0; c < VEC; ++c) u[rr].v[c] = fmaf(beta, u[rr].v[c], g[rr].v[c]);
          stv_s<VEC, NT>(at_row(urow[rr], j), u[rr]);
#pragma unroll
          for (int c = 0; c < VEC; ++c) mv.v[c] = LOAD_E ? u[rr].v[c] + e[rr].v[c] : u[rr].v[c];
        } else {
#pragma unroll
          for (int c = 0; c < VEC; ++c) mv.v[c] = LOAD_E ? g[rr].v[c] + e[rr].v[c] : g[rr].v[c];
        }
        if constexpr (MODE != 0) stv_s<VEC, NT>(at_row(erow[rr], j), mv);
#pragma unroll
        for (int k = 0; k < R; ++k)
#pragma unroll
          for (int c = 0; c < VEC; ++c) acc[rr][k] = fmaf(mv.v[c], qv[k].v[c], acc[rr][k]);
      }
    }
  }

  row_sums<R, 0>(acc, lane, nrows, m, row0, pdst);
}

// Row tile and column range of a pass-1 / pass-3 workgroup: the matrix's
// workgroups (`local` counts from its first one) run over (row tile, column
// split), splits fastest; `splits` of `cols` columns each.
struct RowTile {
  int row0, c0, c1, split;
};

__device__ __forceinline__ RowTile row_tile(const MatDesc& d, int local, int splits, int cols, int wave) {
  const int tile = local / splits, split = local - tile * splits;
  const int c0 = split * cols;
  return RowTile{tile * kRowsPerWG + wave * kWaveRows, c0, min(d.n, c0 + cols), split};
}

// P (or, for a column-split matrix, the split's partial in ppart, summed
// afterwards in fixed order) at the plan's offsets or at p_fixed.
// Workgroups from nrow_wg on pack the pass-through tensors (the launch's
// extra workgroups, when pack_dst is given).
// NT: streaming hints on E, M and u (sets far larger than the caches).
template <int R, int MODE, bool GBF16, bool NT>
__global__ __launch_bounds__(kWGThreads) void k_ef_p(const MatDesc* __restrict__ mats,
                                                     const int32_t* __restrict__ map, int wg_base,
                                                     const void* __restrict__ G, float* __restrict__ E,
                                                     float* __restrict__ U, float beta,
                                                     const float* __restrict__ Q, float* P, int64_t p_fixed,
                                                     const float* Pold, float* __restrict__ ppart, int nrow_wg,
                                                     const PassDesc* __restrict__ pass,
                                                     const int32_t* __restrict__ pass_map, float* pack_dst) {
  if constexpr (MODE != 0) {
    if ((int)blockIdx.x >= nrow_wg) {
      constexpr bool MOM = MODE == 2 || MODE == 4 || MODE == 6;
      pass_pack_wg<MOM, GBF16>(pass, pass_map, blockIdx.x - nrow_wg, G, U, beta, pack_dst);
      return;
    }
  }
  const int wg = blockIdx.x + wg_base;
  const MatDesc d = mats[map[wg]];
  // wave index made provably uniform: row addressing and P_hat loads go scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const RowTile t = row_tile(d, wg - d.wg_rows0, d.s1, d.s1_cols, wave);
  if (t.row0 >= d.m) return;
  float* pdst = d.s1 > 1 ? ppart + d.ppart_off + (int64_t)t.split * R * d.m : P + (p_fixed >= 0 ? p_fixed : d.p_off);
  if (d.vec == 4)
    ef_p_wave<R, 4, MODE, GBF16, NT>(d, t.row0, t.c0, t.c1, lane, G, E, U, beta, Q, pdst, Pold);
  else if (d.vec == 2)
    ef_p_wave<R, 2, MODE, GBF16, NT>(d, t.row0, t.c0, t.c1, lane, G, E, U, beta, Q, pdst, Pold);
  else
    ef_p_wave<R, 1, MODE, GBF16, NT>(d, t.row0, t.c0, t.c1, lane, G, E, U, beta, Q, pdst, Pold);
}

// ---------------------------------------------------------------------------
// Pass 2: Q = M^T P_hat, partial sums per row block
// ---------------------------------------------------------------------------

// One wavefront: 64*VEC consecutive columns of one row block.  P_hat values
// of a row are wavefront-uniform (scalar loads); each lane accumulates VEC x R
// dot products over the block's rows.  NT: M is read with the non-temporal
// hint, for sets far larger than the caches (7B-shaped set 4.49 -> 4.19 ms,
// the step 33.4 -> 32.4-32.9 ms); a set that fits the 256 MB last-level cache
// keeps plain loads, so that M is still cached for the residual pass that
// reads it next.
template <int R, int VEC, bool NT>
__device__ __forceinline__ Vec<VEC> ld_m(const float* p) {
  if constexpr (NT) return ldv_nt<VEC>(p);
  else return ldv<VEC>(p);
}

template <int R, int VEC, bool NT>
__device__ __forceinline__ void mtp_wave(const MatDesc& d, int rb, int j, const float* __restrict__ M,
                                         const float* __restrict__ Ph, int64_t ph_fixed, float* __restrict__ Q,
                                         float* __restrict__ part) {
  const int m = d.m, n = d.n;
  const int i0 = rb * d.rb_rows;
  const int i1 = min(m, i0 + d.rb_rows);
  const float* ph = Ph + (ph_fixed >= 0 ? ph_fixed : d.p_off);
  const float* mp = M + d.off + j;
  float acc[VEC][R];
#pragma unroll
  for (int c = 0; c < VEC; ++c)
#pragma unroll
    for (int k = 0; k < R; ++k) acc[c][k] = 0.f;

  constexpr int U = 8;
  int i = i0;
  for (; i + U <= i1; i += U) {
    Vec<VEC> x[U];
#pragma unroll
    for (int t = 0; t < U; ++t) x[t] = ld_m<R, VEC, NT>(mp + (int64_t)(i + t) * n);
#pragma unroll
    for (int t = 0; t < U; ++t)
#pragma unroll
      for (int k = 0; k < R; ++k) {
        const float w = ph[(int64_t)k * m + i + t];
#pragma unroll
        for (int c = 0; c < VEC; ++c) acc[c][k] = fmaf(x[t].v[c], w, acc[c][k]);
      }
  }
  for (; i < i1; ++i) {
    const Vec<VEC> x = ld_m<R, VEC, NT>(mp + (int64_t)i * n);
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const float w = ph[(int64_t)k * m + i];
#pragma unroll
      for (int c = 0; c < VEC; ++c) acc[c][k] = fmaf(x.v[c], w, acc[c][k]);
    }
  }
  float* out = d.nrb > 1 ? part + d.part_off + (int64_t)rb * R * n : Q + d.q_off;
#pragma unroll
  for (int k = 0; k < R; ++k) {
    Vec<VEC> o;
#pragma unroll
    for (int c = 0; c < VEC; ++c) o.v[c] = acc[c][k];
    stv<VEC>(out + (int64_t)k * n + j, o);
  }
}

template <int R, bool NT>
__global__ __launch_bounds__(kWGThreads) void k_mtp(const MatDesc* __restrict__ mats, const int32_t* __restrict__ map,
                                                    int wg_base, const float* __restrict__ M,
                                                    const float* __restrict__ Ph, int64_t ph_fixed,
                                                    float* __restrict__ Q, float* __restrict__ part) {
  const int wg = blockIdx.x + wg_base;
  const MatDesc d = mats[map[wg]];
  const int local = wg - d.wg_mtp0;
  const int rb = local / d.ncb, cb = local - rb * d.ncb;
  // wave index made provably uniform: row addressing and P_hat loads go scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int j = (cb * kMtpWaves + wave) * 64 * d.vec + lane * d.vec;
  if (j >= d.n) return;
  if (d.vec == 4)
    mtp_wave<R, 4, NT>(d, rb, j, M, Ph, ph_fixed, Q, part);
  else if (d.vec == 2)
    mtp_wave<R, 2, NT>(d, rb, j, M, Ph, ph_fixed, Q, part);
  else
    mtp_wave<R, 1, NT>(d, rb, j, M, Ph, ph_fixed, Q, part);
}

// Fixed-order sum of the row-block partials: Q[k*n + j] = sum_b part_b[k*n + j].
// A workgroup of kRedWaves wavefronts.  Lane l of a wavefront owns output
// element l of a 64-element slice (256-byte loads per block); the matrix's
// red_split S wavefronts share a slice, wavefront s summing the blocks
// b = s, s + S, ... in two running sums, and the S totals are added in
// wavefront order through LDS.  The order is fixed: deterministic.
__global__ __launch_bounds__(64 * kRedWaves) void k_qreduce(const MatDesc* __restrict__ mats,
                                                            const int32_t* __restrict__ map, int wg_base, int R,
                                                            const float* __restrict__ part, float* __restrict__ Q) {
  __shared__ float tot[kRedWaves][64];
  const int wg = blockIdx.x + wg_base;
  const MatDesc d = mats[map[wg]];
  const int S = d.red_split;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int grp = wave / S, s = wave - grp * S;
  const int64_t len = (int64_t)R * d.n;
  const int64_t idx = ((int64_t)(wg - d.wg_red0) * (kRedWaves / S) + grp) * 64 + lane;
  float acc = 0.f;
  if (idx < len) {
    const float* src = part + d.part_off + idx;
    float s0 = 0.f, s1 = 0.f;
    int b = s;
    for (; b + S < d.nrb; b += 2 * S) {
      s0 += src[(int64_t)b * len];
      s1 += src[(int64_t)(b + S) * len];
    }
    if (b < d.nrb) s0 += src[(int64_t)b * len];
    acc = s0 + s1;
  }
  if (S == 1) {  // uniform over the workgroup
    if (idx < len) Q[d.q_off + idx] = acc;
    return;
  }
  tot[wave][lane] = acc;
  __syncthreads();
  if (s == 0 && idx < len) {
    float t = tot[wave][lane];
    for (int u = 1; u < S; ++u) t += tot[wave + u][lane];
    Q[d.q_off + idx] = t;
  }
}

// ---------------------------------------------------------------------------
// Pass 3: residual E = M - P_hat Q^T (+ M_hat); decompression
// ---------------------------------------------------------------------------

// RESID: E <- M - M_hat (M read from E).  WRITE_MHAT: M_hat stored.  SGD:
// post-compression heavy-ball step with the decompressed update M_hat,
// m <- mu m + M_hat, x <- x - lr m (X = parameters, Mb = momentum buffer).
template <int R, int VEC, bool RESID, bool WRITE_MHAT, bool SGD>
__device__ __forceinline__ void recon_wave(const MatDesc& d, int row0, int c0, int c1, int lane, float* __restrict__ E,
                                           const float* __restrict__ Q, const float* __restrict__ Ph,
                                           float* __restrict__ Mhat, const SgdArgs& sg) {
  const int m = d.m, n = d.n;
  const int nrows = min(kWaveRows, m - row0);
  float ph[kWaveRows][R];
#pragma unroll
  for (int rr = 0; rr < kWaveRows; ++rr)
#pragma unroll
    for (int k = 0; k < R; ++k) ph[rr][k] = Ph[d.p_off + (int64_t)k * m + row0 + min(rr, nrows - 1)];
  const float* q = Q + d.q_off;
  const int64_t base = d.off + (int64_t)row0 * n;
  for (int j = c0 + lane * VEC; j < c1; j += 64 * VEC) {
    Vec<VEC> qv[R];
#pragma unroll
    for (int k = 0; k < R; ++k) qv[k] = ldv<VEC>(q + (int64_t)k * n + j);
    Vec<VEC> x[kWaveRows], xp[kWaveRows], xm[kWaveRows];
#pragma unroll
    for (int rr = 0; rr < kWaveRows; ++rr) {
      const int64_t idx = base + (int64_t)min(rr, nrows - 1) * n + j;
      if constexpr (RESID) x[rr] = ldv_nt<VEC>(E + idx);
      if constexpr (SGD) {
        xp[rr] = ldv<VEC>(sg.x + idx);
        xm[rr] = ldv<VEC>(sg.m + idx);
      }
    }
#pragma unroll
    for (int rr = 0; rr < kWaveRows; ++rr) {
      if (rr < nrows) {
        const int64_t idx = base + (int64_t)rr * n + j;
        const Vec<VEC> mh = recon_row<R, VEC>(ph[rr], qv);
        if constexpr (RESID) {
          Vec<VEC> e;
#pragma unroll
          for (int c = 0; c < VEC; ++c) e.v[c] = x[rr].v[c] - mh.v[c];
          stv_nt<VEC>(E + idx, e);
        }
        // M_hat is consumed by the optimizer after the step, not by this
        // pipeline: streaming store.
        if constexpr (WRITE_MHAT) stv_nt<VEC>(Mhat + idx, mh);
        if constexpr (SGD) {
#pragma unroll
          for (int c = 0; c < VEC; ++c) {
            xm[rr].v[c] = fmaf(sg.mu, xm[rr].v[c], mh.v[c]);
            const float dir = sg.nesterov ? fmaf(sg.mu, xm[rr].v[c], mh.v[c]) : xm[rr].v[c];
            xp[rr].v[c] = fmaf(-sg.lr, dir, xp[rr].v[c]);
          }
          stv<VEC>(sg.m + idx, xm[rr]);
          stv<VEC>(sg.x + idx, xp[rr]);
        }
      }
    }
  }
}

// Flat tiling (a matrix with d.s3 == 0, see psgd_flat.h): the workgroup's
// d.s3_cols elements (1 to kFlatSub pieces of kFlatChunk), 8 float4 per thread and piece (each wavefront load or store one
// aligned 1 KB stretch).  Q is staged in LDS transposed (row j: the RQ
// values Q[j][k], zero past the rank) and so are the P_hat rows the chunk
// touches; each value is formed with recon_row, the arithmetic of the row
// tiles and of the deferred residual.  The last float4 of a matrix whose
// size is not a multiple of 4 is handled element by element.
extern __shared__ float4 psgd_flat_lds[];

template <int R, bool RESID, bool WRITE_MHAT, bool SGD>
__device__ __forceinline__ void recon_flat(const MatDesc& d, int chunk, float* __restrict__ E,
                                           const float* __restrict__ Q, const float* __restrict__ Ph,
                                           float* __restrict__ Mhat, const SgdArgs& sg) {
  constexpr int RQ = flat_rq(R);
  constexpr int NV = kFlatChunk / 4 / kWGThreads;  // float4 per thread
  const int m = d.m, n = d.n;
  const uint32_t total = (uint32_t)m * (uint32_t)n;
  const uint32_t GW = (uint32_t)d.s3_cols;  // elements per workgroup (a multiple of kFlatChunk)
  const int nsub = (int)(GW / kFlatChunk);
  const uint32_t g0 = (uint32_t)chunk * GW;
  const uint32_t g1 = min(total, g0 + GW);
  const int row_a = (int)(g0 / (uint32_t)n), row_b = (int)((g1 - 1) / (uint32_t)n);
  float* qs = reinterpret_cast<float*>(psgd_flat_lds);  // [n][RQ]
  float* ps = qs + n * RQ;                              // [row_b - row_a + 1][RQ]
  for (int e = threadIdx.x; e < RQ * n; e += kWGThreads) {
    const int k = e / n, j = e - k * n;
    qs[j * RQ + k] = k < R ? Q[d.q_off + (int64_t)k * n + j] : 0.f;
  }
  const int nr = row_b - row_a + 1;
  for (int e = threadIdx.x; e < RQ * nr; e += kWGThreads) {
    const int k = e / nr, rr = e - k * nr;
    ps[rr * RQ + k] = k < R ? Ph[d.p_off + (int64_t)k * m + row_a + rr] : 0.f;
  }
  __syncthreads();
  const int64_t base = d.off;
  // nsub pieces of kFlatChunk elements, one after the other, on the
  // staged Q and P_hat rows
  for (int sc = 0; sc < nsub; ++sc) {
  const uint32_t f0 = g0 + (uint32_t)sc * kFlatChunk;
  if (f0 >= g1) break;
  const uint32_t f1 = min(g1, f0 + (uint32_t)kFlatChunk);
  Vec<4> x[NV], xp[NV], xm[NV];
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const uint32_t f = f0 + 4u * (threadIdx.x + kWGThreads * u);
    if (f + 4 <= f1) {
      if constexpr (RESID) x[u] = ldv_nt<4>(E + base + f);
      if constexpr (SGD) {
        xp[u] = ldv<4>(sg.x + base + f);
        xm[u] = ldv<4>(sg.m + base + f);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const uint32_t f = f0 + 4u * (threadIdx.x + kWGThreads * u);
    if (f >= f1) continue;
    const int cnt = (int)min(4u, f1 - f);
    int i = (int)(f / (uint32_t)n);
    int j = (int)(f - (uint32_t)i * (uint32_t)n);
    Vec<4> mh;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (j >= n) {
        j -= n;
        ++i;
      }
      // (past the matrix's end, in its last float4, i may reach row_b + 1:
      // clamped to a staged row, the value is discarded)
      const int prow = min(i, row_b) - row_a;
      float ph[R];
      Vec<1> qv[R];
#pragma unroll
      for (int k = 0; k < R; ++k) {
        ph[k] = ps[prow * RQ + k];
        qv[k].v[0] = qs[j * RQ + k];
      }
      mh.v[c] = recon_row<R, 1>(ph, qv).v[0];
      ++j;
    }
    const int64_t idx = base + f;
    if (cnt == 4) {
      if constexpr (RESID) {
        Vec<4> e;
#pragma unroll
        for (int c = 0; c < 4; ++c) e.v[c] = x[u].v[c] - mh.v[c];
        stv_nt<4>(E + idx, e);
      }
      if constexpr (WRITE_MHAT) stv_nt<4>(Mhat + idx, mh);
      if constexpr (SGD) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          xm[u].v[c] = fmaf(sg.mu, xm[u].v[c], mh.v[c]);
          const float dir = sg.nesterov ? fmaf(sg.mu, xm[u].v[c], mh.v[c]) : xm[u].v[c];
          xp[u].v[c] = fmaf(-sg.lr, dir, xp[u].v[c]);
        }
        stv<4>(sg.m + idx, xm[u]);
        stv<4>(sg.x + idx, xp[u]);
      }
    } else {  // the matrix's last, partial float4 (constant indices into mh)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (c >= cnt) break;
        if constexpr (RESID) E[idx + c] = E[idx + c] - mh.v[c];
        if constexpr (WRITE_MHAT) Mhat[idx + c] = mh.v[c];
        if constexpr (SGD) {
          float mm = fmaf(sg.mu, sg.m[idx + c], mh.v[c]);
          const float dir = sg.nesterov ? fmaf(sg.mu, mm, mh.v[c]) : mm;
          sg.x[idx + c] = fmaf(-sg.lr, dir, sg.x[idx + c]);
          sg.m[idx + c] = mm;
        }
      }
    }
  }
  }  // sub-chunks
}

// Workgroups from nrec_wg on unpack the pass-through tensors (the launch's
// extra workgroups, when unpack_src is given).
template <int R, bool RESID, bool WRITE_MHAT, bool SGD>
__global__ __launch_bounds__(kWGThreads) void k_recon(const MatDesc* __restrict__ mats, const int32_t* __restrict__ map,
                                                      float* __restrict__ E, const float* __restrict__ Q,
                                                      const float* __restrict__ Ph, float* __restrict__ Mhat,
                                                      SgdArgs sg, int nrec_wg, const PassDesc* __restrict__ pass,
                                                      const int32_t* __restrict__ pass_map,
                                                      const float* __restrict__ unpack_src) {
  if ((int)blockIdx.x >= nrec_wg) {
    pass_unpack_wg<SGD>(pass, pass_map, blockIdx.x - nrec_wg, unpack_src, Mhat, sg);
    return;
  }
  const int wg = blockIdx.x;
  const MatDesc d = mats[map[wg]];
  if (d.s3 == 0) {  // flat tiling (uniform over the workgroup)
    recon_flat<R, RESID, WRITE_MHAT, SGD>(d, wg - d.wg_rec0, E, Q, Ph, Mhat, sg);
    return;
  }
  // wave index made provably uniform: row addressing and P_hat loads go scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const RowTile t = row_tile(d, wg - d.wg_rec0, d.s3, d.s3_cols, wave);
  if (t.row0 >= d.m) return;
  if (d.vec == 4)
    recon_wave<R, 4, RESID, WRITE_MHAT, SGD>(d, t.row0, t.c0, t.c1, lane, E, Q, Ph, Mhat, sg);
  else if (d.vec == 2)
    recon_wave<R, 2, RESID, WRITE_MHAT, SGD>(d, t.row0, t.c0, t.c1, lane, E, Q, Ph, Mhat, sg);
  else
    recon_wave<R, 1, RESID, WRITE_MHAT, SGD>(d, t.row0, t.c0, t.c1, lane, E, Q, Ph, Mhat, sg);
}

// ---------------------------------------------------------------------------
// Pass-through tensors
// ---------------------------------------------------------------------------

template <bool MOM, bool GBF16>
__global__ __launch_bounds__(256) void k_pass_pack(const PassDesc* __restrict__ pass, const int32_t* __restrict__ map,
                                                   const void* __restrict__ G, float* __restrict__ U, float beta,
                                                   float* __restrict__ Pbuf) {
  pass_pack_wg<MOM, GBF16>(pass, map, blockIdx.x, G, U, beta, Pbuf);
}

template <bool SGD>
__global__ __launch_bounds__(256) void k_pass_unpack(const PassDesc* __restrict__ pass, const int32_t* __restrict__ map,
                                                     const float* __restrict__ Pbuf, float* __restrict__ out,
                                                     SgdArgs sg) {
  pass_unpack_wg<SGD>(pass, map, blockIdx.x, Pbuf, out, sg);
}

// Payload quantiser: every value rounded to the nearest bfloat16 (ties to
// even), kept in fp32 storage.  Adding 0x7fff plus the lowest kept bit to the
// fp32 pattern and clearing the low half rounds the magnitude to 8
// significant bits with ties to even (a carry moves into the exponent, which
// is the next binade).  Inf and NaN are left as they are.
__device__ __forceinline__ float round_bf16(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7f800000u) == 0x7f800000u) return x;
  return __uint_as_float((u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u);
}

__global__ __launch_bounds__(256) void k_round_bf16(float* __restrict__ buf, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  const int64_t n4 = n / 4;
  float4* b4 = reinterpret_cast<float4*>(buf);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
    float4 v = b4[i];
    v.x = round_bf16(v.x);
    v.y = round_bf16(v.y);
    v.z = round_bf16(v.z);
    v.w = round_bf16(v.w);
    b4[i] = v;
  }
  for (int64_t i = 4 * n4 + (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) buf[i] = round_bf16(buf[i]);
}

// ---------------------------------------------------------------------------
// Host-side launchers
// ---------------------------------------------------------------------------

template <int R, bool GBF16>
static hipError_t launch_ef_p_rg(const LaunchCtx& c, const GridRange& g, int mode, const void* G, float* E, float* U,
                                 float beta, const float* Q, float* P, int64_t p_fixed) {
  const int extra = c.pack_dst ? c.wg_pass : 0;
  if (g.count + extra == 0) return hipSuccess;
  const dim3 gr(g.count + extra), b(kWGThreads);
#define PSGD_EFP(MD)              \
  do {                            \
    if (c.stream_hint) {          \
      PSGD_EFP_NT(MD, true);      \
    } else {                      \
      PSGD_EFP_NT(MD, false);     \
    }                             \
  } while (0)
#define PSGD_EFP_NT(MD, NT_)                                                                                      \
  hipLaunchKernelGGL((k_ef_p<R, MD, GBF16, NT_>), gr, b, 0, c.stream, c.mats, c.rows_map, g.base, G, E, U, beta, Q, P, \
                     p_fixed, c.p_prev, static_cast<float*>(c.ppart), g.count, c.pass, c.pass_map, c.pack_dst)
  switch (mode) {
    case 1: PSGD_EFP(1); break;
    case 2: PSGD_EFP(2); break;
    case 3: PSGD_EFP(3); break;
    case 4: PSGD_EFP(4); break;
    case 5: PSGD_EFP(5); break;
    default: PSGD_EFP(6); break;
  }
#undef PSGD_EFP
#undef PSGD_EFP_NT
  return hipGetLastError();
}

template <int R>
static hipError_t launch_ef_p_r(const LaunchCtx& c, const GridRange& g, int mode, const void* G, float* E, float* U,
                                float beta, const float* Q, float* P, int64_t p_fixed) {
  if (mode == 0) {  // P = M Q with M read from E: no gradient involved, no packing
    if (g.count == 0) return hipSuccess;
    if (c.stream_hint)
      hipLaunchKernelGGL((k_ef_p<R, 0, false, true>), dim3(g.count), dim3(kWGThreads), 0, c.stream, c.mats,
                         c.rows_map, g.base, G, E, U, beta, Q, P, p_fixed, nullptr, static_cast<float*>(c.ppart),
                         g.count, c.pass, c.pass_map, nullptr);
    else
      hipLaunchKernelGGL((k_ef_p<R, 0, false, false>), dim3(g.count), dim3(kWGThreads), 0, c.stream, c.mats,
                         c.rows_map, g.base, G, E, U, beta, Q, P, p_fixed, nullptr, static_cast<float*>(c.ppart),
                         g.count, c.pass, c.pass_map, nullptr);
    return hipGetLastError();
  }
  return c.g_bf16 ? launch_ef_p_rg<R, true>(c, g, mode, G, E, U, beta, Q, P, p_fixed)
                  : launch_ef_p_rg<R, false>(c, g, mode, G, E, U, beta, Q, P, p_fixed);
}

template <int R>
static hipError_t launch_mtp_r(const LaunchCtx& c, const GridRange& g, const float* M, const float* Ph,
                               int64_t ph_fixed, float* Q) {
  if (g.count == 0) return hipSuccess;
  if (c.stream_hint)
    hipLaunchKernelGGL((k_mtp<R, true>), dim3(g.count), dim3(kWGThreads), 0, c.stream, c.mats, c.mtp_map, g.base, M,
                       Ph, ph_fixed, Q, c.part);
  else
    hipLaunchKernelGGL((k_mtp<R, false>), dim3(g.count), dim3(kWGThreads), 0, c.stream, c.mats, c.mtp_map, g.base, M,
                       Ph, ph_fixed, Q, c.part);
  return hipGetLastError();
}

template <int R>
static hipError_t launch_recon_r(const LaunchCtx& c, float* E, const float* Q, const float* Ph, float* Mhat,
                                 bool residual, const SgdArgs& sg, size_t lds) {
  const int extra = c.unpack_src ? c.wg_pass : 0;
  if (c.wg_rec + extra == 0) return hipSuccess;
  const dim3 g(c.wg_rec + extra), b(kWGThreads);
  const bool mh = Mhat != nullptr, sgd = sg.x != nullptr;
#define PSGD_RECON(RS, MH, SG)                                                                                  \
  hipLaunchKernelGGL((k_recon<R, RS, MH, SG>), g, b, lds, c.stream, c.mats, c.rec_map, E, Q, Ph, Mhat, sg, c.wg_rec, \
                     c.pass, c.pass_map, c.unpack_src)
  if (residual) {
    if (mh && sgd) PSGD_RECON(true, true, true);
    else if (mh) PSGD_RECON(true, true, false);
    else if (sgd) PSGD_RECON(true, false, true);
    else PSGD_RECON(true, false, false);
  } else {
    if (mh && sgd) PSGD_RECON(false, true, true);
    else if (mh) PSGD_RECON(false, true, false);
    else if (sgd) PSGD_RECON(false, false, true);
    else return hipSuccess;
  }
#undef PSGD_RECON
  return hipGetLastError();
}

#define PSGD_RANK_SWITCH(R_, CALL)  \
  switch (R_) {                     \
    case 1: { constexpr int RR = 1; return CALL; } \
    case 2: { constexpr int RR = 2; return CALL; } \
    case 3: { constexpr int RR = 3; return CALL; } \
    case 4: { constexpr int RR = 4; return CALL; } \
    case 5: { constexpr int RR = 5; return CALL; } \
    case 6: { constexpr int RR = 6; return CALL; } \
    case 7: { constexpr int RR = 7; return CALL; } \
    case 8: { constexpr int RR = 8; return CALL; } \
    default: return hipErrorInvalidValue;           \
  }

hipError_t launch_ef_p(const LaunchCtx& c, const GridRange& g, int mode, const void* G, float* E, float* U,
                       float beta, const float* Q, float* P, int64_t p_fixed) {
  PSGD_RANK_SWITCH(c.rank, launch_ef_p_r<RR>(c, g, mode, G, E, U, beta, Q, P, p_fixed));
}

hipError_t launch_mtp(const LaunchCtx& c, const GridRange& g, const float* M, const float* Ph, int64_t ph_fixed,
                      float* Q) {
  PSGD_RANK_SWITCH(c.rank, launch_mtp_r<RR>(c, g, M, Ph, ph_fixed, Q));
}

hipError_t launch_qreduce(const LaunchCtx& c, const GridRange& g, float* Q) {
  if (g.count == 0) return hipSuccess;
  hipLaunchKernelGGL(k_qreduce, dim3(g.count), dim3(64 * kRedWaves), 0, c.stream, c.mats, c.red_map, g.base, c.rank,
                     c.part, Q);
  return hipGetLastError();
}

// Without the plan's figure: the most any flat-tiled matrix can need.
hipError_t launch_recon(const LaunchCtx& c, float* E, const float* Q, const float* Ph, float* Mhat, bool residual,
                        const SgdArgs& sg) {
  PSGD_RANK_SWITCH(c.rank, launch_recon_r<RR>(c, E, Q, Ph, Mhat, residual, sg, (size_t)kFlatReconLdsMax));
}

hipError_t launch_recon_lds(const LaunchCtx& c, float* E, const float* Q, const float* Ph, float* Mhat,
                            bool residual, const SgdArgs& sg, size_t lds_bytes) {
  PSGD_RANK_SWITCH(c.rank, launch_recon_r<RR>(c, E, Q, Ph, Mhat, residual, sg, lds_bytes));
}

hipError_t launch_pass_pack(const LaunchCtx& c, const void* G, float* U, float beta, float* Pbuf) {
  if (c.wg_pass == 0) return hipSuccess;
  const dim3 g(c.wg_pass), b(256);
  if (U && c.g_bf16)
    hipLaunchKernelGGL((k_pass_pack<true, true>), g, b, 0, c.stream, c.pass, c.pass_map, G, U, beta, Pbuf);
  else if (U)
    hipLaunchKernelGGL((k_pass_pack<true, false>), g, b, 0, c.stream, c.pass, c.pass_map, G, U, beta, Pbuf);
  else if (c.g_bf16)
    hipLaunchKernelGGL((k_pass_pack<false, true>), g, b, 0, c.stream, c.pass, c.pass_map, G, U, beta, Pbuf);
  else
    hipLaunchKernelGGL((k_pass_pack<false, false>), g, b, 0, c.stream, c.pass, c.pass_map, G, U, beta, Pbuf);
  return hipGetLastError();
}

hipError_t launch_pass_unpack(const LaunchCtx& c, const float* Pbuf, float* out, const SgdArgs& sg) {
  if (c.wg_pass == 0 || (!out && !sg.x)) return hipSuccess;
  if (sg.x)
    hipLaunchKernelGGL((k_pass_unpack<true>), dim3(c.wg_pass), dim3(256), 0, c.stream, c.pass, c.pass_map, Pbuf, out,
                       sg);
  else
    hipLaunchKernelGGL((k_pass_unpack<false>), dim3(c.wg_pass), dim3(256), 0, c.stream, c.pass, c.pass_map, Pbuf, out,
                       sg);
  return hipGetLastError();
}

hipError_t launch_round_bf16(float* buf, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n / 4 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_round_bf16, dim3((unsigned)blocks), dim3(256), 0, stream, buf, n);
  return hipGetLastError();
}

}  // namespace psgd
