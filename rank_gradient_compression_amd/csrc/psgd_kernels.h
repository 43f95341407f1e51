// Kernel launchers of the PowerSGD library (host declarations).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "psgd_tables.h"

namespace psgd {

// A set whose compressed matrices hold more bytes than this streams through
// the caches whatever the access hints; smaller ones can stay in the 256 MB
// last-level cache from one pass to the next.
constexpr int64_t kStreamHintBytes = int64_t(1) << 30;

// Relative threshold under which a Gram-Schmidt column counts as dependent
// and is set to zero.
constexpr float kZeroColumnRel = 1e-4f;

// Device table pointers (inside an initialised workspace) and grid sizes of
// one plan, plus the stream every launch goes to.
struct LaunchCtx {
  hipStream_t stream;
  int rank, rank_pad;
  bool mfma;
  bool g_bf16;  // gradients stored as bfloat16
  bool stream_hint;  // the compressed matrices exceed kStreamHintBytes: read M non-temporally where it pays
  const float* p_prev;  // deferred residual: the previous step's P_hat (plan offsets)
  int nmat, npass;
  int wg_rows, wg_rec, wg_mtp, wg_red, wg_pass, wg_pred, wg_gram, wg_gramq;
  int wg_rows_v4;  // matrix cores: the pass-1 grid's 16-byte-row part is [0, wg_rows_v4)
  const MatDesc* mats;
  const PassDesc* pass;
  const OrthDesc* orth;
  const int32_t* rows_map;  // pass-1 row tiles
  const int32_t* rec_map;   // residual / decompression pass row tiles
  const int32_t* mtp_map;
  const int32_t* red_map;
  const int32_t* pass_map;
  const int32_t* pred_map;
  const int32_t* gram_map;
  const int32_t* gramq_map;
  float* part;    // partial-Q scratch
  void* ppart;    // partial-P scratch (column splits of pass 1): fp32 on the
                  // vector path, fp64 on the matrix cores
  // Vector-ALU path: the pass-through packing runs as extra workgroups of
  // the pass-1 launch (into pack_dst, when non-null) and the unpacking as
  // extra workgroups of the residual-pass launch (from unpack_src).
  float* pack_dst;
  const float* unpack_src;
  double* gram;   // orthonormalisation scratch
  float* rscr;    // refresh scratch
};

// Fused post-compression momentum SGD (x = parameters, m = momentum buffer,
// flat plan layout); x == nullptr disables it.
struct SgdArgs {
  float* x;
  float* m;
  float lr;
  float mu;
  int nesterov;  // step along D + mu m instead of m
};

// A contiguous range of workgroups of one of the plan's grids (the whole grid
// for the grouped launches, one matrix's workgroups inside the refresh).
struct GridRange {
  int base;
  int count;
};

// ---- ranks up to kValuMaxRank (vector ALU kernels)
// mode 0: P = M Q with M read from E; 1: M = G + E stored over E; 2: also
// u = beta u + G first (M = u + E); 3: M = G; 4: u = beta u + G, M = u
// (3 and 4: no error feedback); 5 and 6: as 1 and 2 with E formed from a
// deferred residual, E = E_in - p_prev Q^T (also in launch_mfma_p).
// p_fixed >= 0 replaces the plan's P offset.
hipError_t launch_ef_p(const LaunchCtx& c, const GridRange& g, int mode, const void* G, float* E, float* U,
                       float beta, const float* Q, float* P, int64_t p_fixed);
hipError_t launch_mtp(const LaunchCtx& c, const GridRange& g, const float* M, const float* Ph, int64_t ph_fixed,
                      float* Q);
// residual = true: E <- M - P_hat Q^T (M read from E); residual = false:
// decompression only.  M_hat written if non-null; fused SGD if sg.x.
hipError_t launch_recon(const LaunchCtx& c, float* E, const float* Q, const float* Ph, float* Mhat, bool residual,
                        const SgdArgs& sg);

// ---- ranks above kValuMaxRank (matrix-core kernels)
hipError_t launch_mfma_p(const LaunchCtx& c, const GridRange& g, int mode, const void* G, float* E, float* U,
                         float beta, const float* Q, float* P, int64_t p_fixed);
hipError_t launch_psum(const LaunchCtx& c, const GridRange& g, float* P, int64_t p_fixed);
hipError_t launch_mfma_qt(const LaunchCtx& c, const GridRange& g, const float* M, const float* Ph, int64_t ph_fixed,
                          float* Q);
hipError_t launch_mfma_recon(const LaunchCtx& c, float* E, const float* Q, const float* Ph, float* Mhat,
                             bool residual, const SgdArgs& sg);
// With a map: descriptors first + [0, count) over a grouped Gram grid of
// nblocks workgroups (map gives the matrix of each workgroup).  Without: the
// single descriptor `first` with nblocks Gram blocks.  zcount (nullable)
// receives, per descriptor, the number of columns set to zero.
hipError_t launch_gram_orth(const LaunchCtx& c, int first, int count, const int32_t* map, int nblocks,
                            float* base, int32_t* zcount = nullptr);

// Block partials (RP x RP doubles each, at the descriptors' Gram offsets)
// summed into the T slots: descriptors first + [0, count).
hipError_t launch_gram_reduce(const LaunchCtx& c, int first, int count);

// ---- diagnostics (outside the step)
// out[2k], out[2k + 1] = ||E_k||^2, ||M_hat_k + E_k||^2 for matrix k (fp64),
// from kStatsWGs partial sums per matrix in its Gram scratch.
constexpr int kStatsWGs = 64;
hipError_t launch_sumsq(const LaunchCtx& c, const float* E, const float* Mh, double* out);
// out[k] = mean cosine of the principal angles between the spans of two
// orthonormalised factors laid out as the Q buffer (descriptors first + k).
constexpr int kJacobiSweeps = 12;
hipError_t launch_overlap(const LaunchCtx& c, int first, const float* a, const float* b, double* out);

// ---- shared
hipError_t launch_qreduce(const LaunchCtx& c, const GridRange& g, float* Q);
hipError_t launch_pass_pack(const LaunchCtx& c, const void* G, float* U, float beta, float* Pbuf);
hipError_t launch_pass_unpack(const LaunchCtx& c, const float* Pbuf, float* out, const SgdArgs& sg);
// Seeded N(0, 1) start Q of every compressed tensor (max_blocks: the largest
// ceil(n * rank / 4) over the matrices).
hipError_t launch_init_q(const LaunchCtx& c, float* Q, uint64_t seed, int64_t max_blocks);

// Round n floats (16-byte aligned) to bfloat16 values in place.
hipError_t launch_round_bf16(float* buf, int64_t n, hipStream_t stream);

hipError_t launch_stream_copy(float* dst, const float* src, size_t n, hipStream_t stream);

// Streaming-bandwidth probe (psgd_stream_probe): up to 3 inputs, 2 outputs,
// n4 16-byte vectors each; without outputs each wavefront adds its sum into
// one of the sink's kProbeSinkFloats floats.  The copy moves kStreamUnroll
// vectors per thread and grid step on at most kCopyMaxBlocks workgroups.
constexpr int kStreamUnroll = 8;
constexpr int kProbeSinkFloats = 16384;
constexpr int kCopyMaxBlocks = 16384;
struct ProbeArgs {
  const float4* in[3];
  float4* out[2];
  float* sink;
  int64_t n4;
};
hipError_t launch_stream_probe(const ProbeArgs& a, int nin, int nout, hipStream_t stream);

}  // namespace psgd
