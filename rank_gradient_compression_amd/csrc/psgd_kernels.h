// Kernel launchers of the PowerSGD library (host declarations).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "psgd_tables.h"

namespace psgd {

// Relative threshold under which a Gram-Schmidt column counts as dependent
// and is set to zero.
constexpr float kZeroColumnRel = 1e-4f;

// Device table pointers (inside an initialised workspace) and grid sizes of
// one plan, plus the stream every launch goes to.
struct LaunchCtx {
  hipStream_t stream;
  int rank;
  int nmat, npass;
  int wg_rows, wg_mtp, wg_red, wg_pass;
  const MatDesc* mats;
  const PassDesc* pass;
  const int32_t* rows_map;
  const int32_t* mtp_map;
  const int32_t* red_map;
  const int32_t* pass_map;
  float* part;    // partial-Q scratch
  double* gram;   // orthonormalisation scratch
  float* rscr;    // refresh scratch
};

hipError_t launch_ef_p(const LaunchCtx& c, const float* G, float* E, float* U, float beta, const float* Q, float* P);
hipError_t launch_orth(const LaunchCtx& c, float* P);
hipError_t launch_mtp(const LaunchCtx& c, const float* M, const float* Ph, float* Q, float* part);
hipError_t launch_qreduce(const LaunchCtx& c, const float* part, float* Q);
// residual = true: E <- M - P_hat Q^T (M read from E), M_hat written if non-null.
// residual = false: Mhat <- P_hat Q^T only (decompression).
hipError_t launch_recon(const LaunchCtx& c, float* E, const float* Q, const float* Ph, float* Mhat, bool residual);
hipError_t launch_pass_pack(const LaunchCtx& c, const float* G, float* U, float beta, float* Pbuf);
hipError_t launch_pass_unpack(const LaunchCtx& c, const float* Pbuf, float* out);
hipError_t launch_stream_copy(float* dst, const float* src, size_t n, hipStream_t stream);

}  // namespace psgd
