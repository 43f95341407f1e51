// Flat tiling of the vector-path residual / decompression pass (host and
// device declarations).
//
// A matrix whose rows do not start on 128-byte lines (row length not a
// multiple of 32 floats) makes every row-contiguous 1 KB store of a
// wavefront cover two partly written lines; the passes that write two
// arrays then stream far below their bandwidth (33278 x 650 at rank 4:
// 68 us against 41 us for 33278 x 640).  Such matrices are tiled flat
// instead: workgroup w of the matrix covers the elements [w * G,
// (w + 1) * G) of its row-major storage, G = S * kFlatChunk with S pieces
// (1 to kFlatSub: more where staging Q costs more per piece), whose start is line
// aligned, and each element's row and column are computed from its index.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "psgd_kernels.h"

namespace psgd {

constexpr int kFlatChunk = 8192;  // elements per piece (256 threads x 8 float4)
constexpr int kFlatSub = 4;       // most pieces per workgroup, on one staging of Q and P_hat rows
constexpr int kFlatQMax = 8192;   // largest n * flat_rq(r) staged in LDS (floats)
constexpr int kFlatMinCols = 64;  // shorter rows keep the row tiles
// Q and P_hat rows staged in LDS with the rank padded to 4 or 8 floats.
constexpr int flat_rq(int r) { return r <= 4 ? 4 : 8; }
// The most dynamic LDS a flat-tiled residual pass needs: Q (n * rq <=
// kFlatQMax floats) and the P_hat rows one workgroup can touch (at most
// kFlatSub * kFlatChunk / kFlatMinCols + 2 rows of 8 floats).
constexpr int kFlatReconLdsMax = (kFlatQMax + (kFlatSub * kFlatChunk / kFlatMinCols + 2) * 8) * 4;

// The residual / decompression pass as launch_recon, with lds_bytes of
// dynamic LDS for the flat-tiled matrices (0 when the plan has none).
hipError_t launch_recon_lds(const LaunchCtx& c, float* E, const float* Q, const float* Ph, float* Mhat,
                            bool residual, const SgdArgs& sg, size_t lds_bytes);

}  // namespace psgd
