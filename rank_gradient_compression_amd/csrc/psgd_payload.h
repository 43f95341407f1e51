// Quantisers of the transmitted factors beyond bfloat16 (host declarations).
#pragma once

#include <hip/hip_runtime.h>

#include "psgd_kernels.h"

namespace psgd {

// Round every column of the factors of descriptors first + [0, nmat) (rank
// columns of `rows` floats at base + off, the orthonormalisation descriptors'
// layout) to E4M3 values times the column's power-of-two scale, in place.
hipError_t launch_round_fp8_cols(const LaunchCtx& c, int first, float* base);

}  // namespace psgd
