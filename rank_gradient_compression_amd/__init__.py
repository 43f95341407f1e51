"""PowerSGD gradient compression for AMD Instinct MI355X (gfx950).

The compute path is libpsgd.so (hand-written HIP kernels behind the C ABI of
include/psgd.h); `binding` exposes it with the same names, and `torch_api`
holds a thin buffer-owning convenience layer over PyTorch device memory.
"""
from . import binding  # noqa: F401  (loads libpsgd.so; raises if it is not built)
from .binding import (PSGD_FLAG_GRADS_BF16, PSGD_FLAG_MOMENTUM, PSGD_KIND_COMPRESSED,  # noqa: F401
                      PSGD_KIND_PASSTHRU, PSGD_KIND_VECTOR, PSGD_STEP_DEFER_RESIDUAL, PSGD_STEP_NESTEROV,
                      PSGD_STEP_NO_ERROR_FEEDBACK, PSGD_STEP_PAYLOAD_BF16, PSGD_STEP_PAYLOAD_FP8,
                      PSGD_STEP_RESIDUAL_DEFERRED,
                      PsgdError, psgd_compress, psgd_compress_noalloc, psgd_decompress, psgd_init_q, psgd_last_error, psgd_plan_create,
                      psgd_plan_destroy, psgd_plan_get_info, psgd_plan_tensor, psgd_refresh, psgd_stream_copy,
                      psgd_step_stats, psgd_stream_probe, psgd_subspace_overlap,
                      psgd_timing_enable, psgd_timing_read, psgd_timing_stages, psgd_version, psgd_workspace_init,
                      step_opts)

__all__ = [n for n in dir() if n.startswith("psgd_") or n.startswith("PSGD_")] + ["PsgdError", "binding"]
