"""fp64 reference oracle for the PowerSGD compression step (test
infrastructure: imported only by tests, the smoke entry and the benchmark's
CPU-baseline leg)."""
from .powersgd import *  # noqa: F401,F403
from .powersgd import (KIND_COMPRESSED, KIND_PASSTHRU, KIND_VECTOR, Plan, SetResult, SetState,  # noqa: F401
                       ZERO_COLUMN_REL, classify, compress_matrix, compress_workers, decompress,
                       compression_error, gram_schmidt, init_state, matrix_view, momentum_input, orthonormality_error,
                       principal_angle_sines, refresh, round_bf16, sgd_momentum_step, step_set, subspace_overlap,
                       FP8_E4M3_MAX, fp8_column_exponent, round_fp8_columns, round_fp8_e4m3)
from .philox import init_q, init_q_set, normal_stream, philox4x64  # noqa: F401
