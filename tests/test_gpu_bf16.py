"""Parity with bfloat16 gradients as input (PSGD_FLAG_GRADS_BF16): the kernels
widen each bfloat16 value exactly to fp32 on load, so the oracle, given the
same rounded values in fp64, is held to the fp32 tolerances."""
import functools

import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import workloads as W  # noqa: E402
from test_gpu_parity import run_set_parity  # noqa: E402

pytestmark = pytest.mark.gpu
BF16 = torch.bfloat16

RAGGED = [(300, 650), (257, 4099), (97, 1030), (33, 27), (1000, 1), (5,), (640, 4096), (70, 130), (2, 2)]


@pytest.mark.parametrize("rank", [1, 4, 7, 16, 64])
def test_bf16_ragged_shapes(rank):
    tensors = [(str(i), s) for i, s in enumerate(RAGGED)]
    wl = W.ModelSetWorkload(tensors, "plain", seed=110 + rank)
    run_set_parity(tensors, rank, 2, wl.grad, lambda i: wl.q0(i, rank), grads_dtype=BF16, tag=f"bf16 r={rank}")


@pytest.mark.parametrize("rank", [4, 32])
def test_bf16_momentum_odd_offsets(rank):
    # odd element offsets force the narrow (1- and 2-element) load paths
    shapes = [(300, 512), (200, 650), (13,)]
    offsets = [1, 300 * 512 + 3, 300 * 512 + 3 + 200 * 650 + 2]
    tensors = [(str(i), s) for i, s in enumerate(shapes)]
    wl = W.ModelSetWorkload(tensors, "plain", seed=120 + rank)
    run_set_parity(tensors, rank, 3, wl.grad, lambda i: wl.q0(i, rank), beta=0.9, offsets=offsets,
                   grads_dtype=BF16, tag=f"bf16 momentum offsets r={rank}")


@pytest.mark.parametrize("rank,beta", [(4, None), (16, 0.9)])
def test_bf16_no_error_feedback_power_iterations(rank, beta):
    shapes = [(300, 650), (400, 512), (9,)]
    tensors = [(str(i), s) for i, s in enumerate(shapes)]
    wl = W.ModelSetWorkload(tensors, "plain", seed=130 + rank)
    run_set_parity(tensors, rank, 2, wl.grad, lambda i: wl.q0(i, rank), beta=beta, grads_dtype=BF16,
                   power_iters=2, error_feedback=False, tag=f"bf16 no-EF x2 r={rank}")


@functools.lru_cache(maxsize=1)
def _sweep_matrix():
    return W.decaying_spectrum_matrix(11008, 4096, seed=5)


@pytest.mark.parametrize("rank", [4, 32])
def test_bf16_11008x4096(rank):
    A, _, _ = _sweep_matrix()
    q0 = W.gaussian_q0(4096, rank, 5)
    run_set_parity([("A", (11008, 4096))], rank, 2, lambda i, t: A, lambda i: q0, grads_dtype=BF16,
                   tag=f"bf16 11008x4096 r={rank}")
