"""psgd_init_q (seeded N(0, 1) start Q) against the oracle's Philox-4x64-10 +
Box-Muller stream, and the cold-start ablation (a fresh seeded Q every step)
against the oracle's step from the same Q."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle  # noqa: E402
import workloads as W  # noqa: E402
from gpu_util import compare_set, cpu, say  # noqa: E402
from rank_gradient_compression_amd.torch_api import PowerSGD  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

SHAPES = [(300, 650), (257, 4099), (5,), (33, 27), (1000, 1), (97, 1031), (2, 2), (64, 3, 3, 3)]


def _check_q(ps, oplan, seed, tag):
    want = oracle.init_q_set(oplan, seed)
    for i in ps.compressed():
        got = cpu(ps.q_of(i))
        w = want[i]
        # fp64 transform on both sides, one rounding to fp32: at most 1 ulp apart
        ulp = np.spacing(np.abs(w).astype(np.float32)).astype(np.float64)
        err = np.abs(got - w)
        assert np.all(err <= ulp), f"{tag} tensor {i}: max |diff| {err.max():.3e}"
        say(f"[{tag}] tensor {i} {ps.shapes[i]}: max |GPU - oracle| = {err.max():.2e}")


@pytest.mark.parametrize("rank", [1, 4, 7, 32, 64])
def test_init_q_matches_oracle(rank):
    ps = PowerSGD(SHAPES, rank, device=DEV, with_mhat=False)
    oplan = oracle.Plan(SHAPES, rank)
    ps.q.fill_(123.0)
    ps.init_q(2024 + rank)
    torch.cuda.synchronize()
    _check_q(ps, oplan, 2024 + rank, f"init_q r={rank}")
    # padding between the packed factors is left alone
    covered = torch.zeros_like(ps.q, dtype=torch.bool)
    for i in ps.compressed():
        _, _, _, qoff = ps.tensors[i]
        covered[qoff: qoff + rank * ps.views[i][1]] = True
    assert torch.all(ps.q[~covered] == 123.0)


def test_init_q_large_seed_and_repeat():
    ps = PowerSGD([(4096, 11008), (11008, 4096)], 4, device=DEV, with_mhat=False)
    oplan = oracle.Plan([(4096, 11008), (11008, 4096)], 4)
    seed = (1 << 64) - 3
    ps.init_q(seed)
    torch.cuda.synchronize()
    first = ps.q.clone()
    ps.init_q(seed)
    torch.cuda.synchronize()
    assert torch.equal(first, ps.q)
    _check_q(ps, oplan, seed, "init_q 7B shapes")


@pytest.mark.parametrize("rank", [2, 16])
def test_cold_start_steps(rank):
    shapes = [(300, 650), (400, 512), (9,)]
    tensors = [(str(i), s) for i, s in enumerate(shapes)]
    wl = W.ModelSetWorkload(tensors, "resnet18", seed=140 + rank)
    ps = PowerSGD(shapes, rank, device=DEV)
    oplan = oracle.Plan(shapes, rank)
    ost = oracle.init_state(oplan, oracle.init_q_set(oplan, 1000))
    for t in range(1, 4):
        grads = [wl.grad(i, t) for i in range(len(shapes))]
        for i, g in enumerate(grads):
            ps.view(ps.grads, i).copy_(torch.from_numpy(g).to(DEV))
        ps.init_q(1000 + t)
        ost.Q = oracle.init_q_set(oplan, 1000 + t)
        say(f"[cold start r={rank}] step {t}")
        ps.compress(mhat=True)
        torch.cuda.synchronize()
        res = oracle.step_set(oplan, grads, ost)
        compare_set(ps, oplan, res, ost, tag=f"cold start r={rank} step {t}")
