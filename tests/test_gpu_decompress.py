"""Standalone decompression (psgd_decompress) against the fp64 oracle.

The receiver's whole job is the product of the two transmitted factors,
M_hat = P_hat Q^T (glossary entry "PowerSGD", factorisation paragraph), plus
the pass-through tensors copied out of the P buffer.  After compress steps on
the GPU, psgd_decompress writes into a fresh buffer (filled with a sentinel)
and is compared with
  * oracle.decompress of the oracle's own P_hat and Q for the same inputs
    (relative Frobenius error <= 1e-4 per matrix), and
  * oracle.decompress of the GPU's P_hat and Q, upcast (the product alone:
    one fp32 rounding per term, <= 1e-6),
with every pass-through value exact and nothing outside the tensors written.
Ranks 2 and 4 take the vector path, 16 and 64 the matrix-core one (tiles with
ragged row and column tails)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle  # noqa: E402
import workloads as W  # noqa: E402
from gpu_util import REL_TOL, cpu, rel, say  # noqa: E402
from rank_gradient_compression_amd.torch_api import PowerSGD  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

SHAPES = [(300, 650), (257, 1030), (5,), (97, 1030), (33, 27), (1000, 1), (70, 130), (640, 512), (3, 3)]
SENTINEL = -7.25


@pytest.mark.parametrize("rank", [2, 4, 16, 64])
def test_decompress_matches_oracle(rank):
    tensors = [(str(i), s) for i, s in enumerate(SHAPES)]
    wl = W.ModelSetWorkload(tensors, "plain", seed=400 + rank)
    ps = PowerSGD(SHAPES, rank, device=DEV)
    oplan = oracle.Plan(SHAPES, rank)
    kinds = oplan.kinds
    assert sum(k == oracle.KIND_COMPRESSED for k in kinds) >= 3
    assert sum(k != oracle.KIND_COMPRESSED for k in kinds) >= 3
    q0 = [wl.q0(i, rank) if kinds[i] == oracle.KIND_COMPRESSED else None for i in range(len(SHAPES))]
    ost = oracle.init_state(oplan, q0)
    for i in ps.compressed():
        ps.set_q(i, q0[i])
    covered = torch.zeros(ps.info["flat_elems"], dtype=torch.bool)
    for i in range(len(SHAPES)):
        _, off, _, _ = ps.tensors[i]
        covered[off: off + int(np.prod(SHAPES[i]))] = True
    for t in (1, 2):
        grads = [wl.grad(i, t) for i in range(len(SHAPES))]
        for i, g in enumerate(grads):
            ps.view(ps.grads, i).copy_(torch.from_numpy(g).to(DEV))
        say(f"[decompress r={rank}] step {t}: compress, then decompress into a fresh buffer")
        ps.compress(mhat=False)
        out = torch.full_like(ps.err, SENTINEL)
        ps.decompress(out)
        torch.cuda.synchronize()
        res = oracle.step_set(oplan, grads, ost)
        worst = 0.0
        for i in range(len(SHAPES)):
            got = cpu(ps.view(out, i))
            if kinds[i] == oracle.KIND_COMPRESSED:
                want = oracle.decompress(res.P_hat[i], res.Q[i])
                e = rel(got, want)
                assert e <= REL_TOL, f"r={rank} step {t} tensor {i} {SHAPES[i]}: rel err {e:.3e} against the oracle"
                own = oracle.decompress(cpu(ps.p_hat(i)), cpu(ps.q_of(i)))
                e2 = rel(got, own)
                assert e2 <= 1e-6, f"r={rank} step {t} tensor {i}: product of the GPU's factors, rel err {e2:.3e}"
                worst = max(worst, e)
            else:
                # pass-through: the value sent, bit for bit
                assert np.array_equal(got.reshape(-1), grads[i].astype(np.float32).reshape(-1).astype(np.float64)), \
                    f"r={rank} step {t} pass-through tensor {i}"
        # nothing outside the tensors (the alignment gaps) was written
        assert torch.all(out.cpu()[~covered] == SENTINEL)
        say(f"[decompress r={rank}] step {t}: worst rel err against the oracle {worst:.2e}")
    ps.close()
