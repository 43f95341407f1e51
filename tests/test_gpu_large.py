"""Largest sizes: one matrix of more than 2^31 elements (32768 x 65600), so
every flat index past row 32736 needs 64-bit arithmetic, on the vector-ALU
and the matrix-core paths.  The oracle's quantities are computed in fp64
over row chunks copied from the device: P = G Q0 and Q = G^T P_hat in full
(P_hat by the oracle's Gram-Schmidt), E and M_hat on sampled rows, including
the rows on both sides of element 2^31."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle  # noqa: E402
import workloads as W  # noqa: E402
from gpu_util import ORTH_TOL, REL_TOL, cpu, rel, say  # noqa: E402
from rank_gradient_compression_amd.torch_api import PowerSGD  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
M_ROWS, N_COLS = 32768, 65600  # 2,149,580,800 elements
CHUNK = 2048


@pytest.mark.parametrize("rank", [4, 16, 64])
def test_matrix_beyond_2_31_elements(rank):
    m, n = M_ROWS, N_COLS
    assert m * n > 2 ** 31
    say(f"[large r={rank}] allocating {m}x{n}")
    ps = PowerSGD([(m, n)], rank, device=DEV)
    try:
        G = ps.view(ps.grads, 0)
        W.llama7b_grad_(G, m, n, 0, step=1, seed=9)
        q0 = W.gaussian_q0(n, rank, 9).astype(np.float64)
        ps.set_q(0, q0)
        torch.cuda.synchronize()
        say(f"[large r={rank}] compress")
        ps.compress(mhat=True)
        torch.cuda.synchronize()

        say(f"[large r={rank}] oracle P = G Q0 over row chunks")
        P = np.concatenate([cpu(G[a:a + CHUNK]) @ q0 for a in range(0, m, CHUNK)])
        Ph = oracle.gram_schmidt(P)
        say(f"[large r={rank}] oracle Q = G^T P_hat over row chunks")
        Qo = np.zeros((n, rank))
        for a in range(0, m, CHUNK):
            Qo += cpu(G[a:a + CHUNK]).T @ Ph[a:a + CHUNK]

        Ph_gpu = cpu(ps.p_hat(0))
        orth = oracle.orthonormality_error(Ph_gpu)
        e_p, e_q = rel(Ph_gpu, Ph), rel(cpu(ps.q_of(0)), Qo)
        say(f"[large r={rank}] P_hat {e_p:.2e}  Q {e_q:.2e}  orth {orth:.2e}")
        assert orth <= ORTH_TOL and e_p <= REL_TOL and e_q <= REL_TOL

        g = np.random.default_rng(9)
        rows = sorted(set([0, 1, 2 ** 31 // n - 1, 2 ** 31 // n, 2 ** 31 // n + 1, m - 1]
                          + list(g.integers(0, m, 26))))
        idx = torch.tensor(rows, device=DEV)
        Gs, Es, Mh = (cpu(buf.index_select(0, idx)) for buf in (G, ps.view(ps.err, 0), ps.view(ps.mhat, 0)))
        Mh_o = Ph[rows] @ Qo.T
        e_e, e_m = rel(Es, Gs - Mh_o), rel(Mh, Mh_o)
        say(f"[large r={rank}] sampled rows {len(rows)}: E {e_e:.2e}  M_hat {e_m:.2e}")
        assert e_e <= REL_TOL and e_m <= REL_TOL
    finally:
        ps.close()
        del ps
        torch.cuda.empty_cache()
