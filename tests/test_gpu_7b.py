"""Full-size parity on the 7B-shaped gradient set (226 matrices, 6.74e9
elements), in the launch configurations the benchmark times: one grouped
psgd_compress over the whole set with the fused decompression -- plain,
compressing momentum, with the residual deferred into the next step, and with
bfloat16 gradients.  The oracle checks sampled matrices one by one (their
gradients are copied from the device generator, or from the bfloat16 buffer),
free-running over the steps."""
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
RANK = 4
# embed, layer-0 q / gate / down, layer-31 v, head
SAMPLE = [0, 1, 5, 7, 1 + 31 * 7 + 2, 225]


def fill(ps, tensors, step):
    if ps.grads.dtype == torch.float32:
        for i, (_, s) in enumerate(tensors):
            W.llama7b_grad_(ps.view(ps.grads, i), s[0], s[1], i, step=step)
        return
    for i, (_, s) in enumerate(tensors):
        tmp = torch.empty(s, dtype=torch.float32, device=DEV)
        W.llama7b_grad_(tmp, s[0], s[1], i, step=step)
        ps.view(ps.grads, i).copy_(tmp)
        del tmp


@pytest.mark.parametrize("mode", ["plain", "momentum", "deferred", "bf16"])
def test_7b_set_sampled_parity(mode):
    beta = 0.9 if mode == "momentum" else None
    deferred = mode == "deferred"
    steps = (1, 2, 3) if deferred else (1, 2)
    tensors = W.llama7b_set()
    shapes = [s for _, s in tensors]
    say(f"[7b {mode}] allocating the full set")
    ps = PowerSGD(shapes, RANK, device=DEV, momentum_beta=beta,
                  grads_dtype=torch.bfloat16 if mode == "bf16" else torch.float32)
    q0 = {}
    for i, (_, s) in enumerate(tensors):
        q = W.llama7b_q0(s[1], RANK, i, device=DEV)
        ps.set_q(i, q)
        if i in SAMPLE:
            q0[i] = q.cpu().numpy()
    E = {i: np.zeros(shapes[i]) for i in SAMPLE}
    Qw = {i: q0[i].astype(np.float64) for i in SAMPLE}
    U = {i: np.zeros(shapes[i]) for i in SAMPLE}
    try:
        for step in steps:
            say(f"[7b {mode}] step {step}: generate + compress")
            fill(ps, tensors, step)
            torch.cuda.synchronize()
            G = {i: cpu(ps.view(ps.grads, i)) for i in SAMPLE}
            # deferred: defer at every step but the last, which ends with an explicit E
            defer_out = deferred and step != steps[-1]
            ps.compress(mhat=True, defer_residual=defer_out, residual_deferred=deferred and step > 1)
            torch.cuda.synchronize()
            for i in SAMPLE:
                X = G[i]
                if beta is not None:
                    U[i] = oracle.momentum_input(U[i], G[i], beta)
                    X = U[i]
                M = X + E[i]
                res = oracle.compress_matrix(M, Qw[i])
                E[i], Qw[i] = res.E, res.Q
                Ph = cpu(ps.p_hat(i))
                errs = {"P_hat": rel(Ph, res.P_hat), "Q": rel(cpu(ps.q_of(i)), res.Q),
                        "M_hat": rel(cpu(ps.view(ps.mhat, i)), res.M_hat)}
                if defer_out:
                    errs["M (err buffer)"] = rel(cpu(ps.view(ps.err, i)), M)
                else:
                    errs["E"] = rel(cpu(ps.view(ps.err, i)), res.E)
                if beta is not None:
                    errs["u"] = rel(cpu(ps.view(ps.mom, i)), U[i])
                orth = oracle.orthonormality_error(Ph)
                say(f"[7b {mode}] step {step} {tensors[i][0]} {shapes[i]}: "
                    + " ".join(f"{k}={v:.2e}" for k, v in errs.items()) + f" orth={orth:.2e}")
                assert orth <= ORTH_TOL
                for k, v in errs.items():
                    assert v <= REL_TOL, (i, k, v)
    finally:
        ps.close()
        del ps
        torch.cuda.empty_cache()
