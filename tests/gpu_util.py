"""Helpers shared by the GPU tests: run the HIP path and the fp64 oracle on the
same seeded inputs and compare per matrix."""
from __future__ import annotations

import sys

import numpy as np

import oracle

REL_TOL = 1e-4     # relative Frobenius error on P_hat, Q, E (and M_hat)
ORTH_TOL = 1e-5    # ||P_hat^T P_hat - I||_F over the non-zero columns


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    if nb == 0.0:
        return float(np.linalg.norm(a))
    return float(np.linalg.norm(a - b) / nb)


def cpu(t) -> np.ndarray:
    return t.detach().to("cpu").double().numpy()


def compare_set(ps, oplan, ores, ostate, idx=None, mhat=True, tol=REL_TOL, tag="", check_e=True):
    """Compare the GPU buffers of `ps` against one oracle step result."""
    import rank_gradient_compression_amd.binding as B

    idx = range(len(oplan.shapes)) if idx is None else idx
    worst = {}
    for i in idx:
        if oplan.kinds[i] == oracle.KIND_COMPRESSED:
            Ph = cpu(ps.p_hat(i))
            errs = {"P_hat": rel(Ph, ores.P_hat[i]), "Q": rel(cpu(ps.q_of(i)), ores.Q[i])}
            if check_e:
                errs["E"] = rel(cpu(ps.view(ps.err, i)), ostate.E[i])
            if mhat:
                errs["M_hat"] = rel(cpu(ps.view(ps.mhat, i)), ores.M_hat[i])
            orth = oracle.orthonormality_error(Ph)
            assert orth <= ORTH_TOL, f"{tag} tensor {i}: orthonormality {orth:.3e}"
            for k, v in errs.items():
                assert v <= tol, f"{tag} tensor {i} {ps.shapes[i]}: {k} rel err {v:.3e}"
                worst[k] = max(worst.get(k, 0.0), v)
        else:
            if mhat:
                got = cpu(ps.view(ps.mhat, i)).reshape(-1)
                want = np.asarray(ores.M_hat[i]).reshape(-1)
                e = rel(got, want)
                assert e <= 1e-6, f"{tag} pass-through tensor {i}: rel err {e:.3e}"
            kind, _, poff, _ = ps.tensors[i]
            assert kind != B.PSGD_KIND_COMPRESSED
    return worst
