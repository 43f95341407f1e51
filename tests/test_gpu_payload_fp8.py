"""fp8 payload (PSGD_STEP_PAYLOAD_FP8) against the oracle's quantiser.

Each column of each factor is rounded to E4M3 values times a power of two
chosen from the column's largest magnitude.  Both the exponent and the
rounded values are decided by floating point: the GPU sums in fp32, the
oracle in fp64, so a column maximum next to 448 * 2^k, or a value next to a
rounding midpoint, can go either way.  Each factor the hook receives is
therefore checked as a valid rounding: every column on the E4M3 grid of one
exponent (the oracle's, or one next to it when the oracle's column maximum
lies within the fp32 accumulation error of that boundary), and every value
within half an E4M3 step of a value inside the fp32 accumulation error of
the oracle's exact one.  The oracle then continues from the factors the GPU
sent (teacher forcing at the hooks, what an aggregation hands every worker),
and P_hat, E and M_hat are compared to the usual tolerance.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle  # noqa: E402
import workloads as W  # noqa: E402
from gpu_util import ORTH_TOL, REL_TOL, cpu, rel, say  # noqa: E402
from rank_gradient_compression_amd import binding as B  # noqa: E402
from rank_gradient_compression_amd.torch_api import PowerSGD  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
ACC_REL = 2e-5  # fp32 accumulation error bound, relative to the factor's largest entry


def _e4m3_half_step(y):
    """Half the E4M3 spacing at |y| (scaled values, |y| <= 448)."""
    a = np.abs(y)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return 0.5 * 2.0 ** (np.maximum(e, -6.0) - 3.0)


def check_valid_column(gpu, exact, tag):
    """gpu: one column as the hook saw it; exact: the oracle's unrounded
    column.  Returns the number of values that differ from the oracle's own
    rounding."""
    ex32 = exact.astype(np.float32).astype(np.float64)
    amax = np.abs(ex32).max()
    if amax == 0.0:
        assert np.all(gpu == 0.0), f"{tag}: zero column not kept zero"
        return 0
    tol = ACC_REL * amax
    k_o = oracle.fp8_column_exponent(amax)
    cands = [k_o] + [k for k in (k_o - 1, k_o + 1)
                     if oracle.fp8_column_exponent(amax + tol) == k or oracle.fp8_column_exponent(amax - tol) == k]
    for k in cands:
        y = gpu / 2.0 ** k
        if np.abs(y).max() > 448.0 or not np.array_equal(oracle.round_fp8_e4m3(y), y):
            continue
        yx = ex32 / 2.0 ** k
        far = np.abs(y - yx) > _e4m3_half_step(np.where(y != 0, y, yx)) * (1 + 1e-12) + tol / 2.0 ** k
        if far.any():
            continue
        # the oracle's values rounded at the same exponent (clipped where an
        # exponent one below the oracle's leaves them just above 448)
        want = np.ldexp(oracle.round_fp8_e4m3(np.clip(yx, -448.0, 448.0)), k)
        return int((gpu != want).sum())
    raise AssertionError(f"{tag}: no exponent near the oracle's ({k_o}) makes the column a valid E4M3 rounding")


def check_valid_factor(gpu, exact, tag):
    flips = sum(check_valid_column(gpu[:, c], exact[:, c], f"{tag} column {c}") for c in range(gpu.shape[1]))
    assert flips <= 2 + gpu.size // 50, f"{tag}: {flips} rounding differences"
    return flips


@pytest.mark.parametrize("rank", [2, 4, 16, 32])
def test_fp8_payload_steps(rank):
    shapes = [(300, 650), (257, 1030), (33, 27), (5,), (2, 2)] if rank <= 16 else \
        [(700, 512), (1030, 257), (5,)]
    tensors = [(str(i), s) for i, s in enumerate(shapes)]
    wl = W.ModelSetWorkload(tensors, "lstm3", seed=280 + rank)
    ps = PowerSGD(shapes, rank, device=DEV)
    oplan = oracle.Plan(shapes, rank)
    comp = ps.compressed()
    Qw = {i: wl.q0(i, rank).astype(np.float64) for i in comp}
    Qw[comp[0]][:, rank // 2] = 0.0  # a zero Q column: its P column is zero and stays zero
    E = {i: np.zeros(oplan.views[i]) for i in comp}
    for i in comp:
        ps.set_q(i, Qw[i])
    seen = {}

    def hook(buf, count, stream):
        torch.cuda.synchronize()
        if buf == ps.p.data_ptr():
            seen["P"] = ps.p.clone()
        elif buf == ps.q.data_ptr():
            seen["Q"] = ps.q.clone()
        else:
            return 1
        return 0

    h = B.make_hook(hook)
    flips = 0
    for t in range(1, 4):
        grads = [wl.grad(i, t) for i in range(len(shapes))]
        for i, g in enumerate(grads):
            ps.view(ps.grads, i).copy_(torch.from_numpy(np.ascontiguousarray(g)).to(DEV))
        say(f"[fp8 payload r={rank}] step {t}")
        ps.compress(mhat=True, hook=h, payload_fp8=True)
        torch.cuda.synchronize()
        for i in comp:
            _, _, poff, qoff = ps.tensors[i]
            m, n = oplan.views[i]
            gP = cpu(seen["P"][poff: poff + rank * m].view(rank, m).t())
            gQ = cpu(seen["Q"][qoff: qoff + rank * n].view(rank, n).t())
            raw = {}

            def quantize(X, raw=raw):
                raw["P" if "P" not in raw else "Q"] = X.copy()
                return oracle.round_fp8_columns(X)

            def hook_p(P, gP=gP, raw=raw, i=i):
                nonlocal flips
                flips += check_valid_factor(gP, raw["P"], f"r={rank} step {t} tensor {i} P")
                return gP

            def hook_q(Q, gQ=gQ, raw=raw, i=i):
                nonlocal flips
                flips += check_valid_factor(gQ, raw["Q"], f"r={rank} step {t} tensor {i} Q")
                return gQ

            M = np.asarray(grads[i], np.float64).reshape(m, n) + E[i]
            res = oracle.compress_matrix(M, Qw[i], hook_p, hook_q, quantize=quantize)
            E[i], Qw[i] = res.E, res.Q
            Ph = cpu(ps.p_hat(i))
            assert oracle.orthonormality_error(Ph) <= ORTH_TOL
            if i == comp[0]:
                assert np.all(Ph[:, rank // 2] == 0.0) and np.all(gQ[:, rank // 2] == 0.0)
            for name, got, want in (("P_hat", Ph, res.P_hat), ("Q", cpu(ps.q_of(i)), res.Q),
                                    ("E", cpu(ps.view(ps.err, i)), res.E),
                                    ("M_hat", cpu(ps.view(ps.mhat, i)), res.M_hat)):
                e = rel(got, want)
                assert e <= REL_TOL, f"r={rank} step {t} tensor {i} {name}: rel err {e:.3e}"
        for i in range(len(shapes)):
            if i not in comp:  # pass-through values are not rounded
                assert np.array_equal(cpu(ps.view(ps.mhat, i)).reshape(-1),
                                      np.asarray(grads[i], np.float32).astype(np.float64).reshape(-1))
    say(f"[fp8 payload r={rank}] rounding differences against the fp64 oracle: {flips}")


def test_fp8_payload_on_the_7b_shapes_with_one_layer():
    """One layer of the 7B-shaped set (4096 x 4096, 11008 x 4096, 4096 x
    11008) at rank 4: the quantiser's grid covers matrices with up to 11008
    rows per column."""
    shapes = [(4096, 4096), (11008, 4096), (4096, 11008)]
    tensors = [(str(i), s) for i, s in enumerate(shapes)]
    wl = W.ModelSetWorkload(tensors, "resnet18", seed=290)
    rank = 4
    ps = PowerSGD(shapes, rank, device=DEV)
    seen = {}

    def hook(buf, count, stream):
        torch.cuda.synchronize()
        seen["P" if buf == ps.p.data_ptr() else "Q"] = (ps.p if buf == ps.p.data_ptr() else ps.q).clone()
        return 0

    h = B.make_hook(hook)
    for i in ps.compressed():
        ps.set_q(i, wl.q0(i, rank))
    for i in range(len(shapes)):
        ps.view(ps.grads, i).copy_(torch.from_numpy(np.ascontiguousarray(wl.grad(i, 1))).to(DEV))
    say("[fp8 payload 7B layer r=4] step 1")
    ps.compress(mhat=True, hook=h, payload_fp8=True)
    torch.cuda.synchronize()
    flips = 0
    for i in ps.compressed():
        _, _, poff, qoff = ps.tensors[i]
        m, n = shapes[i]
        G = np.asarray(wl.grad(i, 1), np.float32).astype(np.float64).reshape(m, n)
        Q0 = np.asarray(wl.q0(i, rank), np.float32).astype(np.float64)
        gP = cpu(seen["P"][poff: poff + rank * m].view(rank, m).t())
        gQ = cpu(seen["Q"][qoff: qoff + rank * n].view(rank, n).t())
        flips += check_valid_factor(gP, G @ Q0, f"tensor {i} P")
        flips += check_valid_factor(gQ, G.T @ oracle.gram_schmidt(gP), f"tensor {i} Q")
    say(f"[fp8 payload 7B layer r=4] rounding differences: {flips}")
