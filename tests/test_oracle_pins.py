"""Pins for the fp64 oracle, against what the PowerSGD pages and the
mathematics fix.  The pages print no worked numerical example, so every pin is
a closed form, an invariant, a library routine (LAPACK QR / SVD), or brute
force on tiny inputs.  Several tests plant a mistake in a copy of the oracle
and check that a pin catches it.
"""
import math
import os

import numpy as np
import pytest

import oracle
from oracle import powersgd as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(autouse=True)
def _strict_fp():
    with np.errstate(over="raise", invalid="raise", divide="raise"):
        yield


def rand(g, *shape):
    return g.standard_normal(shape)


def qr_positive(P):
    """Q factor of LAPACK's QR with signs fixed so that diag(R) > 0."""
    Qf, R = np.linalg.qr(P)
    s = np.sign(np.diag(R))
    s[s == 0] = 1.0
    return Qf * s


# ---------------------------------------------------------------- Gram-Schmidt

@pytest.mark.parametrize("m,r", [(7, 1), (64, 2), (256, 4), (1000, 7), (513, 16), (300, 64)])
def test_gs_equals_qr_factor(m, r):
    g = np.random.default_rng(m * 100 + r)
    P = rand(g, m, r)
    Ph = oracle.gram_schmidt(P)
    assert np.abs(Ph - qr_positive(P)).max() <= 1e-12


def test_gs_orthonormal_and_triangular_relation():
    g = np.random.default_rng(11)
    P = rand(g, 500, 8) @ np.diag(np.logspace(0, -3, 8))  # moderately ill-conditioned
    Ph = oracle.gram_schmidt(P)
    assert oracle.orthonormality_error(Ph) <= 1e-12
    R = Ph.T @ P  # P = Ph R with R upper triangular, positive diagonal
    assert np.abs(np.tril(R, -1)).max() <= 1e-12 * np.abs(R).max()
    assert (np.diag(R) > 0).all()


def test_gs_zero_and_dependent_columns():
    g = np.random.default_rng(3)
    a = rand(g, 50)
    b = rand(g, 50)
    P = np.stack([a, np.zeros(50), 2.0 * a, b, a - 3.0 * b], axis=1)
    Ph = oracle.gram_schmidt(P)
    assert np.all(Ph[:, 1] == 0) and np.all(Ph[:, 2] == 0) and np.all(Ph[:, 4] == 0)
    np.testing.assert_allclose(Ph[:, 0], a / np.linalg.norm(a), atol=1e-14)
    assert abs(Ph[:, 3] @ Ph[:, 0]) <= 1e-14
    assert abs(np.linalg.norm(Ph[:, 3]) - 1.0) <= 1e-14


def test_gs_threshold_is_relative():
    # A column whose component off the span is 1e-3 of its norm survives;
    # one at 1e-6 is zeroed (threshold 1e-4, reading R3).
    g = np.random.default_rng(5)
    a = rand(g, 40)
    a /= np.linalg.norm(a)
    z = rand(g, 40)
    z -= (a @ z) * a
    z /= np.linalg.norm(z)
    keep = oracle.gram_schmidt(np.stack([a, a + 1e-3 * z], 1))
    drop = oracle.gram_schmidt(np.stack([a, a + 1e-6 * z], 1))
    np.testing.assert_allclose(keep[:, 1], z, atol=1e-9)
    assert np.all(drop[:, 1] == 0)


# -------------------------------------------------------------- one compression

def test_residual_identity_exact():
    g = np.random.default_rng(7)
    M = rand(g, 96, 80)
    Q = rand(g, 80, 3)
    res = oracle.compress_matrix(M, Q)
    scale = np.maximum(np.abs(M), np.abs(res.M_hat))
    ulp = np.spacing(scale)
    assert np.all(np.abs(res.M_hat + res.E - M) <= ulp)


def test_orthonormal_output():
    wl = W.SmallMatrixWorkload()
    res = oracle.compress_matrix(wl.grads[0], wl.Q0)
    assert oracle.orthonormality_error(res.P_hat) <= 1e-12


@pytest.mark.parametrize("m,n,k,r", [(60, 40, 1, 1), (60, 40, 2, 2), (128, 64, 3, 4), (33, 27, 4, 4)])
def test_exact_recovery_low_rank(m, n, k, r):
    g = np.random.default_rng(m + n + k + r)
    M = rand(g, m, k) @ rand(g, n, k).T
    Q = rand(g, n, r)  # generic Q: rank(B^T Q) = k
    res = oracle.compress_matrix(M, Q)
    assert np.linalg.norm(res.E) <= 1e-12 * np.linalg.norm(M)
    assert np.linalg.norm(res.M_hat - M) <= 1e-12 * np.linalg.norm(M)


def test_eckart_young_limit():
    # Fixed M, error memory reset to zero every round: repeated warm-started
    # single iterations are subspace iteration on M^T M, so the residual tends
    # to the best rank-r error sqrt(sum_{k>r} sigma_k^2) (LAPACK SVD).
    g = np.random.default_rng(1)
    m, n, r = 256, 128, 2
    U = W.orthonormal(g, m, n)
    V = W.orthonormal(g, n, n)
    s = 1.0 / np.arange(1, n + 1)
    M = (U * s) @ V.T
    Q = rand(g, n, r)
    for _ in range(40):
        res = oracle.compress_matrix(M, Q)
        Q = res.Q
    sv = np.linalg.svd(M, compute_uv=False)
    best = math.sqrt(float(np.sum(sv[r:] ** 2)))
    assert abs(np.linalg.norm(res.E) - best) <= 1e-10 * best
    # and the reconstruction is the truncated SVD itself
    Uf, sf, Vf = np.linalg.svd(M)
    trunc = (Uf[:, :r] * sf[:r]) @ Vf[:r]
    assert np.linalg.norm(res.M_hat - trunc) <= 1e-9 * np.linalg.norm(trunc)


def test_eckart_young_rate():
    # Error of the rank-r subspace decays like (sigma_{r+1}/sigma_r)^(2t).
    g = np.random.default_rng(2)
    m, n, r = 120, 80, 3
    U = W.orthonormal(g, m, n)
    V = W.orthonormal(g, n, n)
    s = 0.9 ** np.arange(n)
    M = (U * s) @ V.T
    Q = rand(g, n, r)
    sines = []
    for _ in range(12):
        res = oracle.compress_matrix(M, Q)
        Q = res.Q
        sines.append(oracle.principal_angle_sines(Q, V[:, :r])[0])
    ratios = np.array(sines[5:]) / np.array(sines[4:-1])
    np.testing.assert_allclose(ratios, (s[r] / s[r - 1]) ** 2, rtol=2e-2)


def test_zero_matrix():
    res = oracle.compress_matrix(np.zeros((30, 20)), np.ones((20, 2)))
    assert not res.P_hat.any() and not res.Q.any() and not res.E.any() and not res.M_hat.any()


def test_rank1_power_method():
    # r = 1 is the power method: q/||q|| -> +-v1 and ||M^T p_hat|| -> sigma_1.
    g = np.random.default_rng(9)
    m, n = 90, 70
    U = W.orthonormal(g, m, n)
    V = W.orthonormal(g, n, n)
    s = np.concatenate([[3.0], np.linspace(1.5, 0.1, n - 1)])
    M = (U * s) @ V.T
    q = rand(g, n, 1)
    for _ in range(200):
        q = oracle.compress_matrix(M, q).Q
    v = q[:, 0] / np.linalg.norm(q)
    assert abs(abs(v @ V[:, 0]) - 1.0) <= 1e-12
    assert abs(np.linalg.norm(q) - 3.0) <= 1e-12


def test_triangular_invariance_of_warm_start():
    # GS(M Q T) = GS(M Q) for upper-triangular T with positive diagonal
    # (uniqueness of thin QR), so P_hat does not depend on rescaling or
    # orthonormalising the warm start (reading R2 is immaterial for P_hat).
    g = np.random.default_rng(4)
    M = rand(g, 70, 50)
    Q = rand(g, 50, 4)
    T = np.triu(rand(g, 4, 4))
    np.fill_diagonal(T, np.abs(np.diag(T)) + 0.5)
    a = oracle.compress_matrix(M, Q)
    b = oracle.compress_matrix(M, Q @ T)
    assert np.abs(a.P_hat - b.P_hat).max() <= 1e-12
    assert np.abs(a.Q - b.Q).max() <= 1e-12


# ---------------------------------------------------------------- linearity

def test_linearity_of_p_and_q_stages():
    g = np.random.default_rng(12)
    M1, M2 = rand(g, 64, 48), rand(g, 64, 48)
    Q = rand(g, 48, 3)
    a, b = 0.7, -1.3
    P = lambda M: oracle.compress_matrix(M, Q).P
    assert np.abs(P(a * M1 + b * M2) - (a * P(M1) + b * P(M2))).max() <= 1e-13
    Ph = oracle.gram_schmidt(rand(g, 64, 3))
    Qs = lambda M: M.T @ Ph
    assert np.abs(Qs(a * M1 + b * M2) - (a * Qs(M1) + b * Qs(M2))).max() <= 1e-13


@pytest.mark.parametrize("power_iters", [1, 3])
def test_mean_hook_over_workers_equals_compressing_the_mean(power_iters):
    g = np.random.default_rng(13)
    Ms = [rand(g, 80, 60) for _ in range(4)]
    Q = rand(g, 60, 2)
    Ph, Qn, Es = oracle.compress_workers(Ms, Q, power_iters=power_iters)
    ref = oracle.compress_matrix(sum(Ms) / 4, Q, power_iters=power_iters)
    assert np.abs(Ph - ref.P_hat).max() <= 1e-13
    assert np.abs(Qn - ref.Q).max() <= 1e-13
    # each worker keeps its own residual against the shared reconstruction
    for M, E in zip(Ms, Es):
        assert np.abs(M - E - ref.M_hat).max() <= 1e-13


def test_mean_hooks_in_step_set_match_workers():
    # The hook arguments of compress_matrix carry the aggregation.
    g = np.random.default_rng(14)
    Ms = [rand(g, 40, 30) for _ in range(3)]
    Q = rand(g, 30, 2)
    Ps = [M @ Q for M in Ms]
    mean_p = lambda P: sum(Ps) / 3
    Ph = oracle.gram_schmidt(sum(Ps) / 3)
    mean_q = lambda Qx: sum(M.T @ Ph for M in Ms) / 3
    r = oracle.compress_matrix(Ms[0], Q, hook_p=mean_p, hook_q=mean_q)
    Ph2, Q2, Es = oracle.compress_workers(Ms, Q)
    assert np.abs(r.P_hat - Ph2).max() <= 1e-13
    assert np.abs(r.Q - Q2).max() <= 1e-13
    assert np.abs(r.E - Es[0]).max() <= 1e-13


def test_worker_power_iterations_with_one_worker_are_the_step():
    """One worker: the mean is the identity, so compress_workers with k
    iterations is compress_matrix with k iterations, and k = 2 is two single
    iterations chained (the second starting from the first's Q)."""
    g = np.random.default_rng(15)
    M, Q = rand(g, 50, 40), rand(g, 40, 3)
    Ph, Qn, Es = oracle.compress_workers([M], Q, power_iters=2)
    ref = oracle.compress_matrix(M, Q, power_iters=2)
    assert np.array_equal(Ph, ref.P_hat) and np.array_equal(Qn, ref.Q)
    first = oracle.compress_matrix(M, Q)
    second = oracle.compress_matrix(M, first.Q)
    assert np.abs(Ph - second.P_hat).max() <= 1e-13
    assert np.abs(Es[0] - second.E).max() <= 1e-13


# ----------------------------------------------------------- error feedback

def test_error_feedback_telescopes():
    # No information is discarded, only delayed: sum_t M_hat_t + E_T = sum_t G_t.
    wl = W.SmallMatrixWorkload()
    plan = oracle.Plan([(256, 128)], 2)
    st = oracle.init_state(plan, [wl.Q0])
    acc = np.zeros((256, 128))
    gsum = np.zeros((256, 128))
    for t in range(wl.steps):
        res = oracle.step_set(plan, [wl.grads[t]], st)
        acc += res.M_hat[0]
        gsum += wl.grads[t].astype(np.float64)
    err = np.linalg.norm(acc + st.E[0] - gsum) / np.linalg.norm(gsum)
    assert err <= 1e-12


def test_error_feedback_telescopes_with_momentum():
    g = np.random.default_rng(21)
    plan = oracle.Plan([(40, 30), (30,)], 2)
    st = oracle.init_state(plan, [rand(g, 30, 2), None], momentum=True)
    beta = 0.9
    acc = np.zeros((40, 30))
    usum = np.zeros((40, 30))
    u = np.zeros((40, 30))
    for t in range(6):
        G = rand(g, 40, 30)
        res = oracle.step_set(plan, [G, rand(g, 30)], st, beta=beta)
        u = beta * u + G
        usum += u
        acc += res.M_hat[0]
    assert np.linalg.norm(acc + st.E[0] - usum) <= 1e-12 * np.linalg.norm(usum)


def test_momentum_closed_form():
    # Constant G: u_t = G (1 - beta^t) / (1 - beta).
    G = np.arange(12.0).reshape(3, 4)
    u = np.zeros_like(G)
    beta = 0.9
    for t in range(1, 8):
        u = oracle.momentum_input(u, G, beta)
        np.testing.assert_allclose(u, G * (1 - beta ** t) / (1 - beta), rtol=1e-14)


def test_passthrough_tensors_sent_unchanged():
    g = np.random.default_rng(22)
    plan = oracle.Plan([(5,), (2, 2), (64, 32)], 1)
    assert plan.kinds == [O.KIND_VECTOR, O.KIND_PASSTHRU, O.KIND_COMPRESSED]
    st = oracle.init_state(plan, [None, None, rand(g, 32, 1)])
    grads = [rand(g, 5), rand(g, 2, 2), rand(g, 64, 32)]
    res = oracle.step_set(plan, grads, st)
    assert np.array_equal(res.M_hat[0], grads[0]) and np.array_equal(res.M_hat[1], grads[1])
    assert st.E[0] is None and st.E[1] is None


# ------------------------------------------------------------- plan / payload

def _golden_payload():
    rows = {}
    with open(os.path.join(GOLDEN, "payload_counts.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            name, r, nm, el, fl, vec = line.split()
            rows[name] = tuple(int(x) for x in (r, nm, el, fl, vec))
    return rows


@pytest.mark.parametrize("name,tensors", [("resnet18", W.resnet18_cifar_set()),
                                          ("lstm3", W.lstm3_wikitext_set()),
                                          ("llama7b", W.llama7b_set())])
def test_payload_counts(name, tensors):
    r, nm, el, fl, vec = _golden_payload()[name]
    plan = oracle.Plan([s for _, s in tensors], r)
    pm, qn, pt = plan.payload()
    assert len(plan.compressed) == nm
    assert plan.dense_elems() == el
    assert pm + qn == fl
    assert pt == vec
    assert el / fl > 100  # "ratios above 100x" at r = 1..4


def test_classification_rule():
    assert oracle.classify((7,), 1) == O.KIND_VECTOR
    assert oracle.classify((2, 2), 1) == O.KIND_PASSTHRU       # 1*(2+2) = 4 = mn
    assert oracle.classify((3, 3), 1) == O.KIND_COMPRESSED     # 6 < 9
    assert oracle.classify((10, 512), 2) == O.KIND_COMPRESSED
    assert oracle.classify((10, 10), 5) == O.KIND_PASSTHRU     # 100 = 100
    assert oracle.classify((64, 3, 3, 3), 2) == O.KIND_COMPRESSED
    assert oracle.matrix_view((64, 3, 3, 3)) == (64, 27)
    assert oracle.classify((1, 4096), 1) == O.KIND_PASSTHRU    # 4097 >= 4096


# ---------------------------------------------------------------- brute force

def _scalar_compress(M, Q):
    """Scalar-loop PowerSGD step for tiny sizes (no BLAS, no numpy reductions)."""
    m, n = len(M), len(M[0])
    r = len(Q[0])
    P = [[sum(M[i][j] * Q[j][k] for j in range(n)) for k in range(r)] for i in range(m)]
    Ph = [[0.0] * r for _ in range(m)]
    for k in range(r):
        v = [P[i][k] for i in range(m)]
        nu0 = math.sqrt(sum(x * x for x in v))
        for j in range(k):
            d = sum(Ph[i][j] * v[i] for i in range(m))
            v = [v[i] - d * Ph[i][j] for i in range(m)]
        nv = math.sqrt(sum(x * x for x in v))
        if nu0 > 0 and nv > 1e-4 * nu0:
            for i in range(m):
                Ph[i][k] = v[i] / nv
    Qn = [[sum(M[i][j] * Ph[i][k] for i in range(m)) for k in range(r)] for j in range(n)]
    E = [[M[i][j] - sum(Ph[i][k] * Qn[j][k] for k in range(r)) for j in range(n)] for i in range(m)]
    return Ph, Qn, E


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_tiny(seed):
    g = np.random.default_rng(100 + seed)
    m, n = int(g.integers(2, 7)), int(g.integers(2, 7))
    r = int(g.integers(1, min(m, n) + 1))
    M = rand(g, m, n)
    Q = rand(g, n, r)
    Ph, Qn, E = _scalar_compress(M.tolist(), Q.tolist())
    res = oracle.compress_matrix(M, Q)
    assert np.abs(np.array(Ph) - res.P_hat).max() <= 1e-13
    assert np.abs(np.array(Qn) - res.Q).max() <= 1e-13
    assert np.abs(np.array(E) - res.E).max() <= 1e-13


# ---------------------------------------------------------------- refresh

def test_refresh_converges_to_svd_subspace():
    # Well separated leading spectrum: 8 rounds reach the LAPACK subspace.
    g = np.random.default_rng(31)
    m, n, r = 300, 200, 4
    U = W.orthonormal(g, m, n)
    V = W.orthonormal(g, n, n)
    s = np.concatenate([[10.0, 8.0, 6.0, 4.0], 0.5 * 0.99 ** np.arange(n - 4)])
    M = (U * s) @ V.T
    Q = oracle.refresh(M, rand(g, n, r), 8)
    _, _, Vt = np.linalg.svd(M)
    assert oracle.orthonormality_error(Q) <= 1e-12
    bound = (0.5 / 4.0) ** 16 * 1e3
    assert oracle.principal_angle_sines(Q, Vt[:r].T)[0] <= bound


def test_refresh_fused_form_same_subspace():
    # GS(M^T (M Q)) spans the same space as GS(M^T GS(M Q)) and, both being
    # Q factors with positive diagonal of matrices differing by an
    # upper-triangular factor, they are equal.
    g = np.random.default_rng(32)
    M = rand(g, 120, 90)
    Q = rand(g, 90, 6)
    two = oracle.gram_schmidt(M.T @ oracle.gram_schmidt(M @ Q))
    fused = oracle.gram_schmidt(M.T @ (M @ Q))
    assert np.abs(two - fused).max() <= 1e-12
    assert np.abs(oracle.refresh(M, Q, 1) - two).max() == 0.0


def test_refresh_decaying_spectrum_small_analogue():
    # sigma_k = exp(-k/20): the first few directions converge in 8 rounds,
    # the tail of a 32-wide block does not (gap e^{-1/20}).
    A, V, s = W.decaying_spectrum_matrix(512, 384, seed=5, K=256)
    A = A.astype(np.float64)
    Q0 = W.gaussian_q0(384, 32, 5).astype(np.float64)
    Q = oracle.refresh(A, Q0, 8)
    _, _, Vt = np.linalg.svd(A)
    # sin(theta(V_k, span Q)) for the leading k right singular vectors
    assert oracle.principal_angle_sines(Q, Vt[:1].T)[0] <= 1e-9
    assert oracle.principal_angle_sines(Q, Vt[:8].T)[0] <= 1e-7
    assert oracle.principal_angle_sines(Q, Vt[:32].T)[0] > 0.1


def test_principal_angles_closed_form():
    # Two planes in R^3 at a known dihedral angle.
    th = 0.3
    A = np.array([[1.0, 0], [0, 1], [0, 0]])
    B = np.array([[1.0, 0], [0, math.cos(th)], [0, math.sin(th)]])
    s = oracle.principal_angle_sines(A, B)
    np.testing.assert_allclose(s, [math.sin(th), 0.0], atol=1e-15)


# ------------------------------------------- planted mistakes fail the pins

def test_planted_mistakes_are_caught(monkeypatch):
    g = np.random.default_rng(41)
    M = rand(g, 50, 40)
    Q = rand(g, 40, 3)
    low = rand(g, 50, 2) @ rand(g, 40, 2).T

    # (a) Gram-Schmidt that forgets one projection term
    def gs_missing_term(P):
        P = np.asarray(P, float)
        out = np.zeros_like(P)
        for k in range(P.shape[1]):
            v = P[:, k].copy()
            for j in range(max(0, k - 1)):
                v -= (out[:, j] @ v) * out[:, j]
            out[:, k] = v / np.linalg.norm(v)
        return out

    assert oracle.orthonormality_error(gs_missing_term(rand(g, 50, 3))) > 1e-3

    # (b) sign flipped normalisation fails the QR pin
    Pm = rand(g, 30, 3)
    assert np.abs(-oracle.gram_schmidt(Pm) - qr_positive(Pm)).max() > 0.1

    # (c) Q computed from the raw P instead of P_hat breaks exact recovery
    P = low @ Q[:, :3]
    Qbad = low.T @ P
    Ebad = low - oracle.gram_schmidt(P) @ Qbad.T
    assert np.linalg.norm(Ebad) > 1e-3 * np.linalg.norm(low)

    # (d) a transposed operand in the left multiply fails on a square case
    Ms = rand(g, 40, 40)
    good = oracle.compress_matrix(Ms, Q)
    Ph = good.P_hat
    assert np.abs(Ms @ Ph - good.Q).max() > 1e-3

    # (e) forgetting to add E breaks the telescoping pin
    wl = W.SmallMatrixWorkload()
    plan = oracle.Plan([(256, 128)], 2)
    st = oracle.init_state(plan, [wl.Q0])
    orig = O.compress_matrix

    def no_ef(Mx, Qw, hp=None, hq=None, power_iters=1, quantize=None):
        return orig(Mx - st.E[0], Qw, hp, hq, power_iters=power_iters, quantize=quantize)

    monkeypatch.setattr(O, "compress_matrix", no_ef)
    acc = np.zeros((256, 128))
    gsum = np.zeros((256, 128))
    for t in range(3):
        res = O.step_set(plan, [wl.grads[t]], st)
        acc += res.M_hat[0]
        gsum += wl.grads[t]
    assert np.linalg.norm(acc + st.E[0] - gsum) > 1e-3 * np.linalg.norm(gsum)


# ------------------------------------------- power iterations, ablations, SGD

def test_power_iterations_equal_repeated_single_iterations():
    # k iterations in one step = k warm-started single iterations on the same
    # M with the error memory reset (reading R8).
    g = np.random.default_rng(61)
    M = rand(g, 80, 60)
    Q = rand(g, 60, 3)
    multi = oracle.compress_matrix(M, Q, power_iters=4)
    q = Q
    for _ in range(4):
        single = oracle.compress_matrix(M, q)
        q = single.Q
    assert np.abs(multi.Q - single.Q).max() <= 1e-12
    assert np.abs(multi.P_hat - single.P_hat).max() <= 1e-12
    assert np.abs(multi.E - single.E).max() <= 1e-12


def _approx_error(kind, iters, seed, steps=30, m=256, n=128, r=2):
    g = np.random.default_rng(seed)
    U = W.orthonormal(g, m, 16)
    V = W.orthonormal(g, n, 16)
    S = (U / np.arange(1, 17)) @ V.T
    Q = g.standard_normal((n, r))
    errs = []
    for _ in range(steps):
        M = S + 0.01 * g.standard_normal((m, n))
        if kind == "cold":
            Q = g.standard_normal((n, r))
        res = oracle.compress_matrix(M, Q, power_iters=iters)
        Q = res.Q
        errs.append(np.linalg.norm(M - res.M_hat) / np.linalg.norm(M))
    return float(np.mean(errs[5:]))


def test_warm_start_matches_several_cold_iterations():
    # Glossary entry "PowerSGD", temporal-coherence paragraph: one warm-started
    # power iteration matches the accuracy of 2-4 iterations from scratch.
    # Fixed rank-16 signal (sigma ~ 1/j) plus fresh noise, rank 2, no error
    # feedback (approximation quality alone).
    for seed in range(3):
        warm1 = _approx_error("warm", 1, seed)
        cold1, cold2, cold4 = (_approx_error("cold", k, seed) for k in (1, 2, 4))
        assert warm1 < cold1 and warm1 <= cold2
        assert warm1 <= cold4 * 1.001


def test_no_error_feedback_ignores_memory():
    g = np.random.default_rng(62)
    plan = oracle.Plan([(40, 30)], 2)
    q0 = rand(g, 30, 2)
    st = oracle.init_state(plan, [q0])
    st.E[0] = rand(g, 40, 30)  # would be added with error feedback on
    G = rand(g, 40, 30)
    res = oracle.step_set(plan, [G], st, error_feedback=False)
    ref = oracle.compress_matrix(G, q0)
    assert np.abs(res.M_hat[0] - ref.M_hat).max() <= 1e-13
    assert np.abs(st.E[0] - ref.E).max() <= 1e-13


def test_sgd_momentum_closed_form():
    # Constant update D: m_t = D (1 - mu^t)/(1 - mu), x_t = x_0 - lr sum_t m_t.
    D = np.linspace(-1.0, 1.0, 7)
    x = np.ones(7)
    m = np.zeros(7)
    lr, mu = 0.1, 0.9
    xs = x.copy()
    for t in range(1, 6):
        x, m = oracle.sgd_momentum_step(x, m, D, lr, mu)
        np.testing.assert_allclose(m, D * (1 - mu ** t) / (1 - mu), rtol=1e-14)
        xs = xs - lr * D * (1 - mu ** t) / (1 - mu)
        np.testing.assert_allclose(x, xs, rtol=1e-13, atol=1e-15)


def test_sgd_nesterov_closed_form():
    # Constant D: the Nesterov direction D + mu m_t equals D (1 - mu^(t+1))/(1 - mu).
    D = np.linspace(-1.0, 1.0, 7)
    x = np.ones(7)
    m = np.zeros(7)
    lr, mu = 0.1, 0.9
    xs = x.copy()
    for t in range(1, 6):
        x, m = oracle.sgd_momentum_step(x, m, D, lr, mu, nesterov=True)
        np.testing.assert_allclose(m, D * (1 - mu ** t) / (1 - mu), rtol=1e-14)
        xs = xs - lr * D * (1 - mu ** (t + 1)) / (1 - mu)
        np.testing.assert_allclose(x, xs, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("nesterov", [False, True])
def test_sgd_matches_torch_optimizer(nesterov):
    # Library routine: torch.optim.SGD (dampening 0) on the CPU in float64,
    # fed the same sequence of updates.
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(17)
    x0 = g.standard_normal(11)
    lr, mu = 0.05, 0.8
    p = torch.nn.Parameter(torch.from_numpy(x0.copy()))
    opt = torch.optim.SGD([p], lr=lr, momentum=mu, nesterov=nesterov)
    x, m = x0.copy(), np.zeros(11)
    for _ in range(6):
        D = g.standard_normal(11)
        p.grad = torch.from_numpy(D.copy())
        opt.step()
        x, m = oracle.sgd_momentum_step(x, m, D, lr, mu, nesterov=nesterov)
        np.testing.assert_allclose(x, p.detach().numpy(), rtol=1e-14, atol=1e-15)


# ------------------------------------------------------- seeded start for Q

@pytest.mark.parametrize("key,counter", [
    ((5, 7), (0, 0, 0, 0)),
    ((0, 0), (0, 0, 0, 0)),
    ((2 ** 64 - 1, 2 ** 64 - 1), (2 ** 64 - 2, 3, 2 ** 63, 9)),
    ((1234, 17), (2 ** 64 - 1, 0, 0, 0)),  # the library's counter carries into word 1
])
def test_philox_matches_numpy_bit_generator(key, counter):
    # numpy's Philox is Philox-4x64-10; it advances its 256-bit counter by one
    # before producing each block of four words.
    from oracle import philox as PH
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(counter, dtype=np.uint64))
    raw = [int(v) for v in bg.random_raw(12)]
    c = sum(int(w) << (64 * i) for i, w in enumerate(counter))
    for blk in range(3):
        cc = (c + 1 + blk) % (1 << 256)
        words = [(cc >> (64 * i)) & PH.MASK64 for i in range(4)]
        assert list(PH.philox4x64(words, key)) == raw[4 * blk: 4 * blk + 4]


def test_box_muller_inverts_to_its_uniforms():
    # From each pair (z0, z1): exp(-(z0^2 + z1^2)/2) is u1 and the polar angle
    # is 2 pi u2, for the uniforms built from the block's words.
    from oracle import philox as PH
    for b in range(50):
        w = PH.philox4x64((b, 0, 0, 0), (99, 3))
        z = PH.normal_stream(99, 3, 4 * b + 4)[4 * b: 4 * b + 4]
        for (wa, wb), (z0, z1) in (((w[0], w[1]), z[:2]), ((w[2], w[3]), z[2:])):
            u1 = 1.0 - (wa >> 11) / 2.0 ** 53
            u2 = (wb >> 11) / 2.0 ** 53
            assert abs(np.exp(-(z0 * z0 + z1 * z1) / 2) - u1) <= 1e-12
            ang = np.arctan2(z1, z0) % (2 * np.pi)
            assert min(abs(ang - 2 * np.pi * u2), 2 * np.pi - abs(ang - 2 * np.pi * u2)) <= 1e-9


def test_seeded_q_is_standard_normal():
    # Kolmogorov-Smirnov against N(0, 1) over 2^16 draws of one stream, and
    # between-stream independence: correlation of two keys' streams.
    scipy_stats = pytest.importorskip("scipy.stats")
    z = oracle.normal_stream(2024, 0, 1 << 16)
    assert scipy_stats.kstest(z, "norm").pvalue > 1e-3
    assert abs(z.mean()) < 5 / np.sqrt(z.size) and abs(z.var() - 1) < 0.03
    z2 = oracle.normal_stream(2024, 1, 1 << 16)
    assert abs(np.corrcoef(z, z2)[0, 1]) < 5 / np.sqrt(z.size)


def test_seeded_q_layout():
    # Column c of the n x r start Q is the stream's slice [c n, (c + 1) n): the
    # same column at every rank, different for another seed or tensor.
    q4 = oracle.init_q(37, 4, 7, 2)
    q9 = oracle.init_q(37, 9, 7, 2)
    s = oracle.normal_stream(7, 2, 37 * 9)
    assert np.array_equal(q9[:, :4], q4)
    assert np.array_equal(q9, s.reshape(9, 37).T)
    assert not np.array_equal(oracle.init_q(37, 4, 8, 2), q4)
    assert not np.array_equal(oracle.init_q(37, 4, 7, 3), q4)
    plan = oracle.Plan([(300, 40), (5,), (2, 2)], 4)
    qs = oracle.init_q_set(plan, 11)
    assert qs[1] is None and qs[2] is None and np.array_equal(qs[0], oracle.init_q(40, 4, 11, 0))


# ------------------------------------------------- bfloat16 payload (R11)

def test_round_bf16_matches_torch_conversion():
    # Library routine: torch's float32 -> bfloat16 conversion (round to
    # nearest even) on the CPU, over normal, subnormal, tie and carry cases.
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(23)
    x = np.concatenate([
        g.standard_normal(20000) * 10.0 ** g.integers(-30, 30, 20000),
        g.standard_normal(2000) * 1e-39,                       # fp32 subnormals
        np.array([1.0, -1.0, 2.0 ** -126, 3.0, 0.0, 65280.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8,
                  -(1.0 + 2 ** -8), 255.5, 2.0 ** -133, 1.5 * 2.0 ** -133, 2.5 * 2.0 ** -133]),
    ]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_bf16(x)
    assert np.array_equal(got, want)


def test_quantised_payload_rounds_both_factors_before_the_hooks():
    # The hooks see bfloat16-representable factors; the residual is formed
    # from the received factors, so M_hat + E = M still holds.
    g = np.random.default_rng(24)
    M = rand(g, 40, 30)
    Q0 = rand(g, 30, 3)
    seen = {}

    def keep(name):
        def h(X):
            seen[name] = X.copy()
            return X
        return h

    res = oracle.compress_matrix(M, Q0, keep("P"), keep("Q"), quantize=oracle.round_bf16)
    for name in ("P", "Q"):
        assert np.array_equal(oracle.round_bf16(seen[name]), seen[name])
    np.testing.assert_array_equal(seen["P"], oracle.round_bf16(M @ Q0))
    np.testing.assert_allclose(res.M_hat + res.E, M, rtol=0, atol=1e-14)
    plain = oracle.compress_matrix(M, Q0)
    # bfloat16 keeps about 3 significant digits: close to, but not equal to, fp64
    d = np.linalg.norm(res.M_hat - plain.M_hat) / np.linalg.norm(plain.M_hat)
    assert 1e-5 < d < 2e-2


# ------------------------------------------------ fp8 (E4M3) payload (R12)

def _e4m3_grid():
    """Every finite non-negative OCP FP8 E4M3 value, from the format's
    definition: subnormals m/8 * 2^-6 (m = 0..7), normals (1 + m/8) * 2^e for
    e = -6..8, except e = 8, m = 7 (the NaN code); the codes in order."""
    vals = [m / 8.0 * 2.0 ** -6 for m in range(8)]
    vals += [(1.0 + m / 8.0) * 2.0 ** e for e in range(-6, 9) for m in range(8) if not (e == 8 and m == 7)]
    return np.array(vals)


def test_e4m3_grid_definition():
    grid = _e4m3_grid()
    assert grid.size == 127 and grid[-1] == oracle.FP8_E4M3_MAX == 448.0
    assert np.all(np.diff(grid) > 0)


def test_round_fp8_e4m3_matches_torch_conversion():
    # Library routine: torch's float32 -> float8_e4m3fn conversion (round to
    # nearest even) on the CPU, over normals, subnormals, ties and carries.
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(41)
    grid = _e4m3_grid()
    mids = 0.5 * (grid[1:] + grid[:-1])
    x = np.concatenate([
        g.uniform(-448.0, 448.0, 20000),
        g.standard_normal(20000) * 2.0 ** g.integers(-14, 8, 20000),
        grid, -grid, mids, -mids,                                # grid values and every midpoint (ties)
        np.array([2.0 ** -10, 3 * 2.0 ** -11, 2.0 ** -12, 1e-30, 0.0, 447.9, 2.0 ** -6 * (1 - 2 ** -5)]),
    ])
    x = x[np.abs(x) <= 448.0].astype(np.float32)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.round_fp8_e4m3(x)
    assert np.array_equal(got, want)


def test_round_fp8_e4m3_is_the_nearest_grid_value_brute_force():
    # Brute force over the format's 127 magnitudes: the nearest value, and on
    # a tie the one with the even code (an even index into the ordered grid).
    grid = _e4m3_grid()
    g = np.random.default_rng(42)
    mids = 0.5 * (grid[1:] + grid[:-1])
    x = np.concatenate([g.uniform(0, 448.0, 3000), g.uniform(0, 2.0 ** -5, 1000), mids, grid])
    for v in x:
        d = np.abs(grid - v)
        best = np.flatnonzero(d == d.min())
        idx = best[0] if best.size == 1 else [b for b in best if b % 2 == 0][0]
        assert oracle.round_fp8_e4m3(np.array([v]))[0] == grid[idx]
        assert oracle.round_fp8_e4m3(np.array([-v]))[0] == -grid[idx]


def test_fp8_column_exponent_is_the_smallest_sufficient_power():
    g = np.random.default_rng(43)
    amax = np.concatenate([np.abs(g.standard_normal(3000)) * 10.0 ** g.integers(-20, 20, 3000),
                           448.0 * 2.0 ** np.arange(-30, 30), np.nextafter(448.0 * 2.0 ** np.arange(-30, 30), np.inf),
                           np.nextafter(448.0 * 2.0 ** np.arange(-30, 30), 0)])
    for a in amax:
        k = oracle.fp8_column_exponent(a)
        assert a <= 448.0 * 2.0 ** k and not a <= 448.0 * 2.0 ** (k - 1), a
    assert oracle.fp8_column_exponent(0.0) == 0


def test_round_fp8_columns_scales_each_column_on_its_own():
    g = np.random.default_rng(44)
    F = g.standard_normal((300, 5)) * np.array([1e-3, 1.0, 40.0, 1e4, 0.0])
    F[:, 4] = 0.0
    out = oracle.round_fp8_columns(F)
    assert np.all(out[:, 4] == 0.0)
    for c in range(4):
        f32 = F[:, c].astype(np.float32).astype(np.float64)
        k = oracle.fp8_column_exponent(np.abs(f32).max())
        y = out[:, c] / 2.0 ** k
        assert 224.0 < np.abs(y).max() <= 448.0
        assert np.array_equal(oracle.round_fp8_e4m3(y), y)       # on the E4M3 grid
        # the nearest value: within half a step of the binade the scaled value lies in
        a = np.abs(f32 / 2.0 ** k)
        e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -6)
        assert np.all(np.abs(y - f32 / 2.0 ** k) <= 0.5 * 2.0 ** (e - 3) * (1 + 1e-12))
    # scaling one column by a power of two scales only its result, exactly
    G = F.copy()
    G[:, 2] *= 2.0 ** 7
    out2 = oracle.round_fp8_columns(G)
    assert np.array_equal(out2[:, 2], out[:, 2] * 2.0 ** 7)
    assert np.array_equal(np.delete(out2, 2, axis=1), np.delete(out, 2, axis=1))
    # planted mistake: one scale for the whole factor loses the small columns
    k_all = oracle.fp8_column_exponent(np.abs(F).max())
    one_scale = np.ldexp(oracle.round_fp8_e4m3(np.ldexp(F.astype(np.float32).astype(np.float64), -k_all)), k_all)
    assert not np.array_equal(one_scale, out)


def test_fp8_payload_rounds_both_factors_before_the_hooks():
    g = np.random.default_rng(45)
    M = rand(g, 40, 30)
    Q0 = rand(g, 30, 3)
    seen = {}

    def keep(name):
        def h(X):
            seen[name] = X.copy()
            return X
        return h

    res = oracle.compress_matrix(M, Q0, keep("P"), keep("Q"), quantize=oracle.round_fp8_columns)
    for name in ("P", "Q"):
        assert np.array_equal(oracle.round_fp8_columns(seen[name]), seen[name])
    np.testing.assert_array_equal(seen["P"], oracle.round_fp8_columns(M @ Q0))
    np.testing.assert_allclose(res.M_hat + res.E, M, rtol=0, atol=1e-14)
    plain = oracle.compress_matrix(M, Q0)
    # E4M3 keeps 4 significant bits: a few percent from fp64, more than bfloat16
    d = np.linalg.norm(res.M_hat - plain.M_hat) / np.linalg.norm(plain.M_hat)
    db = np.linalg.norm(oracle.compress_matrix(M, Q0, quantize=oracle.round_bf16).M_hat - plain.M_hat) \
        / np.linalg.norm(plain.M_hat)
    assert db < d < 0.2


# ---------------------------------------------------------------- decompression
#
# The receiver rebuilds the gradient from the two transmitted factors as their
# product P_hat Q^T (glossary entry "PowerSGD", factorisation paragraph).

def _scalar_decompress(Ph, Q):
    m, r, n = len(Ph), len(Ph[0]), len(Q)
    return [[sum(Ph[i][k] * Q[j][k] for k in range(r)) for j in range(n)] for i in range(m)]


@pytest.mark.parametrize("m,n,r", [(1, 1, 1), (2, 5, 1), (6, 4, 3), (5, 6, 2), (4, 4, 4)])
def test_decompress_brute_force(m, n, r):
    g = np.random.default_rng(300 + 10 * m + n + r)
    Ph, Q = rand(g, m, r), rand(g, n, r)
    want = np.array(_scalar_decompress(Ph.tolist(), Q.tolist()))
    got = oracle.decompress(Ph, Q)
    assert got.shape == (m, n)
    assert np.abs(got - want).max() <= 1e-14


@pytest.mark.parametrize("m,n,k,r", [(60, 40, 1, 1), (60, 40, 2, 5), (128, 64, 3, 4), (33, 27, 4, 4)])
def test_decompress_exact_recovery_from_any_basis_of_the_column_space(m, n, k, r):
    """M = A B^T of rank k <= r, P_hat any orthonormal m x r basis whose span
    holds the columns of A, Q = M^T P_hat: the product is P_hat P_hat^T M = M
    (a projection onto a space that holds M's columns)."""
    g = np.random.default_rng(310 + k + r)
    A, Bm = rand(g, m, k), rand(g, n, k)
    M = A @ Bm.T
    # the first k columns span A; the rest are random directions
    Ph = qr_positive(np.hstack([A, rand(g, m, r - k)]))
    Q = M.T @ Ph
    assert np.linalg.norm(oracle.decompress(Ph, Q) - M) <= 1e-12 * np.linalg.norm(M)


def test_decompress_equals_step_reconstruction_and_residual():
    """decompress(P_hat, Q) of a step's outputs is the step's M_hat, and
    M - decompress = E (error feedback keeps exactly what was not sent)."""
    g = np.random.default_rng(320)
    M, Q0 = rand(g, 90, 70), rand(g, 70, 3)
    res = oracle.compress_matrix(M, Q0)
    D = oracle.decompress(res.P_hat, res.Q)
    assert np.array_equal(D, res.M_hat)
    assert np.abs(M - D - res.E).max() <= 4 * np.spacing(np.abs(M).max())


def test_decompress_planted_mistakes_are_caught():
    """Plausible wrong forms of the product each fail a pin above."""
    g = np.random.default_rng(330)
    m, n, r = 6, 5, 2
    Ph, Q = rand(g, m, r), rand(g, n, r)
    want = np.array(_scalar_decompress(Ph.tolist(), Q.tolist()))
    wrong = [
        lambda P, Qf: P[:, :1] @ Qf[:, :1].T,           # drops the last rank term
        lambda P, Qf: -(P @ Qf.T),                       # flipped sign
        lambda P, Qf: P @ np.flip(Qf, axis=1).T,         # columns paired wrongly
        lambda P, Qf: (P @ Qf.T)[::-1],                  # rows permuted
    ]
    for f in wrong:
        assert np.abs(f(Ph, Q) - want).max() > 1e-3
    # a transposed operand does not even give an m x n matrix
    with pytest.raises(ValueError):
        np.asarray(Ph.T @ Q)


# ---------------------------------------------------------------- diagnostics

def test_compression_error_closed_form_at_the_svd_subspace():
    # Warm start on the exact top-r right singular vectors: P_hat spans the
    # top-r left singular vectors, so E = M - U_r U_r^T M and
    # ||E||^2 = sum_{k > r} sigma_k^2 (Eckart-Young).
    g = np.random.default_rng(41)
    m, n, r = 60, 40, 3
    U = W.orthonormal(g, m, n)
    V = W.orthonormal(g, n, n)
    s = np.linspace(5.0, 0.1, n)
    M = (U * s) @ V.T
    res = oracle.compress_matrix(M, V[:, :r] @ np.diag([2.0, 0.5, 1.0]))
    want = math.sqrt(np.sum(s[r:] ** 2) / np.sum(s ** 2))
    assert abs(oracle.compression_error(res.E, M) - want) <= 1e-12
    # exact rank r: nothing is left for later steps
    Mr = (U[:, :r] * s[:r]) @ V[:, :r].T
    res = oracle.compress_matrix(Mr, rand(g, n, r))
    assert oracle.compression_error(res.E, Mr) <= 1e-12
    assert oracle.compression_error(np.zeros((3, 4)), np.zeros((3, 4))) == 0.0
    assert abs(oracle.compression_error(2.0 * res.E + 1.0, 2.0 * Mr + 2.0)
               - np.linalg.norm(2.0 * res.E + 1.0) / np.linalg.norm(2.0 * Mr + 2.0)) <= 1e-15


def test_subspace_overlap_special_cases():
    g = np.random.default_rng(42)
    n, r = 30, 4
    A = rand(g, n, r)
    # the same span, other basis: every cosine is 1
    assert abs(oracle.subspace_overlap(A, A @ rand(g, r, r)) - 1.0) <= 1e-12
    I = np.eye(n)
    # orthogonal spans: 0; one shared direction of r: 1 / r
    assert abs(oracle.subspace_overlap(I[:, :r], I[:, r:2 * r])) <= 1e-15
    assert abs(oracle.subspace_overlap(I[:, :r], np.c_[I[:, :1], I[:, r:2 * r - 1]]) - 1.0 / r) <= 1e-15
    # one direction turned by theta: (r - 1 + cos theta) / r
    th = 0.3
    B = I[:, :r].copy()
    B[:, r - 1] = math.cos(th) * I[:, r - 1] + math.sin(th) * I[:, r]
    assert abs(oracle.subspace_overlap(I[:, :r], B) - (r - 1 + math.cos(th)) / r) <= 1e-14
    # a dependent column counts as a cosine of 0
    C = I[:, :r].copy()
    C[:, 2] = C[:, 0] + C[:, 1]
    assert abs(oracle.subspace_overlap(I[:, :r], C) - (r - 1) / r) <= 1e-14


def test_subspace_overlap_equals_scipy_principal_angles():
    scipy_linalg = pytest.importorskip("scipy.linalg")
    g = np.random.default_rng(43)
    for n, r in ((50, 3), (200, 16), (90, 32)):
        A = rand(g, n, r)
        B = A + 0.3 * rand(g, n, r)
        want = float(np.mean(np.cos(scipy_linalg.subspace_angles(A, B))))
        assert abs(oracle.subspace_overlap(A, B) - want) <= 1e-12
