"""Parity of the HIP path (through the C ABI) with the fp64 oracle on the
seeded workloads, plus edge cases, determinism and the ABI's device-side
contracts.  Tolerances: relative Frobenius error <= 1e-4 on P_hat, Q, E and
M_hat per matrix and step, ||P_hat^T P_hat - I||_F <= 1e-5."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle  # noqa: E402
import workloads as W  # noqa: E402
from gpu_util import (DRIFT_STEPS, ORTH_TOL, REL_TOL, TELESCOPE_TOL, DriftTolerance, Telescope,  # noqa: E402
                      compare_set, cpu, rel, say, snapshot_state)
from rank_gradient_compression_amd import binding as B  # noqa: E402
from rank_gradient_compression_amd.torch_api import PowerSGD  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def run_set_parity(tensors, rank, steps, grad_fn, q0_fn, beta=None, tag="", check_every=1, offsets=None,
                   grads_dtype=None, power_iters=0, error_feedback=True, refresh_at=(), refresh_iters=8):
    """Run `steps` compress calls on the GPU and the oracle's step on the same
    inputs.  Every `check_every` steps (and the first, the last and every
    refresh step): the teacher-forced gate (the oracle starts the step from
    the GPU's own state) at REL_TOL, and the free-running oracle's trajectory,
    asserted at the drift tolerance up to step DRIFT_STEPS and reported
    after it; with error feedback, error feedback's telescoping sum over the
    whole GPU trajectory.  Steps in `refresh_at` are PowerSGD+ steps with
    `refresh_iters` rounds.  With grads_dtype=bfloat16 the gradients are
    rounded to bfloat16 on the host first and the oracle gets the rounded
    values, widened exactly."""
    shapes = [s for _, s in tensors]
    say(f"[{tag}] plan: {len(shapes)} tensors, rank {rank}, {steps} steps")
    gdt = grads_dtype or torch.float32
    ps = PowerSGD(shapes, rank, device=DEV, momentum_beta=beta, offsets=offsets, grads_dtype=gdt)
    oplan = oracle.Plan(shapes, rank)
    q0 = [q0_fn(i) if oplan.kinds[i] == oracle.KIND_COMPRESSED else None for i in range(len(shapes))]
    ost = oracle.init_state(oplan, q0, momentum=beta is not None)
    for i in ps.compressed():
        ps.set_q(i, q0[i])
    drift = DriftTolerance()
    tele = Telescope(ps) if error_feedback else None
    worst, worst_drift = {}, {}
    for t in range(1, steps + 1):
        it = refresh_iters if t in refresh_at else 0
        kw = dict(beta=beta or 0.0, power_iters=max(1, power_iters), error_feedback=error_feedback, refresh_iters=it)
        grads = [grad_fn(i, t) for i in range(len(shapes))]
        if gdt != torch.float32:
            host = [torch.from_numpy(np.ascontiguousarray(g, dtype=np.float32)).to(gdt) for g in grads]
            grads = [h.double().numpy() for h in host]
        else:
            host = [torch.from_numpy(np.ascontiguousarray(g)) for g in grads]
        for i, h in enumerate(host):
            ps.view(ps.grads, i).copy_(h.to(DEV))
        check = t == 1 or t % check_every == 0 or t == steps or t in refresh_at
        if check:
            forced = snapshot_state(ps, oplan, momentum=beta is not None)
        if check or steps <= 20:
            say(f"[{tag}] step {t}: compress" + (f" with a {it}-round refresh" if it else ""))
        ps.compress(mhat=True, power_iters=power_iters, error_feedback=error_feedback, refresh_iters=it)
        if tele is not None:
            tele.add()
        torch.cuda.synchronize()
        ores = oracle.step_set(oplan, grads, ost, **kw)
        drift.update(ores)
        if check:
            gres = oracle.step_set(oplan, grads, forced, **kw)
            g = compare_set(ps, oplan, gres, forced, tag=f"{tag} step {t} (teacher-forced)")
            d = compare_set(ps, oplan, ores, ost, tag=f"{tag} step {t} (free-running)",
                            tol=drift.tols() if t <= DRIFT_STEPS else float("inf"))
            say(f"[{tag}] step {t}: gate " + " ".join(f"{k}={v:.2e}" for k, v in g.items())
                + " | drift " + " ".join(f"{k}={v:.2e}" for k, v in d.items()))
            for k, v in g.items():
                worst[k] = max(worst.get(k, 0.0), v)
            for k, v in d.items():
                worst_drift[k] = max(worst_drift.get(k, 0.0), v)
    say(f"[{tag}] worst teacher-forced rel errors: {worst}; worst free-running: {worst_drift}")
    if tele is not None:
        e = tele.error()
        say(f"[{tag}] error-feedback telescoping sum over {steps} steps: rel err {e:.2e}")
        assert e <= TELESCOPE_TOL, f"{tag}: sum M_hat + E_T - sum X, rel err {e:.3e}"
    return ps, oplan, ost


def test_single_256x128_rank2_ten_steps():
    wl = W.SmallMatrixWorkload()
    ps, oplan, ost = run_set_parity([("w", (256, 128))], 2, wl.steps, lambda i, t: wl.grads[t - 1],
                                    lambda i: wl.Q0, tag="256x128")


def test_residual_identity_on_gpu():
    # M_hat + E reproduces M = G + E_old up to the rounding of one subtraction.
    wl = W.SmallMatrixWorkload()
    ps = PowerSGD([(256, 128)], 2, device=DEV)
    ps.set_q(0, wl.Q0)
    for t in range(3):
        e_old = ps.view(ps.err, 0).clone()
        ps.view(ps.grads, 0).copy_(torch.from_numpy(wl.grads[t]).to(DEV))
        ps.compress(mhat=True)
        torch.cuda.synchronize()
        M = (ps.view(ps.grads, 0) + e_old).cpu().numpy()  # fp32 add, as the kernel
        Mh = ps.view(ps.mhat, 0).cpu().numpy()
        E = ps.view(ps.err, 0).cpu().numpy()
        ulp = np.spacing(np.maximum(np.abs(M), np.abs(Mh)).astype(np.float32))
        assert np.all(np.abs((Mh.astype(np.float64) + E) - M) <= 2 * ulp)


@pytest.mark.parametrize("rank", [1, 2, 3, 4, 5, 6, 7, 8])
def test_ragged_shapes_every_rank(rank):
    # rows not a multiple of the 32-row workgroup tile, columns not a multiple
    # of the 256-column step, odd column counts (scalar path), even (2-wide)
    shapes = [(97, 1030), (33, 27), (1, 3), (300, 650), (64, 64), (1000, 1), (257, 4099), (45, 2002),
              (8, 9), (5,), (129, 384)]
    tensors = [(str(i), s) for i, s in enumerate(shapes)]
    wl = W.ModelSetWorkload(tensors, "plain", seed=10 + rank)
    run_set_parity(tensors, rank, 2, wl.grad, lambda i: wl.q0(i, rank), tag=f"ragged r={rank}")


def test_unaligned_caller_offsets():
    # offsets that force the 1- and 2-wide load paths on 4-divisible widths
    shapes = [(70, 256), (50, 512), (40, 300)]
    offsets = [1, 70 * 256 + 3, 70 * 256 + 3 + 50 * 512 + 2]
    tensors = [(str(i), s) for i, s in enumerate(shapes)]
    wl = W.ModelSetWorkload(tensors, "plain", seed=77)
    run_set_parity(tensors, 3, 2, wl.grad, lambda i: wl.q0(i, 3), tag="offsets", offsets=offsets)


def test_momentum_variant_small_set():
    wl = W.ModelSetWorkload(W.resnet18_cifar_set(), "resnet18", seed=2)
    run_set_parity(wl.tensors, 2, 5, wl.grad, lambda i: wl.q0(i, 2), beta=0.9, tag="resnet18 momentum")


def test_zero_gradient_gives_zero_factors():
    ps = PowerSGD([(200, 300), (7,)], 3, device=DEV)
    ps.set_q(0, np.ones((300, 3), np.float32))
    ps.compress(mhat=True)
    torch.cuda.synchronize()
    assert not ps.p_hat(0).any() and not ps.q_of(0).any()
    assert not ps.view(ps.err, 0).any() and not ps.view(ps.mhat, 0).any()


def test_exact_recovery_low_rank():
    g = np.random.default_rng(5)
    m, n, k, r = 700, 520, 3, 4
    M = (g.standard_normal((m, k)) @ g.standard_normal((k, n))).astype(np.float32)
    ps = PowerSGD([(m, n)], r, device=DEV)
    ps.set_q(0, g.standard_normal((n, r)).astype(np.float32))
    ps.view(ps.grads, 0).copy_(torch.from_numpy(M).to(DEV))
    ps.compress(mhat=True)
    torch.cuda.synchronize()
    # rank-3 input at r = 4: the fourth column is dependent and zeroed
    assert rel(cpu(ps.view(ps.mhat, 0)), M) <= 1e-5
    assert np.linalg.norm(cpu(ps.view(ps.err, 0))) <= 1e-5 * np.linalg.norm(M)
    Ph = cpu(ps.p_hat(0))
    assert oracle.orthonormality_error(Ph) <= ORTH_TOL


@pytest.mark.parametrize("m,n,k,r", [(1000, 700, 5, 20), (777, 1290, 16, 33), (1500, 600, 30, 50)])
def test_rank_deficient_matrix_core(m, n, k, r):
    # An exactly rank-k matrix at rank r > k on the matrix-core path (padded
    # ranks 32 / 48 / 64, ragged row and column tails): columns k .. r-1 of
    # P = M Q are dependent, so the Gram-Schmidt rule zeroes them exactly;
    # the first k match the oracle's Gram-Schmidt of the same P, and M is
    # recovered with E ~ 0.
    g = np.random.default_rng(100 + r)
    M = (g.standard_normal((m, k)) @ g.standard_normal((k, n))).astype(np.float32)
    q0 = g.standard_normal((n, r)).astype(np.float32)
    say(f"[rank-deficient] {m}x{n}, true rank {k}, r = {r}")
    ps = PowerSGD([(m, n)], r, device=DEV)
    ps.set_q(0, q0)
    ps.view(ps.grads, 0).copy_(torch.from_numpy(M).to(DEV))
    ps.compress(mhat=True)
    torch.cuda.synchronize()
    Ph = cpu(ps.p_hat(0))
    assert not Ph[:, k:].any(), "dependent columns must be zero"
    assert oracle.orthonormality_error(Ph[:, :k]) <= ORTH_TOL
    Ph_ref = oracle.gram_schmidt(M.astype(np.float64) @ q0.astype(np.float64))
    assert not Ph_ref[:, k:].any()
    assert rel(Ph, Ph_ref) <= REL_TOL
    assert rel(cpu(ps.view(ps.mhat, 0)), M) <= 1e-5
    assert np.linalg.norm(cpu(ps.view(ps.err, 0))) <= 1e-5 * np.linalg.norm(M)


def test_decompress_equals_fused_and_is_deterministic():
    wl = W.ModelSetWorkload(W.resnet18_cifar_set(), "resnet18", seed=2)
    shapes = [s for _, s in wl.tensors]
    outs = []
    for rep in range(2):
        ps = PowerSGD(shapes, 2, device=DEV)
        for i in ps.compressed():
            ps.set_q(i, wl.q0(i, 2))
        for t in (1, 2):
            for i in range(len(shapes)):
                ps.view(ps.grads, i).copy_(torch.from_numpy(wl.grad(i, t)).to(DEV))
            ps.compress(mhat=True)
        other = torch.zeros_like(ps.mhat)
        ps.decompress(other)
        torch.cuda.synchronize()
        assert torch.equal(other, ps.mhat)
        outs.append((ps.p.clone(), ps.q.clone(), ps.err.clone(), ps.mhat.clone()))
    for a, b in zip(*outs):
        assert torch.equal(a, b), "run-to-run results differ"


def test_mhat_may_alias_grads():
    wl = W.SmallMatrixWorkload()
    ref = PowerSGD([(256, 128)], 2, device=DEV)
    ali = PowerSGD([(256, 128)], 2, device=DEV)
    for ps in (ref, ali):
        ps.set_q(0, wl.Q0)
        ps.view(ps.grads, 0).copy_(torch.from_numpy(wl.grads[0]).to(DEV))
    ref.compress(mhat=True)
    ali.compress(mhat_buf=ali.grads)
    torch.cuda.synchronize()
    assert torch.equal(ref.mhat, ali.grads) and torch.equal(ref.err, ali.err)


def test_hooks_identity_and_failure():
    wl = W.SmallMatrixWorkload()
    calls = []

    def ident(buf, count, stream):
        calls.append(count)
        return 0

    hook = B.make_hook(ident)
    a = PowerSGD([(256, 128), (33,)], 2, device=DEV)
    b = PowerSGD([(256, 128), (33,)], 2, device=DEV)
    for ps in (a, b):
        ps.set_q(0, wl.Q0)
        ps.view(ps.grads, 0).copy_(torch.from_numpy(wl.grads[0]).to(DEV))
        ps.view(ps.grads, 1).fill_(0.5)
    a.compress(mhat=True, hook=hook)
    b.compress(mhat=True)
    torch.cuda.synchronize()
    assert calls == [a.info["p_buffer_elems"], a.info["q_elems"]]
    assert torch.equal(a.mhat, b.mhat) and torch.equal(a.err, b.err)
    assert torch.all(a.view(a.mhat, 1) == 0.5)

    # a failing hook aborts the call with PSGD_ERR_HOOK
    fail = B.make_hook(lambda buf, count, stream: 1)
    c = PowerSGD([(256, 128)], 2, device=DEV)
    c.set_q(0, wl.Q0)
    c.view(c.grads, 0).copy_(torch.from_numpy(wl.grads[0]).to(DEV))
    with pytest.raises(B.PsgdError) as e:
        c.compress(mhat=True, hook=fail)
    assert e.value.status == B.PSGD_ERR_HOOK
    torch.cuda.synchronize()
    # after a failure past the first pass E holds M = G + E_old (= G here)
    assert torch.equal(c.view(c.err, 0), c.view(c.grads, 0))


@pytest.mark.parametrize("power_iters", [1, 3])
def test_mean_hook_over_simulated_workers_matches_oracle(power_iters):
    # W workers in lockstep on one GPU: each hook call averages the buffer
    # across workers (device-side, on the stream), as an all-reduce-mean would.
    # Linearity ("Linearity of compressor", anthology note 152, Concepts)
    # makes the shared P_hat and Q equal those of the averaged gradient.  The
    # pass-through vector is averaged once, with the first P, whatever the
    # number of iterations: its value is the single mean, bit for bit.
    import threading

    Wn, m, n, r, nv = 3, 300, 200, 2, 333
    g = np.random.default_rng(9)
    Ms = [g.standard_normal((m, n)).astype(np.float32) for _ in range(Wn)]
    vs = [g.standard_normal(nv).astype(np.float32) for _ in range(Wn)]
    q0 = g.standard_normal((n, r)).astype(np.float32)
    workers = [PowerSGD([(m, n), (nv,)], r, device=DEV) for _ in range(Wn)]
    for w, M, v in zip(workers, Ms, vs):
        w.set_q(0, q0)
        w.view(w.grads, 0).copy_(torch.from_numpy(M).to(DEV))
        w.view(w.grads, 1).copy_(torch.from_numpy(v).to(DEV))
    torch.cuda.synchronize()
    barrier = threading.Barrier(Wn)
    bufs = {}
    lock = threading.Lock()

    def make(wid):
        def hook(buf, count, stream):
            torch.cuda.synchronize()
            with lock:
                bufs[wid] = (buf, count)
            barrier.wait()
            if wid == 0:
                views = []
                for k in range(Wn):
                    ptr, cnt = bufs[k]
                    full = workers[k].p if ptr == workers[k].p.data_ptr() else workers[k].q
                    assert full.data_ptr() == ptr
                    views.append(full[:cnt])
                mean = sum(views) / Wn
                for v in views:
                    v.copy_(mean)
                torch.cuda.synchronize()
            barrier.wait()
            return 0
        return B.make_hook(hook)

    hooks = [make(k) for k in range(Wn)]
    errs = []

    def run(k):
        try:
            workers[k].compress(mhat=True, hook=hooks[k], power_iters=power_iters)
            torch.cuda.synchronize()
        except Exception as ex:  # pragma: no cover
            errs.append(ex)

    th = [threading.Thread(target=run, args=(k,)) for k in range(Wn)]
    for t in th:
        t.start()
    for t in th:
        t.join(60)
    assert not errs
    Ph, Qn, Es = oracle.compress_workers(Ms, q0, power_iters=power_iters)
    vmean = (sum(torch.from_numpy(v).to(DEV) for v in vs) / Wn).cpu()  # the hook's own fp32 mean, once
    for k, w in enumerate(workers):
        assert rel(cpu(w.p_hat(0)), Ph) <= REL_TOL
        assert rel(cpu(w.q_of(0)), Qn) <= REL_TOL
        assert rel(cpu(w.view(w.err, 0)), Es[k]) <= REL_TOL
        assert torch.equal(w.view(w.mhat, 1).cpu(), vmean), "pass-through values averaged more than once"


def test_timing_records_every_stage():
    wl = W.SmallMatrixWorkload()
    ps = PowerSGD([(256, 128), (9,)], 2, device=DEV)
    ps.set_q(0, wl.Q0)
    B.psgd_timing_enable(ps.plan, True)
    for _ in range(3):
        ps.compress(mhat=True)
    ms, n = B.psgd_timing_read(ps.plan)
    assert n[B.PSGD_STAGE_EF_P] == 3 and n[B.PSGD_STAGE_RESIDUAL] == 3 and n[B.PSGD_STAGE_GS] == 3
    assert all(x >= 0 for x in ms) and ms[B.PSGD_STAGE_EF_P] > 0
    ms2, n2 = B.psgd_timing_read(ps.plan)
    assert sum(n2) == 0


def test_stream_copy():
    x = torch.randn(1 << 20, device=DEV)
    y = torch.empty_like(x)
    B.psgd_stream_copy(y.data_ptr(), x.data_ptr(), x.numel(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(x, y)


@pytest.mark.parametrize("nin,nout", [(0, 1), (1, 0), (1, 1), (2, 1), (1, 2), (3, 2), (3, 0)])
def test_stream_probe(nin, nout):
    """The bandwidth probe moves the bytes it claims: every output is the
    sum of the inputs, and without outputs the per-workgroup sums add up to
    the total (a ragged length exercises the bounds)."""
    n = (1 << 20) + 4 * 37
    ins = [torch.randn(n, device=DEV) for _ in range(nin)]
    outs = [torch.full((n,), 7.0, device=DEV) for _ in range(nout)]
    sink = torch.zeros(B.PSGD_PROBE_SINK_FLOATS, device=DEV)
    B.psgd_stream_probe([t.data_ptr() for t in ins], [t.data_ptr() for t in outs], n, sink.data_ptr(),
                        torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    want = sum(t.double() for t in ins) if ins else torch.zeros(n, dtype=torch.float64, device=DEV)
    for o in outs:
        assert torch.allclose(o.double(), want, rtol=0, atol=1e-5)
    if nout == 0:
        got = sink.double().sum().item()
        assert abs(got - want.sum().item()) <= 1e-3 * max(1.0, want.abs().sum().item() / n ** 0.5)


def test_stream_probe_sink_shared_by_workgroups():
    """More workgroups than sink floats: the wavefront sums still add up to
    the total."""
    n = (1 << 27) + 4 * 37
    x = torch.randn(n, device=DEV)
    sink = torch.zeros(B.PSGD_PROBE_SINK_FLOATS, device=DEV)
    B.psgd_stream_probe([x.data_ptr()], [], n, sink.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    want = x.double().sum().item()
    assert abs(sink.double().sum().item() - want) <= 1e-3 * max(1.0, x.abs().double().sum().item() / n ** 0.5)
    del x


@pytest.mark.parametrize("nin,nout,alias", [(1, 1, (0,)), (2, 1, (1,)), (1, 2, (0, None)), (3, 2, (1, 2))])
def test_stream_probe_in_place(nin, nout, alias):
    """The in-place forms of the passes' patterns: an output that is one of
    the inputs ends as the sum of the inputs' values before the call."""
    n = (1 << 20) + 4 * 37
    ins = [torch.randn(n, device=DEV) for _ in range(nin)]
    want = sum(t.double() for t in ins)
    extra = [torch.full((n,), 7.0, device=DEV) for _ in range(nout)]
    outs = [ins[alias[j]] if alias[j] is not None else extra[j] for j in range(nout)]
    sink = torch.zeros(B.PSGD_PROBE_SINK_FLOATS, device=DEV)
    B.psgd_stream_probe([t.data_ptr() for t in ins], [t.data_ptr() for t in outs], n, sink.data_ptr(),
                        torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for o in outs:
        assert torch.allclose(o.double(), want, rtol=0, atol=1e-5)


def test_empty_and_vector_only_plans_run():
    ps = PowerSGD([(5,), (7,)], 2, device=DEV)
    ps.view(ps.grads, 0).fill_(1.0)
    ps.view(ps.grads, 1).fill_(2.0)
    ps.compress(mhat=True)
    torch.cuda.synchronize()
    assert torch.all(ps.view(ps.mhat, 0) == 1.0) and torch.all(ps.view(ps.mhat, 1) == 2.0)
    e = PowerSGD([], 3, device=DEV)
    e.compress(mhat=True)
    torch.cuda.synchronize()
