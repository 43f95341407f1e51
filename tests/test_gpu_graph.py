"""psgd_compress and psgd_refresh captured in a HIP graph (no hook, timing
off: the calls then only enqueue kernels) and replayed: every replay, with eager work and
synchronisations in between, must give bit for bit what the same sequence of
eager calls gives on an identical twin (the kernels are deterministic)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import workloads as W  # noqa: E402
from gpu_util import say  # noqa: E402
from rank_gradient_compression_amd.torch_api import PowerSGD  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.mark.parametrize("rank,beta,payload", [(2, None, None), (4, 0.9, None), (16, None, None),
                                                (4, None, "bf16"), (4, None, "fp8"), (32, None, "fp8")])
def test_graph_replays_match_eager_calls(rank, beta, payload):
    shapes = [(300, 650), (257, 1030), (64, 3, 3, 3), (11,), (2, 2)]
    tensors = [(str(i), s) for i, s in enumerate(shapes)]
    wl = W.ModelSetWorkload(tensors, "plain", seed=190 + rank)
    a = PowerSGD(shapes, rank, device=DEV, momentum_beta=beta)
    b = PowerSGD(shapes, rank, device=DEV, momentum_beta=beta)
    kw = {"payload_bf16": payload == "bf16", "payload_fp8": payload == "fp8"}
    for ps in (a, b):
        for i in ps.compressed():
            ps.set_q(i, wl.q0(i, rank))
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        a.compress(mhat=True, **kw)
    for t in range(1, 5):
        for ps in (a, b):
            for i in range(len(shapes)):
                ps.view(ps.grads, i).copy_(torch.from_numpy(np.ascontiguousarray(wl.grad(i, t))).to(DEV))
        torch.cuda.synchronize()
        say(f"[graph r={rank} beta={beta} payload={payload}] replay {t}")
        graph.replay()
        b.compress(mhat=True, **kw)
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device=DEV).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        del junk
        for name in ("p", "q", "err", "mhat") + (("mom",) if beta is not None else ()):
            assert torch.equal(getattr(a, name), getattr(b, name)), f"replay {t}: {name} differs"


@pytest.mark.parametrize("rank", [4, 32])
def test_refresh_graph_replays_match_eager_calls(rank):
    """psgd_refresh (setting the start Q, then the rounds) captured once and
    replayed on changing matrices: bit for bit the eager calls' Q."""
    m, n = 700, 520
    a = PowerSGD([(m, n)], rank, device=DEV)
    b = PowerSGD([(m, n)], rank, device=DEV)
    q0 = torch.from_numpy(W.gaussian_q0(n, rank, 77)).float().to(DEV)
    ma = torch.zeros(a.grads.numel(), device=DEV)
    mb = torch.zeros_like(ma)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        a.set_q(0, q0)
        a.refresh(0, ma, 3)
    g = torch.Generator(device=DEV).manual_seed(rank)
    for t in range(1, 4):
        x = torch.randn(m, n, device=DEV, generator=g)
        a.view(ma, 0).copy_(x)
        b.view(mb, 0).copy_(x)
        torch.cuda.synchronize()
        say(f"[graph refresh r={rank}] replay {t}")
        graph.replay()
        b.set_q(0, q0)
        b.refresh(0, mb, 3)
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        del junk
        assert torch.equal(a.q_of(0), b.q_of(0)), f"replay {t}: Q differs"
