"""psgd_compress_noalloc, the entry point that uses the library's static
device scratch instead of a caller workspace, against psgd_compress: the same
kernels on the same inputs, so every output must agree bit for bit.  Two calls
in a row with different plans, the second on a smaller input, so the second
finds the first one's tables and scratch in the static array; then further
calls with the second plan (tables kept) and the first again (uploaded
again)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import workloads as W  # noqa: E402
from gpu_util import say  # noqa: E402
from rank_gradient_compression_amd import binding as B  # noqa: E402
from rank_gradient_compression_amd.torch_api import PowerSGD  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

# larger set on the matrix-core path (rank 16: P partials, Q partials and
# Gram scratch all in use), smaller set on the vector path
BIG = ([(300, 650), (257, 4099), (97, 1030), (33, 27), (5,), (640, 512)], 16, 201)
SMALL = ([(256, 128), (9,), (70, 40)], 2, 202)


class Pair:
    """The same plan twice: one object steps with psgd_compress (its own
    workspace), the other with psgd_compress_noalloc."""

    def __init__(self, shapes, rank, seed):
        tensors = [(str(i), s) for i, s in enumerate(shapes)]
        self.wl = W.ModelSetWorkload(tensors, "plain", seed=seed)
        self.n = len(shapes)
        self.ref = PowerSGD(shapes, rank, device=DEV)
        self.new = PowerSGD(shapes, rank, device=DEV)
        assert self.ref.info["workspace_bytes"] <= B.PSGD_NOALLOC_SCRATCH_BYTES
        for ps in (self.ref, self.new):
            for i in ps.compressed():
                ps.set_q(i, self.wl.q0(i, rank))
        self.t = 0

    def step(self, tag):
        self.t += 1
        for i in range(self.n):
            g = torch.from_numpy(self.wl.grad(i, self.t)).to(DEV)
            self.ref.view(self.ref.grads, i).copy_(g)
            self.new.view(self.new.grads, i).copy_(g)
        say(f"[noalloc] {tag}: step {self.t}")
        self.ref.compress(mhat=True)
        self.new.compress(mhat=True, noalloc=True)
        torch.cuda.synchronize()
        for name in ("p", "q", "err", "mhat"):
            a, b = getattr(self.ref, name), getattr(self.new, name)
            assert torch.equal(a, b), f"{tag} step {self.t}: {name} differs"


def test_noalloc_matches_workspace_entry_point():
    big = Pair(*BIG)
    small = Pair(*SMALL)
    assert small.ref.info["flat_elems"] < big.ref.info["flat_elems"]
    big.step("larger set, rank 16")
    small.step("smaller set, rank 2 (after the larger one)")
    small.step("smaller set again (tables kept)")
    big.step("larger set again (tables uploaded again)")
    for ps in (big.ref, big.new, small.ref, small.new):
        ps.close()


def test_noalloc_rejects_a_plan_beyond_the_static_scratch():
    shapes = [s for _, s in W.llama7b_set()]
    rows = [s[0] for s in shapes]
    cols = [s[1] for s in shapes]
    p = B.psgd_plan_create(rows, cols, 4)
    try:
        x = torch.zeros(64, device=DEV)
        with pytest.raises(B.PsgdError) as e:
            B.psgd_compress_noalloc(p, x.data_ptr(), x.data_ptr(), 0, x.data_ptr(), x.data_ptr(), 0, None, None,
                                    torch.cuda.current_stream().cuda_stream)
        assert e.value.status == B.PSGD_ERR_WORKSPACE
    finally:
        B.psgd_plan_destroy(p)
