"""The plain C client (csrc/c_smoke.c, built by build() with gcc against
libpsgd.so and the HIP runtime, no Python in the process) on the GPU: exact
recovery of a rank-2 matrix at rank 4 and an exact bias pass-through."""
import os
import subprocess

import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import rank_gradient_compression_amd as R  # noqa: E402
from gpu_util import say  # noqa: E402

pytestmark = pytest.mark.gpu


def test_c_client_runs_the_whole_call_sequence():
    exe = os.path.join(os.path.dirname(R.__file__), "psgd_c_smoke")
    assert os.path.exists(exe)
    say("[c-abi] running the C client")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    say(res.stdout.strip() + (" | " + res.stderr.strip() if res.stderr.strip() else ""))
    assert res.returncode == 0 and "c-abi smoke: ok" in res.stdout
