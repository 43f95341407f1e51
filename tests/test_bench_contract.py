"""Host-side checks of bench.py's contract: one GPU only, the algorithmic
bytes per element of each step variant, and the measured-traffic lookup that
feeds the roofline's `traffic` field."""
import json
import os
import subprocess
import sys

import pytest

import bench
from rank_gradient_compression_amd import profile_summary as PS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ELEMS_7B = 6738149376  # fp32 elements of the 226-matrix 7B-shaped set


def test_more_than_one_gpu_exits_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    line = json.loads(p.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_algorithmic_bytes_per_element():
    # pass 1 reads G, E and writes M (12 B; +8 for u), pass 2 reads M (4 B),
    # pass 3 reads M, writes E (8 B; +4 for M_hat); the deferred residual
    # moves the E update into pass 1 and leaves pass 3 the M_hat write
    assert sum(bench.step_bytes(False).values()) == 28.0
    assert sum(bench.step_bytes(False, mhat=False).values()) == 24.0
    assert sum(bench.step_bytes(False, momentum=True, mhat=False).values()) == 32.0
    assert sum(bench.step_bytes(False, deferred=True).values()) == 20.0


def test_headline_traffic_matches_algorithmic_bytes():
    prof = "hbm_bytes_llama7b_r4_fused.md"
    assert os.path.exists(os.path.join(ROOT, "profiles", prof))
    t = bench.measured_traffic("k_ef_p", prof)
    if t is None:
        pytest.skip("the kernel source changed since the byte counters were taken")
    alg = 12.0 * ELEMS_7B
    assert abs(t - alg) <= 0.02 * alg, (t, alg)


def test_traffic_is_null_for_a_missing_profile_or_a_changed_source(monkeypatch):
    assert bench.measured_traffic("k_ef_p", "no_such_profile.md") is None
    monkeypatch.setattr(PS, "source_hash", lambda kernel: "0000000000000000")
    assert bench.measured_traffic("k_ef_p", "hbm_bytes_llama7b_r4_fused.md") is None
