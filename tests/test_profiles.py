"""Host-side checks of the committed rocprofv3 summaries and of the
summariser that writes them: every kernel in a byte summary is attributed to
the source file that defines it (the file whose code hash decides whether the
counters still describe the kernel), and the summaries' figures are
self-consistent."""
import glob
import json
import os
import re

from rank_gradient_compression_amd import profile_summary as PS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rank_gradient_compression_amd", "csrc")


def _blob(path):
    text = open(path).read()
    return json.loads(text.split("```json", 1)[1].split("```", 1)[0])


def _base_name(kernel):
    k = kernel.replace("void ", "").replace("psgd::", "").strip()
    return re.match(r"[A-Za-z_][A-Za-z0-9_]*", k).group(0)


def _defines(source, name):
    code = open(os.path.join(CSRC, source)).read()
    return re.search(r"__global__[^;{]*\b" + name + r"\s*\(", code) is not None


def test_byte_summaries_exist():
    assert glob.glob(os.path.join(ROOT, "profiles", "hbm_bytes_*.md"))


def test_kernels_attributed_to_their_defining_file():
    for path in glob.glob(os.path.join(ROOT, "profiles", "hbm_bytes_*.md")):
        for kernel, rec in _blob(path)["kernels"].items():
            name = _base_name(kernel)
            assert rec["source"] == PS.source_file(kernel), (path, kernel)
            assert _defines(rec["source"], name), f"{os.path.basename(path)}: {name} is not defined in {rec['source']}"


def test_source_file_map_covers_every_kernel():
    # every __global__ kernel of the library maps to the file that defines it
    for source in ("kernels_valu.hip", "kernels_mfma.hip", "kernels_rng.hip", "kernels_probe.hip", "kernels_diag.hip",
                   "kernels_payload.hip"):
        code = open(os.path.join(CSRC, source)).read()
        for name in set(re.findall(r"__global__[^;{(]*?\b(k_[A-Za-z0-9_]+)\s*\(", code)):
            assert PS.source_file(f"void {name}<4>") == source, (name, source)
            assert PS.source_file(name) == source, (name, source)


def test_scaled_bytes_match_raw_counters():
    # per kernel: read bytes = FETCH_SIZE (KiB, the table's raw column) x 1024
    # x fetch_scale, write bytes likewise with write_scale (the table prints
    # six significant digits)
    row = re.compile(r"^\| `([^`]+)` \| (\d+) \| ([0-9.e+-]+) \| ([0-9.e+-]+) \| ([0-9.]+) \| ([0-9.]+) \|$")
    for path in glob.glob(os.path.join(ROOT, "profiles", "hbm_bytes_*.md")):
        b = _blob(path)
        assert 1.5 < b["fetch_scale"] < 2.5 and 0.5 < b["write_scale"] < 1.5
        seen = 0
        for line in open(path):
            m = row.match(line.strip())
            if not m:
                continue
            kernel, launches, fetch_kib, write_kib = m.group(1), int(m.group(2)), float(m.group(3)), float(m.group(4))
            rec = b["kernels"][kernel]
            assert rec["launches"] == launches
            for raw, scale, got in ((fetch_kib, b["fetch_scale"], rec["read_bytes"]),
                                    (write_kib, b["write_scale"], rec["write_bytes"])):
                want = raw * 1024.0 * scale
                assert abs(got - want) <= 1e-5 * max(want, 1.0) + 1024.0, (path, kernel, got, want)
            seen += 1
        assert seen == len(b["kernels"]), path
