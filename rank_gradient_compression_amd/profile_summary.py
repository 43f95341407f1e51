"""Short markdown summaries of rocprofv3 output for the library's kernels.

    python -m rank_gradient_compression_amd.profile_summary trace STATS_CSV "COMMAND" "TITLE"
    python -m rank_gradient_compression_amd.profile_summary bytes FETCH_CSV WRITE_CSV "CMD_FETCH" "CMD_WRITE" "TITLE"
    python -m rank_gradient_compression_amd.profile_summary dispatches KERNEL TRACE_CSV "CMD_TRACE"
        COUNTER_CSV "CMD_COUNTERS" [COUNTER_CSV "CMD_COUNTERS" ...] "TITLE"
    python -m rank_gradient_compression_amd.profile_summary counters COUNTER_CSV "CMD" [COUNTER_CSV "CMD" ...]
        "TITLE"

`counters` averages every counter of one or more `--pmc` runs per dispatch of
each library kernel, and derives the matrix-core busy fraction (of SIMD
cycles while the kernel runs), the matrix-core fp32 / fp64 flops (512 per
MOPS count), LDS
bank-conflict cycles per LDS instruction and the share of wave time spent
waiting to issue, where the counters they need are present.

`dispatches` lists every dispatch of one kernel in launch order: its duration
from a `--kernel-trace` kernel_trace.csv and its counters from one or more
`--pmc` counter_collection.csv files of the same program (the n-th dispatch
of the kernel in each file).  `trace` reads a `--kernel-trace --stats`
kernel_stats.csv; `bytes` reads the
counter_collection.csv of one `--pmc FETCH_SIZE` run and one `--pmc
WRITE_SIZE` run of the same program.  The byte counters are calibrated with
the library's 16-byte copy kernel over 4 GiB (`psgd_stream_copy`, which the
benchmark runs first): each counter is scaled so that the copy reads and
writes exactly 4 GiB.  The machine-readable block records, per kernel, the
scaled bytes per launch and a hash of the code (comments stripped) of the
source file that defines the kernel and of the shared headers, so a reader can
tell when the counters no longer describe the code.
"""
from __future__ import annotations

import collections
import csv
import hashlib
import json
import os
import re
import statistics
import sys

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
SHARED_HEADERS = ("psgd_kernels.h", "psgd_tables.h")
COPY_BYTES = 4 * (1 << 30)


def source_file(kernel: str) -> str:
    """The source file that defines a library kernel (by its name)."""
    k = kernel.replace("psgd::", "").replace("void ", "").strip()
    if k.startswith(("k_mfma", "k_psum", "k_gram", "k_apply")):
        return "kernels_mfma.hip"
    if "k_init_q" in k:
        return "kernels_rng.hip"
    if k.startswith("k_stream"):
        return "kernels_probe.hip"
    if k.startswith(("k_sumsq", "k_cross", "k_overlap")):
        return "kernels_diag.hip"
    if k.startswith("k_round_fp8"):
        return "kernels_payload.hip"
    return "kernels_valu.hip"


def _code_only(text: str) -> str:
    """C++ source without comments and blank-line / trailing-space noise, so
    that editing a comment does not count as changing the kernel.  (The
    kernel sources hold no string literals with comment markers.)"""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def source_hash(kernel: str) -> str:
    """Hash of the code (comments stripped) of the file that defines the
    kernel and of the shared headers."""
    h = hashlib.sha256()
    for f in (source_file(kernel),) + SHARED_HEADERS:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def short(k: str) -> str:
    k = k.replace("psgd::", "")
    i = k.find("(")
    return k[:i] if i > 0 else k


def trace(stats_csv: str, cmd: str, title: str) -> str:
    rows = list(csv.DictReader(open(stats_csv)))
    out = [f"# {title}\n", "Command:\n", f"```\n{cmd}\n```\n",
           "| kernel | calls | avg (us) | min (us) | max (us) | share of GPU time |", "|---|---|---|---|---|---|"]
    for r in rows:
        if "psgd" not in r["Name"]:
            continue
        out.append(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f}% |")
    out.append(f"\nSummarised from `{os.path.basename(stats_csv)}` by "
               "`python -m rank_gradient_compression_amd.profile_summary trace`.")
    return "\n".join(out) + "\n"


def _counters(path: str, counter: str):
    agg = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            agg[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return agg


def hbm_bytes(fetch_csv: str, write_csv: str, cmd_f: str, cmd_w: str, title: str) -> str:
    f = _counters(fetch_csv, "FETCH_SIZE")
    w = _counters(write_csv, "WRITE_SIZE")
    copy = [k for k in f if "k_stream_copy" in k][0]
    ff = COPY_BYTES / 1024 / statistics.mean(f[copy])
    wf = COPY_BYTES / 1024 / statistics.mean(w[copy])
    out = [f"# {title}\n", "Commands (one counter per run):\n", f"```\n{cmd_f}\n{cmd_w}\n```\n",
           f"Calibration: `k_stream_copy` over 4 GiB (reads 4 GiB, writes 4 GiB) reads FETCH_SIZE = "
           f"{statistics.mean(f[copy]):.4g} KiB and WRITE_SIZE = {statistics.mean(w[copy]):.4g} KiB per launch, so "
           f"FETCH_SIZE is scaled by {ff:.3f} and WRITE_SIZE by {wf:.3f} below.\n",
           "| kernel | launches | FETCH_SIZE (KiB, raw) | WRITE_SIZE (KiB, raw) | read GB (scaled) | write GB (scaled) |",
           "|---|---|---|---|---|---|"]
    blob = {}
    for k in f:
        if "psgd" not in k or k == copy:
            continue
        fr = statistics.mean(f[k])
        wr = statistics.mean(w.get(k, [0.0]))
        out.append(f"| `{short(k)}` | {len(f[k])} | {fr:.6g} | {wr:.6g} | {fr * ff * 1024 / 1e9:.3f} | "
                   f"{wr * wf * 1024 / 1e9:.3f} |")
        blob[short(k)] = {"launches": len(f[k]), "read_bytes": fr * ff * 1024, "write_bytes": wr * wf * 1024,
                          "source": source_file(k), "source_hash": source_hash(k)}
    out.append("\nMachine-readable (per launch, scaled bytes; `source_hash` = sha256 prefix of the kernel's source "
               "file and the shared headers when the counters were taken):\n")
    out.append("```json\n" + json.dumps({"fetch_scale": ff, "write_scale": wf, "kernels": blob}) + "\n```")
    out.append("\nSummarised from the two runs' `counter_collection.csv` by "
               "`python -m rank_gradient_compression_amd.profile_summary bytes`.")
    return "\n".join(out) + "\n"


def dispatches(kernel: str, trace_csv: str, cmd_trace: str, counter_runs, title: str) -> str:
    """Every dispatch of `kernel` in launch order: duration from a kernel
    trace, counters from one or more counter-collection runs (matched by the
    dispatch's position among the kernel's dispatches in each file)."""
    rows = [r for r in csv.DictReader(open(trace_csv)) if kernel in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6 for r in rows]
    cols, per = [], []
    for path, _ in counter_runs:
        by = collections.OrderedDict()
        for r in csv.DictReader(open(path)):
            if kernel in r["Kernel_Name"]:
                by.setdefault(int(r["Dispatch_Id"]), {})[r["Counter_Name"]] = float(r["Counter_Value"])
        seq = [by[k] for k in sorted(by)]
        names = sorted({n for c in seq for n in c})
        cols += names
        per.append((names, seq))
    out = [f"# {title}\n", "Commands:\n", "```\n" + "\n".join([cmd_trace] + [c for _, c in counter_runs]) + "\n```\n",
           "| dispatch | duration (ms, trace run) | " + " | ".join(cols) + " |", "|---" * (2 + len(cols)) + "|"]
    n = max([len(durs)] + [len(seq) for _, seq in per])
    for i in range(n):
        cells = [str(i), f"{durs[i]:.3f}" if i < len(durs) else ""]
        for names, seq in per:
            cells += [f"{seq[i][c]:.4g}" if i < len(seq) and c in seq[i] else "" for c in names]
        out.append("| " + " | ".join(cells) + " |")
    out.append("\nSummarised by `python -m rank_gradient_compression_amd.profile_summary dispatches`.")
    return "\n".join(out) + "\n"


N_CU = 256  # compute units of the device the counters are read on (MI355X)
N_XCD = 8   # its accelerator dies: GRBM_GUI_ACTIVE is summed over them


def counters(runs, title: str) -> str:
    """Mean per dispatch of every counter of the given `--pmc` runs, per
    library kernel, with derived figures (see the module docstring)."""
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    order = []
    for path, _ in runs:
        per = collections.defaultdict(dict)
        for r in csv.DictReader(open(path)):
            if "psgd" not in r["Kernel_Name"]:
                continue
            per[(short(r["Kernel_Name"]), int(r["Dispatch_Id"]))][r["Counter_Name"]] = float(r["Counter_Value"])
        for (k, _), cs in per.items():
            if k not in order:
                order.append(k)
            for c, v in cs.items():
                vals[k][c].append(v)
    names = sorted({c for k in vals for c in vals[k]})
    out = [f"# {title}\n", "Commands (one counter set per run):\n",
           "```\n" + "\n".join(c for _, c in runs) + "\n```\n",
           "Mean per dispatch.  Derived: matrix-core busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / "
           f"{N_XCD} dies x {N_CU} CUs x 4 SIMDs) (the busy count is 32 cycles per 16x16x4 fp32 instruction, "
           "summed over the SIMDs; GRBM_GUI_ACTIVE is summed over the dies); fp32 / fp64 matrix-core GFLOP = "
           "512 x SQ_INSTS_VALU_MFMA_MOPS_F32 / F64; "
           "LDS conflict cycles per LDS instruction = SQ_LDS_BANK_CONFLICT / SQ_INSTS_LDS; issue wait = "
           "SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (both in quad-cycles).\n"]
    derived = [("MFMA busy", lambda m: m["SQ_VALU_MFMA_BUSY_CYCLES"] / (m["GRBM_GUI_ACTIVE"] / N_XCD * N_CU * 4),
                "{:.1%}"),
               ("MFMA f32 GFLOP", lambda m: 512 * m["SQ_INSTS_VALU_MFMA_MOPS_F32"] / 1e9, "{:.3f}"),
               ("MFMA f64 GFLOP", lambda m: 512 * m["SQ_INSTS_VALU_MFMA_MOPS_F64"] / 1e9, "{:.3f}"),
               ("LDS conflict cyc / LDS inst", lambda m: m["SQ_LDS_BANK_CONFLICT"] / m["SQ_INSTS_LDS"], "{:.3f}"),
               ("issue wait", lambda m: m["SQ_WAIT_INST_ANY"] / m["SQ_WAVE_CYCLES"], "{:.1%}")]
    rows = []
    for k in order:
        m = {c: statistics.mean(v) for c, v in vals[k].items()}
        cells = [f"`{k}`", str(max(len(v) for v in vals[k].values()))]
        dcells = []
        for _, f, fmt in derived:
            try:
                dcells.append(fmt.format(f(m)))
            except (KeyError, ZeroDivisionError):
                dcells.append("")
        cells += dcells + [f"{m[c]:.4g}" if c in m else "" for c in names]
        rows.append("| " + " | ".join(cells) + " |")
    head = ["kernel", "dispatches"] + [d[0] for d in derived] + names
    out += ["| " + " | ".join(head) + " |", "|---" * len(head) + "|"] + rows
    out.append("\nSummarised by `python -m rank_gradient_compression_amd.profile_summary counters`.")
    return "\n".join(out) + "\n"


def main(argv) -> int:
    if len(argv) >= 5 and argv[1] == "trace":
        sys.stdout.write(trace(argv[2], argv[3], argv[4]))
        return 0
    if len(argv) >= 7 and argv[1] == "bytes":
        sys.stdout.write(hbm_bytes(*argv[2:7]))
        return 0
    if len(argv) >= 8 and argv[1] == "dispatches" and len(argv) % 2 == 0:
        runs = [(argv[i], argv[i + 1]) for i in range(5, len(argv) - 1, 2)]
        sys.stdout.write(dispatches(argv[2], argv[3], argv[4], runs, argv[-1]))
        return 0
    if len(argv) >= 5 and argv[1] == "counters" and len(argv) % 2 == 1:
        runs = [(argv[i], argv[i + 1]) for i in range(2, len(argv) - 1, 2)]
        sys.stdout.write(counters(runs, argv[-1]))
        return 0
    sys.stderr.write(__doc__)
    return 2


if __name__ == "__main__":
    sys.exit(main(sys.argv))
