"""Short markdown summaries of rocprofv3 output for the library's kernels.

    python -m rank_gradient_compression_amd.profile_summary trace STATS_CSV "COMMAND" "TITLE"
    python -m rank_gradient_compression_amd.profile_summary bytes FETCH_CSV WRITE_CSV "CMD_FETCH" "CMD_WRITE" "TITLE"
    python -m rank_gradient_compression_amd.profile_summary dispatches KERNEL TRACE_CSV "CMD_TRACE"
        COUNTER_CSV "CMD_COUNTERS" [COUNTER_CSV "CMD_COUNTERS" ...] "TITLE"

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
    sys.stderr.write(__doc__)
    return 2


if __name__ == "__main__":
    sys.exit(main(sys.argv))
