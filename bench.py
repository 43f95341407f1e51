"""Throughput of the PowerSGD compression step on one MI355X.

Workload: the 7B-transformer shaped gradient set (32 layers of q,k,v,o
4096x4096, gate/up 11008x4096, down 4096x11008, plus 32000x4096 embedding and
head: 226 fp32 matrices, 6,738,149,376 elements), rank 4.  A step is one
psgd_compress call with the fused decompression: EF-add, P = M Q,
orthogonalisation, Q = M^T P_hat, residual E = M - P_hat Q^T and M_hat, all in
the library's HIP kernels.  The gradients are synthetic (seeded rank-16 signal
plus Gaussian noise, unit Frobenius norm per matrix) and resident in HBM
before timing starts.

Prints ONE JSON line.  `value` is gradient GB compressed per second
(4 bytes x elements / step time).
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "gradient GB compressed/s (EF+P+Q+E) and % HBM peak, 1×MI355X, r=2/4"
HBM_PEAK_GBS = 8000.0
# Algorithmic HBM bytes per gradient element for each kernel (fp32):
#   EF-add + P = M Q: read G, E, write M                  12 (20 with momentum: + read/write u)
#   Q = M^T P_hat: read M                                  4
#   residual (+ M_hat): read M, write E (+ write M_hat)    8 (12)
B_STAGE = {"ef_p": 12.0, "mtp": 4.0, "residual": 8.0}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--rank", type=int, default=4)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true", help="skip the plain-compress and momentum lines")
    ap.add_argument("--no-stage-timing", action="store_true")
    return ap.parse_args()


KERNEL_OF_STAGE = {"ef_p": "k_ef_p", "mtp": "k_mtp", "residual": "k_recon"}


def source_hash():
    import hashlib

    csrc = os.path.join(ROOT, "rank_gradient_compression_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(stage, rank, mhat):
    """HBM bytes per launch of the stage's kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary, or None when the summary does not cover
    this configuration or the library sources changed since it was taken."""
    if rank != 4 or not mhat:
        return None
    path = os.path.join(ROOT, "profiles", "hbm_bytes_llama7b_r4_fused.md")
    try:
        text = open(path).read()
        blob = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (OSError, IndexError, ValueError):
        return None
    if blob.get("source_hash") != source_hash():
        return None
    for name, v in blob["kernels"].items():
        if KERNEL_OF_STAGE.get(stage, "?") in name:
            return v["read_bytes"] + v["write_bytes"]
    return None


def stage_roofline(plan, B, n_steps, dense, momentum=False, mhat=True):
    ms, n = B.psgd_timing_read(plan)
    stages = {}
    for i, name in enumerate(B.STAGE_NAMES):
        if n[i]:
            stages[name] = {"ms_avg": ms[i] / n[i], "launches": n[i]}
    b = dict(B_STAGE)
    if momentum:
        b["ef_p"] = 20.0
    if mhat:
        b["residual"] = 12.0
    for name, s in stages.items():
        if name in b:
            s["bytes_alg"] = b[name] * dense
            s["gbs"] = s["bytes_alg"] / (s["ms_avg"] * 1e-3) / 1e9
            s["frac_hbm"] = s["gbs"] / HBM_PEAK_GBS
    return stages


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; multi-GPU aggregation is a caller hook "
                          "(all-reduce of P and Q) and is not benchmarked here", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    import workloads as W
    from rank_gradient_compression_amd import binding as B
    from rank_gradient_compression_amd.torch_api import PowerSGD

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tensors = W.llama7b_set(args.layers)
    shapes = [s for _, s in tensors]
    rank = args.rank
    log(f"bench: building plan for {len(shapes)} matrices, rank {rank}")
    ps = PowerSGD(shapes, rank, device=dev, with_mhat=True)
    dense = ps.info["dense_elems"]
    log(f"bench: generating {dense} synthetic gradient elements on the device")
    t0 = time.time()
    for i, (_, s) in enumerate(tensors):
        W.llama7b_grad_(ps.view(ps.grads, i), s[0], s[1], i, step=1)
        ps.set_q(i, W.llama7b_q0(s[1], rank, i, device=dev))
    torch.cuda.synchronize()
    log(f"bench: inputs ready in {time.time() - t0:.1f} s")
    stream = torch.cuda.current_stream()

    def run(label, call, steps, warmup, stage_timing=True):
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        B.psgd_timing_read(ps.plan)  # drop warm-up records
        if stage_timing:
            B.psgd_timing_enable(ps.plan, True)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        t_wall = time.perf_counter()
        ev[0].record(stream)
        for k in range(steps):
            call()
            ev[k + 1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_wall
        B.psgd_timing_enable(ps.plan, False)
        per = [ev[k].elapsed_time(ev[k + 1]) for k in range(steps)]
        total_ms = ev[0].elapsed_time(ev[steps])
        log(f"bench: {label}: {total_ms / steps:.3f} ms/step (median {statistics.median(per):.3f}, "
            f"wall {wall * 1e3 / steps:.3f})")
        return total_ms / steps, per

    # stream-copy ceiling on a 4 GiB buffer
    ncopy = 1 << 30
    src = torch.empty(ncopy, dtype=torch.float32, device=dev).normal_()
    dst = torch.empty_like(src)
    for _ in range(2):
        B.psgd_stream_copy(dst.data_ptr(), src.data_ptr(), ncopy, stream.cuda_stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(5):
        B.psgd_stream_copy(dst.data_ptr(), src.data_ptr(), ncopy, stream.cuda_stream)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 5 * 8 * ncopy / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    log(f"bench: stream copy ceiling {copy_gbs:.0f} GB/s")

    # headline: compress + fused decompression
    fused = lambda: ps.compress(mhat=True)  # noqa: E731
    ms_step, per = run("compress+decompress (fused)", fused, args.steps, args.warmup,
                       stage_timing=not args.no_stage_timing)
    stages = stage_roofline(ps.plan, B, args.steps, dense, mhat=True) if not args.no_stage_timing else {}
    grad_gbs = 4.0 * dense / (ms_step * 1e-3) / 1e9
    alg_bytes = 28.0 * dense
    result = {
        "metric": METRIC,
        "value": round(grad_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"7B-shaped gradient set: {len(shapes)} fp32 matrices, {dense} elements, rank {rank}, "
                        "compress with fused decompression (EF+P+Q+E+M_hat)",
            "rank": rank,
            "matrices": len(shapes),
            "elements": dense,
            "alg_bytes_per_step": alg_bytes,
            "step_hbm_frac": round(alg_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "median_ms": round(statistics.median(per), 4),
            "p10_ms": round(sorted(per)[max(0, int(0.1 * len(per)) - 0)], 4),
            "p90_ms": round(sorted(per)[min(len(per) - 1, int(0.9 * len(per)))], 4),
            "copy_ceiling_gbs": round(copy_gbs, 1),
        },
    }
    if stages:
        dom = max((s for s in stages if s in B_STAGE), key=lambda s: stages[s]["ms_avg"] * stages[s]["launches"])
        d = stages[dom]
        tr = measured_traffic(dom, rank, True)
        result["roofline"] = {"bound": "hbm", "kernel": KERNEL_OF_STAGE[dom], "achieved": round(d["gbs"], 1),
                              "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(d["gbs"] / HBM_PEAK_GBS, 4),
                              "traffic": round(tr) if tr else None,
                              "alg_bytes_per_launch": d["bytes_alg"], "avg_launch_ms": round(d["ms_avg"], 4)}
        result["stages"] = {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                            for k, v in stages.items()}

    if not args.no_variants:
        ms_c, _ = run("compress only", lambda: ps.compress(mhat=False), max(3, args.steps // 2), 1,
                      stage_timing=False)
        result["config"]["compress_only"] = {"ms_per_step": round(ms_c, 4),
                                             "grad_gbs": round(4.0 * dense / (ms_c * 1e-3) / 1e9, 2),
                                             "hbm_frac": round(24.0 * dense / (ms_c * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        ps.close()
        del ps
        torch.cuda.empty_cache()
        psm = PowerSGD(shapes, rank, device=dev, momentum_beta=0.9, with_mhat=False)
        for i, (_, s) in enumerate(tensors):
            W.llama7b_grad_(psm.view(psm.grads, i), s[0], s[1], i, step=1)
            psm.set_q(i, W.llama7b_q0(s[1], rank, i, device=dev))
        torch.cuda.synchronize()
        ps = psm
        ms_m, _ = run("momentum compress", lambda: psm.compress(mhat=False), max(3, args.steps // 2), 1,
                      stage_timing=False)
        result["config"]["momentum_compress"] = {"beta": 0.9, "ms_per_step": round(ms_m, 4),
                                                 "grad_gbs": round(4.0 * dense / (ms_m * 1e-3) / 1e9, 2),
                                                 "hbm_frac": round(32.0 * dense / (ms_m * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                                                   4)}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(tensors, rank)
    print(json.dumps(result), flush=True)


def cpu_baseline(tensors, rank):
    """The fp64 oracle on the host cores: one step of each distinct matrix
    shape of the set, scaled by how often the shape occurs (an extrapolated
    whole-set step)."""
    import numpy as np

    import oracle

    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info

        blas_threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = cores
    counts = {}
    for _, s in tensors:
        counts[tuple(s)] = counts.get(tuple(s), 0) + 1
    g = np.random.default_rng(0)
    total = 0.0
    detail = {}
    for shape, c in counts.items():
        m, n = shape
        G = g.standard_normal((m, n), dtype=np.float32)
        E = np.zeros((m, n))
        Q = g.standard_normal((n, rank))
        t0 = time.perf_counter()
        res = oracle.compress_matrix(G.astype(np.float64) + E, Q)
        dt = time.perf_counter() - t0
        del res, G, E
        detail[f"{m}x{n}"] = {"s": round(dt, 3), "count": c}
        total += dt * c
    dense = sum(a * b for (a, b), c in counts.items() for _ in range(c))
    return {"value": round(4.0 * dense / total / 1e9, 4), "unit": "GB/s", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": "one fp64 oracle step per distinct matrix shape (" + ", ".join(detail) + "), "
                      f"scaled by shape counts to the {len(tensors)}-matrix set: extrapolated "
                      f"{total:.1f} s per step",
            "host_cores": cores, "detail": detail}


if __name__ == "__main__":
    main()
