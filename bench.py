"""Throughput of the PowerSGD compression step on one MI355X.

Default workload: the 7B-transformer shaped gradient set (32 layers of
q,k,v,o 4096x4096, gate/up 11008x4096, down 4096x11008, plus 32000x4096
embedding and head: 226 fp32 matrices, 6,738,149,376 elements), rank 4.  A
step is one psgd_compress call with the fused decompression: EF-add, P = M Q,
orthogonalisation, Q = M^T P_hat, residual E = M - P_hat Q^T and M_hat, all in
the library's HIP kernels.  The gradients are synthetic (seeded rank-16 signal
plus Gaussian noise, unit Frobenius norm per matrix) and resident in HBM
before timing starts.

The default run also times the other seeded workloads and nests them in the
same JSON line under "configs", each with its own roofline (dominant kernel
named) and the fp64 oracle timed on the host cores beside it: the single
256x128 matrix at rank 2, the ResNet18-shaped set at rank 2, the LSTM-shaped
set at rank 4, the 11008x4096 decaying-spectrum matrix at ranks 1..64 and the
PowerSGD+ refresh (8 rounds at rank 32 on 8192x8192).  --no-configs skips
them.

Other workloads (--workload): `single`, `sweep`, `refresh`, `resnet18`,
`lstm3`, each printed as a JSON line of its own.

`value` is gradient GB compressed per second (4 bytes x elements / step
time).
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
MFMA_FP32_PEAK_TFLOPS = 157.3
# the streaming passes: the stages whose launches move the matrix and carry its bytes
STREAM_STAGES = ("ef_p", "mtp", "residual")
KERNEL_OF_STAGE = {"ef_p": "k_ef_p", "mtp": "k_mtp", "residual": "k_recon"}
KERNEL_OF_STAGE_MFMA = {"ef_p": "k_mfma_p", "mtp": "k_mfma_qt", "residual": "k_mfma_recon"}
# Byte pattern of each pass (arrays read, arrays written, and for each output
# the input it overwrites or None), measured with the library's streaming
# probe: the practical bandwidth of that pattern.  The passes write in place:
# EF-add stores M over E (and u over u with momentum), the residual stores E
# over M; the "_sep" forms write separate arrays, for comparison.
PATTERNS = {"r2w1": (2, 1, (1,)), "r2w1_sep": (2, 1, (None,)), "r1": (1, 0, ()),
            "r1w1": (1, 1, (0,)), "r1w2": (1, 2, (0, None)), "r1w2_sep": (1, 2, (None, None)),
            "r3w2": (3, 2, (1, 2)), "r3w2_sep": (3, 2, (None, None)), "w1": (0, 1, (None,))}
PROBE_PLACEMENTS = 3  # array sets the probe is run on; each pattern's best counts


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama7b",
                    choices=["llama7b", "single", "sweep", "refresh", "resnet18", "lstm3", "matrix"])
    ap.add_argument("--shape", default="33278x650",
                    help="matrix workload: comma-separated MxN shapes, each timed on its own (Gaussian gradients)")
    ap.add_argument("--no-configs", action="store_true",
                    help="7B workload: skip the other workloads nested under 'configs'")
    ap.add_argument("--rank", type=int, default=None)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true", help="skip the plain-compress and momentum figures")
    ap.add_argument("--no-stage-timing", action="store_true")
    ap.add_argument("--mhat-buffers", type=int, default=0,
                    help="7B workload: also time the fused step with this many further M_hat buffers, each "
                         "allocated on its own (the residual pass's speed depends on where M_hat lands)")
    ap.add_argument("--residual", default="explicit", choices=["explicit", "deferred"],
                    help="7B workload: time the step that writes E (default) or the steady-state step with the "
                         "residual deferred into the next step's first pass")
    return ap.parse_args()


def measured_traffic(kernel, profile):
    """HBM bytes per launch of `kernel` from a committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary, or None when there is none or the
    kernel's source changed since the counters were taken."""
    from rank_gradient_compression_amd.profile_summary import source_hash

    path = os.path.join(ROOT, "profiles", profile)
    try:
        text = open(path).read()
        blob = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (OSError, IndexError, ValueError):
        return None
    # the most-launched instantiation of the kernel in the profiled run
    hits = [v for name, v in blob["kernels"].items()
            if name.split("<")[0].split()[-1] == kernel and v.get("source_hash") == source_hash(name)]
    if not hits:
        return None
    v = max(hits, key=lambda h: h.get("launches", 0))
    return v["read_bytes"] + v["write_bytes"]


def stage_table(B, R, bytes_per_el, flops_per_el, elems):
    """Per-stage average launch time from the library's HIP events and the
    algorithmic bytes / flops of one launch: every stage from the breakdown
    steps of the last Runner.time call, except the stage timed inside the
    headline steps (`"timed": "headline"`), whose figures are taken there."""
    ms, n = (list(v) for v in R.breakdown)
    focus = R.focus
    if focus is not None:
        ms[focus[0]], n[focus[0]] = focus[1], focus[2]
    out = {}
    for i, name in enumerate(B.STAGE_NAMES):
        if not n[i]:
            continue
        s = {"ms_avg": ms[i] / n[i], "launches": n[i],
             "timed": "headline" if focus is not None and i == focus[0] else "breakdown"}
        if name in bytes_per_el:
            s["bytes_alg"] = bytes_per_el[name] * elems
            s["flops_alg"] = flops_per_el[name] * elems
            t = s["ms_avg"] * 1e-3
            s["gbs"] = s["bytes_alg"] / t / 1e9
            s["tflops"] = s["flops_alg"] / t / 1e12
            s["frac_hbm"] = s["gbs"] / HBM_PEAK_GBS
            s["frac_mfma"] = s["tflops"] / MFMA_FP32_PEAK_TFLOPS
        out[name] = s
    return out


def roofline_of(stages, mfma, profile=None):
    cand = [s for s in stages if "bytes_alg" in stages[s]]
    if not cand:
        return None
    # the stage timed inside the headline steps (chosen there as the one that
    # took the most time), else the largest
    head = [s for s in cand if stages[s].get("timed") == "headline"]
    dom = head[0] if head else max(cand, key=lambda s: stages[s]["ms_avg"] * stages[s]["launches"])
    d = stages[dom]
    ridge = MFMA_FP32_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    kernel = (KERNEL_OF_STAGE_MFMA if mfma else KERNEL_OF_STAGE)[dom]
    tr = measured_traffic(kernel, profile) if profile else None
    if mfma and d["flops_alg"] / d["bytes_alg"] > ridge:
        return {"bound": "mfma", "kernel": kernel, "achieved": round(d["tflops"], 2), "peak": MFMA_FP32_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(d["frac_mfma"], 4), "traffic": round(tr) if tr else None,
                "alg_flops_per_launch": d["flops_alg"], "avg_launch_ms": round(d["ms_avg"], 4)}
    return {"bound": "hbm", "kernel": kernel, "achieved": round(d["gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(d["frac_hbm"], 4), "traffic": round(tr) if tr else None,
            "alg_bytes_per_launch": d["bytes_alg"], "avg_launch_ms": round(d["ms_avg"], 4)}


def stage_patterns(momentum=False, mhat=True, deferred=False):
    res = "w1" if deferred else ("r1w2" if mhat else "r1w1")
    return {"ef_p": "r3w2" if momentum else "r2w1", "mtp": "r1", "residual": res}


def attach_ceilings(stages, ceilings, patterns):
    """Each streaming stage against the probe's bandwidth for its byte
    pattern; returns the step time if every pass ran at that bandwidth."""
    total = 0.0
    for name, pat in patterns.items():
        st = stages.get(name)
        if not st or "bytes_alg" not in st:
            continue
        st["pattern"] = pat
        st["ceiling_gbs"] = ceilings[pat]
        st["frac_of_ceiling"] = st["gbs"] / ceilings[pat]
        total += st["bytes_alg"] / (ceilings[pat] * 1e9) * 1e3  # one launch per step
    return total


def round_stages(stages):
    return {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in v.items()} for k, v in stages.items()}


class Runner:
    def __init__(self, torch, B):
        self.torch, self.B = torch, B
        self.stream = torch.cuda.current_stream()

    def time(self, label, call, steps, warmup, plan=None, per_step=True, focus=None):
        """K timed steps between one pair of events (the headline figure).
        With `plan`: first K steps with the library's events on every stage
        (the stage breakdown, kept in self.breakdown), then the headline K
        steps with events around the stage that took the most time (among
        the stage names in `focus`, default all) only, kept in self.focus, so
        that the timed calls carry one event pair per launch of one kernel
        instead of one per stage.  Then, separately, K steps with an event
        after each one for the spread."""
        torch, B = self.torch, self.B
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        self.breakdown = self.focus = None
        if plan is not None:
            B.psgd_timing_read(plan)  # drop warm-up records
            B.psgd_timing_stages(plan, 0xFFFFFFFF)
            B.psgd_timing_enable(plan, True)
            for _ in range(steps):
                call()
            B.psgd_timing_enable(plan, False)
            self.breakdown = B.psgd_timing_read(plan)
            ms_b, n_b = self.breakdown
            cand = [i for i, nm in enumerate(B.STAGE_NAMES) if n_b[i] and (focus is None or nm in focus)]
            dom = max(cand, key=lambda i: ms_b[i]) if cand else None
            if dom is not None:
                B.psgd_timing_stages(plan, 1 << dom)
                B.psgd_timing_enable(plan, True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_wall = time.perf_counter()
        e0.record(self.stream)
        for _ in range(steps):
            call()
        e1.record(self.stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_wall
        if plan is not None:
            B.psgd_timing_enable(plan, False)
            B.psgd_timing_stages(plan, 0xFFFFFFFF)
            ms_f, n_f = B.psgd_timing_read(plan)
            if dom is not None:
                self.focus = (dom, ms_f[dom], n_f[dom])
        total_ms = e0.elapsed_time(e1)
        per = [total_ms / steps]
        if per_step:
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
            ev[0].record(self.stream)
            for k in range(steps):
                call()
                ev[k + 1].record(self.stream)
            torch.cuda.synchronize()
            per = [ev[k].elapsed_time(ev[k + 1]) for k in range(steps)]
        log(f"bench: {label}: {total_ms / steps:.4f} ms/step (per-step median {statistics.median(per):.4f}, "
            f"wall {wall * 1e3 / steps:.4f})")
        return total_ms / steps, per

    def copy_ceiling(self, n=1 << 30):
        torch, B = self.torch, self.B
        src = torch.empty(n, dtype=torch.float32, device="cuda").normal_()
        dst = torch.empty_like(src)
        ms, _ = self.time("stream copy 4 GiB", lambda: B.psgd_stream_copy(dst.data_ptr(), src.data_ptr(), n,
                                                                            self.stream.cuda_stream), 5, 2,
                          per_step=False)
        del src, dst
        torch.cuda.empty_cache()
        return 8 * n / (ms * 1e-3) / 1e9

    def pattern_ceilings(self, n=1 << 30, placements=PROBE_PLACEMENTS):
        """GB/s of bytes moved by the library's streaming probe for each pass
        pattern in PATTERNS, over n-float arrays (4 GiB each, so that a launch
        lasts milliseconds and its ramp-up and drain weigh about 1%): the best of
        `placements` sets of arrays, all allocated before the first is
        measured so that each set lands in other physical memory (the
        passes' own speed moves with where their buffers land)."""
        torch, B = self.torch, self.B
        sets = [[torch.empty(n, dtype=torch.float32, device="cuda").normal_() for _ in range(5)]
                for _ in range(placements)]
        sink = torch.zeros(B.PSGD_PROBE_SINK_FLOATS, dtype=torch.float32, device="cuda")
        out = {}
        for t, arrs in enumerate(sets):
            for name, (nin, nout, alias) in PATTERNS.items():
                ins = [a.data_ptr() for a in arrs[:nin]]
                outs = [ins[alias[j]] if alias[j] is not None else arrs[3 + j].data_ptr() for j in range(nout)]
                ms, _ = self.time(f"probe {name} (arrays {t})",
                                  lambda: B.psgd_stream_probe(ins, outs, n, sink.data_ptr(), self.stream.cuda_stream),
                                  5, 2, per_step=False)
                out[name] = max(out.get(name, 0.0), round(4.0 * n * (nin + nout) / (ms * 1e-3) / 1e9, 1))
        del sets, sink
        torch.cuda.empty_cache()
        return out


def base_result(args, value, ms_step, per, workload, extra):
    cfg = {"workload": workload}
    cfg.update(extra)
    cfg["median_ms"] = round(statistics.median(per), 4)
    srt = sorted(per)
    cfg["p10_ms"] = round(srt[int(0.1 * (len(srt) - 1))], 4)
    cfg["p90_ms"] = round(srt[int(round(0.9 * (len(srt) - 1)))], 4)
    return {"metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f32", "data": "synthetic", "config": cfg}


def step_bytes(rank_mfma, momentum=False, mhat=True, deferred=False):
    if deferred:  # pass 1 rebuilds E from M_prev; the last pass only writes M_hat
        return {"ef_p": 20.0 if momentum else 12.0, "mtp": 4.0, "residual": 4.0}
    return {"ef_p": 20.0 if momentum else 12.0, "mtp": 4.0, "residual": 12.0 if mhat else 8.0}


def step_flops(r, momentum=False, deferred=False):
    if deferred:
        return {"ef_p": 4.0 * r + (4.0 if momentum else 2.0), "mtp": 2.0 * r, "residual": 2.0 * r}
    return {"ef_p": 2.0 * r + (3.0 if momentum else 1.0), "mtp": 2.0 * r, "residual": 2.0 * r + 1.0}


# --------------------------------------------------------------------------- workloads

def run_llama7b(args, torch, B, W, PowerSGD, R):
    rank = args.rank or 4
    tensors = W.llama7b_set(args.layers)
    shapes = [s for _, s in tensors]
    log(f"bench: plan for {len(shapes)} matrices, rank {rank}")
    ps = PowerSGD(shapes, rank, device="cuda", with_mhat=True)
    dense = ps.info["dense_elems"]
    t0 = time.time()
    for i, (_, s) in enumerate(tensors):
        W.llama7b_grad_(ps.view(ps.grads, i), s[0], s[1], i, step=1)
        ps.set_q(i, W.llama7b_q0(s[1], rank, i, device="cuda"))
    torch.cuda.synchronize()
    log(f"bench: {dense} synthetic gradient elements ready in {time.time() - t0:.1f} s")
    copy_gbs = R.copy_ceiling()
    ceilings = R.pattern_ceilings()
    deferred = args.residual == "deferred"
    if deferred:
        ps.compress(mhat=True, defer_residual=True)  # leaves M in err: the steady state below

        def step():
            ps.compress(mhat=True, defer_residual=True, residual_deferred=True)
    else:
        def step():
            ps.compress(mhat=True)
    ms, per = R.time("compress + fused decompress" + (" (deferred residual)" if deferred else ""), step, args.steps,
                     args.warmup, plan=None if args.no_stage_timing else ps.plan, focus=STREAM_STAGES)
    mfma = rank > 8
    bpe = 20.0 if deferred else 28.0
    res = base_result(args, 4.0 * dense / (ms * 1e-3) / 1e9, ms, per,
                      f"7B-shaped gradient set: {len(shapes)} fp32 matrices, {dense} elements, rank {rank}, "
                      "compress with fused decompression (EF+P+Q+E+M_hat)"
                      + (", residual deferred into the next step's first pass" if deferred else ""),
                      {"rank": rank, "matrices": len(shapes), "elements": dense, "residual": args.residual,
                       "alg_bytes_per_step": bpe * dense,
                       "step_hbm_frac": round(bpe * dense / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                       "copy_ceiling_gbs": round(copy_gbs, 1), "pattern_ceilings_gbs": ceilings,
                       "pattern_ceiling_placements": PROBE_PLACEMENTS})
    if not args.no_stage_timing:
        st = stage_table(B, R, step_bytes(mfma, deferred=deferred), step_flops(rank, deferred=deferred), dense)
        at_ceil = attach_ceilings(st, ceilings, stage_patterns(deferred=deferred))
        res["config"]["step_ms_at_pattern_ceilings"] = round(at_ceil, 3)
        res["config"]["frac_of_pattern_ceilings"] = round(at_ceil / ms, 4)
        prof = f"hbm_bytes_llama7b_r4_{'deferred' if deferred else 'fused'}.md" if rank == 4 else None
        res["roofline"] = roofline_of(st, mfma, prof)
        res["stages"] = round_stages(st)
    if args.mhat_buffers > 0 and not deferred:
        res["config"]["mhat_buffers"] = mhat_buffer_sweep(torch, B, ps, args.mhat_buffers)
    if not args.no_variants and not deferred:
        ms_c, _ = R.time("compress only", lambda: ps.compress(mhat=False), max(3, args.steps // 2), 1,
                         per_step=False)
        res["config"]["compress_only"] = {"ms_per_step": round(ms_c, 4),
                                          "grad_gbs": round(4.0 * dense / (ms_c * 1e-3) / 1e9, 2),
                                          "hbm_frac": round(24.0 * dense / (ms_c * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        # Standalone decompression M_hat = P_hat Q^T of the whole set: a
        # write-only pass (4 B per element).
        ms_dd, _ = R.time("decompress", lambda: ps.decompress(), max(3, args.steps // 2), 1, per_step=False)
        res["config"]["decompress"] = {"ms_per_step": round(ms_dd, 4),
                                       "hbm_frac": round(4.0 * dense / (ms_dd * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        # Quantised payloads (compound compression): the factors rounded
        # before their hooks to bfloat16, or to E4M3 codes with one power-of-two
        # exponent per column; the same passes plus the quantiser launches.
        # Bytes on the wire per step: factor values at 4, 2 or 1 B (+ one
        # exponent byte per factor column for E4M3).
        fac = sum(rank * (m + n) for m, n in shapes)
        wire = {"fp32": 4.0 * fac, "bf16": 2.0 * fac, "fp8_e4m3": 1.0 * fac + 2 * rank * len(shapes)}
        pay = {"fp32": {"wire_bytes_per_step": wire["fp32"]}}
        for name, kw in (("bf16", {"payload_bf16": True}), ("fp8_e4m3", {"payload_fp8": True})):
            ms_p, _ = R.time(f"{name} payload, compress + fused decompress",
                             lambda kw=kw: ps.compress(mhat=True, **kw), max(3, args.steps // 2), 1, per_step=False)
            pay[name] = {"ms_per_step": round(ms_p, 4), "grad_gbs": round(4.0 * dense / (ms_p * 1e-3) / 1e9, 2),
                         "wire_bytes_per_step": wire[name]}
        res["config"]["quantised_payload"] = pay
        # Deferred residual: E = M - P_hat Q^T is formed inside the next
        # step's EF-add pass instead of being stored (20 / 16 B per element).
        ps.compress(mhat=True, defer_residual=True)
        ms_d, _ = R.time("deferred residual, compress + fused decompress",
                         lambda: ps.compress(mhat=True, defer_residual=True, residual_deferred=True),
                         max(3, args.steps // 2), 1, per_step=False)
        ms_dc, _ = R.time("deferred residual, compress only",
                          lambda: ps.compress(mhat=False, defer_residual=True, residual_deferred=True),
                          max(3, args.steps // 2), 1, per_step=False)
        res["config"]["deferred_residual"] = {
            "fused": {"ms_per_step": round(ms_d, 4), "grad_gbs": round(4.0 * dense / (ms_d * 1e-3) / 1e9, 2),
                      "bytes_per_el": 20.0,
                      "hbm_frac": round(20.0 * dense / (ms_d * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
            "compress_only": {"ms_per_step": round(ms_dc, 4),
                              "grad_gbs": round(4.0 * dense / (ms_dc * 1e-3) / 1e9, 2), "bytes_per_el": 16.0,
                              "hbm_frac": round(16.0 * dense / (ms_dc * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}}
        ps.close()
        del ps
        torch.cuda.empty_cache()
        psm = PowerSGD(shapes, rank, device="cuda", momentum_beta=0.9, with_mhat=False)
        for i, (_, s) in enumerate(tensors):
            W.llama7b_grad_(psm.view(psm.grads, i), s[0], s[1], i, step=1)
            psm.set_q(i, W.llama7b_q0(s[1], rank, i, device="cuda"))
        torch.cuda.synchronize()
        ms_m, _ = R.time("momentum compress (beta 0.9)", lambda: psm.compress(mhat=False), max(3, args.steps // 2), 1,
                         per_step=False)
        res["config"]["momentum_compress"] = {"beta": 0.9, "ms_per_step": round(ms_m, 4),
                                              "grad_gbs": round(4.0 * dense / (ms_m * 1e-3) / 1e9, 2),
                                              "hbm_frac": round(32.0 * dense / (ms_m * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        psm.close()
        del psm
        torch.cuda.empty_cache()
        # bfloat16 gradients in, fp32 everywhere else: 2 B/el less in pass 1
        psb = PowerSGD(shapes, rank, device="cuda", with_mhat=True, grads_dtype=torch.bfloat16)
        for i, (_, s) in enumerate(tensors):
            tmp = torch.empty(s, dtype=torch.float32, device="cuda")
            W.llama7b_grad_(tmp, s[0], s[1], i, step=1)
            psb.view(psb.grads, i).copy_(tmp)
            psb.set_q(i, W.llama7b_q0(s[1], rank, i, device="cuda"))
            del tmp
        torch.cuda.synchronize()
        ms_b, _ = R.time("bf16 gradients, compress + fused decompress", lambda: psb.compress(mhat=True),
                         max(3, args.steps // 2), 1, per_step=False)
        res["config"]["bf16_grads_fused"] = {"ms_per_step": round(ms_b, 4),
                                             "elements_per_s": round(dense / (ms_b * 1e-3), 1),
                                             "hbm_frac": round(26.0 * dense / (ms_b * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        psb.close()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(tensors, rank)
    return res


def mhat_buffer_sweep(torch, B, ps, count, calls=3):
    """The fused step with `count` further M_hat buffers, each allocated on
    its own, `calls` calls per buffer, twice round-robin: per-call residual
    stage time.  The residual pass runs in one of two speeds per buffer
    (about 12.3 or 13.8 ms on the 7B set), repeatably."""
    bufs = [torch.empty_like(ps.err) for _ in range(count)]
    out = [{"buffer": k, "va_offset_from_err": bufs[k].data_ptr() - ps.err.data_ptr(), "residual_ms": []}
           for k in range(count)]
    torch.cuda.synchronize()
    B.psgd_timing_read(ps.plan)
    B.psgd_timing_enable(ps.plan, True)
    for _ in range(2):
        for k, m in enumerate(bufs):
            for _ in range(calls):
                ps.compress(mhat_buf=m)
                ms, _ = B.psgd_timing_read(ps.plan)
                out[k]["residual_ms"].append(round(ms[B.PSGD_STAGE_RESIDUAL], 3))
    B.psgd_timing_enable(ps.plan, False)
    for o in out:
        log(f"bench: M_hat buffer {o['buffer']}: residual pass {o['residual_ms']} ms")
    del bufs
    torch.cuda.empty_cache()
    return out


def device_decaying(torch, W, m, n, seed, K=512):
    """sigma_k = exp(-k/20) matrix: seeded orthonormal factors from the
    workload generator's host QR, product formed on the device in fp64."""
    import numpy as np

    K = min(K, m, n)
    g = W.rng(seed, m, n)
    U = torch.from_numpy(W.orthonormal(g, m, K)).cuda()
    V = torch.from_numpy(W.orthonormal(g, n, K)).cuda()
    s = torch.from_numpy(np.exp(-np.arange(1, K + 1, dtype=np.float64) / 20.0)).cuda()
    return ((U * s) @ V.T).float()


def run_sweep(args, torch, B, W, PowerSGD, R, nested=False):
    m, n = 11008, 4096
    ranks = [args.rank] if (args.rank and not nested) else [1, 2, 4, 7, 16, 32, 64]
    A = device_decaying(torch, W, m, n, 5)
    if not nested:
        R.copy_ceiling()  # also the byte-counter calibration of a profiled run
    out = []
    for r in ranks:
        ps = PowerSGD([(m, n)], r, device="cuda")
        ps.view(ps.grads, 0).copy_(A)
        ps.set_q(0, torch.from_numpy(W.gaussian_q0(n, r, 5)))
        ms, per = R.time(f"11008x4096 r={r}", lambda: ps.compress(mhat=True), args.steps, args.warmup,
                         plan=None if args.no_stage_timing else ps.plan, focus=STREAM_STAGES)
        mfma = r > 8
        res = base_result(args, 4.0 * m * n / (ms * 1e-3) / 1e9, ms, per,
                          f"one 11008x4096 fp32 matrix (sigma_k = exp(-k/20)), rank {r}, compress with fused "
                          "decompression", {"rank": r, "elements": m * n, "path": "mfma" if mfma else "valu",
                                            "step_hbm_frac": round(28.0 * m * n / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                                                   4)})
        if not args.no_stage_timing:
            st = stage_table(B, R, step_bytes(mfma), step_flops(r), m * n)
            res["roofline"] = roofline_of(st, mfma, f"hbm_bytes_sweep_11008x4096_r{r}.md")
            res["stages"] = round_stages(st)
        if not args.no_cpu_baseline:
            res["cpu_baseline"] = cpu_baseline_sweep(W, m, n, r)
        out.append(res)
        ps.close()
    del A
    torch.cuda.empty_cache()
    return out


def run_matrix(args, torch, B, W, PowerSGD, R):
    """One m x n fp32 matrix per shape of --shape (seeded Gaussian gradients,
    Gaussian Q0), compress with fused decompression at --rank (default 4),
    each shape in its own plan: a probe of how a pass depends on the shape
    (row alignment, row length)."""
    r = args.rank or 4
    out = []
    for spec in args.shape.split(","):
        m, n = (int(x) for x in spec.lower().split("x"))
        ps = PowerSGD([(m, n)], r, device="cuda")
        ps.grads.normal_(generator=torch.Generator(device="cuda").manual_seed(m * 100003 + n))
        ps.set_q(0, torch.from_numpy(W.gaussian_q0(n, r, 5)))
        mfma = r > 8
        ms, per = R.time(f"{m}x{n} r={r}", lambda: ps.compress(mhat=True), args.steps, args.warmup,
                         plan=None if args.no_stage_timing else ps.plan, focus=STREAM_STAGES)
        res = base_result(args, 4.0 * m * n / (ms * 1e-3) / 1e9, ms, per,
                          f"one {m}x{n} fp32 matrix (Gaussian gradients), rank {r}, compress with fused decompression",
                          {"rank": r, "elements": m * n, "path": "mfma" if mfma else "valu",
                           "row_bytes_mod_128": (4 * n) % 128,
                           "step_hbm_frac": round(28.0 * m * n / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
        if not args.no_stage_timing:
            st = stage_table(B, R, step_bytes(mfma), step_flops(r), m * n)
            res["roofline"] = roofline_of(st, mfma)
            res["stages"] = round_stages(st)
        out.append(res)
        ps.close()
        torch.cuda.empty_cache()
    return out


def run_refresh(args, torch, B, W, PowerSGD, R, nested=False):
    m = n = 8192
    r = 32 if nested else (args.rank or 32)
    iters = 8
    A = device_decaying(torch, W, m, n, 5)
    if not nested:
        R.copy_ceiling()  # also the byte-counter calibration of a profiled run
    ps = PowerSGD([(m, n)], r, device="cuda")
    mbuf = torch.zeros_like(ps.grads)
    ps.view(mbuf, 0).copy_(A)
    q0 = torch.from_numpy(W.gaussian_q0(n, r, 5)).float().cuda()

    def call():
        ps.set_q(0, q0)
        ps.refresh(0, mbuf, iters)

    ms, per = R.time(f"refresh 8192^2 r={r} x{iters}", call, args.steps, args.warmup,
                     plan=None if args.no_stage_timing else ps.plan, focus=STREAM_STAGES)
    flops = iters * 4.0 * m * n * r
    res = base_result(args, 4.0 * m * n / (ms * 1e-3) / 1e9, ms, per,
                      f"PowerSGD+ subspace refresh: {iters} rounds of orthonormalised block power iteration at rank "
                      f"{r} on one 8192x8192 fp32 matrix (sigma_k = exp(-k/20))",
                      {"rank": r, "iterations": iters, "elements": m * n, "alg_flops": flops,
                       "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                       "alg_bytes": iters * 8.0 * m * n,
                       "hbm_frac": round(iters * 8.0 * m * n / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
    if not args.no_stage_timing:
        st = stage_table(B, R, {"ef_p": 4.0, "mtp": 4.0}, {"ef_p": 2.0 * r, "mtp": 2.0 * r}, m * n)
        res["roofline"] = roofline_of(st, r > 8, f"hbm_bytes_refresh_8192x8192_r{r}.md")
        res["stages"] = round_stages(st)
    # The same call captured once in a HIP graph and replayed (its 96
    # launches issued together).
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    ms_g, _ = R.time(f"refresh 8192^2 r={r} x{iters}, graph replay", graph.replay, args.steps, args.warmup,
                     per_step=False)
    res["config"]["graph_replay"] = {"ms_per_step": round(ms_g, 4),
                                     "tflops": round(flops / (ms_g * 1e-3) / 1e12, 2)}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_refresh(W, m, n, r, iters)
    ps.close()
    del A, mbuf, graph
    torch.cuda.empty_cache()
    return res


def run_single(args, torch, B, W, PowerSGD, R):
    """The single 256x128 matrix at rank 2 (G = U diag(1/k) V^T + noise)."""
    wl = W.SmallMatrixWorkload()
    ps = PowerSGD([(wl.m, wl.n)], wl.rank, device="cuda")
    ps.view(ps.grads, 0).copy_(torch.from_numpy(wl.grads[0]).cuda())
    ps.set_q(0, wl.Q0)
    dense = wl.m * wl.n
    ms, per = R.time(f"single {wl.m}x{wl.n} r={wl.rank}", lambda: ps.compress(mhat=True), args.steps, args.warmup,
                     plan=None if args.no_stage_timing else ps.plan, focus=STREAM_STAGES)
    res = base_result(args, 4.0 * dense / (ms * 1e-3) / 1e9, ms, per,
                      f"one {wl.m}x{wl.n} fp32 matrix, rank {wl.rank}, compress with fused decompression "
                      "(launch-latency bound: a few tens of kilobytes per step)",
                      {"rank": wl.rank, "elements": dense})
    if not args.no_stage_timing:
        st = stage_table(B, R, step_bytes(False), step_flops(wl.rank), dense)
        res["roofline"] = roofline_of(st, False)
        res["stages"] = round_stages(st)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ps.compress(mhat=True)
    ms_g, _ = R.time(f"single r={wl.rank}, graph replay", graph.replay, args.steps, args.warmup, per_step=False)
    res["config"]["graph_replay"] = {"ms_per_step": round(ms_g, 4),
                                     "grad_gbs": round(4.0 * dense / (ms_g * 1e-3) / 1e9, 3)}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_trajectory(W, "single", wl.rank)
    ps.close()
    return res


def run_small_set(args, torch, B, W, PowerSGD, R, name, nested=False):
    if name == "resnet18":
        tensors, kind, seed, rank = W.resnet18_cifar_set(), "resnet18", 2, (None if nested else args.rank) or 2
    else:
        tensors, kind, seed, rank = W.lstm3_wikitext_set(), "lstm3", 3, (None if nested else args.rank) or 4
    wl = W.ModelSetWorkload(tensors, kind, seed)
    shapes = [s for _, s in tensors]
    ps = PowerSGD(shapes, rank, device="cuda")
    for i in range(len(shapes)):
        ps.view(ps.grads, i).copy_(torch.from_numpy(wl.grad(i, 1)).cuda())
        if ps.kind(i) == B.PSGD_KIND_COMPRESSED:
            ps.set_q(i, wl.q0(i, rank))
    dense = ps.info["dense_elems"]
    ms, per = R.time(f"{name} r={rank}", lambda: ps.compress(mhat=True), args.steps, args.warmup,
                     plan=None if args.no_stage_timing else ps.plan, focus=STREAM_STAGES)
    res = base_result(args, 4.0 * dense / (ms * 1e-3) / 1e9, ms, per,
                      f"{name}-shaped gradient set, rank {rank}, compress with fused decompression (working set "
                      "fits the 256 MB last-level cache)", {"rank": rank, "elements": dense,
                                                           "tensors": len(shapes)})
    if not args.no_stage_timing:
        st = stage_table(B, R, step_bytes(False), step_flops(rank), dense)
        res["roofline"] = roofline_of(st, rank > 8)
        res["stages"] = round_stages(st)
    # The same step captured once in a HIP graph and replayed: these sets are
    # launch-bound, and a replay issues all of the step's kernels at once.
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ps.compress(mhat=True)
    ms_g, _ = R.time(f"{name} r={rank}, graph replay", graph.replay, args.steps, args.warmup, per_step=False)
    res["config"]["graph_replay"] = {"ms_per_step": round(ms_g, 4),
                                     "grad_gbs": round(4.0 * dense / (ms_g * 1e-3) / 1e9, 2)}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_trajectory(W, name, rank)
    ps.close()
    return res


def nested_configs(args, torch, B, W, PowerSGD, R):
    """The other seeded workloads, each as a result object of its own."""
    out = {}
    log("bench: nested workloads")
    out["single_256x128_r2"] = run_single(args, torch, B, W, PowerSGD, R)
    out["resnet18_r2"] = run_small_set(args, torch, B, W, PowerSGD, R, "resnet18", nested=True)
    out["lstm3_r4"] = run_small_set(args, torch, B, W, PowerSGD, R, "lstm3", nested=True)
    for res in run_sweep(args, torch, B, W, PowerSGD, R, nested=True):
        out[f"sweep_11008x4096_r{res['config']['rank']}"] = res
    out["refresh_8192x8192_r32"] = run_refresh(args, torch, B, W, PowerSGD, R, nested=True)
    for v in out.values():  # nested objects carry what differs from the headline line
        for k in ("metric", "n_gpus", "higher_is_better", "scaling", "data", "dtype"):
            v.pop(k, None)
    return out


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(tensors, rank, budget_s=10.0, cap_s=30.0):
    """The fp64 oracle on the host cores: steps of each distinct matrix shape
    of the set, repeated round-robin for about `budget_s` seconds (at least
    three runs per shape), the median per shape scaled by how often the shape
    occurs (an extrapolated whole-set step)."""
    import statistics

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
    inputs = {}
    for shape in counts:
        m, n = shape
        inputs[shape] = (g.standard_normal((m, n), dtype=np.float32), np.zeros((m, n)), g.standard_normal((n, rank)))
    runs = {shape: [] for shape in counts}
    t_start = time.perf_counter()
    while True:
        for shape, (G, E, Q) in inputs.items():
            t0 = time.perf_counter()
            res = oracle.compress_matrix(G.astype(np.float64) + E, Q)
            runs[shape].append(time.perf_counter() - t0)
            del res
        spent = time.perf_counter() - t_start
        if spent >= cap_s or (spent >= budget_s and min(len(v) for v in runs.values()) >= 3):
            break
    del inputs
    total = 0.0
    detail = {}
    for (m, n), c in counts.items():
        med = statistics.median(runs[(m, n)])
        detail[f"{m}x{n}"] = {"s_median": round(med, 4), "runs": len(runs[(m, n)]), "count": c}
        total += med * c
    dense = sum(a * b * c for (a, b), c in counts.items())
    return {"value": round(4.0 * dense / total / 1e9, 4), "unit": "GB/s", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": "fp64 oracle steps (EF-add, P, Gram-Schmidt, Q, residual) of each distinct matrix shape ("
                      + ", ".join(detail) + f"), round-robin for {spent:.1f} s; the median per shape scaled by the "
                      f"shape counts to the {len(tensors)}-matrix set: extrapolated {total:.1f} s per step",
            "host_cores": cores, "cpu_model": cpu_model(), "detail": detail}


def blas_threads(default):
    try:
        from threadpoolctl import threadpool_info

        return max([d.get("num_threads", 1) for d in threadpool_info()] or [default])
    except Exception:  # pragma: no cover
        return default


def cpu_baseline_trajectory(W, name, rank, budget_s=6.0):
    """The fp64 oracle's steps of a seeded set (the whole set, one step after
    another from the seeded start, as the GPU runs it) on the host cores,
    stopped after the step that passes `budget_s` of oracle time (at least 3
    steps, at most the workload's length); the inputs are drawn outside the
    timed calls."""
    import numpy as np

    import oracle

    if name == "single":
        wl = W.SmallMatrixWorkload()
        shapes, total = [(wl.m, wl.n)], wl.steps
        grad = lambda i, t: wl.grads[t - 1]  # noqa: E731
        q0 = [wl.Q0]
    else:
        tensors, kind, seed, total = ((W.resnet18_cifar_set(), "resnet18", 2, 100) if name == "resnet18"
                                      else (W.lstm3_wikitext_set(), "lstm3", 3, 100))
        wl = W.ModelSetWorkload(tensors, kind, seed)
        shapes = [s for _, s in tensors]
        grad = wl.grad
        q0 = None
    plan = oracle.Plan(shapes, rank)
    if q0 is None:
        q0 = [wl.q0(i, rank) if plan.kinds[i] == oracle.KIND_COMPRESSED else None for i in range(len(shapes))]
    spent, steps, reps = 0.0, 0, 0
    # a trajectory shorter than the budget is run again from its start
    while spent < min(budget_s, 0.5) or reps == 0:
        st = oracle.init_state(plan, q0)
        reps += 1
        for t in range(1, total + 1):
            grads = [grad(i, t) for i in range(len(shapes))]
            t0 = time.perf_counter()
            oracle.step_set(plan, grads, st)
            spent += time.perf_counter() - t0
            steps += 1
            if steps >= 3 and spent >= budget_s:
                break
    dense = plan.dense_elems()
    cores = len(os.sched_getaffinity(0))
    what = (f"its whole {total}-step trajectory, {reps} times" if reps > 1 or steps == total
            else f"the first {steps} of its {total} steps")
    return {"value": round(4.0 * dense * steps / spent / 1e9, 5), "unit": "GB/s", "cores": int(blas_threads(cores)),
            "kind": "oracle",
            "sample": f"fp64 oracle steps of the {name} set at rank {rank} from its seeded start: {what} "
                      f"({steps} steps, {spent:.2f} s of oracle time, inputs drawn outside the timed calls)",
            "host_cores": cores}


_DECAYING = {}


def decaying_host(W, m, n):
    """The seeded decaying-spectrum matrix in fp64 on the host (cached)."""
    import numpy as np

    if (m, n) not in _DECAYING:
        _DECAYING[(m, n)] = W.decaying_spectrum_matrix(m, n, seed=5)[0].astype(np.float64)
    return _DECAYING[(m, n)]


def cpu_baseline_sweep(W, m, n, r, runs=2):
    """The oracle's step on the decaying-spectrum matrix at rank r (median of
    `runs`, from the seeded start)."""
    import numpy as np

    import oracle

    A = decaying_host(W, m, n)
    q0 = W.gaussian_q0(n, r, 5).astype(np.float64)
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        oracle.compress_matrix(A, q0)
        ts.append(time.perf_counter() - t0)
    t = statistics.median(ts)
    cores = len(os.sched_getaffinity(0))
    return {"value": round(4.0 * m * n / t / 1e9, 5), "unit": "GB/s", "cores": int(blas_threads(cores)),
            "kind": "oracle",
            "sample": f"one fp64 oracle step of the {m}x{n} matrix at rank {r} (first step, E = 0), median of {runs}: "
                      f"{t:.3f} s",
            "host_cores": cores}


def cpu_baseline_refresh(W, m, n, r, iters):
    """One cold refresh by the oracle: `iters` rounds from the seeded Q0."""
    import numpy as np

    import oracle

    A = decaying_host(W, m, n)
    q0 = W.gaussian_q0(n, r, 5).astype(np.float64)
    t0 = time.perf_counter()
    oracle.refresh(A, q0, iters)
    t = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0))
    return {"value": round(4.0 * m * n / t / 1e9, 5), "unit": "GB/s", "cores": int(blas_threads(cores)),
            "kind": "oracle",
            "sample": f"one cold fp64 oracle refresh of the {m}x{n} matrix at rank {r}, {iters} rounds from the seeded "
                      f"Q0: {t:.2f} s",
            "host_cores": cores}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU: the aggregation between workers is a caller hook "
                          "(all-reduce of P and Q) and is not benchmarked here", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import workloads as W
    from rank_gradient_compression_amd import binding as B
    from rank_gradient_compression_amd.torch_api import PowerSGD

    torch.cuda.set_device(0)
    R = Runner(torch, B)
    if args.workload == "llama7b":
        # the smaller workloads first, on a device that has not yet held the
        # 7B set's 108 GB of buffers
        configs = None if args.no_configs else nested_configs(args, torch, B, W, PowerSGD, R)
        torch.cuda.empty_cache()
        res = run_llama7b(args, torch, B, W, PowerSGD, R)
        if configs is not None:
            res["configs"] = configs
        print(json.dumps(res), flush=True)
    elif args.workload == "single":
        print(json.dumps(run_single(args, torch, B, W, PowerSGD, R)), flush=True)
    elif args.workload == "sweep":
        for res in run_sweep(args, torch, B, W, PowerSGD, R):
            print(json.dumps(res), flush=True)
    elif args.workload == "refresh":
        print(json.dumps(run_refresh(args, torch, B, W, PowerSGD, R)), flush=True)
    elif args.workload == "matrix":
        for res in run_matrix(args, torch, B, W, PowerSGD, R):
            print(json.dumps(res), flush=True)
    else:
        print(json.dumps(run_small_set(args, torch, B, W, PowerSGD, R, args.workload)), flush=True)


if __name__ == "__main__":
    main()
