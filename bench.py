"""Throughput of owner-rank Newton-Schulz on one MI355X.

Workload: one owner rank's share of a 32-layer Llama-3-8B over 8 owner slots,
i.e. the seven projection shapes four times each (28 matrices, bf16 N(0, 1)
synthetic gradients), run through one grouped ns_batched call per step:
fp32 Frobenius normalisation, fp16 cast, five Gram-space NS steps with the
Polar Express table and a restart before step 2. The direct backend is timed
on the same batch as a second line of the report.

One step = one full ns_batched call over all 28 matrices, inputs resident in
HBM. Prints one JSON line.

The roofline object describes the dominant kernel (the grouped MFMA GEMM):
its algorithmic flops per launch (symmetric products counted at s (s + 1) k,
general ones at 2 m n k; zero padding excluded) divided by its average launch
duration, both measured inside the timed region with HIP events that the
library records around each of its launches on the caller's stream.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP16_TFLOPS = 2500.0     # MI355X dense fp16 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
METRIC = "NS matrices/s + TFLOP/s (% fp16 MFMA peak), Llama-8B owner batch"


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=4)
    ap.add_argument("--backend", choices=["gram", "direct"], default="gram",
                    help="headline backend")
    ap.add_argument("--no-second-backend", action="store_true",
                    help="time only the headline backend (also skips the Muon-step and "
                         "sharded-route lines)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the GPU and oracle timings of workloads 1, 2, 3 and 5")
    ap.add_argument("--cpu-budget", type=float, default=25.0,
                    help="seconds of oracle work for the CPU baseline sample")
    ap.add_argument("--only", choices=["muon", "sharded"], default=None,
                    help="time only the Muon step on the batch, or only the 4-shard "
                         "column-sharded route on its gate projection, for --steps "
                         "steps (for profiling those paths), print one JSON line, exit")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run three plain device copies of BYTES bytes (reference "
                         "for the FETCH_SIZE / WRITE_SIZE counters), then exit")
    return ap.parse_args()


def calibrate_copy(nbytes):
    """Three device-to-device copies of a known size, nothing else."""
    import torch
    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n * 4, "copies": 3}), flush=True)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


PROFILE = os.path.join(ROOT, "profiles", "gemm_nt_kernel_llama8b_owner_batch.md")
GEMM_SRC = os.path.join(ROOT, "newton_schulz_matrix_amd", "csrc", "gemm_kernels.hip")


def kernel_code_hash(src: bytes) -> str:
    """sha256 of a kernel source with its // comments and all white space
    removed, so that counters taken on a source stay valid across edits that
    touch only comments or layout (the source holds no // inside strings)."""
    lines = [re.sub(r"//.*", "", ln) for ln in src.decode().splitlines()]
    code = re.sub(r"\s+", "", "".join(lines))
    return hashlib.sha256(code.encode()).hexdigest()


def gemm_traffic_per_launch():
    """HBM bytes per GEMM launch from the committed FETCH_SIZE / WRITE_SIZE
    summary (default workload, gram backend), or None once the kernel code
    differs from the one the counters were taken on."""
    try:
        text = open(PROFILE).read()
        src = open(GEMM_SRC, "rb").read()
    except OSError:
        return None
    m = re.search(r"gemm_nt_kernel_traffic_bytes_per_launch: ([0-9.eE+-]+)", text)
    h = re.search(r"gemm_kernels_hip_code_sha256: ([0-9a-f]{64})", text)
    if not m or not h or h.group(1) != kernel_code_hash(src):
        return None
    return float(m.group(1))


def pages_flops(shapes, steps, restarts):
    """Gram flops per call in the pages' own count: the SYRKs R = X X^T at
    s (s + 1) l (the half-tile saving the pages describe), the restart and
    output products Q X at 2 s^2 l, and every s^3 product of the iteration at
    2 s^3 (no symmetric saving). With r effective restarts the iteration has
    K Z products, K - 1 - r Q updates (the first after a start or restart is
    Q = Z + a I) and two products per R recurrence (k + 1 < K, k + 1 not a
    restart)."""
    K = steps
    S = {int(i) for i in restarts if 0 < int(i) < K}
    r = len(S)
    m3 = K + (K - 1 - r) + 2 * sum(1 for k in range(K - 1) if (k + 1) not in S)
    total = 0.0
    for (m, n) in shapes:
        s_, l_ = min(m, n), max(m, n)
        total += (1 + r) * s_ * (s_ + 1) * l_ + (1 + r) * 2.0 * s_ * s_ * l_ + m3 * 2.0 * s_ ** 3
    return total


def norm_pass_entry(t, steps, Gs):
    """The normalisation pass (sum of squares, norm, scaled cast) per step:
    GB/s on the bytes it moves (G read twice, X written once; the direct
    backend also writes X^T) and on the one-pass minimum (G read once, X
    written once), which no two-pass scheme reaches."""
    ms = t["norm_ms"] / steps
    moved = t["norm_bytes"] / steps
    one_pass = float(sum(G.numel() * (G.element_size() + 2) for G in Gs))
    sec = max(ms * 1e-3, 1e-12)
    return {"ms_per_step": ms, "bytes_per_step": moved, "gbs": moved / sec / 1e9,
            "frac": moved / sec / 1e9 / PEAK_HBM_GBS,
            "one_pass_min_bytes": one_pass, "gbs_on_one_pass_min": one_pass / sec / 1e9,
            "frac_on_one_pass_min": one_pass / sec / 1e9 / PEAK_HBM_GBS,
            "peak_gbs": PEAK_HBM_GBS}


def time_backend(nsmi, torch, Gs, outs, backend, table, restarts, steps, warmup):
    """Warm up, then time exactly `steps` grouped calls; returns a dict."""
    ws = torch.empty(nsmi.ns_workspace_size([tuple(G.shape) for G in Gs], backend, table,
                                            restarts), dtype=torch.uint8, device="cuda")
    for _ in range(warmup):
        nsmi.ns_batched(Gs, backend, table, restarts, outs=outs, workspace=ws)
    torch.cuda.synchronize()
    nsmi.ns_timing_enable(True)
    nsmi.ns_timing_read()  # clear
    # one event between consecutive steps: the block total gives ms_per_step,
    # the per-step spans their median
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record()
    for i in range(steps):
        nsmi.ns_batched(Gs, backend, table, restarts, outs=outs, workspace=ws)
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    nsmi.ns_timing_enable(False)
    rep = nsmi.ns_timing_read()
    ms = evs[0].elapsed_time(evs[-1]) / steps
    per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
    median = (per[(steps - 1) // 2] + per[steps // 2]) / 2
    del ws
    return {"ms_per_step": ms, "median_ms_per_step": median, "wall_s": wall, "timing": rep}


def time_muon(nsmi, torch, Gs, table, restarts, steps):
    """Fused Muon step on the same batch: bf16 gradients, fp32 momentum and
    parameters (updated in place), beta 0.95, lr 0.02, scale 1."""
    Ms = [torch.zeros(G.shape, dtype=torch.float32, device="cuda") for G in Gs]
    Ps = [torch.full(G.shape, 0.01, dtype=torch.float32, device="cuda") for G in Gs]
    nsmi.ns_muon_step(Gs, Ms, Ps, 0.95, 0.02, None, table, restarts)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        nsmi.ns_muon_step(Gs, Ms, Ps, 0.95, 0.02, None, table, restarts)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def time_sharded(nsmi, torch, G, table, restarts, shards, steps):
    """One matrix along the column-sharded route with `shards` virtual
    shards, against the unsharded call."""
    res = {}
    for name, fn in (("unsharded", lambda: nsmi.ns_gram(G, table, restarts)),
                     ("sharded", lambda: nsmi.ns_gram_sharded(G, shards, table, restarts))):
        fn()
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(steps):
            fn()
        end.record()
        torch.cuda.synchronize()
        res[name] = start.elapsed_time(end) / steps
    return res


def cpu_baseline(workload, restarts, budget_s):
    """The fp64 oracle on a bounded sample: one matrix per distinct Gram shape."""
    import numpy as np

    import workloads as W
    from oracle import COEFFICIENT_SETS, gram_newton_schulz

    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max([i.get("num_threads", 0) for i in libs] or [os.cpu_count()])
        if libs:
            blas = " ".join(str(libs[0].get(k, "")) for k in ("internal_api", "version",
                                                              "architecture")).strip()
    except Exception:  # pragma: no cover - informational only
        threads = os.cpu_count()
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((line.split(":", 1)[1].strip() for line in f
                              if line.startswith("model name")), cpu_model)
    except OSError:  # pragma: no cover - informational only
        pass

    w = W.WORKLOADS[workload]
    table = COEFFICIENT_SETS[w.coefficients]   # the oracle's own copy of the table
    classes = {}
    for j, (m, n) in enumerate(w.shapes):
        key = (min(m, n), max(m, n))
        classes.setdefault(key, []).append(j)
    # cheapest class first; oracle flops of one gram call (full fp64 products)
    def oracle_flops(s, l):
        return oracle_gram_flops(s, l, len(table), restarts)

    order = sorted(classes, key=lambda c: oracle_flops(*c))
    measured, spent, rate = {}, 0.0, None
    for key in order:
        est = oracle_flops(*key) / rate if rate else 0.0
        if measured and spent + est > budget_s:
            break
        j = classes[key][0]
        G = W.matrix(workload, j).float().numpy().astype(np.float64)
        t0 = time.perf_counter()
        gram_newton_schulz(G, table, restarts)
        dt = time.perf_counter() - t0
        spent += dt
        measured[key] = dt
        rate = oracle_flops(*key) / dt
        log(f"cpu oracle {key[0]}x{key[1]}: {dt:.2f} s ({rate / 1e9:.1f} GFLOP/s fp64)")
    total = 0.0
    for key, js in classes.items():
        t = measured.get(key, oracle_flops(*key) / rate)
        total += t * len(js)
    sample = ("fp64 numpy oracle (gram backend, same table and restarts) timed on one matrix "
              "of each Gram shape class " + ", ".join(f"{s}x{l}" for s, l in measured) +
              "; whole-batch time = sum over the batch of the measured per-class time"
              + ("" if len(measured) == len(classes) else
                 "; unmeasured classes scaled by fp64 flop count"))
    return {"value": len(w.shapes) / total, "unit": "matrices/s", "cores": int(threads),
            "kind": "oracle", "sample": sample, "batch_seconds_est": total,
            "sample_seconds": spent, "cpu_count": os.cpu_count(), "cpu_model": cpu_model,
            "blas": blas}


def target_status(tflops_step, n, w, ms, steps):
    """The 50%-of-peak target on the work this path does, and, for context
    only, the same time priced at the pages' flop count (see pages_flops),
    which counts every s^3 product at 2 s^3 although this path computes the
    Gram-space products on half the tiles: that figure is not work done and
    is never the target."""
    pct = 100.0 * tflops_step / PEAK_FP16_TFLOPS
    f = pages_flops(w.shapes, steps, w.restarts)
    return {
        "target_pct_fp16_peak": 50.0,
        "pct_fp16_peak_work_done": pct,
        "met": pct >= 50.0,
        "basis": "whole step (normalisation included), algorithmic flops of the work done: "
                 "symmetric products at s(s+1)k, general ones at 2mnk",
        "pages_flop_equivalent": {
            "pages_flops_per_step": f,
            "tflops": f / (ms * 1e-3) / 1e12,
            "note": "the same step time priced at the pages' flop count (SYRK at s(s+1)l, "
                    "Q X at 2s^2 l, every s^3 product at 2s^3); not work done, not the target"},
    }


def oracle_gram_flops(s_, l_, steps, restarts):
    """fp64 flops of one oracle gram call (full products): R = X X^T and every
    Q X at 2 s^2 l (one R and one Q X per effective restart, plus the first R
    and the output), Z = b R + c R R once per step, Q <- Z Q + a Q on every
    step that is not the first after a start or restart, and two products
    per R recurrence (k + 1 < K, k + 1 not a restart): 14 s^3 products for
    five steps with a restart before step 2."""
    K = steps
    S = {int(i) for i in restarts if 0 < int(i) < K}
    r = len(S)
    m3 = K + (K - 1 - r) + 2 * sum(1 for k in range(K - 1) if (k + 1) not in S)
    return (1 + r) * 2.0 * s_ * s_ * l_ + (1 + r) * 2.0 * s_ * s_ * l_ + m3 * 2.0 * s_ ** 3


def time_call(torch, fn, steps, warmup):
    """Median and mean ms of `fn` (one library call per step) on the current
    stream, inputs resident."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for i in range(steps):
        fn()
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
    return {"median_ms": (per[(steps - 1) // 2] + per[steps // 2]) / 2,
            "mean_ms": evs[0].elapsed_time(evs[-1]) / steps}


def graph_replay_ms(torch, fn, steps):
    """The call captured once into a HIP graph, then replayed: median ms per
    replay (None if capture fails)."""
    try:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return time_call(torch, g.replay, steps, 3)["median_ms"]
    except Exception as e:  # pragma: no cover - reported, not fatal
        log(f"graph capture failed: {e}")
        return None


def other_workloads(nsmi, torch, cpu_oracle):
    """Workloads 1, 2, 3 and 5 (the parity configurations): GPU time per call
    and, next to it, the fp64 oracle on the host (workload 1: median of
    three runs; the others: one run over the whole batch)."""
    import numpy as np
    import workloads as W
    from oracle import COEFFICIENT_SETS, direct_newton_schulz, gram_newton_schulz
    res = {}
    for wl, backends in ((1, ("gram", "direct")), (2, ("gram",)), (3, ("gram",)),
                         (5, ("gram",))):
        w = W.WORKLOADS[wl]
        Gs = [W.matrix(wl, j).cuda() for j in range(len(w.shapes))]
        outs = [torch.empty(G.shape, dtype=torch.float16, device="cuda") for G in Gs]
        table = nsmi.COEFFICIENT_SETS[w.coefficients]
        for be in backends:
            rs = w.restarts if be == "gram" else ()
            ws = torch.empty(nsmi.ns_workspace_size([tuple(G.shape) for G in Gs], be, table, rs),
                             dtype=torch.uint8, device="cuda")
            fn = (lambda be=be, rs=rs, ws=ws:
                  nsmi.ns_batched(Gs, be, table, rs, outs=outs, workspace=ws))
            steps = 50 if wl == 1 else 10
            t = time_call(torch, fn, steps, 3)
            key = f"workload{wl}_{be}"
            entry = {"matrices": len(Gs), "shape": list(w.shapes[0]) if len(set(w.shapes)) == 1
                     else "mixed", "coefficients": w.coefficients, "restarts": list(rs),
                     "gpu_median_ms_per_call": t["median_ms"],
                     "gpu_matrices_per_s": len(Gs) / (t["median_ms"] * 1e-3)}
            if wl == 1:
                entry["gpu_graph_replay_median_ms"] = graph_replay_ms(torch, fn, steps)
            if cpu_oracle:
                co = COEFFICIENT_SETS[w.coefficients]
                runs = 3 if wl == 1 else 1
                times = []
                for _ in range(runs):
                    t0 = time.perf_counter()
                    for G in Gs:
                        G64 = G.float().cpu().numpy().astype(np.float64)
                        if be == "gram":
                            gram_newton_schulz(G64, co, rs)
                        else:
                            direct_newton_schulz(G64, co)
                    times.append(time.perf_counter() - t0)
                cpu_s = sorted(times)[len(times) // 2]
                entry["cpu_oracle_s_per_call"] = cpu_s
                entry["cpu_oracle_matrices_per_s"] = len(Gs) / cpu_s
            res[key] = entry
            log(f"{key}: GPU {t['median_ms']:.3f} ms/call"
                + (f", graph replay {entry['gpu_graph_replay_median_ms']:.3f} ms"
                   if entry.get("gpu_graph_replay_median_ms") else "")
                + (f", oracle {entry['cpu_oracle_s_per_call']:.2f} s" if cpu_oracle else ""))
            del ws
        del Gs, outs
        torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}); the owner-"
              "rank Newton-Schulz path has no cross-GPU step to measure here.",
              file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return

    import torch

    import newton_schulz_matrix_amd as nsmi
    import workloads as W

    nsmi.library()
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    w = W.WORKLOADS[args.workload]
    table = nsmi.COEFFICIENT_SETS[w.coefficients]
    restarts = w.restarts
    log(nsmi.ns_backend_info())
    t0 = time.perf_counter()
    Gs = []
    for j in range(len(w.shapes)):
        Gs.append(W.matrix(args.workload, j).cuda())
    torch.cuda.synchronize()
    log(f"inputs: {len(Gs)} matrices generated in {time.perf_counter() - t0:.1f} s")
    outs = [torch.empty(G.shape, dtype=torch.float16, device="cuda") for G in Gs]
    if args.only == "muon":
        mu = time_muon(nsmi, torch, Gs, table, restarts, args.steps)
        print(json.dumps({"only": "muon_step", "ms_per_step": mu, "steps": args.steps,
                          "matrices": len(Gs)}), flush=True)
        return
    if args.only == "sharded":
        gate = next(G for G in Gs if tuple(G.shape) == (14336, 4096))
        sh = time_sharded(nsmi, torch, gate, table, restarts, 4, args.steps)
        print(json.dumps({"only": "tp_emulation", "shards": 4, "steps": args.steps,
                          "ms_sharded": sh["sharded"], "ms_unsharded": sh["unsharded"]}),
              flush=True)
        return

    backends = [args.backend]
    if not args.no_second_backend:
        backends.append("direct" if args.backend == "gram" else "gram")
    results = {}
    for be in backends:
        steps = args.steps if be == args.backend else max(1, min(args.steps, 3))
        r = time_backend(nsmi, torch, Gs, outs, be, table, restarts, steps,
                         args.warmup if be == args.backend else 1)
        r["steps"] = steps
        results[be] = r
        t = r["timing"]
        log(f"{be}: {r['ms_per_step']:.3f} ms/step, gemm {t['gemm_ms'] / steps:.3f} ms/step in "
            f"{t['gemm_launches'] // steps} launches, norm {t['norm_ms'] / steps:.3f} ms/step")

    head = results[args.backend]
    K = head["steps"]
    t = head["timing"]
    ms = head["ms_per_step"]
    n = len(Gs)
    flops_step = (t["gemm_flops"]) / K
    tflops = flops_step / (ms * 1e-3) / 1e12
    avg_launch_ms = t["gemm_ms"] / t["gemm_launches"]
    flops_per_launch = t["gemm_flops"] / t["gemm_launches"]
    achieved = flops_per_launch / (avg_launch_ms * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": n / (ms * 1e-3),
        "unit": "matrices/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "median_ms_per_step": head["median_ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "target": target_status(tflops, n, w, ms, len(table)),
        "config": {"workload": (f"Llama-3-8B owner share: 28 projections (4 x q/k/v/o/gate/"
                                f"up/down), bf16 N(0,1) gradients, one ns_batched call"
                                if args.workload == 4 else f"{w.name}, one ns_batched call"),
                   "matrices": n, "backend": args.backend, "coefficients": w.coefficients,
                   "restarts": list(restarts), "eps": 1e-7, "input_dtype": w.dtype,
                   "output_dtype": "f16"},
        "tflops": tflops,
        "pct_fp16_peak": 100.0 * tflops / PEAK_FP16_TFLOPS,
        "flops_per_step": flops_step,
        "roofline": {"bound": "mfma", "kernel": "gemm_nt_kernel (grouped fp16 MFMA)",
                     "achieved": achieved, "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_FP16_TFLOPS,
                     "traffic": (gemm_traffic_per_launch()
                                 if args.workload == 4 and args.backend == "gram" else None),
                     "traffic_unit": "bytes per launch (FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0)",
                     "launches_per_step": t["gemm_launches"] // K,
                     "avg_launch_ms": avg_launch_ms,
                     "flops_per_launch": flops_per_launch},
        "norm_pass": norm_pass_entry(t, K, Gs),
    }
    for be, r in results.items():
        if be == args.backend:
            continue
        tt = r["timing"]
        out[f"{be}_backend"] = {
            "ms_per_step": r["ms_per_step"], "steps": r["steps"],
            "matrices_per_s": n / (r["ms_per_step"] * 1e-3),
            "tflops": tt["gemm_flops"] / r["steps"] / (r["ms_per_step"] * 1e-3) / 1e12}
    if not args.no_second_backend and args.backend == "gram":
        mu = time_muon(nsmi, torch, Gs, table, restarts, 3)
        out["muon_step"] = {
            "ms_per_step": mu, "ns_ms_per_step": ms,
            "overhead_pct": 100.0 * (mu - ms) / ms,
            "config": "ns_muon_step on the same 28 matrices: bf16 gradients, fp32 momentum "
                      "and parameters, beta 0.95, lr 0.02 (momentum fused into the norm "
                      "pass, update into the final product)"}
        log(f"muon step: {mu:.3f} ms/step ({out['muon_step']['overhead_pct']:+.1f}% vs NS)")
        gate = next(G for G in Gs if tuple(G.shape) == (14336, 4096))
        sh = time_sharded(nsmi, torch, gate, table, restarts, 4, 5)
        out["tp_emulation"] = {
            "matrix": "gate projection 14336 x 4096 (bf16)", "shards": 4,
            "ms_sharded": sh["sharded"], "ms_unsharded": sh["unsharded"],
            "note": "ns_gram_sharded: 4 virtual column shards on one GPU; the shard "
                    "reduction stands in for the all-reduce"}
        log(f"tp emulation (4 shards, gate): {sh['sharded']:.3f} ms vs {sh['unsharded']:.3f} ms")
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.workload, restarts, args.cpu_budget)
    if not args.no_other_workloads and args.workload == 4:
        out["other_workloads"] = other_workloads(nsmi, torch, not args.no_cpu_baseline)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
