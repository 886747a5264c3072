"""Benchmark of the Dion3 optimizer step on one MI355X.

One step = one Dion3 optimizer step over a whole model's weight set: for
every shape group, l1 row scoring, top-k selection, Gram Newton-Schulz on
the selected rows and the row-sparse update with momentum decay, all in the
library's kernels, inputs resident in HBM.  Prints one JSON line.

Default workload: the 7B-like dense transformer weight set (hidden 4096, 32
layers: 128 x 4096x4096, 64 x 11008x4096, 32 x 4096x11008; fp32 W and M) at
f = 1/4, the setting of the pages' largest measured step speedup.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP16_PEAK_TFLOPS = 2500.0      # MI355X dense fp16 MFMA
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
METRIC = "Dion3 optimizer-step ms per model + Gram-NS TFLOP/s (% fp16 MFMA peak)"

# trace name -> the kernel symbol rocprofv3 reports for it
KERNEL_SYMBOLS = {
    "gemm_gram_256": "k_gemm<Cfg<256, 2, 4, 1>, 0, true, false, false>",
    "gemm_poly_256": "k_gemm<Cfg<256, 2, 4, 1>, 1, true, true, false>",
    "gemm_symm_256": "k_gemm<Cfg<256, 2, 4, 1>, 2, true, false, false>",
    "gemm_rect_256": "k_gemm<Cfg<256, 2, 4, 1>, 3, false, false, true>",
    "gemm_nsx_256": "k_gemm<Cfg<256, 2, 4, 1>, 4, false, true, false>",
    "gemm_back_256": "k_gemm<Cfg<256, 2, 4, 1>, 5, false, false, true>",
    "gemm_gram_128": "k_gemm<Cfg<128, 2, 2, 1>, 0, true, false, false>",
    "gemm_poly_128": "k_gemm<Cfg<128, 2, 2, 1>, 1, true, true, false>",
    "gemm_symm_128": "k_gemm<Cfg<128, 2, 2, 1>, 2, true, false, false>",
    "gemm_rect_128": "k_gemm<Cfg<128, 2, 2, 1>, 3, false, false, true>",
    "gemm_nsx_128": "k_gemm<Cfg<128, 2, 2, 1>, 4, false, true, false>",
    "gemm_back_128": "k_gemm<Cfg<128, 2, 2, 1>, 5, false, false, true>",
    "row_score": "k_row_score_f32",
    "accum_score": "k_accum_score_f32",
    "topk": "k_topk",
    "gather": "k_gather<float, true>",
    "gather_rows": "k_gather_rows<float, true>",
    "gram_ns_fused_128": "k_gram_ns_small",
    "gram_ns_fused_64": "k_gram_ns_tiny<2>",
    "gram_ns_fused_32": "k_gram_ns_tiny<1>",
    "norm_rows": "k_norm_rows",
    "norm_stats": "k_norm_stats",
    "norm_update": "k_norm_update",
}


def is_ns_kernel(name: str) -> bool:
    """The orthogonalization's products: tiled GEMMs or the fused small-Gram kernel."""
    return name.startswith("gemm_") or name.startswith("gram_ns_fused")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None,
                   help="timed steps (default: 50 for the small workloads c1-c3, 10 otherwise)")
    p.add_argument("--warmup", type=int, default=None,
                   help="untimed steps first (default: 5 for c1-c3, 2 otherwise)")
    p.add_argument("--workload", default="c4",
                   help="c1, c2, c3, c4 (7B f=1/4), c4h (7B f=1/2), c4f (7B f=1), c5")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--method", default="gram", choices=["gram", "standard"],
                   help="gram: Gram Newton-Schulz (the step); standard: the iteration on X itself "
                        "(the Muon baseline, on the same kernels)")
    p.add_argument("--no-trace", action="store_true")
    p.add_argument("--normalize", action="store_true",
                   help="per-neuron normalization of the update (fp32 second moment per row, "
                        "beta2 = 0.95, eps = 1e-8), the norm argument of dion3_step_groups")
    p.add_argument("--accumulate", action="store_true",
                   help="each step first accumulates a gradient into the momentum (M <- M + G, "
                        "fused into the row scoring); gradients are fixed seeded N(0, 0.1^2)")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="CPU-baseline budget: oracle matrices are taken round-robin over the "
                        "shape groups until this much CPU time is spent (at least one per group)")
    p.add_argument("--streams", type=int, default=1,
                   help="run the shape groups on this many HIP streams (forked from and joined "
                        "back into the current stream each step), each group with its own "
                        "workspace, so that one group's memory-bound kernels overlap another's "
                        "products")
    p.add_argument("--graph", action="store_true",
                   help="capture one whole step (every group's launches) in a HIP graph and time "
                        "its replays (the per-kernel trace is then off)")
    p.add_argument("--per-group", action="store_true",
                   help="one library call per shape group (dion3_step_megabatch's launch "
                        "sequence) instead of one call for all groups")
    p.add_argument("--also-fraction", default="1/2",
                   help="for the 7B set (c4), also step the same resident matrices at this "
                        "fraction and report it in a sub-object (\"none\" to skip)")
    p.add_argument("--paths", action="store_true",
                   help="only time one dion3_gram_ns call on the fused and the tiled path for "
                        "Gram sides up to 128 (the measurements behind the automatic path "
                        "rule) and print the table")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 2 GiB device-to-device copy (a known-size kernel for "
                        "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE) and print its GB/s")
    return p.parse_args()


def copy_calibration():
    """A plain device copy of known size: its FETCH_SIZE / WRITE_SIZE counters
    give the factor between counter units and bytes, and its rate is the
    practical HBM ceiling."""
    import torch
    n = 1 << 29                      # 512 Mi fp32 = 2 GiB read + 2 GiB written
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n,
                      "ms": round(ms, 4), "gbs": round(8 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)


# (matrices, k, m) of the fused / tiled comparison: Gram sides 32, 64 and 128
# at short and long rows, few and many matrices
PATH_SHAPES = [(1, 32, 512), (1, 64, 512), (1, 32, 4096), (16, 32, 8192), (64, 32, 8192),
               (1, 64, 2048), (1, 64, 4096), (16, 64, 4096), (64, 64, 4096), (16, 64, 8192),
               (64, 64, 8192), (512, 32, 256), (512, 64, 256), (2048, 32, 512), (1, 128, 1024),
               (1, 128, 2048), (32, 128, 2048), (16, 128, 4096), (256, 128, 512)]


def path_crossover(reps: int = 20):
    """One dion3_gram_ns call on the fused and on the tiled path (HIP events
    around `reps` eager calls, after one warm-up call), and which path the
    automatic rule takes (from the names of the kernels it launches)."""
    import torch
    import orthogonalizing_optimizer_amd as d3

    def timed(X, path):
        cfg = d3.ns_cfg(path=path)
        d3.gram_ns(X, cfg)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            d3.gram_ns(X, cfg)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3

    rows = []
    for B, k, m in PATH_SHAPES:
        g = torch.Generator(device="cuda:0")
        g.manual_seed(B * 7919 + k * 31 + m)
        X = (torch.randn((B, k, m), generator=g, device="cuda:0") * 0.05).to(torch.float16)
        fused, tiled = timed(X, d3.PATH_FUSED), timed(X, d3.PATH_TILED)
        d3.trace_enable(4096)
        d3.trace_reset()
        d3.gram_ns(X, d3.ns_cfg())
        auto = "fused" if any(r[0].startswith("gram_ns_fused") for r in d3.trace_records()) else "tiled"
        d3.trace_disable()
        rows.append({"matrices": B, "k": k, "m": m, "fused_us": round(fused, 1),
                     "tiled_us": round(tiled, 1), "auto": auto})
        log(f"{B:5d} x {k:4d} x {m:5d}: fused {fused:8.1f} us  tiled {tiled:8.1f} us  "
            f"auto takes {auto}")
        del X
    print(json.dumps({"paths": rows, "reps": reps}), flush=True)


def kernel_source_hash(kernel: str) -> str:
    """Hash of the source file that holds this kernel's device code."""
    if kernel.startswith("gemm_"):
        f = "gemm_f16.hip"
    elif kernel.startswith("gram_ns_fused"):
        f = "gram_small.hip"
    elif kernel.startswith("norm_"):
        f = "normalize.hip"
    else:
        f = "rows.hip"
    with open(os.path.join(ROOT, "orthogonalizing_optimizer_amd", "csrc", f), "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    or None when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
        ent = d.get(workload, {}).get(kernel)
        if not ent or ent.get("source_hash") != kernel_source_hash(kernel):
            return None
        return float(ent["bytes_per_launch"])
    except (ValueError, KeyError, TypeError):
        return None


def kernel_stats(records, steps):
    """Per-kernel totals over the timed region, from the library's trace, and
    per (kernel, work per launch), which tells the shapes apart."""
    kernels, by_shape = {}, {}
    for name, ms, fl, by in records:
        for table, key in ((kernels, name), (by_shape, (name, fl, by))):
            st = table.setdefault(key, {"launches": 0, "ms": 0.0, "flops": 0.0, "bytes": 0.0})
            st["launches"] += 1
            st["ms"] += ms
            st["flops"] += fl
            st["bytes"] += by
    for table in (kernels, by_shape):
        for st in table.values():
            t = st["ms"] * 1e-3
            st["avg_us"] = 1e3 * st["ms"] / st["launches"]
            st["ms_per_step"] = st["ms"] / steps
            st["tflops"] = st["flops"] / t / 1e12 if st["flops"] > 0 else 0.0
            st["gbs"] = st["bytes"] / t / 1e9 if st["bytes"] > 0 else 0.0
            st["frac_fp16_peak"] = st["tflops"] / FP16_PEAK_TFLOPS
            st["frac_hbm"] = st["gbs"] / HBM_PEAK_GBS
            # the roofline of a kernel that does both: the larger of its flop
            # time and its byte time at the peaks, over its measured time
            st["bound"] = "mfma" if st["frac_fp16_peak"] >= st["frac_hbm"] else "hbm"
            st["frac_roofline"] = max(st["frac_fp16_peak"], st["frac_hbm"])
    return kernels, by_shape


def roofline_of(kernels, workload):
    """The roofline object of the dominant kernel (most time per step)."""
    if not kernels:
        return None
    dom = max(kernels, key=lambda nm: kernels[nm]["ms"])
    st = kernels[dom]
    if st["bound"] == "mfma":
        r = {"bound": "mfma", "achieved": round(st["tflops"], 2), "peak": FP16_PEAK_TFLOPS,
             "unit": "TFLOP/s", "frac": round(st["frac_fp16_peak"], 4)}
        work = st["flops"] / st["launches"]
    else:
        r = {"bound": "hbm", "achieved": round(st["gbs"], 1), "peak": HBM_PEAK_GBS,
             "unit": "GB/s", "frac": round(st["frac_hbm"], 4)}
        work = st["bytes"] / st["launches"]
    r["traffic"] = load_traffic(dom, workload)
    r["kernel"] = KERNEL_SYMBOLS.get(dom, dom)
    r["avg_launch_us"] = round(st["avg_us"], 2)
    r["work_per_launch"] = work
    return r


def multiply_back_of(kernels):
    """The final multiply-back with the fused row-sparse update, against both
    of its bounds: its flops (2 s^2 L) and its bytes (X and Q read, the
    selected rows of W read and written)."""
    names = [nm for nm in kernels if nm.startswith("gemm_back_")]
    if not names:
        return None
    st = {"launches": 0, "ms": 0.0, "flops": 0.0, "bytes": 0.0}
    for nm in names:
        for key in st:
            st[key] += kernels[nm][key]
    t = st["ms"] * 1e-3
    tf, gb = st["flops"] / t / 1e12, st["bytes"] / t / 1e9
    return {"kernels": [KERNEL_SYMBOLS.get(nm, nm) for nm in names],
            "avg_launch_us": round(1e3 * st["ms"] / st["launches"], 2),
            "tflops": round(tf, 2), "frac_fp16_peak": round(tf / FP16_PEAK_TFLOPS, 4),
            "gbs": round(gb, 1), "frac_hbm": round(gb / HBM_PEAK_GBS, 4),
            "bound": "mfma" if tf / FP16_PEAK_TFLOPS >= gb / HBM_PEAK_GBS else "hbm",
            "frac_roofline": round(max(tf / FP16_PEAK_TFLOPS, gb / HBM_PEAK_GBS), 4)}


def cpu_baseline_of(samples, fraction, lr, mu, method, budget_s):
    """The fp64 oracle on a bounded sample of the matrices, scaled to one
    whole-model step."""
    from oracle import dion3_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    per_group = {}
    t_cpu = 0.0
    used = 0
    for g, W0, M0 in samples:
        key = (g.n, g.m, g.count)
        if t_cpu >= budget_s and key in per_group:
            continue
        k = orc.k_from_fraction(fraction, g.n)
        t = time.perf_counter()
        orc.dion3_step(W0, M0, k, lr, mu, method=method)
        dt = time.perf_counter() - t
        t_cpu += dt
        used += 1
        per_group.setdefault(key, []).append(dt)
    cpu_ms = 1e3 * sum(g[2] * (sum(v) / len(v)) for g, v in per_group.items())
    log(f"cpu oracle (f = {fraction}): {t_cpu:.1f}s for {used} matrices -> {cpu_ms:.0f} ms/model "
        f"step ({threads} BLAS threads, os.cpu_count()={os.cpu_count()})")
    return {"value": round(cpu_ms, 1), "unit": "ms per model step", "cores": threads,
            "kind": "oracle",
            "sample": f"{used} matrices of the set ("
                      + ", ".join(f"{len(v)} x {n}x{m}" for (n, m, c), v in per_group.items()) +
                      f"), fp64 NumPy oracle, {t_cpu:.1f}s of CPU work; the mean time per matrix "
                      "of each shape group is scaled by the group's matrix count to one "
                      "whole-model step"}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.paths:
        path_crossover()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: every matrix of a Dion3 step is independent, and this "
              "build runs the step on a single MI355X (multi-GPU sharding is a design note only). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    from fractions import Fraction

    import numpy as np
    import torch

    import orthogonalizing_optimizer_amd as d3
    from workloads import WORKLOADS, device_workload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    dev = "cuda:0"
    wl = WORKLOADS[args.workload]
    small = args.workload in ("c1", "c2", "c3")
    if args.steps is None:
        args.steps = 50 if small else 10
    if args.warmup is None:
        args.warmup = 5 if small else 2
    cfg = d3.default_cfg()
    if args.method == "standard":
        cfg.method = d3.NS_STANDARD
    mu = 0.95

    t_gen = time.time()
    data = device_workload(wl, dev)
    torch.cuda.synchronize()
    log(f"generated {wl.name}: {wl.n_matrices} matrices, {wl.n_params / 1e9:.2f} B params "
        f"in {time.time() - t_gen:.1f}s")

    # host copies of the CPU-baseline sample candidates (initial state); at
    # most 8 per group, used round-robin until the CPU budget is spent
    samples = []
    if not args.no_cpu_baseline:
        for j in range(8):
            for g, Ws, Ms in data:
                if j < g.count:
                    samples.append((g, Ws[j].cpu().numpy(), Ms[j].cpu().numpy()))

    grads, norms = {}, {}
    for gi, (g, Ws, Ms) in enumerate(data):
        if args.accumulate:
            gen = torch.Generator(device=dev)
            gen.manual_seed(7000 + gi)
            grads[gi] = [torch.randn(M.shape, generator=gen, device=dev).mul_(0.1) for M in Ms]
        if args.normalize:
            norms[gi] = [torch.zeros(g.n, dtype=torch.float32, device=dev) for _ in Ms]
    norm = (0.95, 1e-8) if args.normalize else None
    ws = d3.Workspace()

    def run(fraction):
        """Warm-up, then the timed steps at this fraction; returns the
        result fields of that run."""
        lr = 0.02 / math.sqrt(float(fraction))
        groups = []
        for gi, (g, Ws, Ms) in enumerate(data):
            k = d3.k_from_fraction(float(fraction), g.n)
            groups.append(d3.Group(Ws, Ms, k, lr, Gs=grads.get(gi), Vs=norms.get(gi)))
        nstreams = max(1, min(args.streams, len(groups)))
        per_group = args.per_group or nstreams > 1
        if per_group:
            wss = [ws] * len(groups) if nstreams == 1 else [d3.Workspace() for _ in groups]
            side = [torch.cuda.Stream() for _ in range(nstreams)] if nstreams > 1 else []
        ws.get(d3.workspace_size_groups(groups, cfg), dev)

        def one_step():
            if not per_group:
                d3.step_groups(groups, mu, cfg, norm=norm, ws=ws)
                return
            if nstreams == 1:
                for gr, w_ in zip(groups, wss):
                    d3.step_groups([gr], mu, cfg, norm=norm, ws=w_)
                return
            main_s = torch.cuda.current_stream()
            for st in side:
                st.wait_stream(main_s)
            for gi, gr in enumerate(groups):
                with torch.cuda.stream(side[gi % nstreams]):
                    d3.step_groups([gr], mu, cfg, norm=norm, ws=wss[gi])
            for st in side:
                main_s.wait_stream(st)

        for _ in range(args.warmup):
            one_step()
        torch.cuda.synchronize()
        graph = None
        no_trace = args.no_trace
        if args.graph:
            no_trace = True
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                one_step()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
        launches_per_step = len(groups) * (3 + 2 * (1 + cfg.n_restart) + 5 * cfg.iters + 8)
        stream = torch.cuda.current_stream()

        def timed(trace):
            # one event before the first step and one after each step: the
            # mean over the whole timed region, and the per-step times for
            # its spread; with `trace`, the library's per-kernel events too
            if trace:
                d3.trace_enable(launches_per_step * args.steps + 64)
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
            torch.cuda.synchronize()
            evs[0].record(stream)
            for i in range(args.steps):
                if graph is not None:
                    graph.replay()
                else:
                    one_step()
                evs[i + 1].record(stream)
            torch.cuda.synchronize()
            recs = None
            if trace:
                recs = d3.trace_records()
                d3.trace_disable()
            return (evs[0].elapsed_time(evs[-1]) / args.steps,
                    sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)), recs)

        # the reported step time comes from steps with the trace off (on small
        # steps its events cost a few microseconds per kernel); the same
        # number of steps then runs again with it on, for the per-kernel
        # figures and the roofline
        ms_per_step, step_ms, _ = timed(False)
        kernels, by_shape = {}, {}
        ms_traced = None
        if not no_trace:
            ms_traced, _, recs = timed(True)
            kernels, by_shape = kernel_stats(recs, args.steps)
        log(f"-- {wl.name} at f = {fraction}: {ms_per_step:.3f} ms per step"
            + (f" ({ms_traced:.3f} with the kernel trace on)" if ms_traced is not None else ""))
        for (name, fl, by), st in sorted(by_shape.items()):
            rate = (f"{st['tflops']:7.1f} TFLOP/s" if fl > 0 else "") + \
                   (f"  {st['gbs']:7.1f} GB/s" if by > 0 else "")
            log(f"  {name:18s} x{st['launches'] / args.steps:4.1f}/step  avg {st['avg_us']:9.1f} us"
                f"  ms/step {st['ms_per_step']:7.3f}  {rate}  roofline {st['frac_roofline']:.3f}"
                f" ({st['bound']})")
        for name, st in kernels.items():
            log(f"  {name:18s} launches/step {st['launches'] / args.steps:5.1f}  "
                f"avg {st['avg_us']:9.1f} us  ms/step {st['ms_per_step']:8.3f}  "
                f"{st['tflops']:7.1f} TFLOP/s ({100 * st['frac_fp16_peak']:.1f}% fp16)  "
                f"{st['gbs']:7.1f} GB/s ({100 * st['frac_hbm']:.1f}% HBM)")
        gemm = [st for nm, st in kernels.items() if is_ns_kernel(nm)]
        gemm_flops = sum(st["flops"] for st in gemm) / max(1, args.steps)
        gemm_ms = sum(st["ms"] for st in gemm) / max(1, args.steps)
        gram_tflops = gemm_flops / (gemm_ms * 1e-3) / 1e12 if gemm_ms > 0 else None
        # standard-NS dense-equivalent work (a labelled "effective" number only)
        eff_flops = 0.0
        for gr in groups:
            s_, L_ = min(gr.k, gr.m), max(gr.k, gr.m)
            eff_flops += gr.batch * cfg.iters * (4.0 * s_ * s_ * L_ + 2.0 * s_ ** 3)
        cpu = (cpu_baseline_of(samples, fraction, lr, mu, args.method, args.cpu_seconds)
               if samples else None)
        return {
            "ms_per_step": round(ms_per_step, 3),
            "ms_per_step_traced": round(ms_traced, 3) if ms_traced is not None else None,
            "k": [gr.k for gr in groups], "lr": round(lr, 6),
            "matrices_per_s": round(wl.n_matrices / (ms_per_step * 1e-3), 1),
            "step_ms": {"median": round(float(np.median(step_ms)), 4),
                        "p10": round(float(np.percentile(step_ms, 10)), 4),
                        "p90": round(float(np.percentile(step_ms, 90)), 4)},
            "gram_ns_tflops": round(gram_tflops, 2) if gram_tflops else None,
            "gram_ns_frac_fp16_peak": round(gram_tflops / FP16_PEAK_TFLOPS, 4) if gram_tflops
            else None,
            "effective_standard_ns_tflops": round(eff_flops / (ms_per_step * 1e-3) / 1e12, 2),
            "roofline": roofline_of(kernels, args.workload if fraction == wl.fraction else
                                    {"1/2": "c4h", "1": "c4f"}.get(str(fraction))),
            "multiply_back": multiply_back_of(kernels),
            "cpu_baseline": cpu,
            "kernels": {nm: {kk: (round(v, 4) if isinstance(v, float) else v)
                             for kk, v in st.items()} for nm, st in kernels.items()},
        }

    head = run(wl.fraction)
    extra = None
    also = None if args.also_fraction in ("", "none") else Fraction(args.also_fraction)
    if also is not None and args.workload == "c4" and also != wl.fraction:
        extra = run(also)

    out = {
        "metric": METRIC,
        "value": head["ms_per_step"],
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "ms_per_step_traced": head["ms_per_step_traced"],
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "matrices": wl.n_matrices,
            "params": wl.n_params,
            "shape_groups": [f"{g.count}x{g.n}x{g.m}" for g in wl.groups],
            "fraction": str(wl.fraction),
            "k": head["k"],
            "lr": head["lr"], "mu": mu, "ns_iters": cfg.iters,
            "restart_at": [cfg.restart_at[i] for i in range(cfg.n_restart)],
            "state_dtype": "fp32 W and M; fp16 X, Gram, polynomials and O with fp32 accumulation",
            "parallelism": "single GPU, " + (
                "one megabatched call per shape group" if (args.per_group or args.streams > 1)
                else "one call for all shape groups (each s x s product one launch over all "
                     "Gram-side sets, each Gram one launch over all groups)") +
                (f", groups on {args.streams} streams" if args.streams > 1 else ""),
            "gradient_accumulation": bool(args.accumulate),
            "per_neuron_normalization": bool(args.normalize),
            "hip_graph": bool(args.graph),
        },
    }
    for key in ("matrices_per_s", "step_ms", "gram_ns_tflops", "gram_ns_frac_fp16_peak",
                "effective_standard_ns_tflops", "roofline", "multiply_back", "cpu_baseline",
                "kernels"):
        out[key] = head[key]
    if extra is not None:
        # the same resident matrices stepped at the other fraction the pages
        # quote for this model (the timed region and protocol are the same)
        out["at_fraction_" + str(also).replace("/", "_")] = {
            "workload": wl.name.replace("f" + str(wl.fraction), "f" + str(also)),
            "fraction": str(also),
            **{key: extra[key] for key in ("ms_per_step", "k", "lr", "matrices_per_s", "step_ms",
                                           "gram_ns_tflops", "gram_ns_frac_fp16_peak",
                                           "effective_standard_ns_tflops", "roofline",
                                           "multiply_back", "cpu_baseline")}}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
