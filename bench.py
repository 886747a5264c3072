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
    "gemm_gram_256": "k_gemm<Cfg<256, 2, 4, 1>, 0, true, false>",
    "gemm_poly_256": "k_gemm<Cfg<256, 2, 4, 1>, 1, true, true>",
    "gemm_symm_256": "k_gemm<Cfg<256, 2, 4, 1>, 2, true, false>",
    "gemm_rect_256": "k_gemm<Cfg<256, 2, 4, 1>, 3, false, false>",
    "gemm_nsx_256": "k_gemm<Cfg<256, 2, 4, 1>, 4, false, true>",
    "gemm_nsx_128": "k_gemm<Cfg<128, 2, 2, 1>, 4, false, true>",
    "gemm_gram_128": "k_gemm<Cfg<128, 2, 2, 1>, 0, true, false>",
    "gemm_poly_128": "k_gemm<Cfg<128, 2, 2, 1>, 1, true, true>",
    "gemm_symm_128": "k_gemm<Cfg<128, 2, 2, 1>, 2, true, false>",
    "gemm_rect_128": "k_gemm<Cfg<128, 2, 2, 1>, 3, false, false>",
    "row_score": "k_row_score_f32",
    "accum_score": "k_accum_score_f32",
    "topk": "k_topk",
    "gather": "k_gather<float, true>",
    "gram_ns_fused_128": "k_gram_ns_small",
    "norm_rows": "k_norm_rows",
    "norm_scale": "k_norm_scale",
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
                        "beta2 = 0.95, eps = 1e-8) through dion3_step_megabatch_norm")
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


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: every matrix of a Dion3 step is independent, and this "
              "build runs the step on a single MI355X (multi-GPU sharding is a design note only). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

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
    lr = wl.lr

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

    groups = []
    grads = {}
    norms = {}
    max_ws = 0
    for gi, (g, Ws, Ms) in enumerate(data):
        k = d3.k_from_fraction(float(wl.fraction), g.n)
        ptrs = (d3.pointer_array(Ws, dev), d3.pointer_array(Ms, dev))
        groups.append((g, Ws, Ms, k, ptrs))
        max_ws = max(max_ws, d3.workspace_size(len(Ms), g.n, g.m, k))
        if args.accumulate:
            gen = torch.Generator(device=dev)
            gen.manual_seed(7000 + gi)
            Gs = [torch.randn(M.shape, generator=gen, device=dev).mul_(0.1) for M in Ms]
            grads[gi] = (Gs, d3.pointer_array(Gs, dev))
        if args.normalize:
            Vs = [torch.zeros(g.n, dtype=torch.float32, device=dev) for _ in Ms]
            norms[gi] = (Vs, d3.pointer_array(Vs, dev))
    nstreams = max(1, min(args.streams, len(groups)))
    if nstreams == 1:
        ws = d3.Workspace()
        ws.get(max_ws, dev)
        wss = [ws] * len(groups)
    else:
        wss = []
        for g, Ws, Ms, k, ptrs in groups:
            w_ = d3.Workspace()
            w_.get(d3.workspace_size(len(Ms), g.n, g.m, k), dev)
            wss.append(w_)
    side = [torch.cuda.Stream() for _ in range(nstreams)] if nstreams > 1 else []

    def one_step():
        if nstreams == 1:
            for gi, (g, Ws, Ms, k, ptrs) in enumerate(groups):
                gp = grads[gi][1] if gi in grads else None
                nrm = (norms[gi][0], 0.95, 1e-8) if gi in norms else None
                d3.step_megabatch(Ws, Ms, k, lr, mu, cfg, ws=wss[gi], ptrs=ptrs, gptrs=gp,
                                  norm=nrm, vptrs=norms[gi][1] if gi in norms else None)
            return
        main = torch.cuda.current_stream()
        for st in side:
            st.wait_stream(main)
        for gi, (g, Ws, Ms, k, ptrs) in enumerate(groups):
            gp = grads[gi][1] if gi in grads else None
            nrm = (norms[gi][0], 0.95, 1e-8) if gi in norms else None
            with torch.cuda.stream(side[gi % nstreams]):
                d3.step_megabatch(Ws, Ms, k, lr, mu, cfg, ws=wss[gi], ptrs=ptrs, gptrs=gp,
                                  norm=nrm, vptrs=norms[gi][1] if gi in norms else None)
        for st in side:
            main.wait_stream(st)

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()

    graph = None
    if args.graph:
        args.no_trace = True
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            one_step()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
    launches_per_step = sum(3 + 1 + 2 * (1 + cfg.n_restart) + 4 * cfg.iters + 3 for _ in groups)
    if not args.no_trace:
        d3.trace_enable(launches_per_step * args.steps + 64)
    stream = torch.cuda.current_stream()
    # one event before the first step and one after each step: the mean over
    # the whole timed region is the reported value; the per-step times give
    # its spread
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
    ms_total = evs[0].elapsed_time(evs[-1])
    ms_per_step = ms_total / args.steps
    step_ms = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))

    # per-kernel statistics over the timed region
    kernels = {}
    by_group = {}
    if not args.no_trace:
        gi = -1
        for name, ms, fl, by in d3.trace_records():
            if name in ("row_score", "accum_score"):   # every group's launch sequence starts so
                gi = (gi + 1) % len(groups)
            for table, key in ((kernels, name), (by_group, (gi, name))):
                st = table.setdefault(key, {"launches": 0, "ms": 0.0, "flops": 0.0, "bytes": 0.0})
                st["launches"] += 1
                st["ms"] += ms
                st["flops"] += fl
                st["bytes"] += by
        d3.trace_disable()
    for (gi, name), st in sorted(by_group.items()):
        g = groups[gi][0]
        rate = (f"{st['flops'] / (st['ms'] * 1e-3) / 1e12:7.1f} TFLOP/s" if st["flops"] > 0 else
                f"{st['bytes'] / (st['ms'] * 1e-3) / 1e9:7.1f} GB/s")
        log(f"  group {gi} ({g.count}x{g.n}x{g.m}, k={groups[gi][3]}) {name:10s} "
            f"avg {1e3 * st['ms'] / st['launches']:9.1f} us  ms/step {st['ms'] / args.steps:7.3f}  {rate}")
    for name, st in kernels.items():
        st["avg_us"] = 1e3 * st["ms"] / st["launches"]
        if st["flops"] > 0:
            st["tflops"] = st["flops"] / (st["ms"] * 1e-3) / 1e12
            st["frac_fp16_peak"] = st["tflops"] / FP16_PEAK_TFLOPS
        else:
            st["gbs"] = st["bytes"] / (st["ms"] * 1e-3) / 1e9
            st["frac_hbm"] = st["gbs"] / HBM_PEAK_GBS
        st["ms_per_step"] = st["ms"] / args.steps
        log(f"  {name:10s} launches/step {st['launches'] / args.steps:5.1f}  "
            f"avg {st['avg_us']:9.1f} us  ms/step {st['ms_per_step']:8.3f}  " +
            (f"{st['tflops']:7.1f} TFLOP/s ({100 * st['frac_fp16_peak']:.1f}% fp16 peak)"
             if st["flops"] > 0 else f"{st['gbs']:7.1f} GB/s ({100 * st['frac_hbm']:.1f}% HBM)"))

    gemm = [st for nm, st in kernels.items() if is_ns_kernel(nm)]
    gemm_flops = sum(st["flops"] for st in gemm) / max(1, args.steps)
    gemm_ms = sum(st["ms"] for st in gemm) / max(1, args.steps)
    gram_tflops = gemm_flops / (gemm_ms * 1e-3) / 1e12 if gemm_ms > 0 else None

    # standard-NS dense-equivalent work (a labelled "effective" number only)
    eff_flops = 0.0
    for g, Ws, Ms, k, ptrs in groups:
        s, L = min(k, g.m), max(k, g.m)
        eff_flops += g.count * cfg.iters * (4.0 * s * s * L + 2.0 * s ** 3)

    roofline = None
    if kernels:
        dom = max(kernels, key=lambda nm: kernels[nm]["ms"])
        st = kernels[dom]
        per_launch_work = (st["flops"] if st["flops"] > 0 else st["bytes"]) / st["launches"]
        if st["flops"] > 0:
            roofline = {"bound": "mfma", "achieved": round(st["tflops"], 2),
                        "peak": FP16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(st["tflops"] / FP16_PEAK_TFLOPS, 4)}
        else:
            roofline = {"bound": "hbm", "achieved": round(st["gbs"], 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(st["gbs"] / HBM_PEAK_GBS, 4)}
        roofline["traffic"] = load_traffic(dom, args.workload)
        roofline["kernel"] = KERNEL_SYMBOLS.get(dom, dom)
        roofline["avg_launch_us"] = round(st["avg_us"], 2)
        roofline["work_per_launch"] = per_launch_work

    # CPU baseline: the fp64 oracle on a bounded sample, scaled to the model
    cpu_baseline = None
    if samples:
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
            if t_cpu >= args.cpu_seconds and key in per_group:
                continue
            k = orc.k_from_fraction(wl.fraction, g.n)
            t = time.perf_counter()
            orc.dion3_step(W0, M0, k, lr, mu, method=args.method)
            dt = time.perf_counter() - t
            t_cpu += dt
            used += 1
            per_group.setdefault(key, []).append(dt)
        cpu_ms = 1e3 * sum(g[2] * (sum(v) / len(v)) for g, v in per_group.items())
        cpu_baseline = {"value": round(cpu_ms, 1), "unit": "ms per model step",
                        "cores": threads, "kind": "oracle",
                        "sample": f"{used} matrices of the set ("
                                  + ", ".join(f"{len(v)} x {n}x{m}" for (n, m, c), v in
                                              per_group.items()) +
                                  f"), fp64 NumPy oracle, {t_cpu:.1f}s of CPU work; the mean time "
                                  "per matrix of each shape group is scaled by the group's "
                                  "matrix count to one whole-model step"}
        log(f"cpu oracle: {t_cpu:.1f}s for {used} matrices -> {cpu_ms:.0f} ms/model step "
            f"({threads} BLAS threads, os.cpu_count()={os.cpu_count()})")

    out = {
        "metric": METRIC,
        "value": round(ms_per_step, 3),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
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
            "k": [k for (_, _, _, k, _) in groups],
            "lr": lr, "mu": mu, "ns_iters": cfg.iters,
            "restart_at": [cfg.restart_at[i] for i in range(cfg.n_restart)],
            "state_dtype": "fp32 W and M; fp16 X, Gram, polynomials and O with fp32 accumulation",
            "parallelism": "single GPU, one megabatched call per shape group" +
                           (f", groups on {nstreams} streams" if nstreams > 1 else ""),
            "gradient_accumulation": bool(args.accumulate),
            "per_neuron_normalization": bool(args.normalize),
            "hip_graph": bool(args.graph),
        },
        "matrices_per_s": round(wl.n_matrices / (ms_per_step * 1e-3), 1),
        "step_ms": {"median": round(float(np.median(step_ms)), 4),
                    "p10": round(float(np.percentile(step_ms, 10)), 4),
                    "p90": round(float(np.percentile(step_ms, 90)), 4)},
        "gram_ns_tflops": round(gram_tflops, 2) if gram_tflops else None,
        "gram_ns_frac_fp16_peak": round(gram_tflops / FP16_PEAK_TFLOPS, 4) if gram_tflops else None,
        "effective_standard_ns_tflops": round(eff_flops / (ms_per_step * 1e-3) / 1e12, 2),
        "roofline": roofline,
        "cpu_baseline": cpu_baseline,
        "kernels": {nm: {kk: (round(v, 4) if isinstance(v, float) else v) for kk, v in st.items()}
                    for nm, st in kernels.items()},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
