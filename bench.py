"""Benchmark of the quantized skinny linear path on one MI355X.

A step is one pass of the hot path over one batch of synthetic inputs: for
every token count M of the workload and every linear layer of the model, the
whole quantized linear (qlin_linear: activation quantization and GEMM, as one
fused kernel or two, per the selection table), replayed from a hipGraph
captured once (the decode path runs only under graph replay).  Weights live in HBM as
R distinct rotating copies (>= 1 GiB in total) so the 256 MiB Infinity Cache
cannot serve them; activations, scales and outputs are resident too.

Prints one JSON line: whole-step throughput (algorithmic bytes / time), the
GEMM roofline entry (its algorithmic bytes over its measured duration, from
HIP events around graphs of the GEMM launches alone) and the CPU oracle timed
on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "skinny W8A8 GEMM achieved HBM GB/s & TFLOP/s at M=1..32, % of roofline"
HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "fp8_dynamic_hidden2048"
DTYPE = {0: "fp8_e4m3", 1: "int8", 2: "fp8_e4m3"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--detail", default=None, help="write per-shape GEMM timings (JSON) here")
    ap.add_argument("--gemm-only-steps", type=int, default=None,
                    help="replay only the GEMM graphs this many times (for profiling)")
    ap.add_argument("--calibrate-copy", type=int, default=0,
                    help="first run a plain device-to-device copy of this many bytes three "
                         "times (reference dispatches for the memory-traffic counters)")
    return ap.parse_args()


class Linear:
    """Device buffers of one (M, layer) linear, for one weight copy set."""

    def __init__(self, fmt, M, layer, wq, ws, dev):
        import torch
        import skinny_bit_gemm_amd as q
        import workloads as wl
        self.fmt, self.M, self.N, self.K = fmt, M, layer.N, layer.K
        self.name = layer.name
        x = wl.activations(fmt, layer.N, layer.K, M)
        self.x = torch.from_numpy(x.view("int16")).to(dev)
        self.xq = torch.empty((M, layer.K), dtype=torch.uint8, device=dev)
        self.xs = torch.empty(q.scales_shape(fmt, M, layer.K, False), dtype=torch.float32, device=dev)
        self.wq, self.ws = wq, ws
        self.y = torch.empty((M, layer.N), dtype=torch.bfloat16, device=dev)
        self.cfg = q.qlin_select_variant(fmt, M, layer.N, layer.K)
        nb = q.qlin_workspace_bytes(fmt, M, layer.N, layer.K, self.cfg)
        self.work = torch.zeros(max(nb, 256), dtype=torch.uint8, device=dev)
        self.bytes = wl.algorithmic_bytes(fmt, M, layer.N, layer.K)
        self.qbytes = wl.quant_bytes(fmt, M, layer.K)
        self.flops = wl.flops(M, layer.N, layer.K)

    def layer(self, stream):
        """The whole decode linear: quantize + GEMM (one or two kernels, as tuned)."""
        import skinny_bit_gemm_amd as q
        q.qlin_linear(self.fmt, self.M, self.N, self.K, self.x, self.K, self.xq, self.xs, self.wq,
                      self.ws, self.y, q.QLIN_OUT_BF16, self.cfg, self.work, stream=stream)

    def gemm(self, stream, wq=None):
        import skinny_bit_gemm_amd as q
        q.qlin_gemm(self.fmt, self.M, self.N, self.K, self.xq, self.xs, self.wq if wq is None else wq,
                    self.ws, self.y, q.QLIN_OUT_BF16, self.cfg, self.work, stream=stream)


def measured_traffic(workload):
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary,
    or None when there is none or the kernels or the table changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"gemm_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    sha = lambda p: hashlib.sha256(open(os.path.join(ROOT, p), "rb").read()).hexdigest()
    if rec.get("kernel_source_sha256") != sha("skinny_bit_gemm_amd/csrc/qlin_kernels.hip") or \
            rec.get("table_sha256") != sha("skinny_bit_gemm_amd/tables/gfx950.tbl"):
        return None
    return rec


def capture(stream, fn):
    import skinny_bit_gemm_amd as q
    q.qlin_graph_begin(stream)
    try:
        fn()
    finally:
        g = q.qlin_graph_end(stream)
    return g


def cpu_baseline(fmt, layers, Ms, budget_s):
    """Time the oracle (as it is) on whole passes over the same workload."""
    import oracle
    import workloads as wl
    oracle.build()
    threads = oracle.num_threads()
    # weights are quantized beforehand (offline on both sides, untimed)
    qweights = {L.name: oracle.quant_weight(fmt, wl.weights(fmt, L.N, L.K)) for L in layers}
    xs = {(M, L.name): wl.activations(fmt, L.N, L.K, M) for M in Ms for L in layers}
    pass_bytes = sum(wl.algorithmic_bytes(fmt, M, L.N, L.K) + wl.quant_bytes(fmt, M, L.K)
                     for M in Ms for L in layers)

    def one_pass():
        t0 = time.perf_counter()
        for M in Ms:
            for L in layers:
                qw, sw = qweights[L.name]
                oracle.linear(fmt, xs[(M, L.name)], qw, sw)
        return time.perf_counter() - t0

    one_pass()                      # warm-up
    times = []
    spent = 0.0
    while len(times) < 3 or (spent < budget_s and len(times) < 50):
        t = one_pass()
        times.append(t)
        spent += t
        if spent > 4 * budget_s:
            break
    best = min(times)
    return {
        "value": round(pass_bytes / best / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"the whole workload ({len(layers) * len(Ms)} linears: quantize + product + "
                  f"epilogue each), best of {len(times)} timed passes after one warm-up, "
                  f"{spent:.1f} s of CPU time in total",
        "ms_per_pass": round(best * 1e3, 2),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import skinny_bit_gemm_amd as q
    import workloads as wl

    if args.workload not in wl.WORKLOADS:
        sys.exit(f"unknown workload {args.workload}; choose from {sorted(wl.WORKLOADS)}")
    fmt, layers, Ms = wl.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q.lib()
    if args.calibrate_copy:
        src = torch.ones(args.calibrate_copy // 4, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # quantized weights (GPU quantizer, offline and untimed), then rotating copies
    base = {}
    for L in layers:
        w = torch.from_numpy(wl.weights(fmt, L.N, L.K)).to(dev)
        wq = torch.empty((L.N, L.K), dtype=torch.uint8, device=dev)
        ws = torch.empty(q.scales_shape(fmt, L.N, L.K, True), dtype=torch.float32, device=dev)
        q.qlin_quantize_weight(fmt, L.N, L.K, w, wq, ws)
        base[L.name] = (wq, ws)
        del w
    torch.cuda.synchronize()
    step_wbytes = sum(L.N * L.K for L in layers) * len(Ms)
    n_sets = max(2, -(-(1 << 30) // step_wbytes))
    sets = []
    for s in range(n_sets):
        lin = []
        for M in Ms:
            for L in layers:
                wq, ws = base[L.name]
                lin.append(Linear(fmt, M, L, wq.clone(), ws, dev))
        sets.append(lin)
    torch.cuda.synchronize()

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        # eager once (also checks every launch is accepted), then capture
        for lin in sets[0]:
            lin.layer(stream)
            lin.gemm(stream)
        torch.cuda.synchronize()
        step_graphs = [capture(stream, lambda ls=ls: [l.layer(stream) for l in ls]) for ls in sets]
        gemm_graphs = [capture(stream, lambda ls=ls: [l.gemm(stream) for l in ls]) for ls in sets]
        torch.cuda.synchronize()

        step_bytes = sum(l.bytes + l.qbytes for l in sets[0])
        gemm_bytes = sum(l.bytes for l in sets[0])
        step_flops = sum(l.flops for l in sets[0])
        n_gemm = len(sets[0])

        if args.gemm_only_steps:
            for i in range(args.gemm_only_steps):
                q.qlin_graph_launch(gemm_graphs[i % n_sets], stream)
            torch.cuda.synchronize()
            print(json.dumps({"gemm_only_steps": args.gemm_only_steps, "launches": n_gemm * args.gemm_only_steps}))
            return

        for i in range(args.warmup):
            q.qlin_graph_launch(step_graphs[i % n_sets], stream)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            q.qlin_graph_launch(step_graphs[i % n_sets], stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms_step = e0.elapsed_time(e1) / args.steps

        # GEMM launches alone (same launches, same order), for the roofline
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        for i in range(2):
            q.qlin_graph_launch(gemm_graphs[i % n_sets], stream)
        g0.record(stream)
        for i in range(args.steps):
            q.qlin_graph_launch(gemm_graphs[i % n_sets], stream)
        g1.record(stream)
        torch.cuda.synchronize()
        ms_gemms = g0.elapsed_time(g1) / args.steps

        detail = []
        if args.detail:
            # per (M, layer): a graph of that GEMM over every weight copy
            for j in range(n_gemm):
                ls = [s_[j] for s_ in sets]
                reps = max(1, -(-64 // len(ls)))
                g = capture(stream, lambda ls=ls: [l.gemm(stream) for _ in range(reps) for l in ls])
                q.qlin_graph_launch(g, stream)
                d0 = torch.cuda.Event(enable_timing=True)
                d1 = torch.cuda.Event(enable_timing=True)
                d0.record(stream)
                for _ in range(5):
                    q.qlin_graph_launch(g, stream)
                d1.record(stream)
                torch.cuda.synchronize()
                us = d0.elapsed_time(d1) * 1e3 / (5 * reps * len(ls))
                q.qlin_graph_destroy(g)
                l0 = ls[0]
                detail.append({"layer": l0.name, "M": l0.M, "N": l0.N, "K": l0.K, "us": round(us, 3),
                               "GBps": round(l0.bytes / us / 1e3, 1),
                               "TFLOPs": round(l0.flops / us / 1e6, 3),
                               "frac_hbm": round(l0.bytes / us / 1e3 / HBM_PEAK_GBS, 4),
                               "cfg": l0.cfg.as_dict()})

    for g in step_graphs + gemm_graphs:
        q.qlin_graph_destroy(g)

    value = step_bytes / (ms_step * 1e-3) / 1e9
    achieved = gemm_bytes / (ms_gemms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE[fmt],
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "format": wl.FORMAT_NAMES[fmt],
            "layers": {L.name: [L.N, L.K] for L in layers},
            "token_counts": list(Ms),
            "linears_per_step": n_gemm,
            "weight_copies": n_sets,
            "graph_replay": True,
        },
        "tflops": round(step_flops / (ms_step * 1e-3) / 1e12, 3),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "kernel": "gemm_kernel (all launches of a step)",
            "avg_launch_us": round(ms_gemms * 1e3 / n_gemm, 3),
            "bytes_per_launch": round(gemm_bytes / n_gemm),
        },
    }
    tr = measured_traffic(args.workload)
    if tr is not None:
        out["roofline"]["traffic"] = tr["per_launch_traffic_bytes"]
        out["roofline"]["traffic_unit"] = "B per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
        out["roofline"]["traffic_vs_algorithmic"] = round(
            tr["per_launch_traffic_bytes"] / tr["per_launch_algorithmic_bytes"], 3)
    if detail:
        with open(args.detail, "w") as f:
            json.dump(detail, f, indent=1)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(fmt, layers, Ms, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
