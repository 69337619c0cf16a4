"""Benchmark of the quantized skinny linear path on one MI355X.

A step is one pass of the hot path over one batch of synthetic inputs: for
every token count M of the workload and every linear layer of the model, the
whole quantized linear (qlin_linear: activation quantization and GEMM, as one
fused kernel or two, per the selection table), replayed from a hipGraph
captured once (the decode path runs only under graph replay).  Weights are
quantized and packed offline (qlin_quantize_weight, qlin_pack_weight) and
live in HBM as R distinct rotating copies (>= 1 GiB in total) so the 256 MiB
Infinity Cache cannot serve them; activations, scales and outputs are
resident too.

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
# the headline: the largest of the three model workloads (BlockFP8 on the
# hidden-5120 layer shapes); the other two are timed beside it (--also)
DEFAULT_WORKLOAD = "block_fp8_hidden5120"
DEFAULT_ALSO = "fp8_dynamic_hidden2048,w8a8_int8_hidden4096"
DTYPE = {0: "fp8_e4m3", 1: "int8", 2: "fp8_e4m3"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--also", default=DEFAULT_ALSO,
                    help="other workloads whose step and GEMM launches are timed the same way and "
                         "reported under other_workloads ('' for none)")
    ap.add_argument("--quant", default=None,
                    help="instead of the step: time every launch shape of the activation quantize kernels "
                         "on the three model workloads' (M, K) and write it (JSON) here")
    ap.add_argument("--floors", default=None,
                    help="instead of the step: time the graph-replayed streaming read of every layer "
                         "size of the three model workloads and write it (JSON) here")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", default=None,
                    help="instead of the step: time the crossover sweep (8B-class shapes, forced "
                         "schedules and the table's pick) and write it (JSON) here")
    ap.add_argument("--moe", default=None,
                    help="write the grouped (mixture-of-experts) measurements to this JSON file and exit")
    ap.add_argument("--moe-tokens", default=None, help="token counts of --moe (default: 1..32)")
    ap.add_argument("--moe-layers", default=None, help="layers of --moe (default: all)")
    ap.add_argument("--moe-schedules", default=None,
                    help="schedules of --moe (rule, forced ones, per_expert_launches; default: all)")
    ap.add_argument("--vendor-sweep", default=None,
                    help="instead of the step: time hipBLASLt's fp8 GEMM (torch._scaled_mm, reference only) "
                         "on the crossover sweep's shapes and token counts and write it (JSON) here")
    ap.add_argument("--vendor-shapes", default="8b",
                    help="shapes of --vendor-sweep: 8b (the crossover sweep's) or a workload name")
    ap.add_argument("--sweep-formats", default="fp8_dynamic,w8a8_int8,block_fp8")
    ap.add_argument("--sweep-m", default="1,2,4,8,16,24,32,64,128,256,512")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip the streaming-read ceiling measurement (1 GiB buffer)")
    ap.add_argument("--detail", default=None,
                    help="write per-shape timings of the whole linear and of its GEMM kernel (JSON) here")
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
        # the weights are in the packed layout (offline preparation)
        self.call_fmt = fmt | q.QLIN_PACKED_WEIGHTS
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

    def layer(self, stream, wq=None):
        """The whole decode linear: quantize + GEMM (one or two kernels, as tuned)."""
        import skinny_bit_gemm_amd as q
        q.qlin_linear(self.call_fmt, self.M, self.N, self.K, self.x, self.K, self.xq, self.xs,
                      self.wq if wq is None else wq, self.ws, self.y, q.QLIN_OUT_BF16, self.cfg, self.work,
                      stream=stream)

    def gemm(self, stream, wq=None):
        import skinny_bit_gemm_amd as q
        q.qlin_gemm(self.call_fmt, self.M, self.N, self.K, self.xq, self.xs, self.wq if wq is None else wq,
                    self.ws, self.y, q.QLIN_OUT_BF16, self.cfg, self.work, stream=stream)

    @property
    def fused(self):
        import skinny_bit_gemm_amd as q
        return self.cfg.act_path == q.QLIN_ACT_FUSED

    def kernel(self, stream, wq=None):
        """The step's GEMM kernel of this linear, as the step runs it: the
        fused quantize + GEMM kernel where the table fuses them, else the
        GEMM kernel alone (its codes come from the step's quantize kernel)."""
        if self.fused:
            self.layer(stream, wq)
        else:
            self.gemm(stream, wq)

    @property
    def kernel_bytes(self):
        return self.bytes + (self.qbytes if self.fused else 0)


# the device code of the path (GEMM and quantization kernels)
KERNEL_SOURCES = ["skinny_bit_gemm_amd/csrc/" + f for f in (
    "qlin_device.h", "qlin_gemm.h", "qlin_gemm_fp8.hip", "qlin_gemm_i8.hip", "qlin_gemm_block.hip",
    "qlin_kernels.hip")]
TABLE = "skinny_bit_gemm_amd/tables/gfx950.tbl"


def source_digests():
    """sha256 of the kernel sources (concatenated in a fixed order) and of
    the selection table's entries that the step runs (its header and the
    entries of the token-count buckets up to 32; entries of the larger
    buckets, which only the crossover sweep uses, do not enter it)."""
    import hashlib
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    t = hashlib.sha256()
    for line in open(os.path.join(ROOT, TABLE), "rb"):
        f = line.split(b"#")[0].split()
        if len(f) == 12 and int(f[3]) > 32:
            continue
        t.update(line)
    return h.hexdigest(), t.hexdigest()


def measured_traffic(workload):
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary,
    or None when there is none or the kernels or the table changed since."""
    path = os.path.join(ROOT, "profiles", f"gemm_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    ksha, tsha = source_digests()
    if rec.get("kernel_source_sha256") != ksha or rec.get("table_sha256") != tsha:
        return None
    return rec


def calibrate_copy(nbytes):
    """Three plain device copies of nbytes (reference dispatches for
    scaling the HBM byte counters)."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


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
    while len(times) < 3 or (spent < budget_s and len(times) < 1000):
        t = one_pass()
        times.append(t)
        spent += t
        if spent > 4 * budget_s:
            break
    best = min(times)
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        pass
    return {
        "value": round(pass_bytes / best / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"the whole workload ({len(layers) * len(Ms)} linears: quantize + product + "
                  f"epilogue each), best of {len(times)} timed passes after one warm-up, "
                  f"{spent:.1f} s of CPU time in total",
        "ms_per_pass": round(best * 1e3, 2),
        "cpu_model": model,
    }


MFMA_PEAK_TFLOPS = 5000.0   # dense fp8 / int8 matrix-core peak of MI355X


def sweep_configs(q, fmt, M):
    """The forced schedules of the crossover sweep (Standard, Swap-AB,
    Split-K 2..16, the skinny kernel's 64-token tiles past 32 tokens, the
    large-M kernel) and the selection table's pick (None)."""
    tm = 16 if M <= 16 else 32
    out = {"standard": q.make_config(0, 1, tm, 64, 4, 2), "swap_ab": q.make_config(1, 1, tm, 64, 4, 2)}
    for sk in (2, 4, 8, 16):
        out[f"splitk{sk}"] = q.make_config(sk % 4 == 0, sk, tm, 64, 4, 2)
    # the skinny kernel's 64-token tiles (one weight read per 64 tokens)
    if M > 32:
        out["skinny64_swap"] = q.make_config(1, 1, 64, 112, 7, 1)
    # the large-M kernel (64- / 128-token tiles), with and without split-K
    for tmb in (64, 128):
        for sk in (1, 2, 4):
            out[f"large_m{tmb}" + (f"_split{sk}" if sk > 1 else "")] = q.make_config(0, sk, tmb, 128, 4, 1)
    out["table"] = None
    return out


def crossover_sweep(path, fmts, Ms):
    """GEMM time of every sweep schedule on the 8B-class shapes, each timed
    as a hipGraph of launches over >= 1 GiB of rotating weight copies."""
    import torch
    import skinny_bit_gemm_amd as q
    from skinny_bit_gemm_amd.tune import warm_graph
    import workloads as wl
    dev = torch.device("cuda:0")
    q.lib()
    st = torch.cuda.Stream()
    rows = []
    with torch.cuda.stream(st):
        for fmt in fmts:
            for L in wl.DENSE_8B:
                N, K = L.N, L.K
                wq, ws = prepare_weights(fmt, L, dev)
                R = max(2, -(-(1 << 30) // (N * K)))
                copies = [wq.clone() for _ in range(R)]
                for M in Ms:
                    x = torch.from_numpy(wl.activations(fmt, N, K, M).view("int16")).to(dev)
                    xq = torch.empty((M, K), dtype=torch.uint8, device=dev)
                    xs = torch.empty(q.scales_shape(fmt, M, K, False), dtype=torch.float32, device=dev)
                    q.qlin_quantize_act(fmt, M, K, x, K, xq, xs, stream=st)
                    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
                    for name, c in sweep_configs(q, fmt, M).items():
                        cfg = c if c is not None else q.qlin_select_variant(fmt, M, N, K)
                        work = torch.zeros(max(256, q.qlin_workspace_bytes(fmt, M, N, K, cfg)),
                                           dtype=torch.uint8, device=dev)
                        run = lambda: [q.qlin_gemm(fmt | q.QLIN_PACKED_WEIGHTS, M, N, K, xq, xs, wc, ws, y,
                                                   q.QLIN_OUT_BF16, cfg, work, stream=st) for wc in copies]
                        run()
                        g = capture(st, run)
                        warm_graph(g, st)
                        e0 = torch.cuda.Event(enable_timing=True)
                        e1 = torch.cuda.Event(enable_timing=True)
                        e0.record(st)
                        for _ in range(3):
                            q.qlin_graph_launch(g, st)
                        e1.record(st)
                        torch.cuda.synchronize()
                        q.qlin_graph_destroy(g)
                        us = e0.elapsed_time(e1) * 1e3 / (3 * R)
                        nbytes = wl.algorithmic_bytes(fmt, M, N, K)
                        tf = wl.flops(M, N, K) / us / 1e6
                        rows.append({"format": wl.FORMAT_NAMES[fmt], "layer": L.name, "N": N, "K": K, "M": M,
                                     "schedule": name, "cfg": cfg.as_dict(), "us": round(us, 3),
                                     "TFLOPs": round(tf, 2), "GBps": round(nbytes / us / 1e3, 1),
                                     "frac_mfma": round(tf / MFMA_PEAK_TFLOPS, 4),
                                     "frac_hbm": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)})
                        del work
                    print(f"[sweep] {wl.FORMAT_NAMES[fmt]} {L.name} M={M}: " + ", ".join(
                        f"{r['schedule']} {r['us']:.1f}us" for r in rows if r["M"] == M and r["N"] == N
                        and r["K"] == K and r["format"] == wl.FORMAT_NAMES[fmt]), file=sys.stderr, flush=True)
                del copies, wq, ws
                torch.cuda.empty_cache()
    with open(path, "w") as f:
        json.dump(rows, f, indent=1)
    best = {}
    for r in rows:
        k = (r["format"], r["layer"], r["M"])
        if k not in best or r["us"] < best[k]["us"]:
            best[k] = r
    return {"mode": "crossover_sweep", "points": len(rows), "file": path,
            "best_frac_mfma_at_512": {f: max((b["frac_mfma"] for k, b in best.items() if k[0] == f and k[2] == 512),
                                             default=None) for f in sorted({k[0] for k in best})}}


def vendor_sweep(path, Ms, shapes="8b"):
    """Reference only (no part of the path): hipBLASLt's fp8 GEMM with a
    scale per token and per channel (torch._scaled_mm, bf16 output) on the
    8B-class shapes, timed like the crossover sweep (a graph of launches
    over >= 1 GiB of rotating weight copies).  The same product as the
    FP8Dynamic GEMM, so it places the large-M kernel against the vendor
    library on the points where the pages hand the work to one."""
    import torch
    import workloads as wl
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    rows = []
    # the 8B-class shapes of the crossover sweep, or a workload's layers
    layers = wl.DENSE_8B if shapes == "8b" else wl.WORKLOADS[shapes][1]
    for L in layers:
        N, K = L.N, L.K
        R = max(2, -(-(1 << 30) // (N * K)))
        copies = [(torch.randn(N, K, device=dev, generator=gen) * 0.02).to(torch.float8_e4m3fn) for _ in range(R)]
        sb = torch.rand(1, N, device=dev, generator=gen) * 1e-2 + 1e-3
        for M in Ms:
            a = torch.randn(M, K, device=dev, generator=gen).to(torch.float8_e4m3fn)
            sa = torch.rand(M, 1, device=dev, generator=gen) * 1e-2 + 1e-3
            y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
            st = torch.cuda.Stream()
            st.wait_stream(torch.cuda.current_stream())

            def run():
                for w in copies:
                    torch._scaled_mm(a, w.t(), scale_a=sa, scale_b=sb, out_dtype=torch.bfloat16, out=y)
            with torch.cuda.stream(st):
                run()   # the library picks its kernels before the capture
            torch.cuda.current_stream().wait_stream(st)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run()
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < 0.02:   # ~20 ms untimed, as the other timings
                g.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(3):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            del g
            us = e0.elapsed_time(e1) * 1e3 / (3 * R)
            tf = wl.flops(M, N, K) / us / 1e6
            nbytes = wl.algorithmic_bytes(wl.FP8_DYNAMIC, M, N, K)
            rows.append({"library": "hipBLASLt (torch._scaled_mm, row-wise scales)", "layer": L.name, "N": N,
                         "K": K, "M": M, "us": round(us, 3), "TFLOPs": round(tf, 2),
                         "frac_mfma": round(tf / MFMA_PEAK_TFLOPS, 4),
                         "frac_hbm": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)})
            print(f"[vendor] {L.name} M={M}: {us:.2f} us, {tf:.0f} TFLOP/s", file=sys.stderr, flush=True)
        del copies
        torch.cuda.empty_cache()
    with open(path, "w") as f:
        json.dump(rows, f, indent=1)
    return {"mode": "vendor_sweep", "points": len(rows), "file": path}


def moe_configs(q, fmt, T):
    """Forced grouped schedules timed beside the built-in rule (None)."""
    tm = 16 if T <= 16 else 32
    red = 1 if fmt != 2 else 0   # packed atomics for the exact formats
    return {"rule": None,
            "swap_n32_kw4": q.make_config(1, 1, tm, 32, 4, 4),
            "standard": q.make_config(0, 1, tm, 64, 4, 2),
            "split2": q.make_config(1, 2, tm, 64, 4, 2, red),
            "split4": q.make_config(1, 4, tm, 64, 4, 2, red)}


def moe_bench(path, fmts, Ts, layers=None, schedules=None):
    """Grouped GEMM over the 128-expert top-8 layers: one launch for all
    experts, timed as a hipGraph of launches that each take another routing
    and another copy of the expert weights (>= 2 GiB of copies in total, so
    the 256 MiB Infinity Cache holds at most a small share of the experts a
    launch reads).  Beside it, the same work as one dense launch per active
    expert (the table's pick for that expert's row count)."""
    import numpy as np
    import torch
    import skinny_bit_gemm_amd as q
    from skinny_bit_gemm_amd.tune import warm_graph
    import workloads as wl
    dev = torch.device("cuda:0")
    q.lib()
    st = torch.cuda.Stream()
    E, topk = wl.MOE_EXPERTS, wl.MOE_TOPK
    rows_out = []

    def timed(fn, n):
        fn()
        g = capture(st, fn)
        warm_graph(g, st)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(3):
            q.qlin_graph_launch(g, st)
        e1.record(st)
        torch.cuda.synchronize()
        q.qlin_graph_destroy(g)
        return e0.elapsed_time(e1) * 1e3 / (3 * n)

    with torch.cuda.stream(st):
        for fmt in fmts:
            for L in wl.MOE_LAYERS:
                if layers and L.name not in layers:
                    continue
                N, K = L.N, L.K
                wq = torch.empty((E, N, K), dtype=torch.uint8, device=dev)
                ws = torch.empty((E,) + tuple(q.scales_shape(fmt, N, K, True)), dtype=torch.float32, device=dev)
                gen = torch.Generator(device=dev)
                gen.manual_seed(7000 + fmt)
                for e in range(E):   # N(0, 0.02) master weights, drawn on the device
                    w = torch.randn((N, K), generator=gen, device=dev) * 0.02
                    q.qlin_quantize_weight(fmt, N, K, w, wq[e], ws[e], stream=st)
                del w
                # the experts' codes in the packed layout, one matrix after another
                wpk = torch.empty((E, q.qlin_packed_weight_bytes(N, K)), dtype=torch.uint8, device=dev)
                q.qlin_pack_weight(E, N, K, wq, wpk, stream=st)
                torch.cuda.synchronize()
                wq = wpk
                fmt_w = fmt | q.QLIN_PACKED_WEIGHTS
                C = max(2, -(-(2 << 30) // (E * N * K)))
                copies = [wq] + [wq.clone() for _ in range(C - 1)]
                for T in Ts:
                    total = T * topk
                    R = 2 * C   # launches per graph: routing i on copy i % C
                    routes = [wl.moe_routing(T, E, topk, 100 + i) for i in range(R)]
                    offs = [torch.from_numpy(o).to(dev) for o, _ in routes]
                    x = torch.from_numpy(wl.random_bf16((total, K), 11).view(np.int16)).to(dev)
                    xq = torch.empty((total, K), dtype=torch.uint8, device=dev)
                    xs = torch.empty(q.scales_shape(fmt, total, K, False), dtype=torch.float32, device=dev)
                    q.qlin_quantize_act(fmt, total, K, x, K, xq, xs, stream=st)
                    y = torch.empty((total, N), dtype=torch.bfloat16, device=dev)
                    nbytes = sum(wl.grouped_algorithmic_bytes(fmt, o, N, K) for o, _ in routes) / R
                    active = sum(int(np.count_nonzero(np.diff(o))) for o, _ in routes) / R
                    point = {"format": wl.FORMAT_NAMES[fmt], "layer": L.name, "N": N, "K": K, "T": T,
                             "rows": total, "active_experts": active, "bytes_per_launch": round(nbytes)}
                    for name, c in moe_configs(q, fmt, T).items():
                        if schedules and name not in schedules:
                            continue
                        cfg = c if c is not None else q.qlin_grouped_select_variant(fmt, E, N, K, T)
                        nb = q.qlin_grouped_workspace_bytes(fmt, E, N, K, total, T, cfg)
                        work = torch.zeros(max(256, nb), dtype=torch.uint8, device=dev)
                        us = timed(lambda: [q.qlin_grouped_gemm(fmt_w, E, N, K, offs[i], total, T, xq, xs,
                                                                copies[i % C], ws, y, q.QLIN_OUT_BF16, cfg, work,
                                                                stream=st) for i in range(R)], R)
                        rows_out.append(dict(point, schedule=name, cfg=cfg.as_dict(), us=round(us, 3),
                                             GBps=round(nbytes / us / 1e3, 1),
                                             frac_hbm=round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)))
                        del work
                    pts = lambda: [r for r in rows_out if r["format"] == point["format"] and r["layer"] == L.name
                                   and r["T"] == T]
                    if schedules and "per_expert_launches" not in schedules:
                        print(f"[moe] {point['format']} {L.name} T={T} active={active:.1f}: " + ", ".join(
                            f"{r['schedule']} {r['us']:.1f}us" for r in pts()), file=sys.stderr, flush=True)
                        continue
                    # one dense launch per active expert, on the same routings and copies
                    launches = []
                    for i, (o, _) in enumerate(routes):
                        for e in range(E):
                            lo, hi = int(o[e]), int(o[e + 1])
                            if hi > lo:
                                cfg = q.qlin_select_variant(fmt, hi - lo, N, K)
                                nb = q.qlin_workspace_bytes(fmt, hi - lo, N, K, cfg)
                                launches.append((i, lo, hi, e, cfg, nb))
                    work = torch.zeros(max(256, max(l[5] for l in launches)), dtype=torch.uint8, device=dev)

                    def per_expert():
                        for i, lo, hi, e, cfg, _ in launches:
                            q.qlin_gemm(fmt_w, hi - lo, N, K, xq[lo:hi], xs[lo:hi],
                                        copies[i % C][e], ws[e], y[lo:hi], q.QLIN_OUT_BF16, cfg, work, stream=st)
                    us = timed(per_expert, R)
                    rows_out.append(dict(point, schedule="per_expert_launches", cfg=None, us=round(us, 3),
                                         GBps=round(nbytes / us / 1e3, 1),
                                         frac_hbm=round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)))
                    del work
                    print(f"[moe] {point['format']} {L.name} T={T} active={active:.1f}: " + ", ".join(
                        f"{r['schedule']} {r['us']:.1f}us" for r in pts()), file=sys.stderr, flush=True)
                del copies, wq, ws
                torch.cuda.empty_cache()
    with open(path, "w") as f:
        json.dump(rows_out, f, indent=1)
    import math

    def geomean(name):
        v = [r["GBps"] for r in rows_out if r["schedule"] == name]
        return round(math.exp(sum(map(math.log, v)) / len(v)), 1) if v else None
    return {"mode": "moe", "points": len({(r["format"], r["layer"], r["T"]) for r in rows_out}), "file": path,
            "geomean_rule_GBps": geomean("rule"), "geomean_per_expert_GBps": geomean("per_expert_launches")}


def prepare_weights(fmt, L, dev):
    """Offline weight preparation of one layer: quantize the N(0, 0.02)
    master weights on the GPU, then reorder the codes into the packed layout
    the kernels stream fastest.  Returns (packed codes, scales)."""
    import torch
    import skinny_bit_gemm_amd as q
    import workloads as wl
    w = torch.from_numpy(wl.weights(fmt, L.N, L.K)).to(dev)
    wq = torch.empty((L.N, L.K), dtype=torch.uint8, device=dev)
    ws = torch.empty(q.scales_shape(fmt, L.N, L.K, True), dtype=torch.float32, device=dev)
    q.qlin_quantize_weight(fmt, L.N, L.K, w, wq, ws)
    del w
    wp = torch.empty(q.qlin_packed_weight_bytes(L.N, L.K), dtype=torch.uint8, device=dev)
    q.qlin_pack_weight(1, L.N, L.K, wq, wp)
    torch.cuda.synchronize()
    return wp, ws


def run_workload(name, steps, warmup, detail=False, gemm_only_steps=None, floors=None):
    """Times one workload's step: every (M, layer) linear of it, replayed
    from hipGraphs over rotating weight copies; then the step's GEMM kernels
    alone (the roofline entry).  With `detail`, also every linear alone
    (`floors`: graph-replayed streaming-read times per weight size, for the
    kernel / floor column).  Returns the numbers as a dict."""
    import torch

    import skinny_bit_gemm_amd as q
    from skinny_bit_gemm_amd.tune import warm_graph
    import workloads as wl

    fmt, layers, Ms = wl.WORKLOADS[name]
    dev = torch.device("cuda:0")
    # quantized and packed weights (GPU quantizer and packer, offline and
    # untimed), then rotating copies
    base = {}
    for L in layers:
        base[L.name] = prepare_weights(fmt, L, dev)
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
            lin.kernel(stream)
        for ls in sets[1:]:
            for lin in ls:
                lin.layer(stream)
        torch.cuda.synchronize()
        step_graphs = [capture(stream, lambda ls=ls: [l.layer(stream) for l in ls]) for ls in sets]
        gemm_graphs = [capture(stream, lambda ls=ls: [l.kernel(stream) for l in ls]) for ls in sets]
        torch.cuda.synchronize()

        step_bytes = sum(l.bytes + l.qbytes for l in sets[0])
        gemm_bytes = sum(l.kernel_bytes for l in sets[0])
        step_flops = sum(l.flops for l in sets[0])
        n_gemm = len(sets[0])

        if gemm_only_steps:
            for i in range(gemm_only_steps):
                q.qlin_graph_launch(gemm_graphs[i % n_sets], stream)
            torch.cuda.synchronize()
            for g in step_graphs + gemm_graphs:
                q.qlin_graph_destroy(g)
            return {"gemm_only_steps": gemm_only_steps, "launches": n_gemm * gemm_only_steps}

        # set-up (weight preparation, the eager pass, capture) leaves the GPU
        # idle; replaying the step for ~20 ms, untimed, before the warm-up
        # steps brings it back to its steady rate whatever --warmup is
        for g in step_graphs:
            warm_graph(g, stream, min_ms=20.0 / n_sets)
        for i in range(warmup):
            q.qlin_graph_launch(step_graphs[i % n_sets], stream)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            q.qlin_graph_launch(step_graphs[i % n_sets], stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms_step = e0.elapsed_time(e1) / steps

        # the step's GEMM kernels alone (same launches, same order; the fused
        # ones include their quantization), for the roofline
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        for i in range(2):
            q.qlin_graph_launch(gemm_graphs[i % n_sets], stream)
        g0.record(stream)
        for i in range(steps):
            q.qlin_graph_launch(gemm_graphs[i % n_sets], stream)
        g1.record(stream)
        torch.cuda.synchronize()
        ms_gemms = g0.elapsed_time(g1) / steps

        rows = []
        if detail:
            # per (M, layer): graphs of the whole linear and of its GEMM
            # kernel over >= 1 GiB of copies of that layer's weights (fewer
            # would leave a small layer's copies in the L2 and Infinity Cache)
            def per_launch_us(ls, fn):
                reps = max(1, -(-64 // len(ls)))
                g = capture(stream, lambda: [fn(l) for _ in range(reps) for l in ls])
                warm_graph(g, stream)
                d0 = torch.cuda.Event(enable_timing=True)
                d1 = torch.cuda.Event(enable_timing=True)
                d0.record(stream)
                for _ in range(5):
                    q.qlin_graph_launch(g, stream)
                d1.record(stream)
                torch.cuda.synchronize()
                q.qlin_graph_destroy(g)
                return d0.elapsed_time(d1) * 1e3 / (5 * reps * len(ls))

            for j in range(n_gemm):
                l0 = sets[0][j]
                n_copies = max(2, -(-(1 << 30) // (l0.N * l0.K)))
                copies = [s_[j].wq for s_ in sets][:n_copies]
                copies += [l0.wq.clone() for _ in range(n_copies - len(copies))]
                layer_us = per_launch_us(copies, lambda w: l0.layer(stream, w))
                kernel_us = per_launch_us(copies, lambda w: l0.kernel(stream, w))
                del copies
                rows.append({"layer": l0.name, "M": l0.M, "N": l0.N, "K": l0.K, "fused": l0.fused,
                             "act_path": ("staged", "fused", "direct")[l0.cfg.act_path],
                             "layer_us": round(layer_us, 3),
                             "layer_GBps": round((l0.bytes + l0.qbytes) / layer_us / 1e3, 1),
                             "layer_TFLOPs": round(l0.flops / layer_us / 1e6, 3),
                             "kernel_us": round(kernel_us, 3),
                             "kernel_GBps": round(l0.kernel_bytes / kernel_us / 1e3, 1),
                             "kernel_frac_hbm": round(l0.kernel_bytes / kernel_us / 1e3 / HBM_PEAK_GBS, 4),
                             "cfg": l0.cfg.as_dict()})

    for g in step_graphs + gemm_graphs:
        q.qlin_graph_destroy(g)
    if floors:
        for d in rows:
            f = floors.get(d["N"] * d["K"])
            if f:
                d["floor_us"] = f
                d["kernel_over_floor"] = round(d["kernel_us"] / f, 3)
    res = {"workload": name, "fmt": fmt, "layers": layers, "Ms": Ms, "n_gemm": n_gemm, "n_sets": n_sets,
           "ms_step": ms_step, "ms_gemms": ms_gemms, "step_bytes": step_bytes, "gemm_bytes": gemm_bytes,
           "step_flops": step_flops, "detail": rows}
    del sets, base
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def floors_bench(path):
    """Graph-replayed streaming-read time of a buffer of each layer's weight
    size (cold copies, >= 1 GiB in all): the floor a kernel that reads the
    layer's weights once would meet under the layer timings' conditions."""
    from skinny_bit_gemm_amd import probe
    import workloads as wl
    rows = []
    seen = set()
    for name in ("fp8_dynamic_hidden2048", "w8a8_int8_hidden4096", "block_fp8_hidden5120"):
        _, layers, _ = wl.WORKLOADS[name]
        for L in layers:
            nb = L.N * L.K
            if nb in seen:
                continue
            seen.add(nb)
            us, blocks = probe.graph_floor_us(nb, with_grid=True)
            rows.append({"workload": name, "layer": L.name, "N": L.N, "K": L.K, "bytes": nb,
                         "floor_us": round(us, 3), "GBps": round(nb / us / 1e3, 1), "best_grid": blocks})
            print(f"[floors] {name} {L.name} {nb} B: {us:.3f} us", file=sys.stderr, flush=True)
    ceiling = probe.read_ceiling_gbs()
    with open(path, "w") as f:
        json.dump({"read_ceiling_GBps": round(ceiling, 1), "floors": rows}, f, indent=1)
    return {"mode": "floors", "sizes": len(rows), "file": path, "read_ceiling_GBps": round(ceiling, 1)}


QUANT_THREADS = {0: (64, 128, 256, 512), 1: (64, 128, 256, 512), 2: (64, 256)}


def quant_bench(path):
    """The activation quantize kernels alone: every launch shape
    (qlin_quantize_act_cfg) at every (token count, K) of the three model
    workloads, each timed as a hipGraph of 64 launches (what a decode step
    pays per unfused layer, launch included)."""
    import torch
    import skinny_bit_gemm_amd as q
    from skinny_bit_gemm_amd.tune import warm_graph
    import workloads as wl
    dev = torch.device("cuda:0")
    st = torch.cuda.Stream()
    rows = []
    with torch.cuda.stream(st):
        for name in ("fp8_dynamic_hidden2048", "w8a8_int8_hidden4096", "block_fp8_hidden5120"):
            fmt, layers, Ms = wl.WORKLOADS[name]
            for K in sorted({L.K for L in layers}):
                for M in Ms:
                    x = torch.from_numpy(wl.activations(fmt, 128, K, M).view("int16")).to(dev)
                    xq = torch.empty((M, K), dtype=torch.uint8, device=dev)
                    xs = torch.empty(q.scales_shape(fmt, M, K, False), dtype=torch.float32, device=dev)
                    point = {"format": wl.FORMAT_NAMES[fmt], "M": M, "K": K, "us": {}}
                    for t in QUANT_THREADS[fmt] + (0,):
                        run = lambda: [q.qlin_quantize_act_cfg(fmt, M, K, x, K, xq, xs, t, stream=st)
                                       for _ in range(64)]
                        run()
                        g = capture(st, run)
                        warm_graph(g, st)
                        e0 = torch.cuda.Event(enable_timing=True)
                        e1 = torch.cuda.Event(enable_timing=True)
                        e0.record(st)
                        for _ in range(5):
                            q.qlin_graph_launch(g, st)
                        e1.record(st)
                        torch.cuda.synchronize()
                        q.qlin_graph_destroy(g)
                        point["us"][str(t) if t else "rule"] = round(e0.elapsed_time(e1) * 1e3 / (5 * 64), 3)
                    rows.append(point)
                    print(f"[quant] {point}", file=sys.stderr, flush=True)
    with open(path, "w") as f:
        json.dump(rows, f, indent=1)
    return {"mode": "quant", "points": len(rows), "file": path}


def workload_summary(r):
    """Step and GEMM-launch numbers of one timed workload."""
    value = r["step_bytes"] / (r["ms_step"] * 1e-3) / 1e9
    achieved = r["gemm_bytes"] / (r["ms_gemms"] * 1e-3) / 1e9
    return {"step_GBps": round(value, 2), "ms_per_step": round(r["ms_step"], 5),
            "step_TFLOPs": round(r["step_flops"] / (r["ms_step"] * 1e-3) / 1e12, 3),
            "gemm_achieved_GBps": round(achieved, 1), "gemm_frac": round(achieved / HBM_PEAK_GBS, 4),
            "gemm_avg_launch_us": round(r["ms_gemms"] * 1e3 / r["n_gemm"], 3),
            "linears_per_step": r["n_gemm"]}


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
    also = [w for w in args.also.split(",") if w and w != args.workload] if args.also else []
    for w in also:
        if w not in wl.WORKLOADS:
            sys.exit(f"unknown workload {w} in --also; choose from {sorted(wl.WORKLOADS)}")
    if args.moe:
        fmts = [wl.FORMAT_IDS[f] for f in args.sweep_formats.split(",")]
        Ts = [int(t) for t in args.moe_tokens.split(",")] if args.moe_tokens else list(wl.MOE_TOKENS)
        if args.calibrate_copy:
            calibrate_copy(args.calibrate_copy)
        print(json.dumps(moe_bench(args.moe, fmts, Ts, args.moe_layers and args.moe_layers.split(","),
                                   args.moe_schedules and args.moe_schedules.split(","))), flush=True)
        return
    if args.vendor_sweep:
        print(json.dumps(vendor_sweep(args.vendor_sweep, [int(m) for m in args.sweep_m.split(",")],
                                      args.vendor_shapes)), flush=True)
        return
    if args.sweep:
        fmts = [wl.FORMAT_IDS[f] for f in args.sweep_formats.split(",")]
        print(json.dumps(crossover_sweep(args.sweep, fmts, [int(m) for m in args.sweep_m.split(",")])),
              flush=True)
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q.lib()
    if args.floors:
        print(json.dumps(floors_bench(args.floors)), flush=True)
        return
    if args.quant:
        print(json.dumps(quant_bench(args.quant)), flush=True)
        return
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
    if args.gemm_only_steps:
        print(json.dumps(run_workload(args.workload, args.steps, args.warmup,
                                      gemm_only_steps=args.gemm_only_steps)), flush=True)
        return

    floors = None
    if args.detail:
        from skinny_bit_gemm_amd import probe
        _, layers, _ = wl.WORKLOADS[args.workload]
        floors = {L.N * L.K: round(probe.graph_floor_us(L.N * L.K), 3) for L in layers}
    r = run_workload(args.workload, args.steps, args.warmup, detail=bool(args.detail), floors=floors)
    print(f"[bench] {args.workload}: {json.dumps(workload_summary(r))}", file=sys.stderr, flush=True)
    fmt, layers, Ms, n_gemm = r["fmt"], r["layers"], r["Ms"], r["n_gemm"]
    detail = r["detail"]
    value = r["step_bytes"] / (r["ms_step"] * 1e-3) / 1e9
    achieved = r["gemm_bytes"] / (r["ms_gemms"] * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_step"], 5),
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
            "weight_copies": r["n_sets"],
            "graph_replay": True,
        },
        "tflops": round(r["step_flops"] / (r["ms_step"] * 1e-3) / 1e12, 3),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "kernel": "gemm_kernel (every launch of a step; the fused ones include their quantization)",
            "avg_launch_us": round(r["ms_gemms"] * 1e3 / n_gemm, 3),
            "bytes_per_launch": round(r["gemm_bytes"] / n_gemm),
        },
    }
    if not args.no_read_ceiling:
        from skinny_bit_gemm_amd import probe
        ceiling = probe.read_ceiling_gbs()
        out["roofline"]["read_ceiling_GBps"] = round(ceiling, 1)
        out["roofline"]["frac_of_read_ceiling"] = round(achieved / ceiling, 4)
    tr = measured_traffic(args.workload)
    if tr is not None:
        out["roofline"]["traffic"] = tr["per_launch_traffic_bytes"]
        out["roofline"]["traffic_unit"] = "B per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
        out["roofline"]["traffic_vs_algorithmic"] = round(
            tr["per_launch_traffic_bytes"] / tr["per_launch_algorithmic_bytes"], 3)
    if detail:
        import math
        ceiling = out["roofline"].get("read_ceiling_GBps")
        for d in detail:
            if ceiling:
                d["kernel_frac_read_ceiling"] = round(d["kernel_GBps"] / ceiling, 4)
        summary = {
            "workload": args.workload,
            "geomean_layer_GBps": round(math.exp(sum(math.log(d["layer_GBps"]) for d in detail) / len(detail)), 1),
            "geomean_kernel_GBps": round(math.exp(sum(math.log(d["kernel_GBps"]) for d in detail) / len(detail)), 1),
            "read_ceiling_GBps": ceiling,
        }
        with open(args.detail, "w") as f:
            json.dump({"summary": summary, "shapes": detail}, f, indent=1)
    if also:
        # the other workloads, step and GEMM launches timed the same way
        # (each with its own traffic record when it matches the sources)
        out["other_workloads"] = {}
        for w in also:
            ro = run_workload(w, args.steps, args.warmup)
            summ = workload_summary(ro)
            tro = measured_traffic(w)
            summ["traffic_vs_algorithmic"] = (round(tro["per_launch_traffic_bytes"] /
                                                    tro["per_launch_algorithmic_bytes"], 3) if tro else None)
            print(f"[bench] {w}: {json.dumps(summ)}", file=sys.stderr, flush=True)
            out["other_workloads"][w] = summ
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(fmt, layers, Ms, args.cpu_seconds)
    print(json.dumps(out), flush=True)




if __name__ == "__main__":
    main()
