"""Offline per-shape tuner: measures candidate schedules on the GPU and writes
the selection table that qlin_select_variant reads.

"Building a High-Performance and Portable vLLM Linear Backend with Helion",
sections "Per-shape Config Tuning" (each (shape, num_tokens) in the tuned
range gets its own configuration) and "Enable CUDA Graph for Autotuner
Benchmarking" (candidates are timed the way they run in production, under
graph replay).  Here the search is exhaustive over a fixed candidate grid
(schedule, tile, split factor, wave layout); each candidate is timed as a
hipGraph of back-to-back layers (qlin_linear: quantize + GEMM) over distinct
weight copies (>= 1 GiB in total, so the Infinity Cache cannot hold them),
in the packed weight layout (--layout row-major for the other).
A coarse pass over the schedule grid (each schedule with each activation
path: codes quantized in their own kernel and staged in the LDS, the same
codes loaded by each wave directly, or quantized inside the GEMM), then the
best few with each
split-K reduction, then the best of those again with more replays.  With
--merge, a point that already has an entry keeps it unless the new best beats
it, timed beside it in the same session, by more than --keep-margin: the
ranking among near-equal schedules changes between runs, and swapping them
on that noise made whole decode steps slower.

Usage:
  python -m skinny_bit_gemm_amd.tune --shape fp8_dynamic,4096,2048 ... \\
      [--m 1,2,4,8,16,24,32] [--out tables/gfx950.tbl] [--merge [--keep-margin 0.02]]
      [--report file.json]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import skinny_bit_gemm_amd as q

FMT_NAMES = {q.QLIN_FP8_DYNAMIC: "fp8_dynamic", q.QLIN_W8A8_INT8: "w8a8_int8",
             q.QLIN_BLOCK_FP8: "block_fp8"}
FMT_IDS = {v: k for k, v in FMT_NAMES.items()}

# (tile_n, waves, k_waves); tile_n = 8 x (waves / k_waves) selects 8-row
# weight sub-tiles.  The last group has 3, 5, 6 or 7 column waves: widths such
# as 24, 48 or 96 rows split N = 6144, 12288 or 24576 into exactly 256 tiles
# (one per compute unit), and 224 rows split N = 51200 into 229, where
# power-of-two widths leave part of the chip idle for a second round.
TILES = [(16, 1, 1), (16, 2, 2), (16, 4, 4), (16, 8, 8), (32, 1, 1), (32, 2, 2), (32, 4, 4),
         (32, 4, 2), (32, 8, 8), (32, 8, 4), (64, 1, 1), (64, 2, 1), (64, 4, 4), (64, 4, 2),
         (64, 4, 1), (64, 8, 4), (64, 8, 2), (128, 4, 1), (128, 8, 2), (128, 8, 1),
         (8, 1, 1), (8, 2, 2), (8, 4, 4), (8, 8, 8), (16, 2, 1), (16, 4, 2), (16, 8, 4), (32, 4, 1),
         (32, 8, 2), (64, 8, 1),
         (24, 3, 1), (24, 6, 2), (48, 3, 1), (48, 6, 2), (96, 3, 1), (96, 6, 2), (40, 5, 1),
         (80, 5, 1), (48, 6, 1), (96, 6, 1), (56, 7, 1), (112, 7, 1), (224, 7, 1)]
SPLITS = [1, 2, 3, 4, 6, 8, 12, 16, 24, 32]


def exact_format(fmt, K):
    return fmt == q.QLIN_W8A8_INT8 or (fmt == q.QLIN_FP8_DYNAMIC and K <= 40960)


def candidates(fmt, M, N, K):
    """Base grid: schedule, tile, split and wave layout, each with staged
    and with direct activation codes (quantized in a separate kernel) and,
    where the tile's rows fit the kernel's registers, quantized inside the
    GEMM; slice reduction."""
    nkb = -(-K // 128)
    seen = set()
    out = []
    # 16-token tiles up to 64 tokens too: two to four token tiles each
    # re-read the weight tile (from the L2 when they run together), but a
    # workgroup stages or loads half the activation rows; past 32 tokens
    # also 64-token tiles, which read each weight tile once per 64 tokens
    tile_ms = (16,) if M <= 16 else (16, 32) if M <= 32 else (16, 32, 64) if M <= 64 else (32, 64)
    for tile_m in tile_ms:
        for swap in (0, 1):
            for (tn, waves, kw) in TILES:
                for split in SPLITS:
                    kbs = -(-nkb // split)
                    eff = -(-nkb // kbs)
                    key = (tile_m, swap, tn, waves, kw, kbs)
                    if key in seen or kbs < kw:
                        continue
                    wgs = -(-N // tn) * -(-M // tile_m) * eff
                    if wgs < 16 or wgs > 16384:
                        continue
                    seen.add(key)
                    acts = (q.QLIN_ACT_STAGED, q.QLIN_ACT_DIRECT) + ((q.QLIN_ACT_FUSED,) if tile_m == 16 else ())
                    for act in acts:
                        c = q.make_config(swap, eff, tile_m, tn, waves, kw, 0, act)
                        if variant_class(c) == "large_m":
                            continue   # the large-M kernel's layout: its candidates follow
                        if q.qlin_validate_config(fmt, M, N, K, c) == 0:
                            out.append(c)
    if M > 32:
        # the large-M kernel: 64- / 128-token tiles of 128 channels
        for tmb in (64, 128):
            for split in (1, 2, 3, 4, 6, 8, 12, 16):
                kbs = -(-nkb // split)
                eff = -(-nkb // kbs)
                c = q.make_config(0, eff, tmb, 128, 4, 1, 0, 0)
                if (tmb, kbs) in seen or q.qlin_validate_config(fmt, M, N, K, c) != 0:
                    continue
                seen.add((tmb, kbs))
                out.append(c)
    return out


def variants(fmt, M, N, K, c):
    """The same schedule with each split-K reduction."""
    out = []
    reds = [0, 1] if (c.split_k > 1 and exact_format(fmt, K)) else [0]
    for r in reds:
        v = q.make_config(c.swap_ab, c.split_k, c.tile_m, c.tile_n, c.waves, c.k_waves, r, c.act_path)
        if q.qlin_validate_config(fmt, M, N, K, v) == 0:
            out.append(v)
    return out


def warm_graph(graph, stream, min_ms=20.0):
    """Replays a captured graph, untimed, for about min_ms (at most 1000
    replays).  After host-side set-up has left the GPU idle, a measurement
    started at once ran up to ~10 % slower (5 ms of replays still left
    3-6 %)."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    q.qlin_graph_launch(graph, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    once = max(e0.elapsed_time(e1), 1e-3)
    for _ in range(min(1000, int(min_ms / once))):
        q.qlin_graph_launch(graph, stream)


# the weight layout the table is tuned for: the packed layout of
# qlin_pack_weight, which the decode path runs (row-major weights use the
# same table)
PACKED = True


class Bench:
    """Device buffers for timing one (fmt, M, N, K) linear layer.  The
    weights are random codes (the timing does not depend on their values),
    laid out as the packed layout's bytes unless `packed` is false."""

    def __init__(self, fmt, M, N, K, min_bytes=1 << 30, packed=None):
        import torch
        self.torch = torch
        self.fmt, self.M, self.N, self.K = fmt, M, N, K
        packed = PACKED if packed is None else packed
        self.call_fmt = fmt | (q.QLIN_PACKED_WEIGHTS if packed else 0)
        wshape = (q.qlin_packed_weight_bytes(N, K),) if packed else (N, K)
        dev = "cuda"
        self.R = max(2, -(-min_bytes // (N * K)))
        g = torch.Generator(device=dev)
        g.manual_seed(0)

        def codes(shape):
            t = torch.randint(-120, 120, shape, dtype=torch.int8, device=dev, generator=g)
            if fmt != q.QLIN_W8A8_INT8:            # finite, modest fp8 codes
                t = (t.view(torch.uint8) & 0xB7)
            return t
        self.W = [codes(wshape) for _ in range(self.R)]
        self.ws = torch.rand(q.scales_shape(fmt, N, K, True), device=dev, generator=g) * 1e-2
        self.x = torch.randn((M, K), device=dev, generator=g).to(torch.bfloat16)
        self.xq = torch.empty((M, K), dtype=torch.uint8, device=dev)
        self.xs = torch.empty(q.scales_shape(fmt, M, K, False), dtype=torch.float32, device=dev)
        self.y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        self.stream = torch.cuda.Stream()
        self.work = torch.zeros(1 << 20, dtype=torch.uint8, device=dev)
        self.warm = False

    def _call(self, cfg, w, st):
        q.qlin_linear(self.call_fmt, self.M, self.N, self.K, self.x, self.K, self.xq, self.xs, w, self.ws,
                      self.y, q.QLIN_OUT_BF16, cfg, self.work, stream=st)

    def time(self, cfg, replays=3):
        """Mean time of one linear (quantize + GEMM) under graph replay."""
        torch = self.torch
        nb = q.qlin_workspace_bytes(self.fmt, self.M, self.N, self.K, cfg)
        if nb > self.work.numel():
            self.work = torch.zeros(nb, dtype=torch.uint8, device="cuda")
        st = self.stream
        with torch.cuda.stream(st):
            self._call(cfg, self.W[0], st)
            q.qlin_graph_begin(st)
            try:
                for w in self.W:
                    self._call(cfg, w, st)
            finally:
                gr = q.qlin_graph_end(st)
            if self.warm:
                q.qlin_graph_launch(gr, st)
            else:   # the first timing after the buffers were set up
                warm_graph(gr, st)
                self.warm = True
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(st)
            for _ in range(replays):
                q.qlin_graph_launch(gr, st)
            e1.record(st)
            torch.cuda.synchronize()
            q.qlin_graph_destroy(gr)
        return e0.elapsed_time(e1) * 1e3 / (replays * self.R)

    def free(self):
        self.W = None
        self.torch.cuda.empty_cache()


def variant_class(c):
    if c.tile_m == 128 or (c.tile_m == 64 and (c.tile_n, c.waves, c.k_waves, c.swap_ab) == (128, 4, 1, 0)
                           and c.reduce == 0):
        return "large_m"
    if c.split_k > 1:
        return "splitk"
    return "swap_ab" if c.swap_ab else "standard"


def keep_or_replace(best_t, best_c, inc_t, inc_c, margin):
    """The entry a merge keeps: the incumbent (an existing table entry, timed
    in the same session) unless the new best is faster by more than `margin`
    (a fraction); near-equal schedules are not swapped on measurement noise.
    Returns (time, config, kept_incumbent)."""
    if inc_c is not None and not best_t < inc_t * (1.0 - margin):
        return inc_t, inc_c, True
    return best_t, best_c, False


def tune_point(fmt, M, N, K, keep=10, final=5, incumbent=None, margin=0.0):
    b = Bench(fmt, M, N, K)
    base = candidates(fmt, M, N, K)
    coarse = sorted(((b.time(c, replays=1), c) for c in base), key=lambda t: t[0])
    best_by_class = {}
    for t, c in coarse:
        best_by_class.setdefault(variant_class(c), (t, c))
    expanded = []
    for _, c in coarse[:keep]:
        for v in variants(fmt, M, N, K, c):
            expanded.append((b.time(v, replays=2), v))
    expanded.sort(key=lambda t: t[0])
    fine = sorted(((b.time(c, replays=5), c) for _, c in expanded[:final]), key=lambda t: t[0])
    inc_t = None
    if incumbent is not None:
        inc_t = min(b.time(incumbent, replays=5) for _ in range(2))
        # the new best is timed again beside it, under the same conditions
        fine[0] = (min(fine[0][0], b.time(fine[0][1], replays=5)), fine[0][1])
    b.free()
    t, c, kept = keep_or_replace(fine[0][0], fine[0][1], inc_t, incumbent, margin)
    return (t, c), best_by_class, len(base) + len(expanded), kept


STANDARD_HEADER = (
    "# measured on MI355X by skinny_bit_gemm_amd.tune (hipGraph replay, rotating weights)",
    "# format N K M swap_ab split_k tile_m tile_n waves k_waves reduce act_path",
    "# (times are of the whole layer, quantize + GEMM; best_by_class in the report",
    "#  compares the schedules' best coarse times, slice reduction)",
)


def read_entries(path):
    """A table's entries {(fmt, N, K, M): [8 fields]} and its comment lines
    other than the standard header."""
    entries, notes = {}, []
    with open(path) as f:
        for line in f:
            if line.startswith("#"):
                if line.rstrip("\n") not in STANDARD_HEADER:
                    notes.append(line.rstrip("\n"))
                continue
            p = line.split("#")[0].split()
            if len(p) == 12:
                entries[(p[0], int(p[1]), int(p[2]), int(p[3]))] = p[4:]
    return entries, notes


def write_entries(path, entries, notes=()):
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        f.write(f"qlin-table {q.qlin_abi_version()} gfx950\n")
        for line in STANDARD_HEADER:
            f.write(line + "\n")
        for line in notes:
            f.write(line + "\n")
        for k in sorted(entries):
            f.write(" ".join([k[0], str(k[1]), str(k[2]), str(k[3])] + entries[k]) + "\n")


def algorithmic_bytes(fmt, M, N, K):
    if fmt == q.QLIN_BLOCK_FP8:
        wsc, asc = 4 * (N // 128) * (K // 128), 4 * M * (K // 128)
    else:
        wsc, asc = 4 * N, 4 * M
    return N * K + wsc + M * K + asc + 2 * M * N


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--shape", action="append", default=[], help="fmt,N,K")
    ap.add_argument("--m", default="1,2,4,8,16,24,32,64,128,256,512")
    ap.add_argument("--out", default=os.path.join(os.path.dirname(__file__), "tables", "gfx950.tbl"))
    ap.add_argument("--merge", action="store_true",
                    help="keep the entries of --out that are not re-tuned; a re-tuned entry is replaced "
                         "only when the new best is faster by more than --keep-margin")
    ap.add_argument("--keep-margin", type=float, default=0.02,
                    help="with --merge: the fraction by which a new schedule must beat the existing entry")
    ap.add_argument("--report", default=None)
    ap.add_argument("--layout", choices=("packed", "row-major"), default="packed",
                    help="weight layout the candidates are timed on (default: packed)")
    args = ap.parse_args(argv)
    global PACKED
    PACKED = args.layout == "packed"
    Ms = [int(v) for v in args.m.split(",")]
    q.lib()
    entries, notes = {}, []
    if args.merge and os.path.exists(args.out):
        entries, notes = read_entries(args.out)
    report = []
    t_start = time.time()
    for spec in args.shape:
        fname, N, K = spec.split(",")
        fmt, N, K = FMT_IDS[fname], int(N), int(K)
        for M in Ms:
            inc = None
            old = entries.get((fname, N, K, M))
            if old is not None:
                inc = q.make_config(*[int(v) for v in old])
                if q.qlin_validate_config(fmt, M, N, K, inc) != 0:
                    inc = None
            (t, c), by_class, n, kept = tune_point(fmt, M, N, K, incumbent=inc, margin=args.keep_margin)
            gbs = algorithmic_bytes(fmt, M, N, K) / t / 1e3
            entries[(fname, N, K, M)] = [str(v) for v in (c.swap_ab, c.split_k, c.tile_m, c.tile_n,
                                                         c.waves, c.k_waves, c.reduce, c.act_path)]
            rec = {"fmt": fname, "N": N, "K": K, "M": M, "us": round(t, 3), "GBps": round(gbs, 1),
                   "cfg": c.as_dict(), "candidates": n, "kept_existing_entry": kept,
                   "best_by_class": {k: {"us": round(v[0], 3), "cfg": v[1].as_dict()}
                                     for k, v in by_class.items()}}
            report.append(rec)
            print(f"[tune {time.time() - t_start:6.1f}s] {fname} N={N} K={K} M={M}: {t:.2f} us "
                  f"{gbs:.0f} GB/s {c}  (" + ", ".join(f"{k} {v[0]:.2f}" for k, v in by_class.items())
                  + ")", flush=True)
    write_entries(args.out, entries, notes)
    if args.report:
        with open(args.report, "w") as f:
            json.dump(report, f, indent=1)
    print(f"wrote {len(entries)} entries to {args.out}", flush=True)


if __name__ == "__main__":
    sys.exit(main())
