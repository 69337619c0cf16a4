"""Binding of the measurement aid libqlin_probe.so (include/qlin_probe.h):
the streaming-read ceiling of HBM that bench.py reports next to the GEMM."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB_PATH = os.path.join(HERE, "libqlin_probe.so")
EXPORTS = ("qlin_probe_read",)

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise RuntimeError(f"{PROBE_LIB_PATH} is missing: build it with "
                               "`python -m skinny_bit_gemm_amd.build`")
        import torch  # noqa: F401  (bind to torch's HIP runtime, as libqlin.so does)
        L = ctypes.CDLL(PROBE_LIB_PATH)
        L.qlin_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                      ctypes.c_void_p]
        L.qlin_probe_read.restype = ctypes.c_int
        _lib = L
    return _lib


def qlin_probe_read(buf, nbytes, sink, blocks, stream=None):
    """Enqueue one streaming read of nbytes of buf; returns the status code."""
    from . import _ptr, _stream
    return lib().qlin_probe_read(_ptr(buf), nbytes, _ptr(sink), blocks, _stream(stream))


def read_ceiling_gbs(nbytes=1 << 30, grids=(256, 512, 8192, 32768), reps=10):
    """GB/s of a plain read of a fresh nbytes buffer: the best over a few
    grid sizes (one workgroup per compute unit streams best on MI355X) and
    reps timed launches each."""
    import torch
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(max(grids), dtype=torch.int32, device="cuda")
    st = torch.cuda.Stream()
    best = None
    with torch.cuda.stream(st):
        for blocks in grids:
            if qlin_probe_read(buf, nbytes, sink, blocks, st) != 0:
                raise RuntimeError("qlin_probe_read was rejected")
            for _ in range(reps):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(st)
                qlin_probe_read(buf, nbytes, sink, blocks, st)
                e1.record(st)
                torch.cuda.synchronize()
                t = e0.elapsed_time(e1) * 1e-3
                best = t if best is None else min(best, t)
    del buf, sink
    return nbytes / best / 1e9


def graph_floor_us(nbytes, grids=(256, 512, 1024, 2048), with_grid=False):
    """Microseconds per launch of the streaming read of an nbytes buffer,
    launched back to back from a hipGraph over cold copies (>= 1 GiB of
    them, so the L2 and the Infinity Cache serve none), the best over a few
    grid sizes: what reading a weight matrix once costs in one kernel under
    the conditions the layer timings run in."""
    import torch
    from . import qlin_graph_begin, qlin_graph_destroy, qlin_graph_end, qlin_graph_launch
    from .tune import warm_graph
    n = max(2, -(-(1 << 30) // nbytes))
    copies = [torch.ones(nbytes // 4, dtype=torch.int32, device="cuda") for _ in range(n)]
    sink = torch.zeros(max(grids), dtype=torch.int32, device="cuda")
    st = torch.cuda.Stream()
    best, best_grid = None, None
    with torch.cuda.stream(st):
        for blocks in grids:
            reps = max(1, -(-64 // n))
            qlin_graph_begin(st)
            try:
                for _ in range(reps):
                    for c in copies:
                        if qlin_probe_read(c, nbytes, sink, blocks, st) != 0:
                            raise RuntimeError("qlin_probe_read was rejected")
            finally:
                g = qlin_graph_end(st)
            warm_graph(g, st)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(st)
            for _ in range(5):
                qlin_graph_launch(g, st)
            e1.record(st)
            torch.cuda.synchronize()
            qlin_graph_destroy(g)
            us = e0.elapsed_time(e1) * 1e3 / (5 * reps * n)
            if best is None or us < best:
                best, best_grid = us, blocks
    del copies, sink
    torch.cuda.empty_cache()
    return (best, best_grid) if with_grid else best
