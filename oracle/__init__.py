"""CPU reference (oracle) for the quantized skinny linear layer.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  The GPU library never imports, links or calls
anything here, and the two share no code.  The arithmetic lives in
``qlin_oracle.c`` (plain loops, fp64 results); this module only builds it
with gcc and marshals numpy arrays.

Source: "Building a High-Performance and Portable vLLM Linear Backend with
Helion", sections "Scope" (formats) and "Kernel Implementation" (the product).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

FP8_DYNAMIC, W8A8_INT8, BLOCK_FP8 = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qlin_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liborc.so")
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64


def build(force: bool = False) -> str:
    """Compile qlin_oracle.c with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < max(
            os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "qlin_oracle.h"))):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB_PATH)
        L.orc_e4m3_decode.restype = ctypes.c_double
        L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_encode.restype = _I
        L.orc_e4m3_encode.argtypes = [ctypes.c_float, _P]
        L.orc_e4m3_encode_array.restype = _I64
        L.orc_e4m3_encode_array.argtypes = [_P, _P, _I64]
        L.orc_quant_act.restype = _I
        L.orc_quant_act.argtypes = [_I, _I, _I, _P, _P, _P]
        L.orc_quant_weight.restype = _I
        L.orc_quant_weight.argtypes = [_I, _I, _I, _P, _P, _P]
        for name in ("orc_acc_int8", "orc_acc_fp8", "orc_acc_fp8_groups"):
            f = getattr(L, name)
            f.restype = _I
            f.argtypes = [_I, _I, _I, _P, _P, _P]
        L.orc_gemm.restype = _I
        L.orc_gemm.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P]
        L.orc_gemm_sampled.restype = _I
        L.orc_gemm_sampled.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, _I64, _P, _P, _P, _P]
        L.orc_linear.restype = _I
        L.orc_linear.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P]
        L.orc_round_bf16.restype = None
        L.orc_round_bf16.argtypes = [_P, _P, _I64]
        L.orc_num_threads.restype = _I
        L.orc_num_threads.argtypes = []
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(st: int, what: str):
    if st != 0:
        raise ValueError(f"oracle {what} failed with status {st}")


def e4m3_decode(codes) -> np.ndarray:
    """Exact value of every E4M3FN code in ``codes`` (fp64)."""
    L = lib()
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([L.orc_e4m3_decode(int(v)) for v in c.ravel()], dtype=np.float64).reshape(c.shape)


def e4m3_encode(values) -> np.ndarray:
    """fp32 -> E4M3FN codes (saturating, nearest-even); raises on non-finite input."""
    v = np.ascontiguousarray(values, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    bad = lib().orc_e4m3_encode_array(_ptr(v), _ptr(out), v.size)
    if bad:
        raise ValueError(f"{bad} non-finite values cannot be encoded")
    return out


def scale_shape(fmt: int, rows: int, K: int, weight: bool) -> tuple:
    if fmt == BLOCK_FP8:
        return ((rows // 128) if weight else rows, K // 128)
    return (rows,)


def quant_act(fmt: int, x_bf16: np.ndarray):
    """Quantize bf16 activations [M, K] (uint16 bits) -> (codes uint8 [M,K], fp32 scales)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    M, K = x.shape
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty(scale_shape(fmt, M, K, False), dtype=np.float32)
    _check(lib().orc_quant_act(fmt, M, K, _ptr(x), _ptr(q), _ptr(s)), "quant_act")
    return q, s


def quant_weight(fmt: int, w: np.ndarray):
    """Quantize fp32 weights [N, K] -> (codes uint8 [N,K], fp32 scales)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    q = np.empty((N, K), dtype=np.uint8)
    s = np.empty(scale_shape(fmt, N, K, True), dtype=np.float32)
    _check(lib().orc_quant_weight(fmt, N, K, _ptr(w), _ptr(q), _ptr(s)), "quant_weight")
    return q, s


def acc_int8(qa: np.ndarray, qw: np.ndarray) -> np.ndarray:
    qa = np.ascontiguousarray(qa, dtype=np.uint8)
    qw = np.ascontiguousarray(qw, dtype=np.uint8)
    M, K = qa.shape
    N = qw.shape[0]
    acc = np.empty((M, N), dtype=np.int32)
    _check(lib().orc_acc_int8(M, N, K, _ptr(qa), _ptr(qw), _ptr(acc)), "acc_int8")
    return acc


def acc_fp8(qa: np.ndarray, qw: np.ndarray) -> np.ndarray:
    qa = np.ascontiguousarray(qa, dtype=np.uint8)
    qw = np.ascontiguousarray(qw, dtype=np.uint8)
    M, K = qa.shape
    N = qw.shape[0]
    acc = np.empty((M, N), dtype=np.float64)
    _check(lib().orc_acc_fp8(M, N, K, _ptr(qa), _ptr(qw), _ptr(acc)), "acc_fp8")
    return acc


def acc_fp8_groups(qa: np.ndarray, qw: np.ndarray) -> np.ndarray:
    qa = np.ascontiguousarray(qa, dtype=np.uint8)
    qw = np.ascontiguousarray(qw, dtype=np.uint8)
    M, K = qa.shape
    N = qw.shape[0]
    acc = np.empty((M, N, K // 128), dtype=np.float64)
    _check(lib().orc_acc_fp8_groups(M, N, K, _ptr(qa), _ptr(qw), _ptr(acc)), "acc_fp8_groups")
    return acc


def gemm(fmt: int, qa, sa, qw, sw, want_acc: bool = False):
    """fp64 dequantized product ref [M, N] (and int32 accumulators for int8)."""
    qa = np.ascontiguousarray(qa, dtype=np.uint8)
    qw = np.ascontiguousarray(qw, dtype=np.uint8)
    sa = np.ascontiguousarray(sa, dtype=np.float32)
    sw = np.ascontiguousarray(sw, dtype=np.float32)
    M, K = qa.shape
    N = qw.shape[0]
    ref = np.empty((M, N), dtype=np.float64)
    acc = np.empty((M, N), dtype=np.int32) if (want_acc and fmt == W8A8_INT8) else None
    _check(lib().orc_gemm(fmt, M, N, K, _ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), _ptr(ref),
                          _ptr(acc) if acc is not None else None), "gemm")
    return (ref, acc) if want_acc else ref


def gemm_sampled(fmt: int, qa, sa, qw, sw, ms, ns, want_acc: bool = False):
    """fp64 ref[i] = ref(ms[i], ns[i]) for selected outputs of a large product."""
    qa = np.ascontiguousarray(qa, dtype=np.uint8)
    qw = np.ascontiguousarray(qw, dtype=np.uint8)
    sa = np.ascontiguousarray(sa, dtype=np.float32)
    sw = np.ascontiguousarray(sw, dtype=np.float32)
    ms = np.ascontiguousarray(ms, dtype=np.int32)
    ns = np.ascontiguousarray(ns, dtype=np.int32)
    M, K = qa.shape
    N = qw.shape[0]
    ref = np.empty(ms.shape, dtype=np.float64)
    acc = np.empty(ms.shape, dtype=np.int32) if (want_acc and fmt == W8A8_INT8) else None
    _check(lib().orc_gemm_sampled(fmt, M, N, K, _ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), ms.size,
                                  _ptr(ms), _ptr(ns), _ptr(ref),
                                  _ptr(acc) if acc is not None else None), "gemm_sampled")
    return (ref, acc) if want_acc else ref


def linear(fmt: int, x_bf16, qw, sw, want_acc: bool = False):
    """Whole layer: (qa, sa, ref[, acc]) for bf16 activations and quantized weights."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    qw = np.ascontiguousarray(qw, dtype=np.uint8)
    sw = np.ascontiguousarray(sw, dtype=np.float32)
    M, K = x.shape
    N = qw.shape[0]
    qa = np.empty((M, K), dtype=np.uint8)
    sa = np.empty(scale_shape(fmt, M, K, False), dtype=np.float32)
    ref = np.empty((M, N), dtype=np.float64)
    acc = np.empty((M, N), dtype=np.int32) if (want_acc and fmt == W8A8_INT8) else None
    _check(lib().orc_linear(fmt, M, N, K, _ptr(x), _ptr(qw), _ptr(sw), _ptr(qa), _ptr(sa),
                            _ptr(ref), _ptr(acc) if acc is not None else None), "linear")
    if want_acc:
        return qa, sa, ref, acc
    return qa, sa, ref


def grouped_gemm(fmt: int, offsets, qa, sa, qw, sw, want_acc: bool = False):
    """Grouped product: rows offsets[e] .. offsets[e+1] - 1 of (qa, sa) times
    the e-th weights (qw[e], sw[e]), each group exactly as gemm(); the rows
    come back in the same order.  A mixture-of-experts layer is this product
    over the experts' row groups; the pages name MoE models as future work
    and give each group's product ("Building a High-Performance and Portable
    vLLM Linear Backend with Helion", sections "Future work", model-coverage
    paragraph, and "Kernel Implementation")."""
    offsets = np.asarray(offsets, dtype=np.int64)
    M, N = int(offsets[-1]), np.asarray(qw).shape[1]
    ref = np.zeros((M, N), dtype=np.float64)
    acc = np.zeros((M, N), dtype=np.int32) if (want_acc and fmt == W8A8_INT8) else None
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        out = gemm(fmt, qa[lo:hi], sa[lo:hi], qw[e], sw[e], want_acc=want_acc)
        if want_acc:
            ref[lo:hi] = out[0]
            if acc is not None:
                acc[lo:hi] = out[1]
        else:
            ref[lo:hi] = out
    return (ref, acc) if want_acc else ref


def round_bf16(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().orc_round_bf16(_ptr(v), _ptr(out), v.size)
    return out


def num_threads() -> int:
    return int(lib().orc_num_threads())


def tolerance_ok(y: np.ndarray, ref: np.ndarray, ref_max: float | None = None):
    """Acceptance rule for bf16 outputs: |y - ref| <= 1e-2 |ref| + 1e-3 max|ref|.

    ``ref_max`` is the max |ref| over the whole output of the call (pass it
    when ``ref`` holds only sampled outputs).  Returns (ok, worst ratio)."""
    ref = np.asarray(ref, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    if ref_max is None:
        ref_max = float(np.max(np.abs(ref))) if ref.size else 0.0
    bound = 1e-2 * np.abs(ref) + 1e-3 * ref_max
    err = np.abs(y - ref)
    if err.size == 0:
        return True, 0.0
    ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))
    return bool(np.all(err <= bound)), float(np.max(ratio))
