"""Python binding of libqlin.so, the gfx950 quantized skinny linear layer.

Argument marshalling only: every step runs in the library's HIP kernels.
Functions carry the C ABI's names (include/qlin.h) and take torch CUDA
tensors (or raw device pointers as ints); torch provides device memory and
the current stream.  A missing or unloadable library raises at import-use
time; there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqlin.so")
TABLE_PATH = os.path.join(HERE, "tables", "gfx950.tbl")

QLIN_FP8_DYNAMIC, QLIN_W8A8_INT8, QLIN_BLOCK_FP8 = 0, 1, 2
QLIN_OUT_BF16, QLIN_OUT_F32_ACC, QLIN_OUT_I32_ACC = 0, 1, 2

STATUS = {
    0: "QLIN_OK", 1: "QLIN_ERR_INVALID_ARG", 2: "QLIN_ERR_ALIGNMENT", 3: "QLIN_ERR_SHAPE",
    4: "QLIN_ERR_WORKSPACE", 5: "QLIN_ERR_NO_CONFIG", 6: "QLIN_ERR_TABLE", 7: "QLIN_ERR_HIP",
}
(QLIN_OK, QLIN_ERR_INVALID_ARG, QLIN_ERR_ALIGNMENT, QLIN_ERR_SHAPE, QLIN_ERR_WORKSPACE,
 QLIN_ERR_NO_CONFIG, QLIN_ERR_TABLE, QLIN_ERR_HIP) = range(8)

# every symbol include/qlin.h declares
EXPORTS = (
    "qlin_quantize_act", "qlin_quantize_weight", "qlin_gemm", "qlin_linear", "qlin_select_variant",
    "qlin_workspace_bytes", "qlin_validate_config", "qlin_load_table", "qlin_set_strict",
    "qlin_table_entries", "qlin_graph_begin", "qlin_graph_end", "qlin_graph_launch",
    "qlin_graph_destroy", "qlin_status_str", "qlin_abi_version", "qlin_last_hip_error",
    "qlin_grouped_gemm", "qlin_grouped_select_variant", "qlin_grouped_workspace_bytes",
    "qlin_linear_scratch", "qlin_packed_weight_bytes", "qlin_pack_weight", "qlin_quantize_act_cfg",
)
# format flag: the weight codes are in the packed layout of qlin_pack_weight
QLIN_PACKED_WEIGHTS = 0x100
# bytes of the static split-K workspace of qlin_linear_scratch (per GPU)
QLIN_SCRATCH_BYTES = 8 << 20


class QlinError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        name = STATUS.get(status, str(status))
        extra = ""
        if status == 7 and _lib is not None:
            extra = f" (hipError {_lib.qlin_last_hip_error()})"
        super().__init__(f"{what}: {name}{extra}")


# qlin_config.act_path: activation codes staged in the LDS, quantized inside
# the GEMM, or loaded by each wave directly
QLIN_ACT_STAGED, QLIN_ACT_FUSED, QLIN_ACT_DIRECT = 0, 1, 2


class qlin_config(ctypes.Structure):
    _fields_ = [("swap_ab", ctypes.c_int32), ("split_k", ctypes.c_int32),
                ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
                ("waves", ctypes.c_int32), ("k_waves", ctypes.c_int32),
                ("reduce", ctypes.c_int32), ("act_path", ctypes.c_int32)]

    def as_dict(self):
        return {f: int(getattr(self, f)) for f, _ in self._fields_}

    def __repr__(self):
        return "qlin_config(%s)" % ", ".join(f"{k}={v}" for k, v in self.as_dict().items())


def make_config(swap_ab=0, split_k=1, tile_m=16, tile_n=32, waves=4, k_waves=4, reduce=0,
                act_path=0) -> qlin_config:
    return qlin_config(swap_ab, split_k, tile_m, tile_n, waves, k_waves, reduce, act_path)


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t


def lib():
    """Load libqlin.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m skinny_bit_gemm_amd.build` (no CPU fallback exists)")
        # torch ships its own HIP runtime (soname libamdhip64.so.7).  Loading
        # torch first makes the dynamic loader bind the library to that same
        # runtime; loading the library first would map the system runtime as
        # a second copy, and torch's streams would be foreign handles to it.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        L.qlin_quantize_act.argtypes = [_I, _I, _I, _P, _I64, _P, _P, _P]
        L.qlin_quantize_weight.argtypes = [_I, _I, _I, _P, _P, _P, _P]
        L.qlin_quantize_act_cfg.argtypes = [_I, _I, _I, _P, _I64, _P, _P, _I, _P]
        L.qlin_gemm.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, _P, _I,
                                ctypes.POINTER(qlin_config), _P, _SZ, _P]
        L.qlin_linear.argtypes = [_I, _I, _I, _I, _P, _I64, _P, _P, _P, _P, _P, _I,
                                  ctypes.POINTER(qlin_config), _P, _SZ, _P]
        L.qlin_linear_scratch.argtypes = [_I, _I, _I, _I, _P, _I64, _P, _P, _P, _P, _P, _I,
                                          ctypes.POINTER(qlin_config), _P]
        L.qlin_packed_weight_bytes.argtypes = [_I, _I, ctypes.POINTER(_SZ)]
        L.qlin_pack_weight.argtypes = [_I, _I, _I, _P, _P, _P]
        L.qlin_select_variant.argtypes = [_I, _I, _I, _I, ctypes.POINTER(qlin_config)]
        L.qlin_workspace_bytes.argtypes = [_I, _I, _I, _I, ctypes.POINTER(qlin_config),
                                           ctypes.POINTER(_SZ)]
        L.qlin_validate_config.argtypes = [_I, _I, _I, _I, ctypes.POINTER(qlin_config)]
        L.qlin_grouped_gemm.argtypes = [_I, _I, _I, _I, _P, _I, _I, _P, _P, _P, _P, _P, _I,
                                        ctypes.POINTER(qlin_config), _P, _SZ, _P]
        L.qlin_grouped_select_variant.argtypes = [_I, _I, _I, _I, _I, ctypes.POINTER(qlin_config)]
        L.qlin_grouped_workspace_bytes.argtypes = [_I, _I, _I, _I, _I, _I, ctypes.POINTER(qlin_config),
                                                   ctypes.POINTER(_SZ)]
        L.qlin_load_table.argtypes = [ctypes.c_char_p]
        L.qlin_set_strict.argtypes = [_I]
        L.qlin_table_entries.argtypes = []
        L.qlin_graph_begin.argtypes = [_P]
        L.qlin_graph_end.argtypes = [_P, ctypes.POINTER(_P)]
        L.qlin_graph_launch.argtypes = [_P, _P]
        L.qlin_graph_destroy.argtypes = [_P]
        L.qlin_status_str.argtypes = [_I]
        L.qlin_status_str.restype = ctypes.c_char_p
        L.qlin_abi_version.argtypes = []
        L.qlin_last_hip_error.argtypes = []
        for name in EXPORTS:
            if name != "qlin_status_str":
                getattr(L, name).restype = _I
        _lib = L
    return _lib


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(st: int, what: str, raise_on_error: bool):
    if raise_on_error and st != 0:
        raise QlinError(st, what)
    return st


def qlin_quantize_act(fmt, M, K, x, ldx, xq, x_scales, stream=None, raise_on_error=True):
    st = lib().qlin_quantize_act(fmt, M, K, _ptr(x), ldx, _ptr(xq), _ptr(x_scales), _stream(stream))
    return _check(st, "qlin_quantize_act", raise_on_error)


def qlin_quantize_act_cfg(fmt, M, K, x, ldx, xq, x_scales, threads, stream=None, raise_on_error=True):
    st = lib().qlin_quantize_act_cfg(fmt, M, K, _ptr(x), ldx, _ptr(xq), _ptr(x_scales), threads, _stream(stream))
    return _check(st, "qlin_quantize_act_cfg", raise_on_error)


def qlin_quantize_weight(fmt, N, K, w, wq, w_scales, stream=None, raise_on_error=True):
    st = lib().qlin_quantize_weight(fmt, N, K, _ptr(w), _ptr(wq), _ptr(w_scales), _stream(stream))
    return _check(st, "qlin_quantize_weight", raise_on_error)


def qlin_gemm(fmt, M, N, K, xq, x_scales, wq, w_scales, y, out_type=QLIN_OUT_BF16, cfg=None,
              workspace=None, ws_bytes=None, stream=None, raise_on_error=True):
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None and \
            not isinstance(workspace, int) else 0
    cptr = ctypes.byref(cfg) if cfg is not None else None
    st = lib().qlin_gemm(fmt, M, N, K, _ptr(xq), _ptr(x_scales), _ptr(wq), _ptr(w_scales), _ptr(y),
                         out_type, cptr, _ptr(workspace), ws_bytes, _stream(stream))
    return _check(st, "qlin_gemm", raise_on_error)


def qlin_linear(fmt, M, N, K, x, ldx, xq, x_scales, wq, w_scales, y, out_type=QLIN_OUT_BF16,
                cfg=None, workspace=None, ws_bytes=None, stream=None, raise_on_error=True):
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None and \
            not isinstance(workspace, int) else 0
    cptr = ctypes.byref(cfg) if cfg is not None else None
    st = lib().qlin_linear(fmt, M, N, K, _ptr(x), ldx, _ptr(xq), _ptr(x_scales), _ptr(wq),
                           _ptr(w_scales), _ptr(y), out_type, cptr, _ptr(workspace), ws_bytes,
                           _stream(stream))
    return _check(st, "qlin_linear", raise_on_error)


def qlin_linear_scratch(fmt, M, N, K, x, ldx, xq, x_scales, wq, w_scales, y, out_type=QLIN_OUT_BF16,
                        cfg=None, stream=None, raise_on_error=True):
    cptr = ctypes.byref(cfg) if cfg is not None else None
    st = lib().qlin_linear_scratch(fmt, M, N, K, _ptr(x), ldx, _ptr(xq), _ptr(x_scales), _ptr(wq),
                                   _ptr(w_scales), _ptr(y), out_type, cptr, _stream(stream))
    return _check(st, "qlin_linear_scratch", raise_on_error)


def qlin_packed_weight_bytes(N, K) -> int:
    out = _SZ(0)
    _check(lib().qlin_packed_weight_bytes(N, K, ctypes.byref(out)), "qlin_packed_weight_bytes", True)
    return int(out.value)


def qlin_pack_weight(batch, N, K, wq, wq_packed, stream=None, raise_on_error=True):
    st = lib().qlin_pack_weight(batch, N, K, _ptr(wq), _ptr(wq_packed), _stream(stream))
    return _check(st, "qlin_pack_weight", raise_on_error)


def qlin_select_variant(fmt, M, N, K) -> qlin_config:
    out = qlin_config()
    st = lib().qlin_select_variant(fmt, M, N, K, ctypes.byref(out))
    _check(st, "qlin_select_variant", True)
    return out


def qlin_workspace_bytes(fmt, M, N, K, cfg=None) -> int:
    out = _SZ(0)
    st = lib().qlin_workspace_bytes(fmt, M, N, K, ctypes.byref(cfg) if cfg is not None else None,
                                    ctypes.byref(out))
    _check(st, "qlin_workspace_bytes", True)
    return int(out.value)


def qlin_grouped_gemm(fmt, groups, N, K, group_offsets, total_rows, max_group_rows, xq, x_scales, wq,
                      w_scales, y, out_type=QLIN_OUT_BF16, cfg=None, workspace=None, ws_bytes=None,
                      stream=None, raise_on_error=True):
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None and \
            not isinstance(workspace, int) else 0
    cptr = ctypes.byref(cfg) if cfg is not None else None
    st = lib().qlin_grouped_gemm(fmt, groups, N, K, _ptr(group_offsets), total_rows, max_group_rows,
                                 _ptr(xq), _ptr(x_scales), _ptr(wq), _ptr(w_scales), _ptr(y), out_type,
                                 cptr, _ptr(workspace), ws_bytes, _stream(stream))
    return _check(st, "qlin_grouped_gemm", raise_on_error)


def qlin_grouped_select_variant(fmt, groups, N, K, max_group_rows) -> qlin_config:
    out = qlin_config()
    st = lib().qlin_grouped_select_variant(fmt, groups, N, K, max_group_rows, ctypes.byref(out))
    _check(st, "qlin_grouped_select_variant", True)
    return out


def qlin_grouped_workspace_bytes(fmt, groups, N, K, total_rows, max_group_rows, cfg=None) -> int:
    out = _SZ(0)
    st = lib().qlin_grouped_workspace_bytes(fmt, groups, N, K, total_rows, max_group_rows,
                                            ctypes.byref(cfg) if cfg is not None else None, ctypes.byref(out))
    _check(st, "qlin_grouped_workspace_bytes", True)
    return int(out.value)


def qlin_validate_config(fmt, M, N, K, cfg) -> int:
    return lib().qlin_validate_config(fmt, M, N, K, ctypes.byref(cfg) if cfg is not None else None)


def qlin_load_table(path=None, raise_on_error=True) -> int:
    st = lib().qlin_load_table(path.encode() if path else None)
    return _check(st, "qlin_load_table", raise_on_error)


def qlin_set_strict(strict: bool) -> None:
    lib().qlin_set_strict(1 if strict else 0)


def qlin_table_entries() -> int:
    return int(lib().qlin_table_entries())


def qlin_graph_begin(stream) -> None:
    _check(lib().qlin_graph_begin(_stream(stream)), "qlin_graph_begin", True)


def qlin_graph_end(stream) -> int:
    h = _P()
    _check(lib().qlin_graph_end(_stream(stream), ctypes.byref(h)), "qlin_graph_end", True)
    return h.value


def qlin_graph_launch(graph: int, stream=None) -> None:
    _check(lib().qlin_graph_launch(graph, _stream(stream)), "qlin_graph_launch", True)


def qlin_graph_destroy(graph: int) -> None:
    _check(lib().qlin_graph_destroy(graph), "qlin_graph_destroy", True)


def qlin_status_str(st: int) -> str:
    return lib().qlin_status_str(st).decode()


def qlin_abi_version() -> int:
    return int(lib().qlin_abi_version())


def qlin_last_hip_error() -> int:
    return int(lib().qlin_last_hip_error())


# ---------------------------------------------------------------- helpers

def scales_shape(fmt: int, rows: int, K: int, weight: bool) -> tuple:
    """Shape of the fp32 scale tensor for an [rows, K] operand."""
    if fmt == QLIN_BLOCK_FP8:
        return ((rows // 128) if weight else rows, K // 128)
    return (rows,)


def code_dtype(fmt: int):
    import torch
    return torch.int8 if fmt == QLIN_W8A8_INT8 else torch.uint8
