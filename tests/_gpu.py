"""Helpers for the GPU parity tests: move numpy inputs to the device, run the
HIP path through the C ABI binding, bring results back as numpy.

Every buffer the library writes (outputs, codes, scales, split-K workspaces)
is allocated by `guarded`: a view into a larger device buffer with 4 KiB
canary bands on both sides.  `check_guards` asserts the bands still hold the
canary byte, so a write past either end of a buffer fails the test, not only
a missed write (which the sentinel fills catch)."""
from __future__ import annotations

import numpy as np
import torch

import skinny_bit_gemm_amd as q

DEV = "cuda:0"
GUARD_BYTES = 4096
CANARY = 0xA7


def guarded(shape, dtype, fill=None) -> torch.Tensor:
    """A device tensor of `shape` / `dtype` placed between two GUARD_BYTES
    bands of CANARY bytes (the start stays 16-byte aligned: the caching
    allocator aligns the base, and the band is a multiple of 16).  `fill`
    initialises the tensor itself (default: left at the canary bytes)."""
    shape = tuple(int(s) for s in (shape if isinstance(shape, (tuple, list)) else (shape,)))
    esize = torch.empty((), dtype=dtype).element_size()
    nbytes = int(np.prod(shape, dtype=np.int64)) * esize
    base = torch.full((2 * GUARD_BYTES + nbytes,), CANARY, dtype=torch.uint8, device=DEV)
    t = base[GUARD_BYTES:GUARD_BYTES + nbytes].view(dtype).view(shape)
    if fill is not None:
        t.fill_(fill)
    t._qlin_guard = (base, nbytes)
    return t


def check_guards(*tensors, what: str = ""):
    """Assert that the canary bands around every guarded tensor are intact
    (tensors without bands are skipped)."""
    for t in tensors:
        g = getattr(t, "_qlin_guard", None)
        if g is None:
            continue
        base, nbytes = g
        lo = base[:GUARD_BYTES]
        hi = base[GUARD_BYTES + nbytes:]
        bad_lo = int((lo != CANARY).sum())
        bad_hi = int((hi != CANARY).sum())
        assert bad_lo == 0 and bad_hi == 0, (
            f"{what}: write outside a {tuple(t.shape)} {t.dtype} buffer "
            f"({bad_lo} bytes changed before it, {bad_hi} after it)")


def check_workspace(work: torch.Tensor, what: str = ""):
    """The split-K workspace is left zero by every call, and nothing is
    written around it."""
    check_guards(work, what=what)
    assert int(work.count_nonzero()) == 0, f"{what}: workspace not left zero"


def base_fmt(fmt: int) -> int:
    """The number format of a format argument (without the weight-layout flag)."""
    return fmt & ~q.QLIN_PACKED_WEIGHTS


def to_dev_bf16(x_bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).to(DEV)


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gpu_quant_act(fmt: int, x_bits: np.ndarray, ldx: int | None = None):
    M, K = x_bits.shape
    ldx = K if ldx is None else ldx
    if ldx != K:
        padded = np.zeros((M, ldx), dtype=np.uint16)
        padded[:, :K] = x_bits
        xd = to_dev_bf16(padded)
    else:
        xd = to_dev_bf16(x_bits)
    xq = guarded((M, K), torch.uint8, 0x55)
    xs = guarded(q.scales_shape(fmt, M, K, False), torch.float32, -1.0)
    q.qlin_quantize_act(fmt, M, K, xd, ldx, xq, xs)
    torch.cuda.synchronize()
    check_guards(xq, xs, what=f"qlin_quantize_act fmt={fmt} M={M} K={K}")
    return xq, xs


def gpu_quant_weight(fmt: int, w: np.ndarray):
    N, K = w.shape
    wd = to_dev(w.astype(np.float32))
    wq = guarded((N, K), torch.uint8, 0x55)
    ws = guarded(q.scales_shape(fmt, N, K, True), torch.float32, -1.0)
    q.qlin_quantize_weight(fmt, N, K, wd, wq, ws)
    torch.cuda.synchronize()
    check_guards(wq, ws, what=f"qlin_quantize_weight fmt={fmt} N={N} K={K}")
    del wd
    return wq, ws


def gpu_pack(wq, N, K, batch=1):
    """Row-major codes ([batch][N][K]) -> the packed layout, guarded."""
    nb = q.qlin_packed_weight_bytes(N, K)
    out = guarded((batch * nb,), torch.uint8, 0x5A)
    q.qlin_pack_weight(batch, N, K, wq, out)
    torch.cuda.synchronize()
    check_guards(out, what=f"qlin_pack_weight batch={batch} N={N} K={K}")
    return out


def workspace_for(fmt, M, N, K, cfg):
    """A zeroed split-K workspace of the size the schedule needs, guarded."""
    nbytes = q.qlin_workspace_bytes(base_fmt(fmt), M, N, K, cfg)
    return guarded((max(nbytes, 16),), torch.uint8, 0)


def out_dtype(out_type):
    return {q.QLIN_OUT_BF16: torch.int16, q.QLIN_OUT_F32_ACC: torch.float32,
            q.QLIN_OUT_I32_ACC: torch.int32}[out_type]


def gpu_gemm(fmt, xq, xs, wq, ws, M, N, K, cfg=None, out_type=q.QLIN_OUT_BF16, workspace=None):
    y = guarded((M, N), out_dtype(out_type), -1)   # sentinel: every element must be written
    if workspace is None:
        workspace = workspace_for(fmt, M, N, K, cfg)
    q.qlin_gemm(fmt, M, N, K, xq, xs, wq, ws, y, out_type, cfg, workspace)
    torch.cuda.synchronize()
    what = f"qlin_gemm fmt={fmt} M={M} N={N} K={K} cfg={cfg}"
    check_guards(y, what=what)
    check_workspace(workspace, what=what)
    return y


def y_to_numpy(y: torch.Tensor, out_type=q.QLIN_OUT_BF16) -> np.ndarray:
    a = y.cpu().numpy()
    if out_type == q.QLIN_OUT_BF16:
        return bf16_to_f64(a.view(np.uint16))
    return a


def as_u8(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint8)


def gpu_linear(fmt, x_bits, wq, ws, N, cfg=None, out_type=q.QLIN_OUT_BF16, workspace=None, ldx=None):
    """The whole layer through qlin_linear: returns (xq, xs, y)."""
    M, K = x_bits.shape
    ldx = K if ldx is None else ldx
    padded = np.zeros((M, ldx), dtype=np.uint16)
    padded[:, :K] = x_bits
    xd = to_dev_bf16(padded)
    xq = guarded((M, K), torch.uint8, 0x55)
    xs = guarded(q.scales_shape(base_fmt(fmt), M, K, False), torch.float32, -1.0)
    y = guarded((M, N), out_dtype(out_type), -1)
    if workspace is None:
        workspace = workspace_for(fmt, M, N, K, cfg)
    q.qlin_linear(fmt, M, N, K, xd, ldx, xq, xs, wq, ws, y, out_type, cfg, workspace)
    torch.cuda.synchronize()
    what = f"qlin_linear fmt={fmt} M={M} N={N} K={K} cfg={cfg}"
    check_guards(xq, xs, y, what=what)
    check_workspace(workspace, what=what)
    return xq, xs, y
