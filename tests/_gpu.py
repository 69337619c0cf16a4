"""Helpers for the GPU parity tests: move numpy inputs to the device, run the
HIP path through the C ABI binding, bring results back as numpy."""
from __future__ import annotations

import numpy as np
import torch

import skinny_bit_gemm_amd as q

DEV = "cuda:0"


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
    xq = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    xs = torch.empty(q.scales_shape(fmt, M, K, False), dtype=torch.float32, device=DEV)
    q.qlin_quantize_act(fmt, M, K, xd, ldx, xq, xs)
    torch.cuda.synchronize()
    return xq, xs


def gpu_quant_weight(fmt: int, w: np.ndarray):
    N, K = w.shape
    wd = to_dev(w.astype(np.float32))
    wq = torch.empty((N, K), dtype=torch.uint8, device=DEV)
    ws = torch.empty(q.scales_shape(fmt, N, K, True), dtype=torch.float32, device=DEV)
    q.qlin_quantize_weight(fmt, N, K, wd, wq, ws)
    torch.cuda.synchronize()
    del wd
    return wq, ws


def workspace_for(fmt, M, N, K, cfg):
    nbytes = q.qlin_workspace_bytes(fmt, M, N, K, cfg)
    return torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=DEV)


def gpu_gemm(fmt, xq, xs, wq, ws, M, N, K, cfg=None, out_type=q.QLIN_OUT_BF16, workspace=None):
    dt = {q.QLIN_OUT_BF16: torch.int16, q.QLIN_OUT_F32_ACC: torch.float32,
          q.QLIN_OUT_I32_ACC: torch.int32}[out_type]
    y = torch.full((M, N), -1, dtype=dt, device=DEV)   # sentinel: every element must be written
    if workspace is None:
        workspace = workspace_for(fmt, M, N, K, cfg)
    q.qlin_gemm(fmt, M, N, K, xq, xs, wq, ws, y, out_type, cfg, workspace)
    torch.cuda.synchronize()
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
    xq = torch.full((M, K), 0x55, dtype=torch.uint8, device=DEV)
    xs = torch.full(q.scales_shape(fmt, M, K, False), -1.0, dtype=torch.float32, device=DEV)
    dt = {q.QLIN_OUT_BF16: torch.int16, q.QLIN_OUT_F32_ACC: torch.float32,
          q.QLIN_OUT_I32_ACC: torch.int32}[out_type]
    y = torch.full((M, N), -1, dtype=dt, device=DEV)
    if workspace is None:
        workspace = workspace_for(fmt, M, N, K, cfg)
    q.qlin_linear(fmt, M, N, K, xd, ldx, xq, xs, wq, ws, y, out_type, cfg, workspace)
    torch.cuda.synchronize()
    return xq, xs, y
