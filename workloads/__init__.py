"""Seeded synthetic workloads for the quantized skinny linear layer.

This module is shared by the tests, the benchmark and the CPU reference
(oracle) harness.  It only draws random numbers and rounds them once to
bfloat16; it holds none of the quantization or GEMM arithmetic.

Shapes are the linear layers of three dense decoder sizes (hidden 2048, 4096
and 5120 with 128-wide heads), standing in for the Qwen3 models benchmarked
in "Building a High-Performance and Portable vLLM Linear Backend with Helion"
(section "Performance Evaluation"), whose weights are not available here.
The token counts are the tuned set of that page's section "Per-shape Config
Tuning": num_tokens in {1, 2, 4, 8, 16, 24, 32}.

Value recipe:
  * activations: fp32 N(0, 1); 1 % of the K channels (ceil(0.01 K), drawn
    without replacement, shared by all tokens) are multiplied by 20; for the
    block-scaled format the outliers are 1 % of the 128-wide K groups (at
    least one group) instead.  The result is rounded once to bfloat16
    (round to nearest, ties to even).
  * weights: fp32 N(0, 0.02), shape [N, K] (row n is output channel n).
  * seeds: numpy default_rng([0, fmt_id, N, K, 0]) for weights and
    default_rng([0, fmt_id, N, K, 1, M]) for activations; the tiny case uses
    default_rng(0), weights drawn first, then activations, no outliers.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

# format ids (same numbering as the C ABI's qlin_format enum)
FP8_DYNAMIC = 0
W8A8_INT8 = 1
BLOCK_FP8 = 2

FORMAT_NAMES = {FP8_DYNAMIC: "fp8_dynamic", W8A8_INT8: "w8a8_int8", BLOCK_FP8: "block_fp8"}
FORMAT_IDS = {v: k for k, v in FORMAT_NAMES.items()}

TUNED_M = (1, 2, 4, 8, 16, 24, 32)
SWEEP_M = (1, 2, 4, 8, 16, 24, 32, 64, 128, 256, 512)


@dataclass(frozen=True)
class Layer:
    name: str
    N: int
    K: int


# hidden 2048, 16 q / 8 kv heads of dim 128, FFN 6144
SMALL_DENSE = (Layer("qkv", 4096, 2048), Layer("o", 2048, 2048),
               Layer("gate_up", 12288, 2048), Layer("down", 2048, 6144))
# hidden 4096, 32 q / 8 kv heads of dim 128, FFN 12288
DENSE_8B = (Layer("qkv", 6144, 4096), Layer("o", 4096, 4096),
            Layer("gate_up", 24576, 4096), Layer("down", 4096, 12288))
# hidden 5120, 64 q / 8 kv heads of dim 128, FFN 25600
DENSE_32B = (Layer("qkv", 10240, 5120), Layer("o", 5120, 8192),
             Layer("gate_up", 51200, 5120), Layer("down", 5120, 25600))

TINY = Layer("tiny", 1024, 512)
TINY_M = 4

WORKLOADS = {
    "tiny_w8a8_int8": (W8A8_INT8, (TINY,), (TINY_M,)),
    "fp8_dynamic_hidden2048": (FP8_DYNAMIC, SMALL_DENSE, TUNED_M),
    "w8a8_int8_hidden4096": (W8A8_INT8, DENSE_8B, TUNED_M),
    "block_fp8_hidden5120": (BLOCK_FP8, DENSE_32B, TUNED_M),
}


def _to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (nearest, ties to even); finite inputs only."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = 0x7FFF + ((u >> 16) & 1)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to fp32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _outlier_mask(rng: np.random.Generator, K: int, fmt: int) -> np.ndarray:
    scale = np.ones(K, dtype=np.float32)
    if fmt == BLOCK_FP8:
        groups = K // 128
        n_out = max(1, math.ceil(0.01 * groups))
        idx = rng.choice(groups, size=n_out, replace=False)
        for g in idx:
            scale[g * 128:(g + 1) * 128] = 20.0
    else:
        n_out = math.ceil(0.01 * K)
        idx = rng.choice(K, size=n_out, replace=False)
        scale[idx] = 20.0
    return scale


def weights(fmt: int, N: int, K: int) -> np.ndarray:
    """fp32 master weights [N, K], N(0, 0.02)."""
    rng = np.random.default_rng([0, fmt, N, K, 0])
    return rng.normal(0.0, 0.02, size=(N, K)).astype(np.float32)


def activations(fmt: int, N: int, K: int, M: int, outliers: bool = True) -> np.ndarray:
    """bfloat16 activations [M, K] as uint16 bit patterns."""
    rng = np.random.default_rng([0, fmt, N, K, 1, M])
    x = rng.normal(0.0, 1.0, size=(M, K)).astype(np.float32)
    if outliers:
        x = x * _outlier_mask(rng, K, fmt)[None, :]
    return _to_bf16_bits(x)


def tiny_case():
    """The tiny int8 linear: M=4, K=512, N=1024, seed 0, no outliers."""
    rng = np.random.default_rng(0)
    w = rng.normal(0.0, 0.02, size=(TINY.N, TINY.K)).astype(np.float32)
    x = rng.normal(0.0, 1.0, size=(TINY_M, TINY.K)).astype(np.float32)
    return _to_bf16_bits(x), w


def random_bf16(shape, seed: int, std: float = 1.0) -> np.ndarray:
    """Plain N(0, std) bfloat16 bit patterns for edge-case tests."""
    rng = np.random.default_rng(seed)
    return _to_bf16_bits(rng.normal(0.0, std, size=shape).astype(np.float32))


def random_weights(N: int, K: int, seed: int, std: float = 0.02) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.normal(0.0, std, size=(N, K)).astype(np.float32)


# A mixture-of-experts layer of the 30B-class, 3B-active shape (hidden 2048,
# 128 experts of width 768, top-8 routing): the grouped product's workload.
# The pages name MoE layers as the next target ("Building a High-Performance
# and Portable vLLM Linear Backend with Helion", section "Future work", its
# model-coverage paragraph); they give no MoE shapes, so this is a
# representative one.
MOE_EXPERTS = 128
MOE_TOPK = 8
MOE_LAYERS = (Layer("expert_gate_up", 1536, 2048), Layer("expert_down", 2048, 768))
MOE_TOKENS = TUNED_M


def moe_routing(T: int, E: int, topk: int, seed: int):
    """Synthetic top-k routing of T tokens to E experts (each token picks topk
    distinct experts uniformly at random; rng = default_rng([2, T, E, topk,
    seed])).  Returns (offsets int32 [E + 1], rows int32 [T * topk]): group e
    owns rows offsets[e] .. offsets[e+1] - 1, and grouped row i holds token
    rows[i]'s activations.  Rows are ordered by expert, then token."""
    rng = np.random.default_rng([2, T, E, topk, seed])
    pairs = [(int(e), t) for t in range(T) for e in rng.choice(E, size=topk, replace=False)]
    pairs.sort()
    counts = np.bincount([e for e, _ in pairs], minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return offsets, np.array([t for _, t in pairs], dtype=np.int32)


def grouped_algorithmic_bytes(fmt: int, offsets, N: int, K: int) -> int:
    """Bytes a perfect grouped product moves: the weights and scales of the
    groups that have rows, and every row's codes, scales and bf16 output."""
    offsets = np.asarray(offsets)
    active = int(np.count_nonzero(np.diff(offsets)))
    rows = int(offsets[-1])
    wsc = 4 * (N // 128) * (K // 128) if fmt == BLOCK_FP8 else 4 * N
    asc = 4 * rows * (K // 128) if fmt == BLOCK_FP8 else 4 * rows
    return active * (N * K + wsc) + rows * K + asc + 2 * rows * N


def algorithmic_bytes(fmt: int, M: int, N: int, K: int) -> int:
    """Bytes a perfect GEMM moves: W, its scales, quantized A, its scales, bf16 Y."""
    if fmt == BLOCK_FP8:
        wsc = 4 * (N // 128) * (K // 128)
        asc = 4 * M * (K // 128)
    else:
        wsc = 4 * N
        asc = 4 * M
    return N * K + wsc + M * K + asc + 2 * M * N


def quant_bytes(fmt: int, M: int, K: int) -> int:
    """Bytes the activation quantizer moves: bf16 in, 8-bit codes and scales out."""
    asc = 4 * M * (K // 128) if fmt == BLOCK_FP8 else 4 * M
    return 2 * M * K + M * K + asc


def flops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K
