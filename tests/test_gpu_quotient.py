"""GPU quantization at the values where the way the quotient is formed
decides the code.

A code is the correctly rounded fp32 quotient x / s rounded to the format
("Building a High-Performance and Portable vLLM Linear Backend with Helion",
section "Scope": dynamic per-token and per-group scales; the rounding rule is
the oracle's).  The kernels form that quotient from a reciprocal and two
residual corrections.  Where x times a once-rounded reciprocal would give
another code (int8 quotients at a tie, e4m3 quotients at a midpoint), the
GPU codes must still equal the oracle's byte for byte, through the
standalone quantize kernels and through the in-kernel quantization of fused
qlin_linear at several wave counts.  The pairs come from the same search the
oracle's own pin uses (tests/_quotient_pairs.py), over more amax values."""
import numpy as np
import pytest
import torch

import oracle
import skinny_bit_gemm_amd as q
import workloads as wl
from _quotient_pairs import quotient_pairs, to_bf16_bits

pytestmark = pytest.mark.gpu

from _gpu import as_u8, gpu_linear, gpu_quant_act, gpu_quant_weight, y_to_numpy  # noqa: E402

FMTS = [wl.FP8_DYNAMIC, wl.W8A8_INT8, wl.BLOCK_FP8]
FMT_IDS = ["fp8_dynamic", "w8a8_int8", "block_fp8"]
QMAX = {wl.FP8_DYNAMIC: 448.0, wl.W8A8_INT8: 127.0, wl.BLOCK_FP8: 448.0}
K = 1024
N = 256


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.lib()
    oracle.build()


def pair_rows(fmt, max_rows=48, seed=2):
    """bf16 activation rows [M, K] built around quotient pairs: per-token
    formats put one amax and its pair values (both signs) in a row, the
    block format one amax and its values in each 128-wide group; the rest
    is zeros, positions shuffled (seeded).  Returns (rows, number of pair
    values placed)."""
    qmax = np.float32(QMAX[fmt])
    encode = None if fmt == wl.W8A8_INT8 else oracle.e4m3_encode
    pairs = quotient_pairs(qmax, encode, n_amax=600, per_amax=16, seed=seed)
    rng = np.random.default_rng(seed)
    run = 128 if fmt == wl.BLOCK_FP8 else K      # values that share one scale
    runs_per_row = K // run
    runs = []
    for a, xs in pairs:
        v = np.zeros(run, dtype=np.float32)
        vals = np.concatenate([[a], xs, -xs])
        v[:vals.size] = vals
        runs.append(rng.permutation(v))
        if len(runs) == max_rows * runs_per_row:
            break
    M = -(-len(runs) // runs_per_row)
    x = np.zeros((M * runs_per_row, run), dtype=np.float32)
    x[:len(runs)] = np.stack(runs)
    placed = sum(2 * xs.size for _, xs in pairs[:len(runs)])
    return to_bf16_bits(x.reshape(M, K)), placed


def reciprocal_codes_differ(fmt, rows):
    """How many elements would get another code from x * fl(1 / s)
    (computed on the CPU from the oracle's scales): the rows really hold
    the discriminating values."""
    _, sa = oracle.quant_act(fmt, rows)
    x = wl.bf16_bits_to_f32(rows)
    s = np.repeat(sa, 128, axis=1) if fmt == wl.BLOCK_FP8 else np.repeat(sa[:, None], K, axis=1)
    live = s > 0
    qd = np.where(live, x / np.where(live, s, 1), 0).astype(np.float32)
    qr = (x * np.where(live, np.float32(1.0) / np.where(live, s, 1), 0)).astype(np.float32)
    if fmt == wl.W8A8_INT8:
        return int(np.count_nonzero(np.rint(qd) != np.rint(qr)))
    return int(np.count_nonzero(oracle.e4m3_encode(qd) != oracle.e4m3_encode(qr)))


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
def test_quotient_pairs_quantize_act(fmt):
    rows, placed = pair_rows(fmt)
    differ = reciprocal_codes_differ(fmt, rows)
    print(f"[quotient] fmt={fmt} rows={rows.shape[0]} pair values={placed} "
          f"reciprocal codes that differ={differ}", flush=True)
    assert differ >= 40, differ            # >= 20 pairs, both signs
    qa, sa = oracle.quant_act(fmt, rows)
    xq, xs = gpu_quant_act(fmt, rows)
    assert np.array_equal(as_u8(xq), qa), "activation codes differ"
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), sa.view(np.uint32)), "scales differ"


def cfg(swap, split, tile_n, waves, k_waves, reduce=0):
    return q.make_config(swap, split, 16, tile_n, waves, k_waves, reduce, 1)


# in-kernel quantization at 8, 6, 4, 3 and 1 waves (the rows spread over
# 512 .. 64 threads), with and without split-K; the token count each
# arrangement can hold (8 register chunks of 8 values per thread)
FUSED = {
    "w8_swap": (cfg(1, 1, 32, 8, 8), 48),
    "w6_std": (cfg(0, 1, 48, 6, 2), 48),
    "w4_swap_split2": (cfg(1, 2, 64, 4, 2), 48),
    "w3_std": (cfg(0, 1, 48, 3, 1), 8),
    "w1_swap_split2": (cfg(1, 2, 16, 1, 1), 2),
}


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("name", list(FUSED))
def test_quotient_pairs_fused_linear(fmt, name):
    c, max_m = FUSED[name]
    rows, _ = pair_rows(fmt)
    rows = rows[:max_m]
    M = rows.shape[0]
    assert q.qlin_validate_config(fmt, M, N, K, c) == 0, (c, M)
    differ = reciprocal_codes_differ(fmt, rows)
    assert differ >= 4, differ
    w = wl.random_weights(N, K, 5)
    qw, sw = oracle.quant_weight(fmt, w)
    qa, sa, ref = oracle.linear(fmt, rows, qw, sw)
    wq, ws = gpu_quant_weight(fmt, w)
    print(f"[quotient-fused] fmt={fmt} {name} M={M} cfg={c} reciprocal codes that differ={differ}", flush=True)
    xq, xs, y = gpu_linear(fmt, rows, wq, ws, N, c)
    assert np.array_equal(as_u8(xq), qa), "activation codes differ"
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), sa.view(np.uint32)), "scales differ"
    ok, worst = oracle.tolerance_ok(y_to_numpy(y), ref)
    assert ok, f"bf16 output outside tolerance (worst ratio {worst:.3g})"
