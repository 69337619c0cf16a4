"""GPU activation quantization against the oracle on every (amax, x) pair of
positive finite bf16 values with x <= amax.

A code is the correctly rounded fp32 quotient x / s, s = amax / qmax,
rounded to the format ("Building a High-Performance and Portable vLLM Linear
Backend with Helion", section "Scope": per-token dynamic scales, and 1 x 128
groups for the block format; the rounding rule is the oracle's).  The
kernels form that quotient from a reciprocal and two residual corrections,
so they equal the division only if the corrections are right everywhere.
Activations are bf16, so for one amax the bf16 values x <= amax are the
whole input domain.  This sweeps all of them, 5.3e8 magnitude pairs per
format and sign:
- per-token formats: one row per amax a, holding every positive bf16 value
  up to a (a is then the row's amax), zero-padded;
- block format: groups of 128 holding a and up to 127 of the values below it;
and the same rows negated.  Codes and the fp32 scale bits must equal the
oracle's byte for byte.
"""
import numpy as np
import pytest
import torch

import oracle
import skinny_bit_gemm_amd as q
import workloads as wl

pytestmark = pytest.mark.gpu

from _gpu import as_u8, gpu_quant_act  # noqa: E402

P = 0x7F7F            # positive finite bf16 bit patterns: 0x0001 .. 0x7F7F
K_TOKEN = 32640       # >= P, a multiple of 128
ROWS = 256            # rows per launch


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.lib()
    oracle.build()


def _compare(fmt, bits, what):
    xq, xs = gpu_quant_act(fmt, bits)
    qo, so = oracle.quant_act(fmt, bits)
    qg = as_u8(xq)
    sg = xs.cpu().numpy().view(np.uint32)
    if not np.array_equal(sg, so.view(np.uint32)):
        i = np.argwhere(sg != so.view(np.uint32))[0]
        pytest.fail(f"{what}: scale differs at {tuple(i)}: gpu {sg[tuple(i)]:#x} oracle {so.view(np.uint32)[tuple(i)]:#x}")
    if not np.array_equal(qg, qo):
        r, c = np.argwhere(qg != qo)[0]
        pytest.fail(f"{what}: code differs at row {r} column {c} (x bits {bits[r, c]:#06x}): "
                    f"gpu {qg[r, c]:#04x} oracle {qo[r, c]:#04x}")


SIGNS = [0, 0x8000]
SIGN_IDS = ["positive", "negative"]


@pytest.mark.parametrize("sign", SIGNS, ids=SIGN_IDS)
@pytest.mark.parametrize("fmt", [wl.FP8_DYNAMIC, wl.W8A8_INT8], ids=["fp8_dynamic", "w8a8_int8"])
def test_every_amax_x_pair_per_token(fmt, sign):
    col = np.arange(K_TOKEN, dtype=np.int32)[None, :]
    for a0 in range(1, P + 1, ROWS):
        a = np.arange(a0, min(a0 + ROWS, P + 1), dtype=np.int32)[:, None]
        bits = np.where(col < a, (col + 1) | sign, 0).astype(np.uint16)   # row r: +-(1 .. a_r), then zeros
        _compare(fmt, bits, f"amax bits {a0:#06x}..{int(a[-1, 0]):#06x} sign {sign:#06x}")


@pytest.mark.parametrize("sign", SIGNS, ids=SIGN_IDS)
def test_every_amax_x_pair_block_groups(sign):
    fmt = wl.BLOCK_FP8
    G = 128
    per_row = K_TOKEN // G              # groups per row
    groups = []
    pending = 0

    def flush(gs):
        n = len(gs)
        rows = -(-n // per_row)
        blk = np.zeros((rows * per_row, G), dtype=np.uint16)
        blk[:n] = np.stack(gs)
        blk[:n] |= np.where(blk[:n] != 0, sign, 0).astype(np.uint16)
        _compare(fmt, blk.reshape(rows, K_TOKEN), f"block groups up to amax bits {int(gs[-1][0]):#06x} sign {sign:#06x}")

    for a in range(1, P + 1):
        xs = np.arange(1, a + 1, dtype=np.uint16)
        n = -(-a // (G - 1))
        g = np.zeros((n, G), dtype=np.uint16)
        g[:, 0] = a                      # the group's amax
        flat = np.zeros(n * (G - 1), dtype=np.uint16)
        flat[:a] = xs
        g[:, 1:] = flat.reshape(n, G - 1)
        groups.extend(g)
        pending += n
        if pending >= ROWS * per_row:
            flush(groups)
            groups, pending = [], 0
    if groups:
        flush(groups)
