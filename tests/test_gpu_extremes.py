"""GPU parity at the limits the library accepts: the largest int8 K
(133120, where a sum of 127 x 127 products comes within 0.02 % of the int32
range) and the largest fp8 K for packed split-K sums (40960), with saturated
codes so that every product is the largest the format has; at these K the
activation rows also span many LDS staging phases.  Accumulators are
compared with the oracle (int8: int32 sums bit for bit; fp8: the exact sums
are representable in fp32, so the fp32 output mode is the oracle's result
up to the two roundings of the scale products)."""
import numpy as np
import pytest
import torch

import oracle
import skinny_bit_gemm_amd as q
import workloads as wl

pytestmark = pytest.mark.gpu

from _gpu import as_u8, gpu_gemm, gpu_quant_act, gpu_quant_weight, y_to_numpy  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.lib()
    oracle.build()


def saturated(M, N, K):
    """Activations and weights whose every element has the row's (or the
    channel's) largest magnitude, with sign patterns that differ per row and
    channel, so that each code is +-qmax; x as bf16 bits, w as fp32."""
    k = np.arange(K)
    xs = np.ones((M, K), dtype=np.float32)
    xs[1::2] *= np.where(k % 3 == 0, -1.0, 1.0)            # odd rows: mixed signs
    ws = np.full((N, K), 0.02, dtype=np.float32)
    ws[1::2] *= np.where(k % 5 == 0, -1.0, 1.0)             # odd channels: mixed signs
    x_bits = (xs.view(np.uint32) >> 16).astype(np.uint16)   # 1.0 is exact in bf16
    return x_bits, ws


def cfg(swap, split, reduce=0):
    return q.make_config(swap, split, 16, 32, 4, 2, reduce, 0)


@pytest.mark.parametrize("name,c", [("table", None), ("std", cfg(0, 1)), ("swap", cfg(1, 1)),
                                    ("split4_packed", cfg(1, 4, 1)), ("split8_slices", cfg(0, 8, 0))])
def test_int8_largest_k_saturated(name, c):
    fmt, M, N, K = wl.W8A8_INT8, 2, 32, 133_120
    x, w = saturated(M, N, K)
    qa, sa = oracle.quant_act(fmt, x)
    qw, sw = oracle.quant_weight(fmt, w)
    assert np.all(np.abs(qa.view(np.int8).astype(int)) == 127) and np.all(np.abs(qw.view(np.int8).astype(int)) == 127)
    _, acc = oracle.gemm(fmt, qa, sa, qw, sw, want_acc=True)
    assert acc.max() == 127 * 127 * K                      # the largest sum the format can reach here
    xq, xs = gpu_quant_act(fmt, x)
    wq, wsd = gpu_quant_weight(fmt, w)
    assert np.array_equal(as_u8(xq), qa) and np.array_equal(as_u8(wq), qw)
    print(f"[extremes] int8 K={K} schedule={name}", flush=True)
    y = gpu_gemm(fmt, xq, xs, wq, wsd, M, N, K, c, out_type=q.QLIN_OUT_I32_ACC)
    assert np.array_equal(y.cpu().numpy(), acc)


@pytest.mark.parametrize("name,c", [("table", None), ("split4_packed", cfg(1, 4, 1)), ("split2_packed_std", cfg(0, 2, 1))])
def test_fp8_largest_packed_k_saturated(name, c):
    fmt, M, N, K = wl.FP8_DYNAMIC, 2, 32, 40_960
    x, w = saturated(M, N, K)
    qa, sa = oracle.quant_act(fmt, x)
    qw, sw = oracle.quant_weight(fmt, w)
    assert np.all((qa & 0x7F) == 0x7E) and np.all((qw & 0x7F) == 0x7E)   # every code is +-448
    # the oracle's exact sums: multiples of 448^2 = 49 * 2^12, at most 40960
    # of them, so integers below 2^24 times a power of two (exact in fp32);
    # the largest has every product positive
    acc = oracle.acc_fp8(qa, qw)
    assert np.abs(acc).max() == 448.0 * 448.0 * K
    ref = oracle.gemm(fmt, qa, sa, qw, sw)
    xq, xs = gpu_quant_act(fmt, x)
    wq, wsd = gpu_quant_weight(fmt, w)
    assert np.array_equal(as_u8(xq), qa) and np.array_equal(as_u8(wq), qw)
    print(f"[extremes] fp8 K={K} schedule={name}", flush=True)
    y = gpu_gemm(fmt, xq, xs, wq, wsd, M, N, K, c, out_type=q.QLIN_OUT_F32_ACC)
    got = y.cpu().numpy().astype(np.float64)
    # the exact sum times s_a and s_w in fp32: two roundings at most
    assert np.allclose(got, ref, rtol=3e-7, atol=0), np.max(np.abs(got - ref) / np.abs(ref))
    # and the bf16 product within the acceptance bound
    yb = gpu_gemm(fmt, xq, xs, wq, wsd, M, N, K, c)
    ok, worst = oracle.tolerance_ok(y_to_numpy(yb), ref)
    assert ok, worst
