"""qlin_linear_scratch (the layer with the library's static per-GPU split-K
workspace, for callers that cannot allocate) against qlin_linear with a
caller-allocated workspace: the same schedule must give the same codes,
scales and outputs, and the oracle's.  Two calls in a row, the second with a
smaller input, for every format and both split-K reductions; then a second
round in the other order, so the scratch array is reused by calls of
different shapes."""
import numpy as np
import pytest
import torch

import oracle
import skinny_bit_gemm_amd as q
import workloads as wl

pytestmark = pytest.mark.gpu

from _gpu import (as_u8, base_fmt, check_guards, gpu_linear, gpu_pack, gpu_quant_weight, guarded,  # noqa: E402
                  out_dtype, to_dev_bf16, y_to_numpy)

FMTS = [wl.FP8_DYNAMIC, wl.W8A8_INT8, wl.BLOCK_FP8]
FMT_IDS = ["fp8_dynamic", "w8a8_int8", "block_fp8"]


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.lib()
    oracle.build()


def scratch_linear(fmt, x_bits, wq, ws, N, cfg, out_type=q.QLIN_OUT_BF16):
    M, K = x_bits.shape
    xd = to_dev_bf16(x_bits)
    xq = guarded((M, K), torch.uint8, 0x55)
    xs = guarded(q.scales_shape(base_fmt(fmt), M, K, False), torch.float32, -1.0)
    y = guarded((M, N), out_dtype(out_type), -1)
    q.qlin_linear_scratch(fmt, M, N, K, xd, K, xq, xs, wq, ws, y, out_type, cfg)
    torch.cuda.synchronize()
    check_guards(xq, xs, y, what=f"qlin_linear_scratch fmt={fmt} M={M} N={N} K={K} cfg={cfg}")
    return xq, xs, y


# (M, N, K, schedule): a larger call, then a smaller one; slices or packed
# sums, Swap-AB and Standard, fused and unfused
def cases(fmt, reduce):
    big = (24, 1024, 4096, q.make_config(1, 8, 32, 32, 4, 4, reduce, 0))
    small = (5, 512, 2048, q.make_config(0, 4, 16, 64, 4, 2, reduce, 1))
    return [big, small]


def check_pair(fmt, M, N, K, c, seed):
    x = wl.activations(fmt, N, K, M)
    w = wl.random_weights(N, K, seed)
    qw, sw = oracle.quant_weight(fmt, w)
    qa, sa, ref = oracle.linear(fmt, x, qw, sw)
    wq, ws = gpu_quant_weight(fmt, w)
    print(f"[no-alloc] fmt={fmt} M={M} N={N} K={K} cfg={c} scratch bytes needed="
          f"{q.qlin_workspace_bytes(fmt, M, N, K, c)}", flush=True)
    xq0, xs0, y0 = gpu_linear(fmt, x, wq, ws, N, c)           # caller's workspace
    xq1, xs1, y1 = scratch_linear(fmt, x, wq, ws, N, c)       # the static scratch
    assert np.array_equal(as_u8(xq1), qa), "codes differ from the oracle's"
    assert np.array_equal(xs1.cpu().numpy().view(np.uint32), sa.view(np.uint32)), "scales differ"
    assert torch.equal(xq0, xq1) and torch.equal(xs0, xs1)
    # both reductions are order-independent: the same schedule gives the same bits
    assert torch.equal(y0, y1), "outputs differ from qlin_linear's"
    ok, worst = oracle.tolerance_ok(y_to_numpy(y1), ref)
    assert ok, f"bf16 output outside tolerance (worst ratio {worst:.3g})"
    # and with the weights packed
    _, _, y2 = scratch_linear(fmt | q.QLIN_PACKED_WEIGHTS, x, gpu_pack(wq, N, K), ws, N, c)
    assert torch.equal(y2, y1), "packed weights: outputs differ"
    if fmt == wl.W8A8_INT8:
        _, acc = oracle.gemm(fmt, qa, sa, qw, sw, want_acc=True)
        _, _, yi = scratch_linear(fmt, x, wq, ws, N, c, q.QLIN_OUT_I32_ACC)
        assert np.array_equal(yi.cpu().numpy(), acc), "int32 accumulators differ"


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("reduce", [0, 1], ids=["slices", "packed"])
def test_scratch_matches_workspace_entry(fmt, reduce):
    if fmt == wl.BLOCK_FP8 and reduce == 1:
        pytest.skip("packed sums are for the exact formats")
    cs = cases(fmt, reduce)
    for i, (M, N, K, c) in enumerate(cs + cs[::-1]):
        assert 0 < q.qlin_workspace_bytes(fmt, M, N, K, c) <= q.QLIN_SCRATCH_BYTES
        check_pair(fmt, M, N, K, c, 100 + i)


def test_scratch_table_schedules_and_no_split():
    """The table's schedule (split or not) and a forced unsplit one."""
    fmt, N, K = wl.W8A8_INT8, 4096, 12288
    for M, c in ((24, None), (3, q.make_config(1, 1, 16, 32, 4, 4, 0, 0))):
        check_pair(fmt, M, N, K, c, 7 + M)


def test_scratch_rejects_oversized_schedule():
    fmt, M, N, K = wl.FP8_DYNAMIC, 32, 8192, 8192
    c = q.make_config(1, 16, 32, 64, 4, 2, 0, 0)          # 16 slices of 32 x 8192 fp32
    assert q.qlin_workspace_bytes(fmt, M, N, K, c) > q.QLIN_SCRATCH_BYTES
    x = torch.zeros((M, K), dtype=torch.int16, device="cuda")
    xq = torch.zeros((M, K), dtype=torch.uint8, device="cuda")
    xs = torch.zeros((M,), dtype=torch.float32, device="cuda")
    w = torch.zeros((N, K), dtype=torch.uint8, device="cuda")
    ws = torch.zeros((N,), dtype=torch.float32, device="cuda")
    y = guarded((M, N), torch.int16, 7)
    st = q.qlin_linear_scratch(fmt, M, N, K, x, K, xq, xs, w, ws, y, q.QLIN_OUT_BF16, c, raise_on_error=False)
    torch.cuda.synchronize()
    assert st == q.QLIN_ERR_WORKSPACE
    assert int((y != 7).sum()) == 0
    check_guards(y, what="rejected call")
