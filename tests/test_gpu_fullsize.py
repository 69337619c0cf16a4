"""GPU parity at the benchmark's full layer sizes, in the configuration the
benchmark times (qlin_linear with the selection table's schedule), and the
crossover sweep above 32 tokens with every schedule forced.

The layers of the three model workloads are compared in full at every token
count, with the weights packed (the benchmark's layout) and row-major:
codes, scales, the whole bf16 output against oracle.gemm (and, for
W8A8_INT8, the whole int32 accumulator array bit for bit).  The crossover
sweep compares whole outputs at 64 tokens and a sample of positions the
oracle computes one by one (corners, tile edges and random positions) above;
there the tolerance's max|ref| is taken over the sampled references, which
is never larger than over the whole output, so the bound is if anything
stricter.  Every output buffer sits between canary bands (tests/_gpu.py)."""
import numpy as np
import pytest
import torch

import oracle
import skinny_bit_gemm_amd as q
import workloads as wl

pytestmark = pytest.mark.gpu

from _gpu import DEV, as_u8, gpu_gemm, gpu_linear, gpu_pack, gpu_quant_weight, to_dev, y_to_numpy  # noqa: E402

PACKED_W = q.QLIN_PACKED_WEIGHTS


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.lib()
    oracle.build()


def sample_positions(M, N, count=1500, seed=0):
    rng = np.random.default_rng(seed)
    ms = [0, M - 1, 0, M - 1] + list(rng.integers(0, M, count))
    ns = [0, 0, N - 1, N - 1] + list(rng.integers(0, N, count))
    # tile and block edges
    for n in (15, 16, 127, 128, N // 2 - 1, N // 2):
        if n < N:
            ms.append(int(rng.integers(0, M)))
            ns.append(n)
    return np.array(ms, dtype=np.int32), np.array(ns, dtype=np.int32)


def check_sampled(fmt, y, qa, sa, qw, sw, M, N, acc_y=None, seed=0):
    ms, ns = sample_positions(M, N, seed=seed)
    if fmt == wl.W8A8_INT8:
        ref, acc = oracle.gemm_sampled(fmt, qa, sa, qw, sw, ms, ns, want_acc=True)
        if acc_y is not None:
            assert np.array_equal(acc_y[ms, ns], acc), "int32 accumulators differ"
    else:
        ref = oracle.gemm_sampled(fmt, qa, sa, qw, sw, ms, ns)
    yv = (y.cpu().numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    ok, worst = oracle.tolerance_ok(yv[ms, ns], ref, float(np.max(np.abs(ref))))
    assert ok, f"outputs outside tolerance (worst ratio {worst:.3g})"


BENCH_SHAPES = [(wl.FP8_DYNAMIC, L) for L in wl.SMALL_DENSE] + \
    [(wl.W8A8_INT8, L) for L in wl.DENSE_8B] + [(wl.BLOCK_FP8, L) for L in wl.DENSE_32B]


def oracle_whole(fmt, qa, sa, qw, sw):
    """(ref, int32 accumulators or None) of the whole product."""
    if fmt == wl.W8A8_INT8:
        return oracle.gemm(fmt, qa, sa, qw, sw, want_acc=True)
    return oracle.gemm(fmt, qa, sa, qw, sw), None


def check_whole(fmt, y, qa, sa, qw, sw, acc_y=None, what="", expected=None):
    """The whole output against oracle.gemm (tolerance with max|ref| over
    the call's whole output), and the int32 accumulators bit for bit.
    `expected` = oracle_whole(...) when already computed."""
    ref, acc = expected if expected is not None else oracle_whole(fmt, qa, sa, qw, sw)
    if acc_y is not None:
        bad = int(np.count_nonzero(acc_y != acc))
        assert bad == 0, f"{what}: {bad} int32 accumulators differ"
    ok, worst = oracle.tolerance_ok(y_to_numpy(y), ref)
    assert ok, f"{what}: outputs outside tolerance (worst ratio {worst:.3g})"


@pytest.mark.parametrize("fmt,layer", BENCH_SHAPES,
                         ids=[f"{wl.FORMAT_NAMES[f]}-{L.name}" for f, L in BENCH_SHAPES])
def test_full_size_layers(fmt, layer):
    N, K = layer.N, layer.K
    print(f"[full] fmt={fmt} {layer.name} N={N} K={K}", flush=True)
    w = wl.weights(fmt, N, K)
    qw, sw = oracle.quant_weight(fmt, w)
    wq, ws = gpu_quant_weight(fmt, w)
    del w
    assert np.array_equal(as_u8(wq), qw), "weight codes differ"
    assert np.array_equal(ws.cpu().numpy().view(np.uint32), sw.view(np.uint32))
    wp = gpu_pack(wq, N, K)          # the layout the benchmark runs
    for M in (1, 2, 4, 7, 16, 24, 32):   # one token count in each tuned bucket
        x = wl.activations(fmt, N, K, M)
        qa, sa = oracle.quant_act(fmt, x)
        print(f"[full]   M={M} schedule={q.qlin_select_variant(fmt, M, N, K)}", flush=True)
        expected = oracle_whole(fmt, qa, sa, qw, sw)
        for layout, (f, wt) in {"packed": (fmt | PACKED_W, wp), "row-major": (fmt, wq)}.items():
            xq, xs, y = gpu_linear(f, x, wt, ws, N, None)       # the table's schedule
            assert np.array_equal(as_u8(xq), qa), f"M={M} {layout}: activation codes differ"
            assert np.array_equal(xs.cpu().numpy().view(np.uint32), sa.view(np.uint32))
            acc_y = None
            if fmt == wl.W8A8_INT8:
                _, _, yi = gpu_linear(f, x, wt, ws, N, None, out_type=q.QLIN_OUT_I32_ACC)
                acc_y = yi.cpu().numpy()
            check_whole(fmt, y, qa, sa, qw, sw, acc_y, what=f"M={M} {layout}", expected=expected)


def forced(fmt, M, N, K):
    """Standard, Swap-AB, Split-K 2..16 (both reductions where allowed), the
    skinny kernel's 64-token tiles, the large-M kernel and the table's pick."""
    tm = 32
    out = {"standard": q.make_config(0, 1, tm, 64, 4, 2), "swap_ab": q.make_config(1, 1, tm, 64, 4, 2)}
    for s in (2, 4, 8, 16):
        out[f"splitk{s}"] = q.make_config(s % 4 == 0, s, tm, 64, 4, 2)
    if fmt != wl.BLOCK_FP8:
        out["splitk4_packed"] = q.make_config(1, 4, tm, 64, 8, 4, 1)
    out["skinny64_swap"] = q.make_config(1, 1, 64, 112, 7, 1)           # 64-token skinny tiles
    out["skinny64_std_split2"] = q.make_config(0, 2, 64, 64, 8, 4)
    out["large_m128"] = q.make_config(0, 1, 128, 128, 4, 1)
    out["large_m64_split2"] = q.make_config(0, 2, 64, 128, 4, 1)
    out["table"] = None
    return out


@pytest.mark.parametrize("fmt", [wl.FP8_DYNAMIC, wl.W8A8_INT8, wl.BLOCK_FP8],
                         ids=["fp8_dynamic", "w8a8_int8", "block_fp8"])
@pytest.mark.parametrize("layer", wl.DENSE_8B, ids=[L.name for L in wl.DENSE_8B])
def test_crossover_sweep_variants(fmt, layer):
    """All three formats on the 8B-class shapes at M = 64 .. 512, every
    schedule forced, against the oracle (whole outputs at 64 tokens, sampled
    outputs above)."""
    N, K = layer.N, layer.K
    print(f"[sweep] fmt={fmt} {layer.name} N={N} K={K}", flush=True)
    w = wl.weights(fmt, N, K)
    qw, sw = oracle.quant_weight(fmt, w)
    wq, ws = gpu_quant_weight(fmt, w)
    del w
    wp = gpu_pack(wq, N, K)
    for M in (64, 128, 256, 512):
        x = wl.activations(fmt, N, K, M)
        qa, sa = oracle.quant_act(fmt, x)
        xq = to_dev(qa)
        xs = to_dev(sa)
        expected = oracle_whole(fmt, qa, sa, qw, sw) if M == 64 else None
        for name, c in forced(fmt, M, N, K).items():
            print(f"[sweep]   M={M} {name} cfg={c}", flush=True)
            y = gpu_gemm(fmt, xq, xs, wq, ws, M, N, K, c)
            acc_y = None
            if fmt == wl.W8A8_INT8:
                acc_y = gpu_gemm(fmt, xq, xs, wq, ws, M, N, K, c, q.QLIN_OUT_I32_ACC).cpu().numpy()
            if M == 64:
                check_whole(fmt, y, qa, sa, qw, sw, acc_y, what=f"M={M} {name}", expected=expected)
            else:
                check_sampled(fmt, y, qa, sa, qw, sw, M, N, acc_y, seed=M + len(name))
            # packed weights: bit-identical to the row-major result
            assert torch.equal(gpu_gemm(fmt | PACKED_W, xq, xs, wp, ws, M, N, K, c), y), f"M={M} {name} packed"
        del xq, xs
