"""GPU parity of the grouped (mixture-of-experts) product against the oracle.

Bars as for the dense product: codes and scales bit-exact, int8 int32
accumulators bit-exact for every schedule, bf16 outputs within
|y - ref| <= 1e-2 |ref| + 1e-3 max|ref|.  Routing is synthetic top-k
(workloads.moe_routing), with empty groups; the offsets live on the device,
so a captured graph is replayed after the routing changes.
"""
import numpy as np
import pytest
import torch

import oracle
import skinny_bit_gemm_amd as q
import workloads as wl

pytestmark = pytest.mark.gpu

from _gpu import (DEV, as_u8, check_guards, check_workspace, gpu_pack, gpu_quant_act, guarded,  # noqa: E402
                  out_dtype, to_dev, y_to_numpy)

PACKED_W = q.QLIN_PACKED_WEIGHTS

FMTS = [wl.FP8_DYNAMIC, wl.W8A8_INT8, wl.BLOCK_FP8]
FMT_IDS = ["fp8_dynamic", "w8a8_int8", "block_fp8"]


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.lib()
    oracle.build()


def cfg(swap=1, split=1, tile_m=16, tile_n=64, waves=4, k_waves=2, reduce=0, act=0):
    return q.make_config(swap, split, tile_m, tile_n, waves, k_waves, reduce, act)


SCHEDULES = {
    "default": None,
    "std": cfg(0, 1, 16, 32, 4, 4),
    "swap_m32": cfg(1, 1, 32, 64, 4, 2),
    "std_nw4": cfg(0, 1, 16, 128, 8, 2),
    "split2": cfg(1, 2, 16, 64, 4, 2),
    "split3_std": cfg(0, 3, 32, 32, 4, 4),
    "half8": cfg(1, 1, 16, 8, 4, 4),
    "half16_std_split2": cfg(0, 2, 16, 16, 2, 1),
    "odd48_w3": cfg(1, 1, 16, 48, 3, 1),
    "odd96_w6kw2_std_m32": cfg(0, 1, 32, 96, 6, 2),
    "odd40_w5_split2": cfg(1, 2, 16, 40, 5, 1),
    # direct activation loads (no LDS staging): each group's rows start
    # at its own offset, rows past the group read out of range
    "direct_swap": cfg(1, 1, 16, 64, 4, 2, act=2),
    "direct_swap_m32_split2": cfg(1, 2, 32, 64, 4, 2, act=2),
}
PACKED = {"packed2": cfg(1, 2, 16, 64, 4, 2, reduce=1), "packed4_std": cfg(0, 4, 16, 32, 4, 2, reduce=1),
          "packed2_half8": cfg(1, 2, 16, 8, 2, 2, reduce=1), "packed3_odd56_w7": cfg(1, 3, 16, 56, 7, 1, reduce=1)}


def experts(fmt, E, N, K, seed):
    """E quantized experts, [E][N][K] codes and their scales (oracle bytes,
    which the device weight quantizer matches bit for bit)."""
    qw, sw = zip(*[oracle.quant_weight(fmt, wl.random_weights(N, K, seed + e)) for e in range(E)])
    return np.stack(qw), np.stack(sw)


def run(fmt, offsets, xq, xs, wqd, wsd, E, N, K, max_rows, c, out_type=q.QLIN_OUT_BF16):
    total = int(offsets[-1])
    y = guarded((total, N), out_dtype(out_type), -1)    # sentinel: every row must be written
    nb = q.qlin_grouped_workspace_bytes(fmt, E, N, K, total, max_rows, c)
    work = guarded((max(nb, 16),), torch.uint8, 0)
    off = to_dev(offsets.astype(np.int32))
    q.qlin_grouped_gemm(fmt, E, N, K, off, total, max_rows, xq, xs, wqd, wsd, y, out_type, c, work)
    torch.cuda.synchronize()
    what = f"qlin_grouped_gemm fmt={fmt} E={E} N={N} K={K} rows={total} cfg={c}"
    check_guards(y, what=what)
    check_workspace(work, what=what)
    return y


def check_case(fmt, E, N, K, T, topk, seed, c, max_rows=None):
    offsets, rows = wl.moe_routing(T, E, topk, seed)
    x = wl.random_bf16((T, K), seed + 7)[rows]
    xq, xs = gpu_quant_act(fmt, x)
    qa, sa = oracle.quant_act(fmt, x)
    assert np.array_equal(as_u8(xq), qa) and np.array_equal(xs.cpu().numpy().view(np.uint32), sa.view(np.uint32))
    qw, sw = experts(fmt, E, N, K, 1000 * seed)
    wqd, wsd = to_dev(qw), to_dev(sw)
    print(f"[grouped] fmt={fmt} E={E} N={N} K={K} T={T} top{topk} cfg={c}", flush=True)
    max_rows = T if max_rows is None else max_rows
    y = run(fmt, offsets, xq, xs, wqd, wsd, E, N, K, max_rows, c)
    ref = oracle.grouped_gemm(fmt, offsets, qa, sa, qw, sw)
    ok, worst = oracle.tolerance_ok(y_to_numpy(y), ref)
    assert ok, f"bf16 output outside tolerance (worst ratio {worst:.3g})"
    # the experts' weights packed (one matrix after another): bit-identical
    wpd = gpu_pack(wqd, N, K, batch=E)
    assert torch.equal(run(fmt | PACKED_W, offsets, xq, xs, wpd, wsd, E, N, K, max_rows, c), y), "packed weights"
    if fmt == wl.W8A8_INT8:
        _, acc = oracle.grouped_gemm(fmt, offsets, qa, sa, qw, sw, want_acc=True)
        yi = run(fmt, offsets, xq, xs, wqd, wsd, E, N, K, max_rows, c, q.QLIN_OUT_I32_ACC)
        assert np.array_equal(yi.cpu().numpy(), acc), "int32 accumulators differ"
        yip = run(fmt | PACKED_W, offsets, xq, xs, wpd, wsd, E, N, K, max_rows, c, q.QLIN_OUT_I32_ACC)
        assert np.array_equal(yip.cpu().numpy(), acc), "packed weights: int32 accumulators differ"


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("name", list(SCHEDULES))
def test_grouped_schedules_match_oracle(fmt, name):
    # 20 experts, top-3 of 13 tokens: 4 experts empty (the first and the last
    # among them), a ragged channel tile (N = 384 over 64- and 128-column tiles)
    check_case(fmt, 20, 384, 640, 13, 3, 1, SCHEDULES[name])


@pytest.mark.parametrize("fmt", [wl.FP8_DYNAMIC, wl.W8A8_INT8], ids=FMT_IDS[:2])
@pytest.mark.parametrize("name", list(PACKED))
def test_grouped_packed_reduction(fmt, name):
    check_case(fmt, 9, 256, 1024, 6, 2, 2, PACKED[name])


@pytest.mark.parametrize("fmt", [wl.FP8_DYNAMIC, wl.W8A8_INT8], ids=FMT_IDS[:2])
@pytest.mark.parametrize("tile_m", [16, 32])
@pytest.mark.parametrize("act", [0, 2], ids=["staged", "direct"])
def test_grouped_ragged_k_and_many_rows(fmt, tile_m, act):
    # K not a multiple of 128; 40 tokens top-2 of 4 experts: groups of 18 to
    # 25 rows, so several token tiles per group with a ragged last one
    check_case(fmt, 4, 256, 1040, 40, 2, 3, cfg(1, 1, tile_m, 64, 4, 2, act=act))


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("max_rows,c", [(2, None), (5, cfg(1, 1, 16, 64, 4, 2)), (3, cfg(0, 2, 32, 32, 4, 2)),
                                        (7, cfg(1, 2, 32, 64, 4, 2, reduce=1))],
                         ids=["tiles_of_2", "tiles_of_5", "tiles_of_3_split2", "tiles_of_7_packed2"])
def test_grouped_groups_larger_than_max_rows(fmt, max_rows, c):
    """max_group_rows below the largest group (13 tokens top-2 of 3 experts:
    groups of 6 to 11 rows): token tiles of min(tile_m, max_group_rows)
    rows, every row still computed."""
    if fmt == wl.BLOCK_FP8 and c is not None and c.reduce:
        c = cfg(1, 2, 32, 64, 4, 2)
    check_case(fmt, 3, 256, 512, 13, 2, 4, c, max_rows=max_rows)


def test_grouped_graph_replays_follow_new_routing():
    """One captured graph; the offsets buffer (and the rows) change between
    replays, the total row count stays T * topk, as in decode."""
    fmt, E, N, K, T, topk = wl.W8A8_INT8, 16, 256, 512, 6, 2
    qw, sw = experts(fmt, E, N, K, 77)
    wqd, wsd = to_dev(qw), to_dev(sw)
    total = T * topk
    xq = torch.empty((total, K), dtype=torch.uint8, device=DEV)
    xs = torch.empty((total,), dtype=torch.float32, device=DEV)
    off = torch.zeros(E + 1, dtype=torch.int32, device=DEV)
    y = guarded((total, N), torch.int32)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        q.qlin_graph_begin(st)
        q.qlin_grouped_gemm(fmt, E, N, K, off, total, T, xq, xs, wqd, wsd, y, q.QLIN_OUT_I32_ACC, None, None,
                            stream=st)
        g = q.qlin_graph_end(st)
    try:
        for seed in range(4):
            offsets, rows = wl.moe_routing(T, E, topk, seed)
            x = wl.random_bf16((T, K), seed)[rows]
            qa, sa = oracle.quant_act(fmt, x)
            off.copy_(torch.from_numpy(offsets))
            xq.copy_(torch.from_numpy(qa))
            xs.copy_(torch.from_numpy(sa))
            torch.cuda.synchronize()
            q.qlin_graph_launch(g, st)
            st.synchronize()
            _, acc = oracle.grouped_gemm(fmt, offsets, qa, sa, qw, sw, want_acc=True)
            assert np.array_equal(y.cpu().numpy(), acc), f"replay {seed}"
            check_guards(y, what=f"grouped graph replay {seed}")
    finally:
        q.qlin_graph_destroy(g)


MOE_CASES = [(f, L, 4) for f in FMTS for L in wl.MOE_LAYERS] + [(wl.W8A8_INT8, wl.MOE_LAYERS[0], 32),
                                                                (wl.BLOCK_FP8, wl.MOE_LAYERS[1], 32)]


@pytest.mark.parametrize("fmt,layer,T", MOE_CASES,
                         ids=[f"{wl.FORMAT_NAMES[f]}-{L.name}-T{T}" for f, L, T in MOE_CASES])
def test_grouped_moe_layer_shape(fmt, layer, T):
    """The 128-expert top-8 layers at their full shapes, with the default
    schedule; only the active experts' weights are quantized (the others
    stay zero and must not matter)."""
    E, topk, N, K = wl.MOE_EXPERTS, wl.MOE_TOPK, layer.N, layer.K
    offsets, rows = wl.moe_routing(T, E, topk, 5)
    x = wl.activations(fmt, N, K, T)[rows]
    xq, xs = gpu_quant_act(fmt, x)
    qa, sa = oracle.quant_act(fmt, x)
    qw = np.zeros((E, N, K), dtype=np.uint8)
    sw = np.ones((E,) + oracle.scale_shape(fmt, N, K, True), dtype=np.float32)
    active = [e for e in range(E) if offsets[e + 1] > offsets[e]]
    for e in active:   # N(0, 0.02) weights, drawn in float32 (seeded per expert)
        w = np.random.default_rng(9000 + e).standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
        qw[e], sw[e] = oracle.quant_weight(fmt, w)
    print(f"[grouped-moe] fmt={fmt} {layer.name} T={T} active={len(active)}", flush=True)
    wpd = gpu_pack(to_dev(qw), N, K, batch=E)
    y = run(fmt | PACKED_W, offsets, xq, xs, wpd, to_dev(sw), E, N, K, T, None)
    ref = oracle.grouped_gemm(fmt, offsets, qa, sa, qw, sw)
    ok, worst = oracle.tolerance_ok(y_to_numpy(y), ref)
    assert ok and len(active) > 16, (worst, len(active))


def test_grouped_no_rows_is_a_no_op():
    E, N, K = 4, 256, 512
    y = guarded((1, N), torch.int16, -1)
    off = torch.zeros(E + 1, dtype=torch.int32, device=DEV)
    z = torch.zeros((E, N, K), dtype=torch.uint8, device=DEV)
    s = torch.zeros((E, N), dtype=torch.float32, device=DEV)
    q.qlin_grouped_gemm(wl.FP8_DYNAMIC, E, N, K, off, 0, 4, z, s, z, s, y)
    torch.cuda.synchronize()
    assert torch.all(y == -1)
    check_guards(y, what="grouped, no rows")
