"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: quantized codes and fp32 scales bit-exact; int8 int32 accumulators
bit-exact for every schedule; bf16 outputs within
|y - ref| <= 1e-2 |ref| + 1e-3 max|ref|.  Every schedule runs on row-major
weights and on the same weights packed by qlin_pack_weight, whose outputs
must be bit-identical.
"""
import numpy as np
import pytest
import torch

import oracle
import skinny_bit_gemm_amd as q
import workloads as wl

pytestmark = pytest.mark.gpu

from _gpu import (as_u8, gpu_gemm, gpu_linear, gpu_pack, gpu_quant_act, gpu_quant_weight,  # noqa: E402
                  workspace_for, y_to_numpy)

PACKED_W = q.QLIN_PACKED_WEIGHTS   # weight-layout flag of the format argument

FMTS = [wl.FP8_DYNAMIC, wl.W8A8_INT8, wl.BLOCK_FP8]
FMT_IDS = ["fp8_dynamic", "w8a8_int8", "block_fp8"]


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.lib()
    oracle.build()


def cfg(swap=0, split=1, tile_m=16, tile_n=32, waves=4, k_waves=4, reduce=0, act=0):
    return q.make_config(swap, split, tile_m, tile_n, waves, k_waves, reduce, act)


# schedules every format is checked with: Standard, Swap-AB, Split-K (with
# and without Swap-AB), several tile shapes and wave arrangements
SCHEDULES = {
    "std": cfg(0, 1, 16, 32, 4, 4),
    "swap": cfg(1, 1, 16, 32, 4, 4),
    "std_m32": cfg(0, 1, 32, 32, 4, 4),
    "swap_m32": cfg(1, 1, 32, 64, 4, 2),
    "splitk2": cfg(0, 2, 16, 32, 4, 4),
    "splitk4_swap": cfg(1, 4, 16, 64, 4, 1),
    "splitk16": cfg(1, 16, 32, 16, 2, 2),
    "nw4": cfg(0, 3, 16, 128, 8, 2),
    "nr4": cfg(1, 2, 32, 64, 1, 1),
    "w8k8": cfg(0, 1, 16, 16, 8, 8),
    # 8-row weight sub-tiles (tile_n = 8 x column waves)
    "half8_swap": cfg(1, 1, 16, 8, 1, 1),
    "half8_std_kw4": cfg(0, 1, 16, 8, 4, 4),
    "half16_nw2_split3": cfg(0, 3, 32, 16, 2, 1),
    "half32_nw4_swap_split2": cfg(1, 2, 32, 32, 4, 1),
    # column-wave counts that are not powers of two (N = 512 leaves a
    # partial last tile for each width)
    "odd3_swap": cfg(1, 1, 16, 48, 3, 1),
    "odd6_std_kw2_m32": cfg(0, 1, 32, 96, 6, 2),
    "odd5_half_swap_split2": cfg(1, 2, 16, 40, 5, 1),
    "odd7_std_split3": cfg(0, 3, 16, 224, 7, 1),
    "odd3_half_std_kw2_m32": cfg(0, 1, 32, 24, 6, 2),
    # the large-M kernel: 64- or 128-token tiles of 128 channels, 4 waves
    "big64": cfg(0, 1, 64, 128, 4, 1),
    "big128_split3": cfg(0, 3, 128, 128, 4, 1),
}
# the same with packed-atomic reduction (exact formats only)
PACKED = {
    "packed4_swap": cfg(1, 4, 16, 64, 4, 1, reduce=1),
    "packed16": cfg(1, 16, 32, 16, 2, 2, reduce=1),
    "packed3_nw4": cfg(0, 3, 16, 128, 8, 2, reduce=1),
    "packed2_half8_swap": cfg(1, 2, 16, 8, 2, 2, reduce=1),
    "packed3_half16_std": cfg(0, 3, 32, 16, 2, 1, reduce=1),
    "packed2_odd6_swap": cfg(1, 2, 16, 96, 6, 2, reduce=1),
    "packed3_odd7_half_std": cfg(0, 3, 32, 56, 7, 1, reduce=1),
}

# direct activations (codes quantized beforehand, each wave loading its own
# fragments with the weight slot they multiply, nothing staged in the LDS);
# the block format has them in the Swap-AB roles only
DIRECT = {
    "direct_swap": cfg(1, 1, 16, 32, 4, 4, act=2),
    "direct_std": cfg(0, 1, 16, 32, 4, 4, act=2),
    "direct_swap_m32": cfg(1, 1, 32, 64, 4, 2, act=2),
    "direct_std_m32_odd6_kw2": cfg(0, 1, 32, 96, 6, 2, act=2),
    "direct_split4_swap": cfg(1, 4, 16, 64, 4, 1, act=2),
    "direct_nr4_m32": cfg(1, 2, 32, 64, 1, 1, act=2),
    "direct_half8_swap": cfg(1, 1, 16, 8, 1, 1, act=2),
    "direct_odd5_half_swap_split2": cfg(1, 2, 16, 40, 5, 1, act=2),
    "direct_packed3_nw4": cfg(0, 3, 16, 128, 8, 2, reduce=1, act=2),
}


def _flush():
    import sys
    sys.stdout.flush()


def check_linear(fmt, M, N, K, x, w, sched, tag=""):
    print(f"[case] fmt={fmt} M={M} N={N} K={K} sched={sched} {tag}", flush=True)
    qw_o, sw_o = oracle.quant_weight(fmt, w)
    qa_o, sa_o, ref = oracle.linear(fmt, x, qw_o, sw_o)
    wq, ws = gpu_quant_weight(fmt, w)
    assert np.array_equal(as_u8(wq), qw_o), "weight codes differ"
    assert np.array_equal(ws.cpu().numpy().view(np.uint32), sw_o.view(np.uint32)), "weight scales differ"
    xq, xs = gpu_quant_act(fmt, x)
    assert np.array_equal(as_u8(xq), qa_o), "activation codes differ"
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), sa_o.view(np.uint32)), "activation scales differ"
    c = SCHEDULES[sched] if isinstance(sched, str) else sched
    yt = gpu_gemm(fmt, xq, xs, wq, ws, M, N, K, c)
    y = y_to_numpy(yt)
    ok, worst = oracle.tolerance_ok(y, ref)
    assert ok, f"bf16 output outside tolerance (worst ratio {worst:.3g})"
    # the same schedule on packed weights: the same operands reach the
    # matrix cores, so the output is bit-identical
    wp = gpu_pack(wq, N, K)
    assert torch.equal(gpu_gemm(fmt | PACKED_W, xq, xs, wp, ws, M, N, K, c), yt), "packed weights: outputs differ"
    if fmt == wl.W8A8_INT8:
        _, acc = oracle.gemm(fmt, qa_o, sa_o, qw_o, sw_o, want_acc=True)
        yi = gpu_gemm(fmt, xq, xs, wq, ws, M, N, K, c, out_type=q.QLIN_OUT_I32_ACC).cpu().numpy()
        assert np.array_equal(yi, acc), "int32 accumulators differ"
        yp = gpu_gemm(fmt | PACKED_W, xq, xs, wp, ws, M, N, K, c, out_type=q.QLIN_OUT_I32_ACC).cpu().numpy()
        assert np.array_equal(yp, acc), "packed weights: int32 accumulators differ"
    return y, ref


def test_tiny_w8a8_int8_all_schedules():
    """The tiny int8 linear (M=4, K=512, N=1024, seed 0) under every schedule."""
    x, w = wl.tiny_case()
    for name in SCHEDULES:
        check_linear(wl.W8A8_INT8, 4, 1024, 512, x, w, name, "tiny")


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("sched", list(SCHEDULES))
def test_schedules_match_oracle(fmt, sched):
    M, N, K = 7, 512, 1024
    x = wl.activations(fmt, N, K, M)
    w = wl.random_weights(N, K, 31)
    check_linear(fmt, M, N, K, x, w, sched)


@pytest.mark.parametrize("fmt", [wl.FP8_DYNAMIC, wl.W8A8_INT8], ids=FMT_IDS[:2])
@pytest.mark.parametrize("sched", list(PACKED))
@pytest.mark.parametrize("M", [1, 7, 32])
def test_packed_reduction_matches_oracle(fmt, sched, M):
    N, K = 512, 2048 + 16
    x = wl.activations(fmt, N, K, M) if K % 128 == 0 else wl.random_bf16((M, K), 3)
    w = wl.random_weights(N, K, 32)
    check_linear(fmt, M, N, K, x, w, PACKED[sched])


def direct_ok(fmt, c):
    """Whether a direct-activation schedule exists for the format."""
    return (fmt != wl.BLOCK_FP8 or c.swap_ab == 1) and (c.reduce == 0 or fmt != wl.BLOCK_FP8)


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("name", list(DIRECT))
@pytest.mark.parametrize("M,K", [(1, 1024), (7, 1040), (32, 2048)])
def test_direct_activations_match_oracle(fmt, name, M, K):
    """qlin_gemm and qlin_linear with direct activation loads: every tile
    shape, ragged K (the last block's bytes past K read as zeros), partial
    token tiles (rows past M read out of range) and split-K."""
    c = DIRECT[name]
    if fmt == wl.BLOCK_FP8 and K % 128:
        K += 128 - K % 128
    if not direct_ok(fmt, c):
        assert q.qlin_validate_config(fmt, M, 512, K, c) == q.QLIN_ERR_INVALID_ARG
        return
    N = 512
    x = wl.activations(fmt, N, K, M) if K % 128 == 0 else wl.random_bf16((M, K), 5)
    w = wl.random_weights(N, K, 60 + M)
    check_linear(fmt, M, N, K, x, w, c, "direct")
    check_layer(fmt, M, N, K, x, w, c)


def test_direct_activations_rejected_for_large_m():
    for fmt in FMTS:
        assert q.qlin_validate_config(fmt, 64, 512, 1024, cfg(0, 1, 64, 128, 4, 1, act=2)) == q.QLIN_ERR_INVALID_ARG


def check_layer(fmt, M, N, K, x, w, c, ldx=None):
    """qlin_linear (quantize + GEMM, fused or not) against the oracle."""
    print(f"[layer] fmt={fmt} M={M} N={N} K={K} cfg={c}", flush=True)
    qw_o, sw_o = oracle.quant_weight(fmt, w)
    qa_o, sa_o, ref = oracle.linear(fmt, x, qw_o, sw_o)
    wq, ws = gpu_quant_weight(fmt, w)
    xq, xs, y = gpu_linear(fmt, x, wq, ws, N, c, ldx=ldx)
    assert np.array_equal(as_u8(xq), qa_o), "activation codes differ"
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), sa_o.view(np.uint32)), "activation scales differ"
    ok, worst = oracle.tolerance_ok(y_to_numpy(y), ref)
    assert ok, f"bf16 output outside tolerance (worst ratio {worst:.3g})"
    wp = gpu_pack(wq, N, K)
    xqp, xsp, yp = gpu_linear(fmt | PACKED_W, x, wp, ws, N, c, ldx=ldx)
    assert torch.equal(xqp, xq) and torch.equal(xsp, xs), "packed weights: codes or scales differ"
    assert torch.equal(yp, y), "packed weights: outputs differ"
    if fmt == wl.W8A8_INT8:
        _, acc = oracle.gemm(fmt, qa_o, sa_o, qw_o, sw_o, want_acc=True)
        _, _, yi = gpu_linear(fmt, x, wq, ws, N, c, out_type=q.QLIN_OUT_I32_ACC, ldx=ldx)
        assert np.array_equal(yi.cpu().numpy(), acc), "int32 accumulators differ"
        _, _, yip = gpu_linear(fmt | PACKED_W, x, wp, ws, N, c, out_type=q.QLIN_OUT_I32_ACC, ldx=ldx)
        assert np.array_equal(yip.cpu().numpy(), acc), "packed weights: int32 accumulators differ"


# In-kernel quantization holds the tile's activation rows (8-value chunks,
# whole rows padded to 64 chunks for the per-token formats, the K range for
# the block format) in at most 8 register chunks per thread: 16 rows of
# K = 1536 need 8 waves.
LAYER_CFGS = {
    "fused": cfg(1, 1, 16, 32, 8, 8, act=1),
    "fused_std": cfg(0, 1, 16, 64, 8, 4, act=1),
    "fused_split": cfg(1, 4, 16, 32, 8, 4, act=1),
    "fused_split_std": cfg(0, 3, 16, 16, 8, 8, act=1),
    "fused_nr4": cfg(1, 2, 16, 256, 8, 2, act=1),
    "unfused": cfg(1, 2, 16, 32, 4, 4),
    "fused_half8": cfg(1, 1, 16, 8, 8, 8, act=1),
    "fused_half16_std_split2": cfg(0, 2, 16, 16, 8, 4, act=1),
    "unfused_m32": cfg(0, 2, 32, 64, 4, 2),
}


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("name", list(LAYER_CFGS))
@pytest.mark.parametrize("M", [1, 3, 16])
def test_linear_fused_and_unfused(fmt, name, M):
    N, K = 512, 1536
    x = wl.activations(fmt, N, K, M)
    w = wl.random_weights(N, K, 50 + M)
    check_layer(fmt, M, N, K, x, w, LAYER_CFGS[name])


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
def test_linear_fused_few_waves(fmt):
    """In-kernel quantization with 1 and 2 waves (4 and 8 register chunks
    per thread), and the rejection of a tile whose rows do not fit."""
    N, K = 512, 1536
    for M, c in ((1, cfg(1, 2, 16, 64, 1, 1, act=1)), (3, cfg(1, 1, 16, 32, 2, 2, act=1))):
        x = wl.activations(fmt, N, K, M)
        w = wl.random_weights(N, K, 90 + M)
        check_layer(fmt, M, N, K, x, w, c)
    assert q.qlin_validate_config(fmt, 16, N, K, cfg(1, 2, 16, 64, 1, 1, act=1)) == q.QLIN_ERR_INVALID_ARG


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
def test_linear_fused_packed_stride_and_phases(fmt):
    """Fused quantization with packed reduction and a row stride larger than
    K; unfused with 16 rows x 8192 codes (one 128 KiB stage on this small
    grid), where the fused form is rejected (16 rows of 1024 chunks do not
    fit 8 register chunks per thread)."""
    N, K = 256, 8192
    w = wl.random_weights(N, K, 61)
    red = 1 if fmt != wl.BLOCK_FP8 else 0
    x4 = wl.activations(fmt, N, K, 4)
    check_layer(fmt, 4, N, K, x4, w, cfg(1, 1, 16, 64, 8, 2, act=1), ldx=K + 32)
    check_layer(fmt, 4, N, K, x4, w, cfg(1, 2, 16, 64, 8, 4, reduce=red, act=1), ldx=K + 32)
    x16 = wl.activations(fmt, N, K, 16)
    check_layer(fmt, 16, N, K, x16, w, cfg(1, 1, 16, 32, 4, 2), ldx=K + 32)
    assert q.qlin_validate_config(fmt, 16, N, K, cfg(1, 1, 16, 64, 8, 2, act=1)) == q.QLIN_ERR_INVALID_ARG


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
def test_staging_phases_ragged(fmt):
    """Activation staging over several LDS phases with a shorter last phase,
    ragged token rows (29 of a 32-row tile) and, for the per-token formats,
    a partial last K block (65 K blocks, each row copied in requests of up
    to 8 blocks).  A launch of at most one workgroup per compute unit stages
    up to 150 KiB at a time (29 rows x 65 blocks take 2 phases); a larger
    grid (N = 4352 in 16-row tiles: 272 workgroups) 78 KiB (4 phases)."""
    M = 29
    K = 8320 if fmt == wl.BLOCK_FP8 else 8240
    for N, cs in ((256, (cfg(1, 1, 32, 32, 4, 2), cfg(0, 2, 32, 64, 8, 2))),
                  (4352, (cfg(1, 1, 32, 16, 4, 4), cfg(0, 1, 32, 16, 2, 1)))):
        x = wl.activations(fmt, N, K, M) if K % 128 == 0 else wl.random_bf16((M, K), 17)
        w = wl.random_weights(N, K, 18)
        for c in cs:
            check_layer(fmt, M, N, K, x, w, c)


@pytest.mark.parametrize("fmt", [wl.FP8_DYNAMIC, wl.W8A8_INT8], ids=FMT_IDS[:2])
def test_linear_fused_ragged_k(fmt):
    M, N, K = 5, 256, 1040
    x = wl.random_bf16((M, K), 70)
    w = wl.random_weights(N, K, 71)
    for c in (cfg(1, 1, 16, 32, 4, 4, act=1), cfg(1, 3, 16, 32, 2, 2, reduce=1, act=1)):
        check_layer(fmt, M, N, K, x, w, c)


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
def test_linear_selected_schedule(fmt):
    for M in (1, 4, 24, 200):
        N, K = 512, 2048
        x = wl.activations(fmt, N, K, M)
        w = wl.random_weights(N, K, 80 + M)
        check_layer(fmt, M, N, K, x, w, None)


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("M", [1, 2, 15, 16, 17, 24, 31, 32])
def test_token_counts(fmt, M):
    N, K = 384, 1280
    x = wl.activations(fmt, N, K, M)
    w = wl.random_weights(N, K, 40 + M)
    for sched in ("swap", "std_m32", "splitk4_swap"):
        check_linear(fmt, M, N, K, x, w, sched)


@pytest.mark.parametrize("fmt", [wl.FP8_DYNAMIC, wl.W8A8_INT8], ids=FMT_IDS[:2])
@pytest.mark.parametrize("K", [16, 48, 1040, 2064])
def test_ragged_k(fmt, K):
    """K not a multiple of 128 (per-channel formats): the last block is partial."""
    M, N = 5, 256
    x = wl.random_bf16((M, K), K)
    w = wl.random_weights(N, K, K + 1)
    for sched in ("std", "swap", "splitk2", "splitk16", "nw4", "big64", "big128_split3"):
        check_linear(fmt, M, N, K, x, w, sched, "ragged K")


@pytest.mark.parametrize("fmt", [wl.FP8_DYNAMIC, wl.W8A8_INT8], ids=FMT_IDS[:2])
def test_half_sub_tiles_ragged_n(fmt):
    """8-row weight sub-tiles with N = 368 = 11.5 tiles of 32: the last
    workgroup has two real sub-tiles and two past N; every schedule family."""
    M, N, K = 5, 368, 1024 + 16
    x = wl.random_bf16((M, K), 8)
    w = wl.random_weights(N, K, 9)
    for c in (cfg(1, 1, 16, 32, 4, 1), cfg(0, 1, 16, 32, 4, 1), cfg(1, 3, 16, 32, 4, 1),
              cfg(0, 2, 16, 32, 4, 1, reduce=1), cfg(1, 1, 16, 8, 2, 2)):
        check_linear(fmt, M, N, K, x, w, c, "half sub-tiles, ragged N")


@pytest.mark.parametrize("fmt", [wl.FP8_DYNAMIC, wl.W8A8_INT8], ids=FMT_IDS[:2])
def test_odd_column_waves_ragged_n(fmt):
    """3, 5, 6 and 7 column waves with N = 368: the last workgroup holds
    a partial tile (16- and 8-row sub-tiles, both roles, both reductions)."""
    M, N, K = 6, 368, 1024 + 16
    x = wl.random_bf16((M, K), 12)
    w = wl.random_weights(N, K, 13)
    for c in (cfg(1, 1, 16, 48, 3, 1), cfg(0, 2, 16, 40, 5, 1), cfg(1, 1, 32, 224, 7, 1),
              cfg(0, 1, 16, 24, 3, 1), cfg(1, 3, 16, 96, 6, 2), cfg(0, 2, 16, 112, 7, 1, reduce=1)):
        check_linear(fmt, M, N, K, x, w, c, "odd column waves, ragged N")


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
def test_linear_fused_odd_column_waves(fmt):
    """In-kernel quantization with 192, 320, 384 and 448 threads: the row
    chunks are spread over a thread count that is not a power of two.  At
    K = 1536 (192 chunks of 8 values per row) 3 waves hold 8 rows in their 8
    register chunks per thread, 5 waves 13; 6 and 7 waves hold the whole
    16-row tile.  (The block format quantizes only the split's K range: with
    two splits, 5 waves hold the whole tile too.)  The largest token count
    each one holds is checked, and the next one is rejected."""
    N, K = 512, 1536
    for c, ms, too_many in ((cfg(1, 1, 16, 24, 3, 1, act=1), (1, 8), 9),
                            (cfg(0, 2, 16, 40, 5, 1, act=1), (2, 13), None if fmt == wl.BLOCK_FP8 else 14),
                            (cfg(1, 1, 16, 48, 6, 2, act=1), (3, 16), None),
                            (cfg(0, 1, 16, 56, 7, 1, act=1), (5, 16), None),
                            (cfg(1, 3, 16, 224, 7, 1, act=1), (1, 23), None)):
        for M in ms:
            assert q.qlin_validate_config(fmt, M, N, K, c) == 0, (c, M)
            x = wl.activations(fmt, N, K, M)
            w = wl.random_weights(N, K, 70 + M)
            check_layer(fmt, M, N, K, x, w, c)
        if too_many is not None:
            assert q.qlin_validate_config(fmt, too_many, N, K, c) != 0, (c, too_many)


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
def test_ragged_n_tiles(fmt):
    """N not a multiple of tile_n: the last workgroup has empty sub-tiles."""
    M, N, K = 3, 384, 512
    x = wl.random_bf16((M, K), 5)
    w = wl.random_weights(N, K, 6)
    check_linear(fmt, M, N, K, x, w, cfg(1, 2, 16, 256, 4, 1))
    check_linear(fmt, M, N, K, x, w, cfg(0, 1, 16, 256, 8, 2))


# 64-token tiles of the skinny kernel (four 16-token fragments per weight
# block; any layout other than the large-M kernel's 128 x 4 x 1 Standard
# one): at K = 2048 + 16 the 64 staged rows take two to three LDS phases
SKINNY64 = {
    "sk64_std": cfg(0, 1, 64, 32, 4, 4),
    "sk64_swap_nr2_nw2": cfg(1, 1, 64, 64, 2, 1),
    "sk64_swap_split3": cfg(1, 3, 64, 32, 2, 2),
    "sk64_half8_swap": cfg(1, 1, 64, 8, 1, 1),
    "sk64_odd3_std": cfg(0, 1, 64, 48, 3, 1),
}
SKINNY64_PACKED = {
    "sk64_packed2_std": cfg(0, 2, 64, 16, 1, 1, reduce=1),
    # the large-M kernel's layout but the packed reduction: the skinny kernel
    "sk64_packed2_big_layout": cfg(0, 2, 64, 128, 4, 1, reduce=1),
}


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("name", list(SKINNY64) + list(SKINNY64_PACKED))
@pytest.mark.parametrize("M", [50, 64, 100])
def test_skinny_64_token_tiles(fmt, name, M):
    c = SKINNY64.get(name) or SKINNY64_PACKED[name]
    if name in SKINNY64_PACKED and fmt == wl.BLOCK_FP8:
        pytest.skip("packed-atomic reduction: exact formats only")
    N, K = 384, (2048 if fmt == wl.BLOCK_FP8 else 2048 + 16)
    assert q.qlin_validate_config(fmt, M, N, K, c) == 0, (name, c)
    x = wl.activations(fmt, N, K, M)
    w = wl.random_weights(N, K, 100 + M)
    check_linear(fmt, M, N, K, x, w, c, "64-token skinny tiles")


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("M", [33, 64, 100])
def test_large_m(fmt, M):
    N, K = 256, 1024
    x = wl.activations(fmt, N, K, M)
    w = wl.random_weights(N, K, 77)
    check_linear(fmt, M, N, K, x, w, "std_m32")
    check_linear(fmt, M, N, K, x, w, "splitk4_swap")


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
def test_default_selection_matches(fmt):
    M, N, K = 9, 512, 2048
    x = wl.activations(fmt, N, K, M)
    w = wl.random_weights(N, K, 8)
    c = q.qlin_select_variant(fmt, M, N, K)
    check_linear(fmt, M, N, K, x, w, c, "selected")


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
def test_zero_and_outlier_rows(fmt):
    """A zero token (scale 0, exact +0 output), a zero weight channel and a
    token whose amax sits in an outlier group."""
    M, N, K = 4, 256, 512
    x = wl.activations(fmt, N, K, M).copy()
    x[1, :] = 0
    w = wl.random_weights(N, K, 3)
    w[:128 if fmt == wl.BLOCK_FP8 else 1, :] = 0.0
    y, ref = check_linear(fmt, M, N, K, x, w, "swap")
    assert np.all(y[1] == 0) and not np.any(np.signbit(y[1]))
    assert np.all(y[:, 0] == 0)


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
def test_quant_act_strided_and_every_bf16(fmt):
    """Row stride ldx > K, and a sweep over every finite bf16 value."""
    x = wl.activations(fmt, 128, 1024, 6)
    qa_o, sa_o = oracle.quant_act(fmt, x)
    xq, xs = gpu_quant_act(fmt, x, ldx=1024 + 64)
    assert np.array_equal(as_u8(xq), qa_o)
    assert np.array_equal(xs.cpu().numpy(), sa_o)
    # every finite bf16 bit pattern, grouped in rows of 1024
    bits = np.arange(2 ** 16, dtype=np.uint32).astype(np.uint16)
    fin = np.isfinite(wl.bf16_bits_to_f32(bits))
    allv = bits[fin]
    allv = allv[: (allv.size // 1024) * 1024].reshape(-1, 1024)
    qa_o, sa_o = oracle.quant_act(fmt, allv)
    xq, xs = gpu_quant_act(fmt, allv)
    assert np.array_equal(as_u8(xq), qa_o)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), sa_o.view(np.uint32))


@pytest.mark.parametrize("fmt,threads", [(f, t) for f in (wl.FP8_DYNAMIC, wl.W8A8_INT8) for t in (64, 128, 256, 512)]
                         + [(wl.BLOCK_FP8, 64), (wl.BLOCK_FP8, 256)],
                         ids=lambda v: str(v))
def test_quant_act_launch_configs(fmt, threads):
    """Every launch shape of the quantize kernels gives the oracle's codes
    and scales: token counts that leave a workgroup's rows partly empty,
    rows of 1 to 40 chunks per thread (and longer, read twice), a row
    stride larger than K, and every finite bf16 value."""
    from _gpu import check_guards, guarded, to_dev_bf16
    cases = [(1, 1024), (3, 2048), (7, 6144), (33, 4096), (5, 12288), (2, 40960)]
    if fmt == wl.BLOCK_FP8:
        cases = [(1, 1024), (3, 2048), (7, 6144), (33, 5120), (5, 25600)]
    bits = np.arange(2 ** 16, dtype=np.uint32).astype(np.uint16)
    allv = bits[np.isfinite(wl.bf16_bits_to_f32(bits))]
    allv = allv[: (allv.size // 1024) * 1024].reshape(-1, 1024)
    for M, K in cases + [(allv.shape[0], 1024)]:
        x = allv if (M, K) == (allv.shape[0], 1024) else wl.activations(fmt, 128, K, M)
        ldx = K + 64
        padded = np.zeros((M, ldx), dtype=np.uint16)
        padded[:, :K] = x
        xq = guarded((M, K), torch.uint8, 0x55)
        xs = guarded(q.scales_shape(fmt, M, K, False), torch.float32, -1.0)
        print(f"[quant-cfg] fmt={fmt} threads={threads} M={M} K={K}", flush=True)
        q.qlin_quantize_act_cfg(fmt, M, K, to_dev_bf16(padded), ldx, xq, xs, threads)
        torch.cuda.synchronize()
        check_guards(xq, xs, what=f"qlin_quantize_act_cfg threads={threads} M={M} K={K}")
        qa_o, sa_o = oracle.quant_act(fmt, x)
        assert np.array_equal(as_u8(xq), qa_o), (M, K)
        assert np.array_equal(xs.cpu().numpy().view(np.uint32), sa_o.view(np.uint32)), (M, K)


def test_e4m3_conversion_exhaustive_at_unit_scale():
    """Rows whose amax is 448 have scale exactly 1, so the codes are the plain
    fp32 -> E4M3 conversion of every bf16 magnitude up to 448 (and 0x80)."""
    bits = np.arange(0, 0x43E1, dtype=np.uint16)   # +0 .. 448 in bf16
    vals = np.concatenate([bits, bits | np.uint16(0x8000)])
    pad = (-vals.size) % 1023
    vals = np.concatenate([vals, np.zeros(pad, dtype=np.uint16)]).reshape(-1, 1023)
    rows = np.concatenate([vals, np.full((vals.shape[0], 1), 0x43E0, dtype=np.uint16)], axis=1)
    K = 1024
    assert rows.shape[1] == K
    qa_o, sa_o = oracle.quant_act(wl.FP8_DYNAMIC, rows)
    assert np.all(sa_o == 1.0)
    xq, xs = gpu_quant_act(wl.FP8_DYNAMIC, rows)
    assert np.array_equal(as_u8(xq), qa_o)


@pytest.mark.parametrize("fmt,red", [(wl.FP8_DYNAMIC, 0), (wl.W8A8_INT8, 0), (wl.BLOCK_FP8, 0),
                                     (wl.FP8_DYNAMIC, 1), (wl.W8A8_INT8, 1)])
def test_splitk_workspace_left_zero_and_reusable(fmt, red):
    M, N, K = 5, 512, 2048
    c = cfg(1, 8, 16, 32, 4, 2, reduce=red)
    x = wl.activations(fmt, N, K, M)
    w = wl.random_weights(N, K, 12)
    wq, ws = gpu_quant_weight(fmt, w)
    xq, xs = gpu_quant_act(fmt, x)
    work = workspace_for(fmt, M, N, K, c)
    y1 = gpu_gemm(fmt, xq, xs, wq, ws, M, N, K, c, workspace=work)
    assert int(work.count_nonzero()) == 0
    y2 = gpu_gemm(fmt, xq, xs, wq, ws, M, N, K, c, workspace=work)
    assert int(work.count_nonzero()) == 0
    if fmt == wl.W8A8_INT8:
        assert torch.equal(y1, y2)


@pytest.mark.parametrize("fmt,red", [(wl.FP8_DYNAMIC, 0), (wl.W8A8_INT8, 0), (wl.BLOCK_FP8, 0),
                                     (wl.FP8_DYNAMIC, 1), (wl.W8A8_INT8, 1)])
def test_splitk_is_deterministic(fmt, red):
    """Slices are added in partition order and packed partials as exact
    integers, so repeated runs give identical bits whatever order the
    partitions finish in."""
    M, N, K = 24, 1024, 4096
    x = wl.activations(fmt, N, K, M)
    w = wl.random_weights(N, K, 14)
    wq, ws = gpu_quant_weight(fmt, w)
    xq, xs = gpu_quant_act(fmt, x)
    c = cfg(1, 16, 32, 32, 4, 4, reduce=red)
    work = workspace_for(fmt, M, N, K, c)
    first = gpu_gemm(fmt, xq, xs, wq, ws, M, N, K, c, q.QLIN_OUT_F32_ACC, work)
    for _ in range(10):
        again = gpu_gemm(fmt, xq, xs, wq, ws, M, N, K, c, q.QLIN_OUT_F32_ACC, work)
        assert torch.equal(first, again)
    assert int(work.count_nonzero()) == 0


def test_int8_splitk_deterministic_accumulators():
    M, N, K = 32, 1024, 4096
    fmt = wl.W8A8_INT8
    x = wl.activations(fmt, N, K, M)
    w = wl.random_weights(N, K, 13)
    wq, ws = gpu_quant_weight(fmt, w)
    xq, xs = gpu_quant_act(fmt, x)
    nbytes = max(q.qlin_workspace_bytes(fmt, M, N, K, cfg(1, 16, 32, 32, 4, 4, reduce=r)) for r in (0, 1))
    work = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    first = gpu_gemm(fmt, xq, xs, wq, ws, M, N, K, cfg(1, 16, 32, 32, 4, 4), q.QLIN_OUT_I32_ACC, work)
    # one workspace serves both reductions and any shape that fits it
    c = cfg(1, 16, 32, 32, 4, 4, reduce=1)
    for _ in range(20):
        again = gpu_gemm(fmt, xq, xs, wq, ws, M, N, K, c, q.QLIN_OUT_I32_ACC, work)
        assert torch.equal(first, again)


def test_zero_tokens_is_a_no_op():
    fmt = wl.W8A8_INT8
    w = wl.random_weights(256, 512, 1)
    wq, ws = gpu_quant_weight(fmt, w)
    xq = torch.empty((1, 512), dtype=torch.uint8, device="cuda")
    xs = torch.empty((1,), dtype=torch.float32, device="cuda")
    y = torch.full((1, 256), 7, dtype=torch.int16, device="cuda")
    assert q.qlin_gemm(fmt, 0, 256, 512, xq, xs, wq, ws, y) == 0
    assert q.qlin_quantize_act(fmt, 0, 512, y, 512, xq, xs) == 0
    torch.cuda.synchronize()
    assert int((y == 7).sum()) == 256


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("M", [63, 64, 129, 200])
def test_large_m_kernel(fmt, M):
    """The large-M kernel across token-tile tails, a channel tail (N = 384 +
    128 for the block format, 3 or 4 tiles of 128) and split-K."""
    N, K = (512 if fmt == wl.BLOCK_FP8 else 400), 1536
    x = wl.activations(fmt, N, K, M)
    w = wl.random_weights(N, K, 120 + M)
    for c in (cfg(0, 1, 64, 128, 4, 1), cfg(0, 1, 128, 128, 4, 1), cfg(0, 4, 128, 128, 4, 1),
              cfg(0, 2, 64, 128, 4, 1)):
        check_linear(fmt, M, N, K, x, w, c, "large M")
    if fmt != wl.BLOCK_FP8:
        # a ragged last K block (K = 1040: 8 blocks and 16 values)
        K = 1040
        x = wl.random_bf16((M, K), 130 + M)
        w = wl.random_weights(N, K, 140 + M)
        for c in (cfg(0, 1, 64, 128, 4, 1), cfg(0, 3, 128, 128, 4, 1)):
            check_linear(fmt, M, N, K, x, w, c, "large M, ragged K")
