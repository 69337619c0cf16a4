"""hipGraph capture of the decode path (qlin_graph_*): replays equal the
eager result, every replay, with eager work and synchronizations in between;
exact formats are bit-identical across many replays."""
import numpy as np
import pytest
import torch

import oracle
import skinny_bit_gemm_amd as q
import workloads as wl

pytestmark = pytest.mark.gpu

from _gpu import (DEV, as_u8, check_guards, check_workspace, gpu_pack, gpu_quant_weight, guarded,  # noqa: E402
                  to_dev_bf16, workspace_for)

FMTS = [wl.FP8_DYNAMIC, wl.W8A8_INT8, wl.BLOCK_FP8]
FMT_IDS = ["fp8_dynamic", "w8a8_int8", "block_fp8"]


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.lib()


class Layer:
    def __init__(self, fmt, M, N, K, seed, cfg=None, packed=False):
        self.fmt, self.M, self.N, self.K = fmt, M, N, K
        self.x_np = wl.activations(fmt, N, K, M)
        self.w_np = wl.random_weights(N, K, seed)
        self.x = to_dev_bf16(self.x_np)
        self.wq, self.ws = gpu_quant_weight(fmt, self.w_np)
        self.call_fmt = fmt
        if packed:   # weights in the packed layout
            self.wq = gpu_pack(self.wq, N, K)
            self.call_fmt = fmt | q.QLIN_PACKED_WEIGHTS
        self.xq = guarded((M, K), torch.uint8)
        self.xs = guarded(q.scales_shape(fmt, M, K, False), torch.float32)
        self.y = guarded((M, N), torch.int16)
        self.cfg = cfg
        self.work = workspace_for(fmt, M, N, K, cfg)

    def check_guards(self, what):
        """Nothing written around the layer's outputs and workspace, and the
        workspace left zero."""
        check_guards(self.xq, self.xs, self.y, what=what)
        check_workspace(self.work, what=what)

    def run(self, stream):
        q.qlin_linear(self.call_fmt, self.M, self.N, self.K, self.x, self.K, self.xq, self.xs, self.wq,
                      self.ws, self.y, q.QLIN_OUT_BF16, self.cfg, self.work, stream=stream)


def capture(stream, layers):
    q.qlin_graph_begin(stream)
    try:
        for l in layers:
            l.run(stream)
    finally:
        g = q.qlin_graph_end(stream)
    return g


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
def test_graph_replays_equal_eager(fmt):
    cfgs = [None,
            q.make_config(1, 4, 16, 32, 4, 2, 0, 1),               # fused, slice reduction
            q.make_config(0, 3, 32, 64, 4, 4, 0, 0),               # unfused, M tile 32
            q.make_config(1, 8, 16, 64, 4, 4, 1 if fmt != wl.BLOCK_FP8 else 0, 0)]
    layers = [Layer(fmt, M, 512, 2048, 10 + i, c, packed=i % 2 == 1)
              for i, (M, c) in enumerate(zip((1, 5, 24, 16), cfgs))]
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for l in layers:
            l.run(stream)
        torch.cuda.synchronize()
        for l in layers:
            l.check_guards("eager")
        eager = [(l.xq.clone(), l.xs.clone(), l.y.clone()) for l in layers]
        g = capture(stream, layers)
        for rep in range(6):
            for l in layers:           # clobber the outputs between replays
                l.y.fill_(0x7FFF)
                l.xq.fill_(0xAA)
            torch.cuda.synchronize()
            q.qlin_graph_launch(g, stream)
            torch.cuda.synchronize()
            for l, (xq, xs, y) in zip(layers, eager):
                assert torch.equal(l.xq, xq), f"replay {rep}: codes differ"
                assert torch.equal(l.xs, xs), f"replay {rep}: scales differ"
                # every reduction is order-independent, so replays are bit-identical
                assert torch.equal(l.y, y), f"replay {rep}: outputs differ"
                l.check_guards(f"replay {rep}")
            # eager work of the program between replays
            for l in layers[:2]:
                l.run(stream)
            torch.cuda.synchronize()
        q.qlin_graph_destroy(g)
    # and the graph's result is the oracle's
    l = layers[1]
    qw, sw = oracle.quant_weight(fmt, l.w_np)
    qa, sa, ref = oracle.linear(fmt, l.x_np, qw, sw)
    assert np.array_equal(as_u8(l.xq), qa)
    yb = (l.y.cpu().numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    assert oracle.tolerance_ok(yb, ref)[0]


def test_graph_int8_bit_identical_over_100_replays():
    l = Layer(wl.W8A8_INT8, 32, 1024, 4096, 3, q.make_config(1, 16, 32, 32, 4, 4, 1, 0))
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        l.run(stream)
        torch.cuda.synchronize()
        first = l.y.clone()
        g = capture(stream, [l])
        for _ in range(100):
            q.qlin_graph_launch(g, stream)
        torch.cuda.synchronize()
        assert torch.equal(l.y, first)
        l.check_guards("after 100 replays")
        q.qlin_graph_destroy(g)


def test_graph_capture_rejects_the_null_stream():
    with pytest.raises(q.QlinError):
        q.qlin_graph_begin(0)
