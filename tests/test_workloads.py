"""Checks of the seeded input generator (CPU only)."""
import math

import numpy as np
import torch

import workloads as wl


def test_deterministic_and_seeded_by_shape():
    a = wl.activations(wl.W8A8_INT8, 4096, 4096, 8)
    b = wl.activations(wl.W8A8_INT8, 4096, 4096, 8)
    c = wl.activations(wl.W8A8_INT8, 4096, 4096, 16)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c[:8])
    w1 = wl.weights(wl.FP8_DYNAMIC, 512, 256)
    w2 = wl.weights(wl.FP8_DYNAMIC, 512, 256)
    assert np.array_equal(w1, w2) and w1.dtype == np.float32 and w1.shape == (512, 256)
    assert abs(float(w1.std()) - 0.02) < 0.001


def test_outlier_channels_and_groups():
    K = 4096
    x = wl.bf16_bits_to_f32(wl.activations(wl.W8A8_INT8, 64, K, 32))
    # outlier channels have ~20x the spread of the rest, the same for all tokens
    std = x.std(axis=0)
    n_out = math.ceil(0.01 * K)
    top = np.argsort(std)[-n_out:]
    assert np.all(std[top] > 8) and np.sum(std > 8) == n_out
    xb = wl.bf16_bits_to_f32(wl.activations(wl.BLOCK_FP8, 128, 5120, 32))
    gstd = xb.reshape(32, 40, 128).std(axis=(0, 2))
    assert np.sum(gstd > 8) == max(1, math.ceil(0.01 * 40))


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    v = rng.normal(0, 3, 100000).astype(np.float32)
    bits = wl._to_bf16_bits(v)
    t = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, t)


def test_tiny_case_and_byte_counts():
    x, w = wl.tiny_case()
    assert x.shape == (4, 512) and w.shape == (1024, 512)
    # algorithmic bytes of the 8B-class o-proj at M=1 and M=32
    assert wl.algorithmic_bytes(wl.W8A8_INT8, 1, 4096, 4096) == 16_805_892
    assert wl.algorithmic_bytes(wl.W8A8_INT8, 32, 4096, 4096) == 17_186_944
    assert wl.algorithmic_bytes(wl.BLOCK_FP8, 32, 51200, 5120) == 265_653_760
