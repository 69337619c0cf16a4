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


def test_moe_routing_is_top_k_of_distinct_experts():
    for T, E, k, seed in ((1, 128, 8, 0), (7, 16, 3, 1), (32, 128, 8, 2)):
        offsets, rows = wl.moe_routing(T, E, k, seed)
        assert offsets.dtype == np.int32 and rows.dtype == np.int32
        assert offsets[0] == 0 and offsets[-1] == T * k and np.all(np.diff(offsets) >= 0)
        assert np.array_equal(np.bincount(rows, minlength=T), np.full(T, k))   # k experts per token
        for e in range(E):
            grp = rows[offsets[e]:offsets[e + 1]]
            assert len(set(grp.tolist())) == len(grp) and np.all(np.diff(grp) > 0)   # distinct, by token
        o2, r2 = wl.moe_routing(T, E, k, seed)
        assert np.array_equal(o2, offsets) and np.array_equal(r2, rows)


def test_grouped_bytes_count_active_groups_only():
    offsets = np.array([0, 2, 2, 5, 5], dtype=np.int32)        # groups 0 and 2 active, 5 rows
    N, K = 256, 512
    b = wl.grouped_algorithmic_bytes(wl.FP8_DYNAMIC, offsets, N, K)
    assert b == 2 * (N * K + 4 * N) + 5 * K + 4 * 5 + 2 * 5 * N
    bb = wl.grouped_algorithmic_bytes(wl.BLOCK_FP8, offsets, N, K)
    assert bb == 2 * (N * K + 4 * 2 * 4) + 5 * K + 4 * 5 * 4 + 2 * 5 * N
