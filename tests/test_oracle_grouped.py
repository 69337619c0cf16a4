"""Pins of the oracle's grouped (mixture-of-experts) product.

grouped_gemm is defined as one gemm() per row group; these tests pin the
grouping itself -- which rows go with which weights, empty groups, order --
against facts that hold for any correct grouped product: a single group is
the plain product, a group whose weights are zero gives exactly zero rows
and leaves the others unchanged, and reordering the groups (weights and row
blocks together) reorders the output rows the same way.
"""
import numpy as np
import pytest

import oracle
import workloads as wl

FMTS = [wl.FP8_DYNAMIC, wl.W8A8_INT8, wl.BLOCK_FP8]


def _case(fmt, E, N, K, T, topk, seed):
    offsets, rows = wl.moe_routing(T, E, topk, seed)
    x = wl.random_bf16((T, K), seed + 1)[rows]                  # gathered token rows
    qa, sa = oracle.quant_act(fmt, x)
    qw, sw = zip(*[oracle.quant_weight(fmt, wl.random_weights(N, K, 100 * seed + e)) for e in range(E)])
    return offsets, qa, sa, np.stack(qw), np.stack(sw)


@pytest.mark.parametrize("fmt", FMTS)
def test_one_group_is_the_plain_product(orc, fmt):
    offsets, qa, sa, qw, sw = _case(fmt, 6, 128, 256, 5, 2, 1)
    one = np.array([0, offsets[-1]], dtype=np.int32)
    for e in range(qw.shape[0]):
        ref = oracle.grouped_gemm(fmt, one, qa, sa, qw[e:e + 1], sw[e:e + 1])
        assert np.array_equal(ref, oracle.gemm(fmt, qa, sa, qw[e], sw[e]))


@pytest.mark.parametrize("fmt", FMTS)
def test_zero_expert_gives_zero_rows_only(orc, fmt):
    offsets, qa, sa, qw, sw = _case(fmt, 6, 128, 256, 7, 3, 2)
    ref = oracle.grouped_gemm(fmt, offsets, qa, sa, qw, sw)
    e = int(np.argmax(np.diff(offsets)))                       # a group with rows
    qz, sz = oracle.quant_weight(fmt, np.zeros((128, 256), np.float32))
    qw2, sw2 = qw.copy(), sw.copy()
    qw2[e], sw2[e] = qz, sz
    ref2 = oracle.grouped_gemm(fmt, offsets, qa, sa, qw2, sw2)
    lo, hi = offsets[e], offsets[e + 1]
    assert hi > lo and np.all(ref2[lo:hi] == 0.0)
    keep = np.r_[0:lo, hi:offsets[-1]]
    assert np.array_equal(ref2[keep], ref[keep])
    assert np.any(ref[lo:hi] != 0.0)


@pytest.mark.parametrize("fmt", FMTS)
def test_reordering_groups_reorders_rows(orc, fmt):
    offsets, qa, sa, qw, sw = _case(fmt, 5, 128, 256, 6, 2, 3)
    ref = oracle.grouped_gemm(fmt, offsets, qa, sa, qw, sw)
    perm = np.array([3, 0, 4, 2, 1])
    counts = np.diff(offsets)[perm]
    off2 = np.zeros(6, dtype=np.int32)
    off2[1:] = np.cumsum(counts)
    rows = np.concatenate([np.arange(offsets[e], offsets[e + 1]) for e in perm])
    ref2 = oracle.grouped_gemm(fmt, off2, qa[rows], sa[rows], qw[perm], sw[perm])
    assert np.array_equal(ref2, ref[rows])


def test_empty_groups_and_no_rows(orc):
    fmt = wl.W8A8_INT8
    offsets, qa, sa, qw, sw = _case(fmt, 4, 128, 256, 3, 2, 4)
    # the same rows with empty groups interleaved (their weights are never used)
    E = qw.shape[0]
    off2 = np.repeat(offsets, 2)[1:-1].copy()                  # groups 2e (real), 2e+1 (empty)
    qw2 = np.repeat(qw, 2, axis=0)
    sw2 = np.repeat(sw, 2, axis=0)
    qw2[1::2] = 0xFF                                            # garbage, never read
    ref, acc = oracle.grouped_gemm(fmt, offsets, qa, sa, qw, sw, want_acc=True)
    ref2, acc2 = oracle.grouped_gemm(fmt, off2, qa, sa, qw2, sw2, want_acc=True)
    assert len(off2) == 2 * E and np.array_equal(ref2, ref) and np.array_equal(acc2, acc)
    none = oracle.grouped_gemm(fmt, np.zeros(E + 1, np.int32), qa[:0], sa[:0], qw, sw)
    assert none.shape == (0, 128)
