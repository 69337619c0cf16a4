"""Pins for the oracle's activation and weight quantization (CPU only).

Formats: "Building a High-Performance and Portable vLLM Linear Backend with
Helion", section "Scope".  Pinned by hand-worked rows (tests/golden), and by
properties the definition fixes whatever the implementation: the element of
largest magnitude maps to +-qmax, scaling by a power of two scales only the
scale, odd symmetry, monotonicity, the per-element dequantization error
bound, zero runs, and group/block locality.
"""
import os

import numpy as np
import pytest

import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FMTS = [wl.FP8_DYNAMIC, wl.W8A8_INT8, wl.BLOCK_FP8]
QMAX = {wl.FP8_DYNAMIC: 448.0, wl.W8A8_INT8: 127.0, wl.BLOCK_FP8: 448.0}


def _f32_to_bf16_exact(vals):
    v = np.asarray(vals, dtype=np.float32)
    bits = v.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0), "fixture value not exactly bf16"
    return (bits >> 16).astype(np.uint16)


def _dequant(orc, fmt, q):
    if fmt == wl.W8A8_INT8:
        return q.view(np.int8).astype(np.float64)
    return orc.e4m3_decode(q)


def _spacing_e4m3(a):
    """Grid spacing of E4M3 around magnitude a (2^-9 below 2^-6)."""
    a = np.maximum(np.abs(a), 2.0 ** -6)
    return 2.0 ** (np.floor(np.log2(a)) - 3)


def test_golden_rows(orc):
    with open(os.path.join(GOLDEN, "quant_rows_hand.txt")) as f:
        rows = [l for l in f if l.strip() and not l.startswith("#")]
    assert len(rows) == 5
    for line in rows:
        fmt_s, xs, sc, codes = [p.strip() for p in line.split("|")]
        fmt = wl.FORMAT_IDS[fmt_s]
        x = _f32_to_bf16_exact([float(t) for t in xs.split()])[None, :]
        q, s = orc.quant_act(fmt, x)
        assert s.tolist() == [float(sc)], line
        if fmt == wl.W8A8_INT8:
            want = [int(c) for c in codes.split()]
            assert q.view(np.int8)[0].tolist() == want, line
        else:
            want = [int(c, 16) for c in codes.split()]
            assert q[0].tolist() == want, line


@pytest.mark.parametrize("fmt", FMTS)
def test_amax_maps_to_qmax_and_scale_definition(orc, fmt):
    x = wl.activations(fmt, 256, 1024, 6)
    q, s = orc.quant_act(fmt, x)
    xf = wl.bf16_bits_to_f32(x).astype(np.float64)
    deq = _dequant(orc, fmt, q)
    if fmt == wl.BLOCK_FP8:
        xg = xf.reshape(6, 8, 128)
        qg = deq.reshape(6, 8, 128)
        amax = np.abs(xg).max(axis=2)
        assert s.shape == (6, 8)
        # scale is the fp32 quotient amax / qmax
        assert np.array_equal(s, (amax.astype(np.float32) / np.float32(448.0)).astype(np.float32))
        idx = np.abs(xg).argmax(axis=2)
        top = np.take_along_axis(qg, idx[..., None], axis=2)[..., 0]
        assert np.all(np.abs(top) == 448.0)
    else:
        amax = np.abs(xf).max(axis=1)
        assert np.array_equal(s, (amax.astype(np.float32) / np.float32(QMAX[fmt])))
        idx = np.abs(xf).argmax(axis=1)
        top = deq[np.arange(6), idx]
        assert np.all(np.abs(top) == QMAX[fmt])
        assert np.all(np.sign(top) == np.sign(xf[np.arange(6), idx]))


@pytest.mark.parametrize("fmt", FMTS)
def test_dequant_error_bound(orc, fmt):
    """|q * s - x| <= s * (half the grid spacing at x/s) plus fp32-division slack."""
    M, K = 8, 2048
    x = wl.activations(fmt, 512, K, M)
    q, s = orc.quant_act(fmt, x)
    xf = wl.bf16_bits_to_f32(x).astype(np.float64)
    deq = _dequant(orc, fmt, q)
    if fmt == wl.BLOCK_FP8:
        sf = np.repeat(s.astype(np.float64), 128, axis=1)
    else:
        sf = np.repeat(s.astype(np.float64)[:, None], K, axis=1)
    err = np.abs(deq * sf - xf)
    t = np.abs(xf) / sf
    if fmt == wl.W8A8_INT8:
        bound = sf * (0.5 + 2.0 ** -17)
    else:
        bound = sf * (_spacing_e4m3(t) / 2 + 448 * 2.0 ** -24)
    assert np.all(err <= bound)
    # the bound is tight: some element uses more than 80 % of it
    assert np.max(err / bound) > 0.8


@pytest.mark.parametrize("fmt", FMTS)
def test_power_of_two_invariance_and_odd_symmetry(orc, fmt):
    x = wl.activations(fmt, 128, 512, 4)
    q, s = orc.quant_act(fmt, x)
    xf = wl.bf16_bits_to_f32(x)
    for j in (-3, 1, 5):
        x2 = (xf * np.float32(2.0 ** j)).view(np.uint32) >> 16
        q2, s2 = orc.quant_act(fmt, x2.astype(np.uint16))
        assert np.array_equal(q2, q)
        assert np.array_equal(s2, s * np.float32(2.0 ** j))
    xn = (x ^ np.uint16(0x8000)).astype(np.uint16)
    qn, sn = orc.quant_act(fmt, xn)
    assert np.array_equal(sn, s)
    assert np.array_equal(_dequant(orc, fmt, qn), -_dequant(orc, fmt, q))


@pytest.mark.parametrize("fmt", FMTS)
def test_monotone_within_a_scale_run(orc, fmt):
    x = wl.activations(fmt, 64, 1024, 3)
    q, s = orc.quant_act(fmt, x)
    xf = wl.bf16_bits_to_f32(x)
    deq = _dequant(orc, fmt, q)
    run = 128 if fmt == wl.BLOCK_FP8 else 1024
    for m in range(3):
        for g in range(0, 1024, run):
            o = np.argsort(xf[m, g:g + run], kind="stable")
            assert np.all(np.diff(deq[m, g:g + run][o]) >= 0)


@pytest.mark.parametrize("fmt", FMTS)
def test_zero_runs_give_zero_scale_and_codes(orc, fmt):
    x = wl.activations(fmt, 64, 512, 3).copy()
    x[1, :] = 0                      # a zero token
    x[2, 128:256] = 0x8000           # a group of negative zeros
    q, s = orc.quant_act(fmt, x)
    if fmt == wl.BLOCK_FP8:
        assert np.all(s[1] == 0) and s[2, 1] == 0 and np.all(s[2, [0, 2, 3]] > 0)
        assert np.all(q[2, 128:256] == 0)
    else:
        assert s[1] == 0 and s[2] > 0
    assert np.all(q[1] == 0)


def test_block_groups_are_local(orc):
    """Changing one 128-group changes only that group's codes and scale."""
    x = wl.activations(wl.BLOCK_FP8, 64, 512, 2).copy()
    q, s = orc.quant_act(wl.BLOCK_FP8, x)
    x2 = x.copy()
    x2[1, 256:384] = wl.random_bf16((128,), 99, std=50.0)
    q2, s2 = orc.quant_act(wl.BLOCK_FP8, x2)
    diff = np.ones((2, 4), dtype=bool)
    diff[1, 2] = False
    assert np.array_equal(s2[diff], s[diff])
    assert s2[1, 2] != s[1, 2]
    mask = np.ones((2, 512), dtype=bool)
    mask[1, 256:384] = False
    assert np.array_equal(q2[mask], q[mask])


@pytest.mark.parametrize("fmt", FMTS)
def test_weight_quant_matches_row_and_block_definitions(orc, fmt):
    N, K = 256, 384
    w = wl.random_weights(N, K, 5)
    w[3, :] = 0.0                                      # a zero channel
    q, s = orc.quant_weight(fmt, w)
    if fmt == wl.BLOCK_FP8:
        assert s.shape == (2, 3)
        for nb in range(2):
            for kb in range(3):
                blk = w[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128]
                assert s[nb, kb] == np.float32(np.abs(blk).max()) / np.float32(448.0)
                # the block's codes depend only on the block
                x = blk.astype(np.float32)
                assert np.abs(_dequant(orc, fmt, q[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128])).max() == 448.0
    else:
        assert s.shape == (N,)
        assert s[3] == 0 and np.all(q[3] == 0)
        amax = np.abs(w).max(axis=1)
        assert np.array_equal(s, amax / np.float32(QMAX[fmt]))
        # weight rows quantize exactly as an activation row of the same values
        xb = (w.view(np.uint32) >> 16).astype(np.uint16)        # truncated to bf16
        wt = wl.bf16_bits_to_f32(xb)
        qa, sa = orc.quant_act(fmt, xb)
        qw2, sw2 = orc.quant_weight(fmt, wt)
        assert np.array_equal(qa, qw2) and np.array_equal(sa, sw2)


def test_nonfinite_input_is_rejected(orc):
    x = wl.activations(wl.W8A8_INT8, 64, 128, 2).copy()
    x[0, 5] = 0x7F80    # +inf
    with pytest.raises(ValueError):
        orc.quant_act(wl.W8A8_INT8, x)


def _f32_nearest(fr):
    """The float32 nearest to a positive rational in float32's normal range
    (ties to the even significand), as an exact Fraction."""
    from fractions import Fraction
    e = fr.numerator.bit_length() - fr.denominator.bit_length()
    if Fraction(2) ** e > fr:
        e -= 1
    if Fraction(2) ** (e + 1) <= fr:
        e += 1
    assert -126 <= e <= 127, "outside float32's normal range"
    unit = Fraction(2) ** (e - 23)             # spacing of 24-bit significands in [2^e, 2^(e+1))
    n, rem = divmod(fr, unit)
    n = int(n)
    if rem * 2 > unit or (rem * 2 == unit and n % 2 == 1):
        n += 1
    return n * unit


def test_codes_come_from_the_ieee_quotient(orc):
    """A code is formed from x / s rounded once to float32, not from x times
    a rounded 1/s.  The two differ in the last bit of the quotient now and
    then, and where that decides a code (a quotient at an int8 tie, or at an
    e4m3 midpoint) the oracle must give the code of the correctly rounded
    quotient, computed here in exact rational arithmetic.  The pairs come
    from a search over bf16 values for those where the two quotients give
    different codes; both formats must meet at least 20 of them."""
    from fractions import Fraction
    from _quotient_pairs import quotient_pairs
    checked = {wl.W8A8_INT8: 0, wl.FP8_DYNAMIC: 0}
    for fmt in checked:
        qmax = np.float32(QMAX[fmt])
        encode = None if fmt == wl.W8A8_INT8 else orc.e4m3_encode
        for a, xsel in quotient_pairs(qmax, encode, n_amax=300, per_amax=8, seed=1):
            row = _f32_to_bf16_exact(np.concatenate([[a], xsel]))[None, :]
            q, sc = orc.quant_act(fmt, row)
            scale = Fraction(float(sc.reshape(-1)[0]))
            assert scale == _f32_nearest(Fraction(float(a)) / Fraction(float(qmax))), (fmt, a)
            for j, x in enumerate(xsel):
                quot = _f32_nearest(Fraction(float(x)) / scale)
                if fmt == wl.W8A8_INT8:
                    n, rem = divmod(quot, 1)
                    n = int(n) + (1 if rem * 2 > 1 or (rem * 2 == 1 and int(n) % 2 == 1) else 0)
                    want = min(n, 127)
                else:
                    want = int(orc.e4m3_encode(np.array([float(quot)], dtype=np.float32))[0])
                got = int(q[0, j + 1]) if fmt != wl.W8A8_INT8 else int(q[0, j + 1].astype(np.int8))
                assert got == want, (fmt, float(a), float(x), got, want)
                checked[fmt] += 1
    assert min(checked.values()) >= 20, checked
