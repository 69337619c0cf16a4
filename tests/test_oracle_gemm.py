"""Pins for the oracle's accumulation and dequantized result (CPU only).

Product: "Building a High-Performance and Portable vLLM Linear Backend with
Helion", section "Kernel Implementation" (out = a @ b, every schedule the
same product) with the scales of section "Scope".  Pinned by exact rational
brute force on tiny shapes, by a second exact route (numpy matmul in
int64 / float64 is exact here), by closed forms (zero, one-hot and identity
weights) and by permutation equivariance.
"""
from fractions import Fraction

import numpy as np
import pytest

import workloads as wl

FMTS = [wl.FP8_DYNAMIC, wl.W8A8_INT8, wl.BLOCK_FP8]
QMAX = {wl.FP8_DYNAMIC: 448, wl.W8A8_INT8: 127, wl.BLOCK_FP8: 448}


def _code_value_fraction(fmt, code):
    """Exact rational value of one code (int8 two's complement or E4M3FN)."""
    if fmt == wl.W8A8_INT8:
        return Fraction(int(np.uint8(code).view(np.int8)))
    s = -1 if code & 0x80 else 1
    e, m = (code >> 3) & 15, code & 7
    assert not (e == 15 and m == 7)
    if e == 0:
        return s * Fraction(m, 512)
    return s * Fraction(8 + m, 8) * Fraction(2) ** (e - 7)


def _quantized_case(orc, fmt, M, N, K, seed):
    w = wl.random_weights(N, K, seed)
    x = wl.random_bf16((M, K), seed + 1, std=1.0)
    qw, sw = orc.quant_weight(fmt, w)
    qa, sa = orc.quant_act(fmt, x)
    return qa, sa, qw, sw


def _brute_one(fmt, qa, sa, qw, sw, m, n):
    """Exact rational result of output (m, n) (no rounding anywhere)."""
    K = qa.shape[1]
    va = [_code_value_fraction(fmt, int(c)) for c in qa[m]]
    vw = [_code_value_fraction(fmt, int(c)) for c in qw[n]]
    if fmt == wl.BLOCK_FP8:
        tot = Fraction(0)
        for g in range(K // 128):
            acc = sum(va[k] * vw[k] for k in range(g * 128, (g + 1) * 128))
            tot += acc * Fraction(float(sa[m, g])) * Fraction(float(sw[n // 128, g]))
        return tot
    acc = sum(va[k] * vw[k] for k in range(K))
    return acc * Fraction(float(sa[m])) * Fraction(float(sw[n]))


@pytest.mark.parametrize("fmt,M,N,K,cols", [
    (wl.W8A8_INT8, 3, 5, 128, None), (wl.W8A8_INT8, 2, 4, 256, None),
    (wl.FP8_DYNAMIC, 3, 5, 128, None), (wl.FP8_DYNAMIC, 2, 4, 256, None),
    (wl.BLOCK_FP8, 2, 256, 256, [0, 1, 127, 128, 200, 255]),
])
def test_brute_force_exact_rationals(orc, fmt, M, N, K, cols):
    qa, sa, qw, sw = _quantized_case(orc, fmt, M, N, K, seed=11 + K)
    ref, acc = orc.gemm(fmt, qa, sa, qw, sw, want_acc=True)
    cols = list(range(N)) if cols is None else cols
    for m in range(M):
        for n in cols:
            e = _brute_one(fmt, qa, sa, qw, sw, m, n)
            # per group: exact accumulator times two scales (two fp64 roundings),
            # then one more rounding per group added
            slack = 3 * (K // 128 if fmt == wl.BLOCK_FP8 else 1)
            assert abs(Fraction(ref[m, n]) - e) <= Fraction(slack, 2 ** 53) * max(abs(e), Fraction(1, 2 ** 60)), (m, n)
    if fmt == wl.W8A8_INT8:
        va = qa.view(np.int8).astype(object)
        vw = qw.view(np.int8).astype(object)
        assert np.array_equal(acc, (va @ vw.T).astype(np.int64))


@pytest.mark.parametrize("fmt", [wl.W8A8_INT8, wl.FP8_DYNAMIC])
def test_accumulator_matches_exact_blas(orc, fmt):
    """Products of codes are small integers times 2^-18, so float64 and int64
    matmuls (any summation order) are exact and must agree bit for bit."""
    qa, sa, qw, sw = _quantized_case(orc, fmt, 7, 96, 4096, seed=3)
    if fmt == wl.W8A8_INT8:
        acc = orc.acc_int8(qa, qw)
        want = qa.view(np.int8).astype(np.int64) @ qw.view(np.int8).astype(np.int64).T
        assert np.array_equal(acc.astype(np.int64), want)
        ref = orc.gemm(fmt, qa, sa, qw, sw)
        assert np.array_equal(ref, want.astype(np.float64) * sa.astype(np.float64)[:, None]
                              * sw.astype(np.float64)[None, :])
    else:
        acc = orc.acc_fp8(qa, qw)
        da = orc.e4m3_decode(np.arange(256))[qa]
        dw = orc.e4m3_decode(np.arange(256))[qw]
        assert np.array_equal(acc, da @ dw.T)


def test_block_accumulators_match_exact_blas(orc):
    qa, sa, qw, sw = _quantized_case(orc, wl.BLOCK_FP8, 3, 256, 512, seed=4)
    accg = orc.acc_fp8_groups(qa, qw)
    dec = orc.e4m3_decode(np.arange(256))
    da, dw = dec[qa], dec[qw]
    for g in range(4):
        sl = slice(g * 128, (g + 1) * 128)
        assert np.array_equal(accg[:, :, g], da[:, sl] @ dw[:, sl].T)
    ref = orc.gemm(wl.BLOCK_FP8, qa, sa, qw, sw)
    want = np.zeros((3, 256))
    for g in range(4):
        want += accg[:, :, g] * sa[:, g:g + 1].astype(np.float64) * \
            np.repeat(sw[:, g].astype(np.float64), 128)[None, :]
    assert np.allclose(ref, want, rtol=1e-14, atol=0)


@pytest.mark.parametrize("fmt", FMTS)
def test_zero_weights_give_exact_positive_zero(orc, fmt):
    M, N, K = 3, 256, 256
    qw, sw = orc.quant_weight(fmt, np.zeros((N, K), dtype=np.float32))
    assert np.all(qw == 0) and np.all(sw == 0)
    x = wl.random_bf16((M, K), 2)
    qa, sa, ref = orc.linear(fmt, x, qw, sw)
    assert np.all(ref == 0) and not np.any(np.signbit(ref))


@pytest.mark.parametrize("fmt", [wl.W8A8_INT8, wl.FP8_DYNAMIC])
def test_one_hot_weights_select_a_permuted_channel(orc, fmt):
    """W[n, pi(n)] = c_n: the weight quantizes to +-qmax there, so
    acc[m, n] = +-qmax * qa[m, pi(n)] and ref = c_n * dequant(x)[m, pi(n)]."""
    M, K, N = 4, 256, 200
    rng = np.random.default_rng(8)
    pi = rng.permutation(K)[:N]
    c = rng.choice([-1.0, 1.0], N) * rng.uniform(0.5, 2.0, N)
    w = np.zeros((N, K), dtype=np.float32)
    w[np.arange(N), pi] = c.astype(np.float32)
    qw, sw = orc.quant_weight(fmt, w)
    x = wl.random_bf16((M, K), 9)
    qa, sa, ref = orc.linear(fmt, x, qw, sw)
    dec = (qa.view(np.int8).astype(np.float64) if fmt == wl.W8A8_INT8
           else orc.e4m3_decode(np.arange(256))[qa])
    dequant_x = dec * sa.astype(np.float64)[:, None]
    want = dequant_x[:, pi] * c.astype(np.float32).astype(np.float64)[None, :]
    assert np.allclose(ref, want, rtol=1e-6, atol=0)
    if fmt == wl.W8A8_INT8:
        acc = orc.acc_int8(qa, qw)
        sign = np.sign(c)[None, :]
        assert np.array_equal(acc, (sign * 127 * qa.view(np.int8)[:, pi]).astype(np.int32))


@pytest.mark.parametrize("fmt", FMTS)
def test_identity_weights(orc, fmt):
    """N = K identity: acc[m, n] = qmax * qa[m, n]; the block format's
    off-diagonal blocks are all zero (scale 0) and contribute nothing."""
    M, K = 3, 256
    w = np.eye(K, dtype=np.float32)
    qw, sw = orc.quant_weight(fmt, w)
    if fmt == wl.BLOCK_FP8:
        assert sw[0, 1] == 0 and sw[1, 0] == 0 and sw[0, 0] == np.float32(1 / 448)
    x = wl.random_bf16((M, K), 10)
    qa, sa, ref = orc.linear(fmt, x, qw, sw)
    dec = (qa.view(np.int8).astype(np.float64) if fmt == wl.W8A8_INT8
           else orc.e4m3_decode(np.arange(256))[qa])
    if fmt == wl.BLOCK_FP8:
        want = dec * np.repeat(sa.astype(np.float64), 128, axis=1) * 448 * (np.float32(1) / np.float32(448))
    else:
        want = dec * sa.astype(np.float64)[:, None] * QMAX[fmt] * sw.astype(np.float64)[None, :]
    assert np.allclose(ref, want, rtol=1e-15, atol=0)
    if fmt == wl.W8A8_INT8:
        assert np.array_equal(orc.acc_int8(qa, qw), 127 * qa.view(np.int8).astype(np.int32))


@pytest.mark.parametrize("fmt", FMTS)
def test_permutation_equivariance(orc, fmt):
    M, N, K = 5, 256, 512
    w = wl.random_weights(N, K, 12)
    x = wl.random_bf16((M, K), 13)
    qw, sw = orc.quant_weight(fmt, w)
    qa, sa, ref = orc.linear(fmt, x, qw, sw)
    pm = np.random.default_rng(1).permutation(M)
    _, _, ref_m = orc.linear(fmt, x[pm], qw, sw)
    assert np.array_equal(ref_m, ref[pm])
    # permute whole 128-row blocks for the block format (scales move with them)
    if fmt == wl.BLOCK_FP8:
        blocks = np.array([1, 0])
        pn = (blocks[:, None] * 128 + np.arange(128)[None, :]).ravel()
        qw2, sw2 = orc.quant_weight(fmt, w[pn])
        assert np.array_equal(sw2, sw[blocks])
    else:
        pn = np.random.default_rng(2).permutation(N)
        qw2, sw2 = orc.quant_weight(fmt, w[pn])
        assert np.array_equal(sw2, sw[pn])
    assert np.array_equal(qw2, qw[pn])
    _, _, ref_n = orc.linear(fmt, x, qw2, sw2)
    assert np.array_equal(ref_n, ref[:, pn])


@pytest.mark.parametrize("fmt", FMTS)
def test_sampled_equals_full(orc, fmt):
    qa, sa, qw, sw = _quantized_case(orc, fmt, 6, 384, 512, seed=21)
    ref = orc.gemm(fmt, qa, sa, qw, sw)
    rng = np.random.default_rng(0)
    ms = rng.integers(0, 6, 100)
    ns = rng.integers(0, 384, 100)
    got = orc.gemm_sampled(fmt, qa, sa, qw, sw, ms, ns)
    assert np.array_equal(got, ref[ms, ns])


def test_int8_accumulator_bound_is_checked(orc):
    """127^2 * K must stay below 2^31: the oracle refuses when it would not."""
    K = 133_248           # 127^2 * K > 2^31 - 1
    qa = np.full((1, K), 127, dtype=np.int8).view(np.uint8)
    qw = np.full((1, K), 127, dtype=np.int8).view(np.uint8)
    with pytest.raises(ValueError):
        orc.acc_int8(qa, qw)
    ok = orc.acc_int8(qa[:, :12288], qw[:, :12288])
    assert ok[0, 0] == 127 * 127 * 12288


def test_round_bf16_matches_torch(orc):
    import torch
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.normal(0, 1, 10000), rng.normal(0, 1e-39, 1000),
                        [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]])
    # torch rounds fp64 -> bf16 in one step too
    t = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.round_bf16(v), t)


def test_tolerance_rule(orc):
    ref = np.array([1.0, -2.0, 100.0])
    ok, worst = orc.tolerance_ok(ref * (1 + 0.009), ref)
    assert ok
    ok, _ = orc.tolerance_ok(ref + np.array([0.0, 0.0, 1.2]), ref)
    assert not ok
