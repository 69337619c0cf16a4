"""Pins for the oracle's fp8 E4M3 decode and encode (CPU only).

The pins are independent of the oracle's own arithmetic: a closed form
enumerated a different way, hand-worked values (tests/golden), a nearest-
in-table search with an explicit tie rule over a stratified-exhaustive set of
fp32 bit patterns, and torch's own float8_e4m3fn cast as a third witness
inside the finite range.
"""
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _closed_form_table():
    """All 256 E4M3FN codes enumerated as integer multiples of 2^-9."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e, m = (code >> 3) & 15, code & 7
        if e == 15 and m == 7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = s * m * 2.0 ** -9
        else:
            # (8 + m) * 2^(e - 10): the implicit leading one as an integer
            vals[code] = s * (8 + m) * 2.0 ** (e - 10)
    return vals


def test_decode_all_codes_closed_form(orc):
    got = orc.e4m3_decode(np.arange(256))
    want = _closed_form_table()
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9
    # every finite value is an integer multiple of 2^-9, |v| <= 229376 * 2^-9
    mult = got[ok] * 2 ** 9
    assert np.all(mult == np.round(mult)) and np.max(np.abs(mult)) == 229376


def test_decode_matches_torch_float8(orc):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    t = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = orc.e4m3_decode(np.arange(256))
    ok = ~np.isnan(t)
    assert np.array_equal(np.isnan(got), np.isnan(t))
    assert np.array_equal(got[ok], t[ok])


def _golden_e4m3():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_hand_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            v, code = line.split()[:2]
            rows.append((float.fromhex(v), int(code, 16)))
    return rows


def test_encode_hand_values(orc):
    rows = _golden_e4m3()
    assert len(rows) >= 15
    vals = np.array([r[0] for r in rows], dtype=np.float32)
    want = np.array([r[1] for r in rows], dtype=np.uint8)
    # the fixture's values must be exactly representable in fp32
    assert np.array_equal(vals.astype(np.float64), np.array([r[0] for r in rows]))
    got = orc.e4m3_encode(vals)
    assert got.tolist() == want.tolist()


def _table_search_encode(v32: np.ndarray) -> np.ndarray:
    """Second encoder: nearest of the 127 non-negative finite codes, ties to
    the even code, after clamping |v| to 448; the sign bit copied over."""
    table = _closed_form_table()[:0x7F]               # codes 0x00..0x7E, ascending
    a = np.minimum(np.abs(v32.astype(np.float64)), 448.0)
    hi = np.clip(np.searchsorted(table, a, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_hi = table[hi] - a
    d_lo = a - table[lo]
    pick = np.where(d_lo < d_hi, lo, hi)
    tie = d_lo == d_hi
    pick = np.where(tie & (lo != hi), np.where(lo % 2 == 0, lo, hi), pick)
    sign = np.signbit(v32).astype(np.uint8) << 7
    return (pick.astype(np.uint8) | sign).astype(np.uint8)


def _stratified_fp32():
    """Every sign, every finite exponent, every value of the top 11 mantissa
    bits, and the low 12 bits set to edge patterns around the round/sticky
    positions (0, 1, just below and at and above a half, all ones)."""
    sign = np.array([0, 1], dtype=np.uint32)[:, None, None, None] << 31
    exp = np.arange(0, 255, dtype=np.uint32)[None, :, None, None] << 23
    top = np.arange(0, 2 ** 11, dtype=np.uint32)[None, None, :, None] << 12
    low = np.array([0x000, 0x001, 0x7FF, 0x800, 0x801, 0xFFF, 0x555, 0xAAA],
                   dtype=np.uint32)[None, None, None, :]
    bits = (sign | exp | top | low).ravel()
    return bits.view(np.float32)


def test_encode_stratified_exhaustive_vs_table_search(orc):
    v = _stratified_fp32()
    assert v.size == 2 * 255 * 2048 * 8
    got = orc.e4m3_encode(v)
    want = _table_search_encode(v)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(v[i]).hex(), hex(got[i]), hex(want[i])) for i in bad[:8]]


def test_encode_random_bits_vs_table_search(orc):
    rng = np.random.default_rng(1234)
    bits = rng.integers(0, 2 ** 32, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    assert np.array_equal(orc.e4m3_encode(v), _table_search_encode(v))


def test_encode_every_bf16_vs_table_search(orc):
    """Every finite bf16 value (activations are bf16) encodes alike."""
    bits = (np.arange(2 ** 16, dtype=np.uint32) << 16).view(np.float32)
    v = bits[np.isfinite(bits)]
    assert np.array_equal(orc.e4m3_encode(v), _table_search_encode(v))


def test_encode_matches_torch_inside_range(orc):
    """torch's float -> float8_e4m3fn cast rounds to nearest even; inside
    +-448 it must give the same bytes (beyond, torch returns NaN and the
    saturating rule gives +-448, so it is no witness there)."""
    rng = np.random.default_rng(7)
    v = np.concatenate([
        rng.uniform(-448, 448, 200_000),
        rng.normal(0, 1, 200_000),
        rng.normal(0, 2 ** -8, 200_000),
    ]).astype(np.float32)
    t = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(orc.e4m3_encode(v), t)


def test_encode_saturates_and_rejects_nonfinite(orc):
    got = orc.e4m3_encode(np.array([1e6, -1e6, 3.0e38, -449.0], dtype=np.float32))
    assert got.tolist() == [0x7E, 0xFE, 0x7E, 0xFE]
    for bad in (np.inf, -np.inf, np.nan):
        with pytest.raises(ValueError):
            orc.e4m3_encode(np.array([bad], dtype=np.float32))


def test_encode_decode_roundtrip_is_identity_on_codes(orc):
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = orc.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(orc.e4m3_encode(vals), codes)
