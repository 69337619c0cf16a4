"""Search for activation values whose code depends on how the quotient
x / scale is formed: the correctly rounded fp32 quotient (the definition the
oracle follows) and x times a rounded reciprocal differ in the last bit now
and then, and where that bit decides a code (an int8 quotient at a tie, an
e4m3 quotient at a midpoint) the two codes differ.  Used by the oracle's
quantization pin and by the GPU quantization parity test."""
from __future__ import annotations

import numpy as np

# every positive normal bf16 value, as float32
BF16_POSITIVE = (np.arange(0x0080, 0x7F80, dtype=np.uint32) << 16).view(np.float32)


def quotient_pairs(qmax, encode=None, n_amax=300, per_amax=8, seed=1):
    """[(amax, xs), ...]: for a seeded sample of n_amax bf16 amax values in
    (1e-3, 1e3), the first per_amax bf16 values x <= amax where the code of
    fl32(x / s) differs from the code of fl32(x * fl32(1 / s)), s =
    fl32(amax / qmax).  `encode` maps fp32 quotients to codes (None: round
    to nearest even, the int8 rule before its saturation, which these
    quotients never reach).  Sample values with no such x are left out."""
    rng = np.random.default_rng(seed)
    bf = BF16_POSITIVE
    amaxes = rng.choice(bf[(bf > 1e-3) & (bf < 1e3)], n_amax, replace=False)
    out = []
    for a in amaxes:
        s = np.float32(a) / np.float32(qmax)
        xs = bf[bf <= a]
        qd, qr = xs / s, xs * (np.float32(1.0) / s)
        if encode is None:
            sel = np.rint(qd) != np.rint(qr)
        else:
            sel = encode(qd) != encode(qr)
        if sel.any():
            out.append((np.float32(a), xs[sel][:per_amax]))
    return out


def to_bf16_bits(vals):
    """float32 values that are exactly bf16 -> bf16 bit patterns (uint16)."""
    v = np.asarray(vals, dtype=np.float32)
    bits = v.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0), "value not exactly bf16"
    return (bits >> 16).astype(np.uint16)
