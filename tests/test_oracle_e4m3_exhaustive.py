"""Exhaustive pin of the oracle's fp32 -> E4M3FN encoder (CPU only).

Every finite fp32 bit pattern, both signs (2^32 - 2^24 values), is encoded
by the oracle and by a second encoder written independently in plain C
(tests/e4m3_table_check.c: nearest entry of a table of the 127 non-negative
finite E4M3 values built from integer significands and powers of two, ties
to the even code, magnitudes clamped to 448, sign bit copied), and the two
must agree everywhere.  This covers round-to-nearest-even at every binade,
subnormals, the sign of zero, and saturation of every finite value above 448
("Building a High-Performance and Portable vLLM Linear Backend with Helion",
section "Scope": FP8 formats; rounding and saturation as the oracle's header
states).

Kept apart from the pin files that the mutation test runs against every
planted mistake: the stratified and hand-valued pins in test_oracle_e4m3.py
already kill the encoder mutants, and this sweep takes ~0.5 minute.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "e4m3_table_check.c")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("e4m3") / "libe4m3check.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
                    "-fno-fast-math", "-Wall", "-o", out, SRC, "-lm"], check=True)
    L = ctypes.CDLL(out)
    L.sweep_mismatches.restype = ctypes.c_int64
    L.sweep_mismatches.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64,
                                   ctypes.POINTER(ctypes.c_uint64)]
    L.table_encode_array.restype = None
    L.table_encode_array.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
    return L


def table_encode(checker, v):
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    checker.table_encode_array(v.ctypes.data, out.ctypes.data, v.size)
    return out


def test_table_encoder_hand_values(checker):
    """The second encoder itself, on values whose codes follow from the format
    definition by hand: 448 and everything above saturate to 0x7E; 464 is the
    midpoint between 448 and the unrepresentable 480, 0x7E being even; 2^-10
    is the midpoint between 0 and 2^-9 (even code 0x00); 3 * 2^-10 between
    codes 0x01 and 0x02 (even 0x02); 2^-6 is the smallest normal (0x08);
    1.0 is 0x38; -2^-11 rounds to a negative zero (0x80); between 16 (0x58)
    and 18 (0x59), 16.5 goes to 16, 17.5 to 18, and the midpoint 17 to the even
    code 0x58."""
    vals = [448.0, 464.0, 1e30, 2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -6, 1.0, -(2.0 ** -11), 16.5, 17.0, 17.5,
            -448.0, 0.0]
    want = [0x7E, 0x7E, 0x7E, 0x00, 0x02, 0x08, 0x38, 0x80, 0x58, 0x58, 0x59, 0xFE, 0x00]
    assert table_encode(checker, np.array(vals)).tolist() == want


def test_every_finite_fp32_matches_the_table_encoder(orc, checker):
    enc = ctypes.cast(orc.lib().orc_e4m3_encode, ctypes.c_void_p).value
    first = ctypes.c_uint64(0)
    bad = checker.sweep_mismatches(enc, 0, 1 << 32, ctypes.byref(first))
    if bad:
        bits = np.array([first.value], dtype=np.uint32)
        v = bits.view(np.float32)
        pytest.fail(f"{bad} fp32 patterns encode differently; the first is {float(v[0]).hex()} "
                    f"(oracle {hex(int(orc.e4m3_encode(v)[0]))}, table {hex(int(table_encode(checker, v)[0]))})")
