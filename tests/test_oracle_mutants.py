"""The oracle's pins catch plausible mistakes.

Each case copies the oracle's C source, plants one mistake of the kind the
pins are meant to catch (a wrong rounding mode, exponent bias or scale, a
multiplication by 1/s in place of the division, a dropped term, factor or
absolute value, a wrong group or block index), builds the copy with the same
gcc flags, and runs the oracle's pin tests against it in a child process:
they must fail.  The unchanged copy, built the same way, must pass them, so
that it is the planted mistake, not the harness, that fails.  No mutant
reads or writes outside its arrays.  CPU only.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "qlin_oracle.c")
HDR = os.path.join(ROOT, "oracle", "qlin_oracle.h")
PINS = ["tests/test_oracle_e4m3.py", "tests/test_oracle_quant.py", "tests/test_oracle_gemm.py",
        "tests/test_oracle_grouped.py"]

# name -> (text in the source, replacement); each text occurs exactly once
MUTANTS = {
    "e4m3_ties_away": ("double r = nearbyint(a / quantum);", "double r = floor(a / quantum + 0.5);"),
    "e4m3_flush_subnormals": ("mag = (uint8_t)(val / ldexp(1.0, -9));", "mag = 0;"),
    "e4m3_no_saturation": ("if (a > E4M3_MAX) a = E4M3_MAX;", ""),
    "decode_bias_8": ("v = ldexp(1.0 + m / 8.0, e - 7);", "v = ldexp(1.0 + m / 8.0, e - 8);"),
    "decode_subnormal_2^-10": ("v = ldexp((double)m, -9);", "v = ldexp((double)m, -10);"),
    "reciprocal_multiply": ("float t = x / s;", "float t = x * (1.0f / s);"),
    "int8_truncates": ("float r = rintf(t);", "float r = truncf(t);"),
    "qmax_swapped": ("return fmt == ORC_W8A8_INT8 ? INT8_QMAX : FP8_QMAX;",
                     "return fmt == ORC_W8A8_INT8 ? FP8_QMAX : INT8_QMAX;"),
    "amax_without_abs": ("float a = fabsf(v[(int64_t)i * stride]);", "float a = v[(int64_t)i * stride];"),
    "act_group_amax_of_group_0": ("scale_of(absmax(row + g * GROUP, GROUP, 1, &bad), fmt)",
                                  "scale_of(absmax(row, GROUP, 1, &bad), fmt)"),
    "weight_block_scale_transposed": ("s[(int64_t)nb * KB + kb] = sc;", "s[(int64_t)kb * NB + nb] = sc;"),
    "weight_block_amax_one_row": ("for (int n = nb * GROUP; n < (nb + 1) * GROUP; ++n)\n"
                                  "                    amax = fmaxf(",
                                  "for (int n = nb * GROUP; n < nb * GROUP + 1; ++n)\n"
                                  "                    amax = fmaxf("),
    "int8_dot_drops_last_term": ("for (int k = 0; k < K; ++k) acc += (int64_t)(int8_t)a[k]",
                                 "for (int k = 0; k < K - 1; ++k) acc += (int64_t)(int8_t)a[k]"),
    "int8_codes_unsigned": ("acc += (int64_t)(int8_t)a[k] * (int64_t)(int8_t)b[k];",
                            "acc += (int64_t)a[k] * (int64_t)b[k];"),
    "fp8_dot_drops_last_term": ("for (int k = 0; k < K; ++k) acc += t[a[k]] * t[b[k]];",
                                "for (int k = 0; k < K - 1; ++k) acc += t[a[k]] * t[b[k]];"),
    "fp8_result_drops_weight_scale": ("return dot_fp8(a, b, K, t) * (double)sa[m] * (double)sw[n];",
                                      "return dot_fp8(a, b, K, t) * (double)sa[m];"),
    "int8_result_channel_0_scale": ("return (double)acc * (double)sa[m] * (double)sw[n];",
                                    "return (double)acc * (double)sa[m] * (double)sw[0];"),
    "block_result_weight_scale_group_0": ("(double)sw[(int64_t)(n / GROUP) * G + g]",
                                          "(double)sw[(int64_t)(n / GROUP) * G]"),
    "block_result_token_scale_group_0": ("(double)sa[(int64_t)m * G + g]", "(double)sa[(int64_t)m * G]"),
    "bf16_truncates": ("double r = nearbyint(a / quantum) * quantum;", "double r = trunc(a / quantum) * quantum;"),
}


def build_copy(tmp, name, edit):
    d = os.path.join(tmp, name)
    os.makedirs(d, exist_ok=True)
    src = open(SRC).read()
    if edit is not None:
        old, new = edit
        assert src.count(old) == 1, f"{name}: the text to replace must occur exactly once"
        src = src.replace(old, new)
    open(os.path.join(d, "qlin_oracle.c"), "w").write(src)
    shutil.copy(HDR, d)
    lib = os.path.join(d, "liborc.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
                    "-fno-fast-math", "-w", "-o", lib, os.path.join(d, "qlin_oracle.c"), "-lm"], check=True)
    return lib


def run_pins(lib):
    env = dict(os.environ, QLIN_ORACLE_MUTANT_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"]
                       + PINS, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


def test_pins_kill_every_planted_mistake(tmp_path):
    tmp = str(tmp_path)
    rc, out = run_pins(build_copy(tmp, "unchanged", None))
    assert rc == 0, "the unchanged copy must pass the pins:\n" + out
    libs = {name: build_copy(tmp, name, edit) for name, edit in MUTANTS.items()}
    with ThreadPoolExecutor(max_workers=4) as ex:
        results = dict(zip(libs, ex.map(run_pins, libs.values())))
    survivors = {n: out for n, (rc, out) in results.items() if rc != 1}
    assert not survivors, "mistakes the pins did not catch (pytest exit code other than 1):\n" + "\n".join(
        f"--- {n} (exit {results[n][0]})\n{out}" for n, out in survivors.items())
