"""CPU checks of bench.py's host logic: the one-GPU contract, the traffic
record's freshness check, the CPU-oracle baseline leg and the MoE mode's
schedule set (nothing here launches a kernel)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as wl  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


def test_traffic_record_matches_the_sources_it_was_taken_on():
    ksha, tsha = bench.source_digests()
    assert len(ksha) == 64 and len(tsha) == 64
    assert bench.source_digests() == (ksha, tsha)        # deterministic
    path = os.path.join(ROOT, "profiles", "gemm_traffic_fp8_dynamic_hidden2048.json")
    rec = json.load(open(path))
    got = bench.measured_traffic("fp8_dynamic_hidden2048")
    if rec["kernel_source_sha256"] == ksha and rec["table_sha256"] == tsha:
        assert got is not None and got["per_launch_traffic_bytes"] > got["per_launch_algorithmic_bytes"] > 0
    else:
        assert got is None                               # stale records are never reported
    assert bench.measured_traffic("no_such_workload") is None


def test_cpu_baseline_leg_on_the_tiny_case():
    fmt, layers, Ms = wl.WORKLOADS["tiny_w8a8_int8"]
    out = bench.cpu_baseline(fmt, layers, Ms, budget_s=0.2)
    assert out["kind"] == "oracle" and out["unit"] == "GB/s"
    assert out["value"] > 0 and out["cores"] >= 1 and out["ms_per_pass"] > 0
    assert "linears" in out["sample"]


def test_moe_schedules_are_valid_grouped_configs():
    q = pytest.importorskip("skinny_bit_gemm_amd")
    q.lib()
    E = wl.MOE_EXPERTS
    for fmt in (wl.FP8_DYNAMIC, wl.W8A8_INT8, wl.BLOCK_FP8):
        for L in wl.MOE_LAYERS:
            for T in wl.MOE_TOKENS:
                for name, c in bench.moe_configs(q, fmt, T).items():
                    # every forced schedule plans for the layer (no launch)
                    assert q.qlin_grouped_workspace_bytes(fmt, E, L.N, L.K, T * wl.MOE_TOPK, T, c) >= 0, name


def test_headline_is_the_largest_workload_and_the_others_ride_along():
    """The default run times BlockFP8 on the hidden-5120 shapes (the largest
    of the three model workloads) and reports the other two beside it."""
    assert bench.DEFAULT_WORKLOAD == "block_fp8_hidden5120"
    fmt, layers, Ms = wl.WORKLOADS[bench.DEFAULT_WORKLOAD]
    sizes = {w: sum(L.N * L.K for L in wl.WORKLOADS[w][1]) for w in
             ("fp8_dynamic_hidden2048", "w8a8_int8_hidden4096", "block_fp8_hidden5120")}
    assert max(sizes, key=sizes.get) == bench.DEFAULT_WORKLOAD
    also = bench.DEFAULT_ALSO.split(",")
    assert sorted(also + [bench.DEFAULT_WORKLOAD]) == sorted(sizes)
    r = {"step_bytes": 2e9, "ms_step": 1.0, "step_flops": 1e12, "gemm_bytes": 4e9, "ms_gemms": 1.0, "n_gemm": 28}
    s = bench.workload_summary(r)
    assert s["step_GBps"] == 2000.0 and s["gemm_achieved_GBps"] == 4000.0 and s["gemm_frac"] == 0.5


def test_table_digest_covers_the_step_buckets_only(tmp_path, monkeypatch):
    """The traffic record stays valid when only entries of the buckets above
    32 tokens (which the step never runs) change; any change to an entry the
    step runs invalidates it."""
    src = os.path.join(bench.ROOT, bench.TABLE)
    lines = open(src).read().splitlines(keepends=True)
    base = tmp_path / "t.tbl"
    base.write_text("".join(lines))
    monkeypatch.setattr(bench, "TABLE", str(base))
    d0 = bench.source_digests()[1]
    big = next(i for i, l in enumerate(lines) if len(l.split()) == 12 and int(l.split()[3]) > 32)
    small = next(i for i, l in enumerate(lines) if len(l.split()) == 12 and int(l.split()[3]) <= 32)
    f = lines[big].split()
    f[5] = str(int(f[5]) + 1)
    base.write_text("".join(lines[:big] + [" ".join(f) + "\n"] + lines[big + 1:]))
    assert bench.source_digests()[1] == d0
    f = lines[small].split()
    f[5] = str(int(f[5]) + 1)
    base.write_text("".join(lines[:small] + [" ".join(f) + "\n"] + lines[small + 1:]))
    assert bench.source_digests()[1] != d0
