"""The C ABI on the host (no GPU): the library loads, exports every symbol
include/qlin.h declares, rejects bad arguments before any HIP call, and
reads / rejects selection tables; the same for the measurement aid
libqlin_probe.so (include/qlin_probe.h).  No call here reaches a kernel
launch."""
import ctypes
import os
import re

import pytest

import skinny_bit_gemm_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlin.h")

FP8, I8, BLK = q.QLIN_FP8_DYNAMIC, q.QLIN_W8A8_INT8, q.QLIN_BLOCK_FP8
OK, EINVAL, EALIGN, ESHAPE, EWS, ENOCFG, ETABLE = 0, 1, 2, 3, 4, 5, 6
A = 1 << 20     # a fake, 16-byte aligned "device address" (never dereferenced)


@pytest.fixture(autouse=True)
def _restore_table():
    yield
    q.qlin_set_strict(False)
    if os.path.exists(q.TABLE_PATH):
        q.qlin_load_table(q.TABLE_PATH)


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(qlin_\w+)\s*\(", text)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    L = q.lib()
    names = declared_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), f"{n} declared in qlin.h but not exported"
    assert set(names) == set(q.EXPORTS)


def test_probe_library_exports_and_validates():
    from skinny_bit_gemm_amd import probe
    L = probe.lib()
    names = declared_functions(os.path.join(ROOT, "include", "qlin_probe.h"))
    assert set(names) == set(probe.EXPORTS)
    for n in names:
        assert hasattr(L, n)
    # rejected before any HIP call: null, misaligned, ragged size, bad grid
    assert probe.qlin_probe_read(0, 1 << 20, A, 64, 0) == 1
    assert probe.qlin_probe_read(A + 4, 1 << 20, A, 64, 0) == 1
    assert probe.qlin_probe_read(A, (1 << 20) + 8, A, 64, 0) == 1
    assert probe.qlin_probe_read(A, 1 << 20, A, 0, 0) == 1
    assert probe.qlin_probe_read(A, 1 << 20, A, 70000, 0) == 1


def test_abi_version_and_status_strings():
    assert q.qlin_abi_version() == 1
    for st in range(8):
        assert q.qlin_status_str(st)
    assert "strict" in q.qlin_status_str(ENOCFG)


def gemm(fmt=FP8, M=4, N=256, K=512, xq=A, xs=A, wq=A, ws=A, y=A, out=0, cfg=None, work=None, wsb=0):
    return q.qlin_gemm(fmt, M, N, K, xq, xs, wq, ws, y, out, cfg, work, wsb, stream=0,
                       raise_on_error=False)


def test_gemm_rejects_bad_arguments():
    assert gemm(fmt=7) == EINVAL
    assert gemm(out=5) == EINVAL
    assert gemm(fmt=FP8, out=q.QLIN_OUT_I32_ACC) == EINVAL      # int32 sums: int8 only
    assert gemm(xq=None) == EINVAL
    assert gemm(y=None) == EINVAL
    assert gemm(wq=A + 8) == EALIGN
    assert gemm(xs=A + 2) == EALIGN
    assert gemm(N=100) == ESHAPE                   # N % 16
    assert gemm(K=520) == ESHAPE                   # K % 16
    assert gemm(M=-1) == ESHAPE
    assert gemm(fmt=BLK, K=640 + 16) == ESHAPE     # block format: K % 128
    assert gemm(fmt=BLK, N=256 + 16) == ESHAPE     # block format: N % 128
    assert gemm(fmt=I8, K=133_120 + 128) == ESHAPE  # int32 sums could overflow


def test_linear_scratch_checks_before_any_hip_call():
    """qlin_linear_scratch validates like qlin_linear and rejects a schedule
    whose workspace does not fit the static scratch array; M = 0 enqueues
    nothing."""
    def call(fmt=FP8, M=4, N=256, K=512, x=A, ldx=512, y=A, cfg=None):
        return q.qlin_linear_scratch(fmt, M, N, K, x, ldx, A, A, A, A, y, 0, cfg, stream=0,
                                     raise_on_error=False)
    assert call(fmt=9) == EINVAL
    assert call(x=None) == EINVAL
    assert call(y=A + 8) == EALIGN
    assert call(ldx=500) == EALIGN
    assert call(K=520, ldx=520) == ESHAPE
    assert call(cfg=q.make_config(split_k=0)) == EINVAL
    big = q.make_config(1, 16, 32, 64, 4, 2, 0, 0)
    need = q.qlin_workspace_bytes(FP8, 32, 8192, 8192, big)
    assert need > q.QLIN_SCRATCH_BYTES
    assert call(M=32, N=8192, K=8192, ldx=8192, cfg=big) == EWS
    assert call(M=0, N=8192, K=8192, ldx=8192, cfg=big) == OK   # nothing to compute
    assert call(M=0) == OK


def test_quantize_act_cfg_checks_before_any_hip_call():
    def call(fmt=FP8, M=4, K=512, threads=64):
        return q.qlin_quantize_act_cfg(fmt, M, K, A, K, A, A, threads, stream=0, raise_on_error=False)
    for t in (0, 64, 128, 256, 512):
        assert call(M=0, threads=t) == OK
        assert call(fmt=I8, M=0, threads=t) == OK
    for t in (0, 64, 256):
        assert call(fmt=BLK, M=0, threads=t) == OK
    for t in (-1, 32, 96, 1024):
        assert call(threads=t) == EINVAL
    assert call(fmt=BLK, threads=128) == EINVAL
    assert call(fmt=BLK, threads=512) == EINVAL
    assert call(K=520) == ESHAPE


def test_pack_weight_checks_before_any_hip_call():
    assert q.qlin_packed_weight_bytes(48, 1040) == 48 * 9 * 128      # blocks of 128 K, zero-padded
    assert q.qlin_packed_weight_bytes(4096, 2048) == 4096 * 2048
    def pack(batch=1, N=256, K=512, src=A, dst=A + (1 << 24)):
        return q.qlin_pack_weight(batch, N, K, src, dst, stream=0, raise_on_error=False)
    assert pack(N=100) == ESHAPE
    assert pack(K=520) == ESHAPE
    assert pack(batch=-1) == ESHAPE
    assert pack(batch=70000) == ESHAPE
    assert pack(src=None) == EINVAL
    assert pack(dst=A + 8) == EALIGN
    assert pack(batch=0) == OK                                       # nothing to do
    # the layout flag on the format argument: accepted by the GEMM calls and
    # the schedule queries, rejected by the quantizers
    flag = q.QLIN_PACKED_WEIGHTS
    assert q.qlin_validate_config(FP8 | flag, 4, 256, 512, q.make_config()) == OK
    assert q.qlin_workspace_bytes(I8 | flag, 4, 256, 512, q.make_config(split_k=2)) == \
        q.qlin_workspace_bytes(I8, 4, 256, 512, q.make_config(split_k=2))
    assert gemm(fmt=BLK | flag, K=640 + 16) == ESHAPE
    assert gemm(fmt=7 | flag) == EINVAL
    assert q.qlin_quantize_act(FP8 | flag, 4, 512, A, 512, A, A, stream=0, raise_on_error=False) == EINVAL


def test_gemm_rejects_bad_configs():
    bad = [q.make_config(swap_ab=2), q.make_config(split_k=0), q.make_config(split_k=65),
           q.make_config(tile_m=8), q.make_config(waves=0, k_waves=1),
           q.make_config(waves=9, k_waves=1), q.make_config(waves=16, k_waves=16),
           q.make_config(waves=4, k_waves=3), q.make_config(tile_n=24, waves=1, k_waves=1),
           q.make_config(tile_n=512, waves=1, k_waves=1),
           q.make_config(tile_n=16, waves=4, k_waves=1),   # 4 column waves need tile_n >= 32
           q.make_config(tile_n=48, waves=4, k_waves=1),   # neither 16-row nor 8-row sub-tiles
           q.make_config(tile_n=48, waves=1, k_waves=1),   # 3 sub-tiles per wave: not built
           q.make_config(tile_n=32, waves=3, k_waves=1),   # 3 column waves: 24, 48, 96 or 192
           q.make_config(tile_n=64, waves=6, k_waves=2)]
    for c in bad:
        assert gemm(cfg=c) == EINVAL, c
        assert q.qlin_validate_config(FP8, 4, 256, 512, c) == EINVAL
    # 8-row weight sub-tiles: tile_n = 8 x (column waves)
    for c in (q.make_config(tile_n=8, waves=1, k_waves=1), q.make_config(tile_n=8, waves=4, k_waves=4),
              q.make_config(tile_n=16, waves=2, k_waves=1), q.make_config(tile_n=32, waves=4, k_waves=1)):
        assert q.qlin_validate_config(FP8, 4, 256, 512, c) == OK, c
    # 64-token tiles: the large-M kernel with its one layout (128 channels,
    # 4 waves, 1 K wave, Standard roles, slice reduction), the skinny kernel
    # with any other (staged codes); 128-token tiles are the large-M kernel's
    for c in (q.make_config(tile_m=64, tile_n=128, waves=4, k_waves=1),
              q.make_config(tile_m=64, tile_n=32, waves=4, k_waves=4),
              q.make_config(tile_m=64, swap_ab=1, tile_n=64, waves=2, k_waves=1),
              q.make_config(tile_m=64, split_k=2, tile_n=128, waves=4, k_waves=1, reduce=1),
              q.make_config(tile_m=128, tile_n=128, waves=4, k_waves=1)):
        assert q.qlin_validate_config(FP8, 64, 256, 512, c) == OK, c
    for c in (q.make_config(tile_m=64, tile_n=256, waves=4, k_waves=1),        # 4 sub-tiles: not built
              q.make_config(tile_m=64, tile_n=32, waves=4, k_waves=4, act_path=2),
              q.make_config(tile_m=128, tile_n=64, waves=4, k_waves=1),
              q.make_config(tile_m=128, swap_ab=1, tile_n=128, waves=4, k_waves=1)):
        assert q.qlin_validate_config(FP8, 64, 256, 512, c) == EINVAL, c
    # column-wave counts that are not powers of two
    for c in (q.make_config(tile_n=24, waves=3, k_waves=1), q.make_config(tile_n=24, waves=6, k_waves=2),
              q.make_config(tile_n=48, waves=3, k_waves=1), q.make_config(tile_n=96, waves=6, k_waves=2),
              q.make_config(tile_n=96, waves=6, k_waves=1), q.make_config(tile_n=40, waves=5, k_waves=1),
              q.make_config(tile_n=80, waves=5, k_waves=1), q.make_config(tile_n=224, waves=7, k_waves=1),
              q.make_config(tile_n=56, waves=7, k_waves=1, act_path=1)):
        assert q.qlin_validate_config(FP8, 4, 256, 512, c) == OK, c


def test_activation_paths():
    """act_path: the header's values, the range check, and where each path
    exists (direct loads: the skinny kernel only, the block format in the
    Swap-AB roles only; fused quantization: 16-token tiles)."""
    with open(HEADER) as f:
        text = f.read()
    for name in ("QLIN_ACT_STAGED", "QLIN_ACT_FUSED", "QLIN_ACT_DIRECT"):
        assert f"#define {name} {getattr(q, name)}" in text, name
    assert q.qlin_validate_config(FP8, 4, 256, 512, q.make_config(act_path=3)) == EINVAL
    assert q.qlin_validate_config(FP8, 4, 256, 512, q.make_config(act_path=-1)) == EINVAL
    D = q.QLIN_ACT_DIRECT
    for fmt in (FP8, I8):
        for c in (q.make_config(0, 1, 16, 32, 4, 4, act_path=D), q.make_config(1, 2, 32, 64, 4, 2, act_path=D),
                  q.make_config(0, 3, 16, 128, 8, 2, reduce=1, act_path=D),
                  q.make_config(1, 1, 16, 8, 1, 1, act_path=D)):
            assert q.qlin_validate_config(fmt, 20, 512, 2048, c) == OK, (fmt, c)
            assert q.qlin_workspace_bytes(fmt, 20, 512, 2048, c) == \
                q.qlin_workspace_bytes(fmt, 20, 512, 2048, q.make_config(**{**c.as_dict(), "act_path": 0}))
    assert q.qlin_validate_config(BLK, 20, 512, 2048, q.make_config(1, 1, 16, 32, 4, 4, act_path=D)) == OK
    assert q.qlin_validate_config(BLK, 20, 512, 2048, q.make_config(0, 1, 16, 32, 4, 4, act_path=D)) == EINVAL
    assert q.qlin_validate_config(FP8, 300, 512, 2048, q.make_config(0, 1, 64, 128, 4, 1, act_path=D)) == EINVAL
    assert q.qlin_validate_config(FP8, 20, 512, 2048, q.make_config(0, 1, 32, 32, 4, 4, act_path=1)) == EINVAL


def test_large_m_configs():
    """Token tiles of 64 / 128 select the large-M kernel: 128-channel tiles,
    4 waves in one K row, Standard roles, slice reduction, no in-kernel
    quantization."""
    for fmt in (FP8, I8, BLK):
        for tm in (64, 128):
            for split in (1, 3):
                assert q.qlin_validate_config(fmt, 300, 512, 2048, q.make_config(0, split, tm, 128, 4, 1)) == OK
        bad = [q.make_config(1, 1, 128, 128, 4, 1), q.make_config(0, 1, 128, 64, 4, 1),
               q.make_config(0, 1, 128, 128, 8, 1), q.make_config(0, 1, 128, 128, 4, 4),
               q.make_config(0, 2, 128, 128, 4, 1, reduce=1), q.make_config(0, 1, 128, 128, 4, 1, act_path=1),
               q.make_config(0, 1, 96, 128, 4, 1)]
        for c in bad:
            assert q.qlin_validate_config(fmt, 300, 512, 2048, c) == EINVAL, (fmt, c)
    # slices: counters for every (M tile, 128-channel tile), one partial per partition
    c = q.make_config(0, 4, 128, 128, 4, 1)
    nbytes = q.qlin_workspace_bytes(FP8, 300, 512, 2048, c)
    counters = -(-(3 * 4 * 4) // 256) * 256
    assert nbytes == counters + -(-(4 * 300 * 512 * 4) // 256) * 256
    assert q.qlin_workspace_bytes(FP8, 300, 512, 2048, q.make_config(0, 1, 128, 128, 4, 1)) == 0


def test_split_k_workspace_is_checked_before_launch():
    c = q.make_config(swap_ab=1, split_k=4, tile_m=16, tile_n=32, waves=4, k_waves=4)
    need = q.qlin_workspace_bytes(FP8, 4, 256, 2048, c)
    assert need >= 4 * 256 * 4
    assert gemm(K=2048, cfg=c, work=None, wsb=0) == EWS
    assert gemm(K=2048, cfg=c, work=A, wsb=need - 1) == EWS
    assert gemm(K=2048, cfg=c, work=A + 4, wsb=need) == EALIGN
    # one partition only (K fits one split): no workspace needed
    c1 = q.make_config(swap_ab=1, split_k=4, tile_m=16, tile_n=32, waves=4, k_waves=4)
    assert q.qlin_workspace_bytes(FP8, 4, 256, 128, c1) == 0


def test_quantize_rejects_bad_arguments():
    f = lambda *a, **k: q.qlin_quantize_act(*a, stream=0, raise_on_error=False, **k)
    assert f(9, 4, 512, A, 512, A, A) == EINVAL
    assert f(FP8, 4, 520, A, 520, A, A) == ESHAPE
    assert f(BLK, 4, 528, A, 528, A, A) == ESHAPE
    assert f(FP8, 4, 512, A, 500, A, A) == EALIGN       # ldx < K
    assert f(FP8, 4, 512, A, 516, A, A) == EALIGN       # ldx % 8
    assert f(FP8, 4, 512, A + 2, 512, A, A) == EALIGN
    assert f(FP8, 4, 512, None, 512, A, A) == EINVAL
    assert f(FP8, 0, 512, A, 512, A, A) == OK           # nothing to do, nothing launched
    g = lambda *a: q.qlin_quantize_weight(*a, stream=0, raise_on_error=False)
    assert g(FP8, 100, 512, A, A, A) == ESHAPE
    assert g(BLK, 256, 384 + 16, A, A, A) == ESHAPE
    assert g(I8, 256, 512, A, None, A) == EINVAL


def test_zero_tokens_gemm_is_ok_without_launch():
    assert gemm(M=0) == OK


def test_any_shape_gets_a_valid_config():
    # listed or not, every token count (also beyond the largest bucket) gets
    # a configuration that fits the shape
    for M in (1, 5, 31, 100, 600):
        for fmt, N, K in ((I8, 2048, 4096), (FP8, 1008, 1040), (BLK, 384, 640)):
            c = q.qlin_select_variant(fmt, M, N, K)
            assert q.qlin_validate_config(fmt, M, N, K, c) == OK


def write_table(tmp_path, body, header="qlin-table 1 gfx950"):
    p = tmp_path / "t.tbl"
    p.write_text(header + "\n" + body)
    return str(p)


def test_table_load_lookup_and_bucket_round_up(tmp_path):
    path = write_table(tmp_path, "# comment\n"
                       "fp8_dynamic 1024 1024 4 1 2 16 64 4 2 0 0\n"
                       "fp8_dynamic 1024 1024 32 0 4 32 32 4 4 0 0   # trailing comment\n")
    assert q.qlin_load_table(path) == OK
    assert q.qlin_table_entries() == 2
    c = q.qlin_select_variant(FP8, 3, 1024, 1024)           # 3 -> bucket 4
    assert (c.swap_ab, c.split_k, c.tile_m, c.tile_n, c.waves, c.k_waves) == (1, 2, 16, 64, 4, 2)
    c = q.qlin_select_variant(FP8, 25, 1024, 1024)          # 25 -> bucket 32
    assert (c.swap_ab, c.split_k, c.tile_m) == (0, 4, 32)


def test_default_rule_without_table_entries(tmp_path):
    # an empty table: the built-in rule.  N = K = 1024: 16 tiles of 64
    # columns; the split doubles while the grid is under 192 workgroups and
    # each of the two K waves keeps a block: 8 K blocks -> split 4 (Swap-AB)
    assert q.qlin_load_table(write_table(tmp_path, "")) == OK
    assert q.qlin_table_entries() == 0
    c = q.qlin_select_variant(FP8, 3, 1024, 1024)
    assert (c.swap_ab, c.split_k, c.tile_m, c.tile_n, c.waves, c.k_waves, c.reduce) == (1, 4, 16, 64, 4, 2, 0)
    assert c.act_path == 1                      # 3 rows of 1024 values fit the registers
    c = q.qlin_select_variant(FP8, 32, 1024, 1024)
    assert (c.split_k, c.tile_m, c.act_path) == (4, 32, 0)
    c = q.qlin_select_variant(I8, 4, 12288, 4096)  # 192 tiles already: no split
    assert (c.swap_ab, c.split_k) == (0, 1)
    c = q.qlin_select_variant(I8, 200, 4096, 4096)
    assert (c.tile_m, c.tile_n, c.k_waves) == (64, 128, 1)


def test_nearest_entry_for_unlisted_shapes(tmp_path):
    path = write_table(tmp_path,
                       "fp8_dynamic 2048 2048 4 0 2 16 32 4 2 1 0\n"
                       "w8a8_int8 1024 1024 4 1 1 16 64 8 4 0 1\n"
                       "fp8_dynamic 1024 1024 8 1 2 16 64 4 2 0 0\n")
    assert q.qlin_load_table(path) == OK
    # same bucket only; a per-token format at distance 0 + 1/2 beats the same
    # format at distance 2
    c = q.qlin_select_variant(FP8, 3, 1024, 1024)
    assert (c.swap_ab, c.split_k, c.tile_n, c.waves, c.k_waves, c.act_path) == (1, 1, 64, 8, 4, 1)
    # nearer in N and K wins within the format
    c = q.qlin_select_variant(FP8, 4, 2048, 4096)
    assert (c.split_k, c.tile_n, c.reduce) == (2, 32, 1)
    # the block format counts a per-token entry at distance + 1; the packed
    # reduction is for exact formats only, so (2048, 2048) is passed over
    c = q.qlin_select_variant(BLK, 4, 2048, 2048)
    assert (c.split_k, c.tile_n, c.waves) == (1, 64, 8)
    # a fused entry whose rows do not fit the registers at this K loses the
    # fused quantization, not the rest
    c = q.qlin_select_variant(I8, 4, 1024, 65536)
    assert (c.swap_ab, c.tile_n, c.waves, c.k_waves, c.act_path) == (1, 64, 8, 4, 0)
    # a direct Standard entry has no block-format kernel: the block format
    # keeps the schedule with staged activations
    path = write_table(tmp_path, "fp8_dynamic 2048 2048 4 0 2 16 32 4 2 0 2\n")
    assert q.qlin_load_table(path) == OK
    c = q.qlin_select_variant(FP8, 4, 2048, 2048)
    assert (c.swap_ab, c.split_k, c.tile_n, c.act_path) == (0, 2, 32, q.QLIN_ACT_DIRECT)
    c = q.qlin_select_variant(BLK, 4, 2048, 2048)
    assert (c.swap_ab, c.split_k, c.tile_n, c.act_path) == (0, 2, 32, q.QLIN_ACT_STAGED)
    path = write_table(tmp_path,
                       "fp8_dynamic 2048 2048 4 0 2 16 32 4 2 1 0\n"
                       "w8a8_int8 1024 1024 4 1 1 16 64 8 4 0 1\n"
                       "fp8_dynamic 1024 1024 8 1 2 16 64 4 2 0 0\n")
    assert q.qlin_load_table(path) == OK
    # another bucket: its own entry, or the built-in rule when it has none
    c = q.qlin_select_variant(FP8, 8, 4096, 4096)
    assert (c.swap_ab, c.split_k, c.tile_n) == (1, 2, 64)
    c = q.qlin_select_variant(FP8, 16, 1024, 1024)
    assert (c.split_k, c.k_waves) == (4, 2)


def test_strict_mode_missing_entry_is_an_error(tmp_path):
    path = write_table(tmp_path, "fp8_dynamic 1024 1024 4 1 2 16 64 4 2 0 0\n")
    assert q.qlin_load_table(path) == OK
    q.qlin_set_strict(True)
    with pytest.raises(q.QlinError) as e:
        q.qlin_select_variant(FP8, 8, 1024, 1024)
    assert e.value.status == ENOCFG
    assert gemm(N=1024, K=1024, M=8) == ENOCFG
    # a present entry and a forced config still work
    assert q.qlin_select_variant(FP8, 4, 1024, 1024).split_k == 2
    q.qlin_set_strict(False)
    assert q.qlin_select_variant(FP8, 8, 1024, 1024).tile_m == 16


@pytest.mark.parametrize("header,body", [
    ("qlin-table 1 gfx942", "fp8_dynamic 1024 1024 4 1 2 16 64 4 2 0 0\n"),     # wrong arch
    ("qlin-table 2 gfx950", "fp8_dynamic 1024 1024 4 1 2 16 64 4 2 0 0\n"),     # wrong version
    ("qlin-table 1 gfx950", "fp4 1024 1024 4 1 2 16 64 4 2 0 0\n"),             # unknown format
    ("qlin-table 1 gfx950", "fp8_dynamic 1024 1024 4 1 2 16 64 4 2 0\n"),   # short line
    ("qlin-table 1 gfx950", "fp8_dynamic 1024 1024 5 1 2 16 64 4 2 0 0\n"),     # 5 is no bucket
    ("qlin-table 1 gfx950", "fp8_dynamic 1024 1024 4 1 2 16 48 4 2 0 0\n"),     # invalid tile
    ("qlin-table 1 gfx950", "block_fp8 1024 1024 4 1 2 16 64 4 2 1 0\n"),  # packed: exact formats only
    ("qlin-table 1 gfx950", "fp8_dynamic 1024 1024 32 1 2 32 64 4 2 0 1\n"),  # fused needs tile_m 16
    ("qlin-table 1 gfx950", "fp8_dynamic 1024 1024 4 1 2 16 64 4 2 0 3\n"),  # no such activation path
    ("qlin-table 1 gfx950", "block_fp8 1024 1024 4 0 2 16 64 4 2 0 2\n"),  # direct block: Swap-AB only
    ("nonsense", ""),
])
def test_corrupt_tables_are_rejected(tmp_path, header, body):
    good = write_table(tmp_path, "fp8_dynamic 1024 1024 4 1 2 16 64 4 2 0 0\n")
    assert q.qlin_load_table(good) == OK
    p = tmp_path / "bad.tbl"
    p.write_text(header + "\n" + body)
    assert q.qlin_load_table(str(p), raise_on_error=False) == ETABLE
    # the previously loaded table stays in force
    assert q.qlin_table_entries() == 1
    assert q.qlin_load_table(str(tmp_path / "missing.tbl"), raise_on_error=False) == ETABLE


def test_installed_table_is_valid():
    if not os.path.exists(q.TABLE_PATH):
        pytest.skip("no installed table")
    assert q.qlin_load_table(q.TABLE_PATH) == OK
    assert q.qlin_table_entries() > 0


def test_graph_calls_reject_null_handles():
    L = q.lib()
    assert L.qlin_graph_launch(None, None) == EINVAL
    assert L.qlin_graph_destroy(None) == EINVAL
    assert L.qlin_graph_begin(None) == EINVAL
    h = ctypes.c_void_p()
    assert L.qlin_graph_end(None, ctypes.byref(h)) == EINVAL


def test_one_hip_runtime_is_mapped():
    """The library binds to torch's HIP runtime instead of mapping a second
    copy (a second runtime would not know torch's stream handles)."""
    import subprocess
    import sys
    code = ("import skinny_bit_gemm_amd as q; q.lib();"
            "m = open('/proc/self/maps').read();"
            "print(len({l.split()[-1] for l in m.splitlines() if 'libamdhip64' in l}))")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT,
                         check=True).stdout.strip().splitlines()[-1]
    assert out == "1"


def test_grouped_gemm_validation():
    def gg(groups=4, N=256, K=512, off=A, total=9, maxr=4, cfg=None, ws=None, wsb=0, fmt=FP8, out=q.QLIN_OUT_BF16):
        return q.qlin_grouped_gemm(fmt, groups, N, K, off, total, maxr, A, A, A, A, A, out, cfg, ws, wsb,
                                   stream=0, raise_on_error=False)
    assert gg(total=0) == OK                                   # nothing to do: no launch
    assert gg(off=None, total=0) == EINVAL
    assert gg(off=A + 2, total=0) == EALIGN
    assert gg(groups=0, total=0) == ESHAPE
    assert gg(total=-1) == ESHAPE
    assert gg(maxr=0, total=0) == ESHAPE
    assert gg(N=100, total=0) == ESHAPE
    assert gg(fmt=BLK, N=192, total=0) == ESHAPE
    assert gg(out=q.QLIN_OUT_I32_ACC, total=0) == EINVAL       # int32 sums: W8A8_INT8 only
    assert gg(cfg=q.make_config(0, 1, 64, 128, 4, 1), total=0) == EINVAL   # large-M tiles: not grouped
    assert gg(cfg=q.make_config(1, 1, 16, 32, 4, 4, 0, 1), total=0) == EINVAL   # codes come quantized
    # grid y: ceil(total / tile rows) + min(groups, total) token tiles, at most 65535
    assert gg(total=70000, maxr=1) == ESHAPE
    assert gg(groups=50000, total=50000, maxr=2) == ESHAPE   # 25000 + 50000 tiles
    assert q.qlin_grouped_workspace_bytes(FP8, 40000, 256, 512, 0, 32) == 0
    split = q.make_config(1, 2, 16, 64, 4, 2)
    need = q.qlin_grouped_workspace_bytes(FP8, 4, 256, 512, 9, 4, split)
    assert need > 0 and q.qlin_grouped_workspace_bytes(FP8, 4, 256, 512, 9, 4) == 0
    assert gg(cfg=split, ws=A, wsb=need - 1) == EWS
    assert gg(cfg=split, ws=None, wsb=need) == EWS
    c = q.qlin_grouped_select_variant(FP8, 128, 1536, 2048, 8)
    assert (c.swap_ab, c.split_k, c.tile_m, c.tile_n, c.act_path) == (1, 1, 16, 64, 0)
    assert q.qlin_grouped_select_variant(I8, 128, 2048, 768, 32).tile_m == 32
    c = q.qlin_grouped_select_variant(FP8, 128, 1536, 2048, 2)
    assert (c.tile_n, c.waves, c.k_waves) == (32, 4, 4)
    assert q.qlin_grouped_select_variant(FP8, 128, 2048, 768, 2).tile_n == 64
    # short rows with more than 2 rows per group: 48-column tiles of 3 waves, whole K per wave
    for fmt, T in ((FP8, 3), (I8, 32), (BLK, 512)):
        c = q.qlin_grouped_select_variant(fmt, 128, 2048, 768, T)
        assert (c.swap_ab, c.split_k, c.tile_m, c.tile_n, c.waves, c.k_waves) == (1, 1, 16 if T <= 16 else 32,
                                                                                    48, 3, 1)
    # 32-token tiles on longer rows: Standard roles
    for K in (1152, 2048):
        c = q.qlin_grouped_select_variant(FP8, 128, 1536, K, 32)
        assert (c.swap_ab, c.tile_m, c.tile_n, c.waves, c.k_waves) == (0, 32, 64, 4, 2)
