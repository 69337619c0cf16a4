"""CPU checks of the offline tuner's host logic: which schedule a merge keeps,
and that tables round-trip (entries and notes) into a file the library loads."""
import os

import skinny_bit_gemm_amd as q
from skinny_bit_gemm_amd import tune


def test_merge_keeps_the_existing_entry_unless_clearly_beaten():
    a, b = q.make_config(1, 1, 16, 16, 4, 4), q.make_config(1, 1, 16, 8, 4, 4)
    # within the margin: the existing entry stays
    assert tune.keep_or_replace(9.9, b, 10.0, a, 0.02) == (10.0, a, True)
    assert tune.keep_or_replace(9.81, b, 10.0, a, 0.02) == (10.0, a, True)
    # faster by more than the margin: replaced
    assert tune.keep_or_replace(9.7, b, 10.0, a, 0.02) == (9.7, b, False)
    # slower: kept
    assert tune.keep_or_replace(10.5, b, 10.0, a, 0.02) == (10.0, a, True)
    # nothing to keep
    assert tune.keep_or_replace(9.9, b, None, None, 0.02) == (9.9, b, False)
    # margin 0: any improvement wins
    assert tune.keep_or_replace(9.99, b, 10.0, a, 0.0) == (9.99, b, False)


def test_table_round_trip_keeps_entries_and_notes(tmp_path):
    entries, notes = tune.read_entries(q.TABLE_PATH)
    assert len(entries) >= 200 and all(len(v) == 8 for v in entries.values())
    out = os.path.join(str(tmp_path), "t.tbl")
    tune.write_entries(out, entries, notes)
    again, notes2 = tune.read_entries(out)
    assert again == entries and notes2 == notes
    try:
        assert q.qlin_load_table(out, raise_on_error=False) == 0
        assert q.qlin_table_entries() == len(entries)
    finally:
        q.qlin_load_table(q.TABLE_PATH)


def test_candidate_grid_token_tiles():
    """The grid's token tiles per bucket: 16 rows up to 16 tokens, 16 and 32
    to 32 tokens, the skinny kernel's 64-token tiles joining past 32 tokens
    and the large-M kernel's layout from 33 tokens on; every candidate is a
    valid schedule, and only the large-M layout is classed as large-M."""
    q.lib()
    fmt, N, K = q.QLIN_FP8_DYNAMIC, 24576, 4096

    def tiles(M):
        return {(c.tile_m, tune.variant_class(c) == "large_m") for c in tune.candidates(fmt, M, N, K)}

    assert tiles(8) == {(16, False)}
    assert tiles(32) == {(16, False), (32, False)}
    assert tiles(64) == {(16, False), (32, False), (64, False), (64, True), (128, True)}
    assert tiles(256) == {(32, False), (64, False), (64, True), (128, True)}
    for M in (8, 64, 256):
        for c in tune.candidates(fmt, M, N, K):
            assert q.qlin_validate_config(fmt, M, N, K, c) == 0, c
            if tune.variant_class(c) == "large_m":
                assert (c.tile_n, c.waves, c.k_waves, c.swap_ab, c.reduce, c.act_path) == (128, 4, 1, 0, 0, 0)
