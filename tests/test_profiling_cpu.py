"""CPU tests of the profile-summary helpers: the kernel-source hash that ties a
counter summary to the code it was taken on follows code, not comments, and
covers exactly the headers a translation unit includes."""
import os
import shutil

import pytest

from modulation_bf16_row_amd import profiling


def test_code_only_strips_comments_and_whitespace_keeps_literals():
    src = 'int a = 1; // note\n/* block\n comment */ const char *s = "x // y"; char q = \'"\';\n'
    assert profiling._code_only(src) == 'inta=1;constchar*s="x // y";charq=\'"\';'


def test_unit_files_follow_local_includes():
    files = profiling.unit_files("dit_ln.hip")
    assert {"dit_ln.hip", "dit_ln.hpp", "dit_rows.hpp", "dit_device.hpp",
            "dit_launch.hpp"} <= set(files)
    assert "dit_qkv.hip" not in files
    assert "dit_divide.hpp" in profiling.unit_files("dit_modtab.hip")


@pytest.fixture
def csrc_copy(tmp_path, monkeypatch):
    d = tmp_path / "csrc"
    shutil.copytree(profiling.CSRC, d)
    monkeypatch.setattr(profiling, "CSRC", str(d))
    return d


def _edit(path, old, new):
    text = path.read_text(encoding="utf-8")
    assert old in text
    path.write_text(text.replace(old, new, 1), encoding="utf-8")


def test_hash_ignores_comment_edits_and_sees_code_edits(csrc_copy):
    h_unit, h_all = profiling.kernel_source_hash("dit_ln.hip"), profiling.kernel_source_hash()
    _edit(csrc_copy / "dit_ln.hip", "// dit_ln.hip", "//   dit_ln.hip (edited comment)")
    assert profiling.kernel_source_hash("dit_ln.hip") == h_unit
    assert profiling.kernel_source_hash() == h_all
    _edit(csrc_copy / "dit_ln.hip", "namespace dit {", "namespace dit {\nconstexpr int kUnused = 1;")
    assert profiling.kernel_source_hash("dit_ln.hip") != h_unit


def test_unit_hash_sees_included_headers_only(csrc_copy):
    h_ln = profiling.kernel_source_hash("dit_ln.hip")
    h_qkv = profiling.kernel_source_hash("dit_qkv.hip")
    _edit(csrc_copy / "dit_rows.hpp", "namespace dit {", "namespace dit {\nconstexpr int kX = 2;")
    assert profiling.kernel_source_hash("dit_ln.hip") != h_ln      # dit_ln.hip includes it
    assert profiling.kernel_source_hash("dit_qkv.hip") == h_qkv    # dit_qkv.hip does not


def test_clock_stats_from_a_grbm_count_table(tmp_path):
    """Effective clock = GRBM_COUNT / 8 XCDs / duration; a kernel whose
    dispatches all take the same core cycles shows a correlation of -1."""
    import sqlite3
    from modulation_bf16_row_amd import profiling
    db = str(tmp_path / "c.db")
    con = sqlite3.connect(db)
    con.execute("create table counters_collection (dispatch_id int, kernel_name text, "
                "grid_size int, counter_name text, value real, duration real)")
    cycles = 1.0e6                                    # per XCD
    for i, ghz in enumerate([2.0, 2.1, 2.2, 2.3, 2.4]):
        dur_ns = cycles / ghz
        con.execute("insert into counters_collection values (?, ?, ?, ?, ?, ?)",
                    (i, "void dit::k_a<1>(dit::Args)", 64, "GRBM_COUNT", 8 * cycles, dur_ns))
    con.execute("insert into counters_collection values (9, 'void k_short()', 64, 'GRBM_COUNT', "
                "8.0, 1000.0)")                        # 1 us: below the 200 us floor
    con.commit()
    rows = profiling.clock_stats(db)
    assert len(rows) == 1
    name, grid, n, med_us, clk, lo, hi, kcyc, r = rows[0]
    assert (name, grid, n) == ("k_a<1>", 64, 5)
    assert abs(clk - 2.2) < 1e-9 and abs(lo - 2.0) < 1e-9 and abs(hi - 2.4) < 1e-9
    assert abs(kcyc - 1000.0) < 1e-6
    assert r < -0.99


def test_counter_table_medians_per_kernel(tmp_path):
    import sqlite3
    from modulation_bf16_row_amd import profiling
    db = str(tmp_path / "q.db")
    con = sqlite3.connect(db)
    con.execute("create table counters_collection (dispatch_id int, kernel_name text, "
                "grid_size int, counter_name text, value real)")
    for d, v in enumerate([100.0, 300.0, 200.0]):
        con.execute("insert into counters_collection values (?, ?, ?, ?, ?)",
                    (d, "void dit::k_b<2>(dit::Args)", 128, "SQ_INSTS_VALU", v))
        con.execute("insert into counters_collection values (?, ?, ?, ?, ?)",
                    (d, "void dit::k_b<2>(dit::Args)", 128, "SQ_WAVES", 2.0))
    con.commit()
    t = profiling.counter_table(db)
    assert t == {("k_b<2>", 128): {"SQ_INSTS_VALU": 200.0, "SQ_WAVES": 2.0}}
