"""Host logic of the profile summaries: kernel-name shortening, per-dispatch
counter sums (one dispatch's counter arrives in several instances, one per
hardware unit) and the derived per-wave and L2 figures, on a small
hand-built database of the rocprofv3 layout."""
import sqlite3

from speculative_decoding_spec_amd import rocprof_summary as rs


def test_short_name():
    n = "void spec::(anonymous namespace)::qmv_kernel<4, 8, 2, 1, 2, 1, false>(uint4 const*, int)"
    assert rs.short_name(n) == "qmv_kernel<4, 8, 2, 1, 2, 1, false>"
    assert rs.short_name("spec::(anonymous namespace)::gdn_commit_kernel(float*, int)") == "gdn_commit_kernel"


def make_db(path):
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (kernel_name text, counter_name text, value real, "
                "dispatch_id integer, grid_size_x integer, grid_size_y integer)")
    k = "void spec::(anonymous namespace)::row_stats_kernel<256, 8>(Rows)"
    rows = []
    for disp in (1, 2):
        rows += [(k, "SQ_WAVES", 100.0, disp, 1024, 1),
                 (k, "SQ_INSTS_VALU", 3000.0, disp, 1024, 1),
                 (k, "SQ_INSTS_SALU", 500.0, disp, 1024, 1)]
        # L2 counters in two instances per dispatch, to be summed
        rows += [(k, "TCC_HIT_sum", 10.0, disp, 1024, 1), (k, "TCC_HIT_sum", 15.0, disp, 1024, 1),
                 (k, "TCC_MISS_sum", 60.0, disp, 1024, 1), (k, "TCC_MISS_sum", 15.0, disp, 1024, 1)]
    rows.append(("void other(int)", "SQ_WAVES", 7.0, 3, 64, 1))
    con.executemany("insert into counters_collection values (?, ?, ?, ?, ?, ?)", rows)
    con.commit()
    con.close()


def test_counter_rows_sum_instances_and_average_dispatches(tmp_path):
    db = str(tmp_path / "c.db")
    make_db(db)
    rows = {(r["kernel"], r["counter"]): r for r in rs.counter_rows(db, ["spec::"])}
    assert ("other", "SQ_WAVES") not in rows
    hit = rows[("row_stats_kernel<256, 8>", "TCC_HIT_sum")]
    assert hit["dispatches"] == 2 and hit["avg"] == 25.0
    assert rows[("row_stats_kernel<256, 8>", "TCC_MISS_sum")]["avg"] == 75.0


def test_derived_per_wave_and_hit_rate(tmp_path, capsys):
    db = str(tmp_path / "c.db")
    make_db(db)
    rs.derived(db, ["spec::"])
    line = [l for l in capsys.readouterr().out.splitlines() if l.startswith("row_stats")][0]
    waves, valu, salu, hit = line.split()[-4:]
    assert float(waves) == 100 and float(valu) == 30.0 and float(salu) == 5.0
    assert float(hit) == 25.0          # 25 / (25 + 75)
