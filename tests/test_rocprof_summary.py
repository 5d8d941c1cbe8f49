"""The profile summaries (block_diffusion_vlm_amd.rocprof_summary) on small
SQLite databases shaped like rocprofv3's views, with known values: the
per-kernel durations of a kernel trace, the counter averages and MFMA busy
fractions of a counter run, and the calibrated HBM bytes of the traffic
summary."""
import json
import sqlite3

import pytest

from block_diffusion_vlm_amd import rocprof_summary as rs

KNAME = "void bd::(anonymous namespace)::dualstream_bf16_kernel<4, false, false>(args)"


def _trace_db(path, rows):
    con = sqlite3.connect(path)
    con.execute("create table kernels (id, name, start, end, grid_x, grid_y, grid_z)")
    con.executemany("insert into kernels values (?, ?, ?, ?, 1, 1, 1)", rows)
    con.commit()
    con.close()


def _pmc_db(path, rows):
    """rows: (dispatch, kernel, counter, value, duration ns)"""
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (dispatch_id, kernel_name, counter_name, "
                "value, duration, vgpr_count, accum_vgpr_count, sgpr_count, lds_block_size, "
                "grid_size_x, grid_size_y, grid_size_z)")
    con.executemany("insert into counters_collection values (?, ?, ?, ?, ?, 128, 64, 40, "
                    "65536, 1, 1, 1)", rows)
    con.commit()
    con.close()


def test_trace_reports_calls_and_durations(tmp_path):
    db = str(tmp_path / "t.db")
    _trace_db(db, [(1, KNAME, 0, 100_000), (2, KNAME, 200_000, 300_000),
                   (3, KNAME, 400_000, 520_000), (4, "copy", 0, 10_000)])
    out = rs.trace(db).splitlines()
    row = next(x for x in out if "dualstream_bf16_kernel" in x).split()
    # calls, avg, median, min, max (us)
    assert row[-6:-1] == ["3", "106.67", "100.00", "100.00", "120.00"]
    assert "(anonymous namespace)" not in out[1]


def test_trace_by_grid_separates_shapes(tmp_path):
    db = str(tmp_path / "g.db")
    con = sqlite3.connect(db)
    con.execute("create table kernels (id, name, start, end, grid_x, grid_y, grid_z)")
    con.executemany("insert into kernels values (?, ?, ?, ?, ?, ?, ?)",
                    [(1, KNAME, 0, 10_000, 21, 2, 1), (2, KNAME, 0, 30_000, 37, 2, 2),
                     (3, KNAME, 0, 12_000, 21, 2, 1)])
    con.commit()
    con.close()
    lines = [x for x in rs.trace(db, by_grid=True).splitlines() if "dualstream" in x]
    assert len(lines) == 2
    small = next(x for x in lines if "(21, 2, 1)" in x).split()
    assert small[-6:-1] == ["2", "11.00", "12.00", "10.00", "12.00"]
    big = next(x for x in lines if "(37, 2, 2)" in x).split()
    assert big[-6:-1] == ["1", "30.00", "30.00", "30.00", "30.00"]
    # without grouping by grid the three dispatches share one line
    assert [x.split()[-6] for x in rs.trace(db).splitlines() if "dualstream" in x] == ["3"]


def test_mfma_summary_fractions(tmp_path):
    pmc, tr = str(tmp_path / "p.db"), str(tmp_path / "t.db")
    busy = 0.25 * rs.SIMD_NUM * 100e-6 * 2.4e9        # a quarter of the pipes' cycles in 100 us
    rows = []
    for d in (1, 2):
        rows += [(d, KNAME, "SQ_VALU_MFMA_BUSY_CYCLES", busy, 110_000),
                 (d, KNAME, "GRBM_GUI_ACTIVE", 8 * 300_000.0, 110_000),
                 (d, KNAME, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 1e8, 110_000),
                 (d, KNAME, "SQ_INSTS_MFMA", 1000.0, 110_000),
                 (d, KNAME, "SQ_INSTS_VALU", 3000.0, 110_000)]
    _pmc_db(pmc, rows)
    _trace_db(tr, [(1, KNAME, 0, 100_000), (2, KNAME, 0, 100_000)])
    text = rs.mfma(pmc, tr)
    vals = {ln[:38].strip(): ln[38:].strip() for ln in text.splitlines() if ln.startswith("    ")}
    assert float(vals["MFMA busy % at 2.4 GHz"]) == pytest.approx(25.0)
    assert float(vals["median duration (us), trace"]) == pytest.approx(100.0)
    # no instance table in this database: GRBM_GUI_ACTIVE counts as one instance
    assert float(vals["MfmaUtil % (per GRBM instance)"]) == pytest.approx(
        100.0 * busy / (8 * 300_000.0 * rs.SIMD_NUM))
    assert float(vals["bf16 MFMA GFLOP executed"]) == pytest.approx(51.2)
    assert float(vals["SQ_INSTS_VALU per MFMA"]) == pytest.approx(3.0)
    # without the trace, the counter run's own durations are used
    vals = {ln[:38].strip(): ln[38:].strip() for ln in rs.mfma(pmc).splitlines()
            if ln.startswith("    ")}
    assert float(vals["median duration (us), pmc run"]) == pytest.approx(110.0)


def test_traffic_scales_by_the_calibration_copy(tmp_path):
    f, w, j = (str(tmp_path / x) for x in ("f.db", "w.db", "o.json"))
    kib = rs.COPY_BYTES / 1024
    for db, cname, copy_val, lm_val in ((f, "FETCH_SIZE", kib / 2, 1000.0),
                                        (w, "WRITE_SIZE", kib, 10.0)):
        con = sqlite3.connect(db)
        con.execute("create table counters_collection (dispatch_id, kernel_name, counter_name, "
                    "value, grid_size_x, grid_size_y, grid_size_z)")
        con.executemany("insert into counters_collection values (?, ?, ?, ?, 1, 1, 1)", [
            (1, "__amd_rocclr_copyBuffer", cname, copy_val),
            (2, "__amd_rocclr_copyBuffer", cname, 0.5),          # a small restore copy
            (3, "void bd::lmhead_bf16_kernel<1, 4>(x)", cname, lm_val),
            (4, "bd::lmhead_combine_kernel(x)", cname, 2.0)])
        con.commit()
        con.close()
    res = rs.traffic(f, w, j, "bf16")
    assert res["fetch"]["scale"] == pytest.approx(2.0)
    assert res["write"]["scale"] == pytest.approx(1.0)
    assert res["hbm_bytes_per_call"] == pytest.approx((1002.0 * 2 + 12.0) * 1024)
    assert json.loads(open(j).read())["kernel_source_sha"] == res["kernel_source_sha"]
