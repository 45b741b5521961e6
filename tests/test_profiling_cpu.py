"""Host logic of the profile summaries (no GPU): counter reduction per
dispatch, scaling by the calibration copy, attention totals, trace tables,
and the bench's rule that a counter summary taken on another kernel source
gives no traffic figure."""
import json
import os
import sqlite3

import pytest

from tree_attention_verification_parent_amd import profiling as P

RING = "void eagle::tree_attn_ring_kernel<eagle::RingShape<128, 2, 2> >(eagle::AttnArgs)"
MERGE = "void eagle::tree_attn_merge_kernel<128>(eagle::AttnArgs, int)"
COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>(int)"


def _db(path, rows, kernels=()):
    """rows: (kernel, dispatch, counter, value, start, end) of counters_collection."""
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (kernel_name text, dispatch_id int, "
                "counter_name text, value real, start int, end int)")
    con.executemany("insert into counters_collection values (?, ?, ?, ?, ?, ?)", rows)
    con.execute("create table kernels (name text, start int, end int)")
    con.executemany("insert into kernels values (?, ?, ?)", kernels)
    con.commit()
    con.close()
    return path


def test_counters_sum_dimensions_and_scale_by_the_copy(tmp_path):
    copy_bytes = 1 << 20
    # FETCH_SIZE reads half the bytes of the copy (KiB): scale 2; two XCD rows per dispatch
    fetch = _db(str(tmp_path / "fetch_results.db"), [
        (COPY, 9, "FETCH_SIZE", copy_bytes / 1024 / 4, 0, 1),
        (COPY, 9, "FETCH_SIZE", copy_bytes / 1024 / 4, 0, 1),
        (RING, 1, "FETCH_SIZE", 100.0, 0, 1), (RING, 1, "FETCH_SIZE", 50.0, 0, 1),
        (RING, 2, "FETCH_SIZE", 160.0, 0, 1),
    ])
    write = _db(str(tmp_path / "write_results.db"), [
        (COPY, 9, "WRITE_SIZE", copy_bytes / 1024, 0, 1),
        (RING, 1, "WRITE_SIZE", 10.0, 0, 1), (RING, 2, "WRITE_SIZE", 10.0, 0, 1),
    ])
    s = P.pmc_summary([fetch], [write], copy_bytes, "f", "w", "toy")
    assert s["scale"]["FETCH_SIZE"] == pytest.approx(2.0)
    assert s["scale"]["WRITE_SIZE"] == pytest.approx(1.0)
    k = s["kernels"][P.short_name(RING)]
    assert k["dispatches"] == 2
    assert k["fetch_kib"] == pytest.approx(155.0)  # median of 150 and 160
    assert s["tree_attn_hbm_bytes_per_launch"] == pytest.approx(155.0 * 1024 * 2 + 10.0 * 1024)


def test_attention_counter_table(tmp_path):
    copy_bytes = 1 << 20
    rows_f = [(COPY, 9, "FETCH_SIZE", copy_bytes / 1024 / 2, 0, 10),
              (RING, 1, "FETCH_SIZE", 1000.0, 0, 10), (MERGE, 2, "FETCH_SIZE", 24.0, 0, 10)]
    rows_w = [(COPY, 9, "WRITE_SIZE", copy_bytes / 1024, 0, 10),
              (RING, 1, "WRITE_SIZE", 100.0, 0, 10), (MERGE, 2, "WRITE_SIZE", 8.0, 0, 10)]
    # 10 us dispatch: busy cycles = 25 % of 10e-6 s x 2.4 GHz x 1024 SIMDs
    busy = 0.25 * 10e-6 * P.CLOCK_HZ * P.SIMD_COUNT
    rows_m = [(RING, 1, "SQ_VALU_MFMA_BUSY_CYCLES", busy, 0, 10000),
              (RING, 1, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 1e6, 0, 10000),
              (RING, 1, "GRBM_GUI_ACTIVE", 8 * 24000.0, 0, 10000),
              (MERGE, 2, "SQ_VALU_MFMA_BUSY_CYCLES", 0.0, 0, 2000),
              (MERGE, 2, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0, 0, 2000)]
    text = P.attn_counters([_db(str(tmp_path / "f_results.db"), rows_f)],
                           [_db(str(tmp_path / "w_results.db"), rows_w)],
                           [_db(str(tmp_path / "m_results.db"), rows_m)],
                           copy_bytes, 2_000_000, 400_000_000, "cmd <COUNTERS>", "toy")
    ring_line = next(l for l in text.splitlines() if "ring_kernel" in l)
    cells = [c.strip() for c in ring_line.split("|")]
    assert cells[3] == f"{1000.0 * 1024 * 2 / 1e6:.2f}"   # fetched MB, scale 2
    assert cells[6] == "25.0"                              # MFMA busy %
    assert cells[7] == f"{512e6 / 1e9:.2f}"                # GFLOP
    assert "cmd FETCH_SIZE" in text and "cmd WRITE_SIZE" in text
    total = (1000.0 + 24.0) * 1024 * 2 + (100.0 + 8.0) * 1024
    assert f"{total / 2_000_000:.3f} x algorithmic" in text


def test_trace_table_orders_by_total_time(tmp_path):
    db = _db(str(tmp_path / "t_results.db"), [],
             kernels=[(RING, 0, 14000), (RING, 0, 16000), (MERGE, 0, 50000)])
    text = P.trace_table([db], "cmd")
    lines = [l for l in text.splitlines() if l.startswith("| `")]
    assert "merge" in lines[0] and "ring" in lines[1]
    assert "| 2 | 15.000 | 15.000 | 14.000 | 16.000 |" in lines[1]


def test_missing_calibration_copy_is_an_error(tmp_path):
    f = _db(str(tmp_path / "f_results.db"), [(RING, 1, "FETCH_SIZE", 1.0, 0, 1)])
    w = _db(str(tmp_path / "w_results.db"), [(RING, 1, "WRITE_SIZE", 1.0, 0, 1)])
    with pytest.raises(SystemExit):
        P.pmc_summary([f], [w], 1 << 20, "f", "w", "toy")


def test_bench_traffic_needs_the_current_kernel_source(tmp_path, monkeypatch):
    import bench
    summary = tmp_path / "pmc.json"
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(summary))
    assert bench.pmc_traffic(1) is None  # no summary
    summary.write_text(json.dumps({"kernel_source_sha": bench.kernel_source_hash(),
                                   "tree_attn_hbm_bytes_per_launch": 123.0}))
    assert bench.pmc_traffic(1) == 123.0
    summary.write_text(json.dumps({"kernel_source_sha": "0" * 16,
                                   "tree_attn_hbm_bytes_per_launch": 123.0}))
    assert bench.pmc_traffic(1) is None  # taken on another source
