"""Host logic of the rocprofv3 summary tool (no GPU): per-kernel trace
statistics split by grid size, counter summaries, and HBM traffic scaled by
the calibration copy."""
from __future__ import annotations

import csv

from transformer_ffn_block_amd import profsum


def _write(path, header, rows):
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(header)
        w.writerows(rows)


def test_stats_splits_a_kernel_by_grid_size(tmp_path):
    p = tmp_path / "trace.csv"
    hdr = ["Kernel_Name", "Grid_Size_X", "Start_Timestamp", "End_Timestamp"]
    rows = [["k_a(int)", 1024, 0, 10000], ["k_a(int)", 1024, 0, 12000],   # 10 / 12 us
            ["k_a(int)", 64, 0, 2000],                                   # 2 us, other grid
            ["k_b(float)", 256, 0, 4000]]                                # one grid only
    _write(p, hdr, rows)
    out = profsum.stats(str(p), "cmd")
    lines = [l for l in out.splitlines() if not l.startswith("#")]
    assert "k_a [grid 1024] | 2 | 11.00 | 11.00 | 10.00 | 12.00" in lines
    assert "k_a [grid 64] | 1 | 2.00 | 2.00 | 2.00 | 2.00" in lines
    assert "k_b | 1 | 4.00 | 4.00 | 4.00 | 4.00" in lines   # no grid tag for a single shape
    assert lines[0].startswith("k_a [grid 1024]")             # sorted by total time


def test_counters_headers_follow_the_counters(tmp_path):
    p = tmp_path / "c.csv"
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    _write(p, hdr, [["kern(int)", "SQ_WAVES", 8], ["kern(int)", "SQ_WAVE_CYCLES", 100],
                    ["kern(int)", "SQ_WAVES", 8], ["kern(int)", "SQ_WAVE_CYCLES", 300]])
    out = profsum.counters(str(p), ["kern"], "cmd")
    assert "wave-cycle shares" in out and "mfma_busy_frac" not in out
    assert "  SQ_WAVE_CYCLES = 200.0" in out and "  dispatches = 2" in out
    q = tmp_path / "m.csv"
    _write(q, hdr, [["g(int)", "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 50], ["g(int)", "GRBM_GUI_ACTIVE", 8 * 100]])
    out = profsum.counters(str(q), ["g"], "cmd")
    assert "mfma_busy_frac = 0.5000" in out          # 51200 / (800 / 8 * 1024)


def test_traffic_scales_by_the_calibration_copy_and_filters_grid(tmp_path):
    hdr = ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    mib = 1 << 20
    # the copy moves 64 MiB each way; its fetch counter reads half of that
    # (scale 2), its write counter all of it (scale 1)
    f = tmp_path / "f.csv"
    _write(f, hdr, [["probe_copy(int)", 1, "FETCH_SIZE", 32 * 1024],
                    ["kern(int)", 4096, "FETCH_SIZE", 1000], ["kern(int)", 4096, "FETCH_SIZE", 1200],
                    ["kern(int)", 64, "FETCH_SIZE", 50]])          # another shape, filtered out
    w = tmp_path / "w.csv"
    _write(w, hdr, [["probe_copy(int)", 1, "WRITE_SIZE", 64 * 1024],
                    ["kern(int)", 4096, "WRITE_SIZE", 10], ["kern(int)", 4096, "WRITE_SIZE", 10],
                    ["kern(int)", 64, "WRITE_SIZE", 1]])
    src = tmp_path / "k.hip"
    src.write_text("kernel source")
    out = profsum.traffic(str(f), str(w), "kern", 64 * mib, str(src), 2_000_000, "PMC run", grid=4096)
    vals = dict(l.split(" = ", 1) for l in out.splitlines() if " = " in l and not l.startswith("#"))
    assert vals["dispatches_fetch"] == "2" and vals["fetch_scale"] == "2.0000" and vals["write_scale"] == "1.0000"
    rd, wr = 1100 * 1024 * 2, 10 * 1024
    assert int(vals["hbm_read_bytes_per_launch"]) == rd and int(vals["hbm_write_bytes_per_launch"]) == wr
    assert vals["traffic_over_algorithmic"] == f"{(rd + wr) / 2_000_000:.4f}"
    assert "FETCH_SIZE run" in out and "WRITE_SIZE run" in out
