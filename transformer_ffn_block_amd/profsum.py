"""Summaries of rocprofv3 CSV output for the profiles/ folder.

  python -m transformer_ffn_block_amd.profsum stats KERNEL_TRACE_CSV --command "..."
      per-kernel dispatch count, average / min / max duration (us)
  python -m transformer_ffn_block_amd.profsum traffic FETCH_CSV WRITE_CSV \\
        --kernel SUBSTRING --copy-bytes N --source FILE --bytes-per-launch B --command "..." [--grid G]
      HBM traffic per launch of the matching kernel from FETCH_SIZE and
      WRITE_SIZE (KiB per dispatch), each scaled by what the same counter
      reads for the library's plain copy kernel (probe_copy) of known size.
  python -m transformer_ffn_block_amd.profsum counters COUNTER_CSV --kernel SUBSTRING [--kernel ...] --command "..."
      per-dispatch means of the counters of one --pmc run, and the MFMA busy
      fraction when its counters are present.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import statistics
import sys


def _rows(path):
    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def stats(trace_csv: str, command: str) -> str:
    """Per-kernel duration statistics; a kernel launched with several grid
    sizes (one template at different shapes) gets one line per grid size."""
    per = collections.defaultdict(list)
    grids = collections.defaultdict(set)
    for r in _rows(trace_csv):
        name = r.get("Kernel_Name") or r.get("Name")
        grid = r.get("Grid_Size_X") or r.get("Grid_Size") or ""
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
        per[(name, grid)].append(dur)
        grids[name].add(grid)
    out = [f"# rocprofv3 kernel trace summary", f"# command: {command}",
           "# kernel | dispatches | avg_us | median_us | min_us | max_us"]
    for (name, grid), d in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        short = name.split("(")[0]
        if len(grids[name]) > 1:
            short += f" [grid {grid}]"
        out.append(f"{short} | {len(d)} | {statistics.fmean(d):.2f} | {statistics.median(d):.2f} | "
                   f"{min(d):.2f} | {max(d):.2f}")
    return "\n".join(out) + "\n"


def _counter(path: str, counter: str, grid=None):
    per = collections.defaultdict(list)
    for r in _rows(path):
        if r["Counter_Name"] != counter:
            continue
        if grid is not None and "probe_copy" not in r["Kernel_Name"] and int(r["Grid_Size"]) != grid:
            continue
        per[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return per


def _pick(per, sub):
    hits = [(k, v) for k, v in per.items() if sub in k]
    if not hits:
        raise SystemExit(f"no kernel matching {sub!r}")
    k, v = max(hits, key=lambda kv: len(kv[1]))
    return k, statistics.fmean(v), len(v)


def traffic(fetch_csv, write_csv, kernel, copy_bytes, source, bytes_per_launch, command,
            grid=None, copy_kernel="probe_copy") -> str:
    f_per, w_per = _counter(fetch_csv, "FETCH_SIZE", grid), _counter(write_csv, "WRITE_SIZE", grid)
    kname, f_kib, nf = _pick(f_per, kernel)
    _, w_kib, nw = _pick(w_per, kernel)
    _, cf_kib, _ = _pick(f_per, copy_kernel)
    _, cw_kib, _ = _pick(w_per, copy_kernel)
    f_scale = copy_bytes / (cf_kib * 1024.0)  # true bytes per counted byte (reads)
    w_scale = copy_bytes / (cw_kib * 1024.0)  # (writes)
    rd = f_kib * 1024.0 * f_scale
    wr = w_kib * 1024.0 * w_scale
    with open(source, "rb") as fh:
        sha = hashlib.sha256(fh.read()).hexdigest()
    lines = [
        "# HBM traffic per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per dispatch),",
        f"# each scaled by the same counter's reading for {copy_kernel} moving copy_bytes",
        f"# command (fetch pass): {command.replace('PMC', 'FETCH_SIZE')}",
        f"# command (write pass): {command.replace('PMC', 'WRITE_SIZE')}",
        f"kernel = {kname.split('(')[0]}",
        f"grid_size = {grid if grid is not None else 'any'}",
        f"dispatches_fetch = {nf}",
        f"dispatches_write = {nw}",
        f"fetch_kib_per_dispatch = {f_kib:.1f}",
        f"write_kib_per_dispatch = {w_kib:.1f}",
        f"copy_bytes = {copy_bytes}",
        f"copy_fetch_kib = {cf_kib:.1f}",
        f"copy_write_kib = {cw_kib:.1f}",
        f"fetch_scale = {f_scale:.4f}",
        f"write_scale = {w_scale:.4f}",
        f"hbm_read_bytes_per_launch = {rd:.0f}",
        f"hbm_write_bytes_per_launch = {wr:.0f}",
        f"hbm_bytes_per_launch = {rd + wr:.0f}",
        f"algorithmic_bytes_per_launch = {bytes_per_launch}",
        f"traffic_over_algorithmic = {(rd + wr) / bytes_per_launch:.4f}",
        f"source = {source.split('/root/repo/')[-1]}",
        f"source_sha256 = {sha}",
    ]
    return "\n".join(lines) + "\n"


def counters(csv_path: str, kernels, command: str, xcds: int = 8, simds: int = 1024) -> str:
    """Per-dispatch means of every counter in one --pmc run for each kernel
    matching a substring; with SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE
    also the MFMA busy fraction = busy cycles summed over SIMDs / (GUI-active
    cycles per XCD x SIMDs)."""
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    names = set()
    for r in _rows(csv_path):
        per[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
        names.add(r["Counter_Name"])
    out = ["# rocprofv3 counter summary (per-dispatch means)", f"# command: {command}"]
    if "SQ_VALU_MFMA_BUSY_CYCLES" in names:
        out.append(f"# mfma_busy_frac = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {xcds} * {simds})")
    if "SQ_WAVE_CYCLES" in names:
        out.append("# wave-cycle shares: SQ_WAIT_INST_ANY, SQ_WAIT_ANY and SQ_ACTIVE_INST_* over SQ_WAVE_CYCLES")
    for sub in kernels:
        hits = [(k, v) for k, v in per.items() if sub in k]
        if not hits:
            raise SystemExit(f"no kernel matching {sub!r}")
        k, cv = max(hits, key=lambda kv: max(len(x) for x in kv[1].values()))
        out.append(f"kernel = {k.split('(')[0]}")
        means = {c: statistics.fmean(v) for c, v in sorted(cv.items())}
        out.append(f"  dispatches = {max(len(v) for v in cv.values())}")
        for c, m in means.items():
            out.append(f"  {c} = {m:.1f}")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in means and means.get("GRBM_GUI_ACTIVE"):
            frac = means["SQ_VALU_MFMA_BUSY_CYCLES"] / (means["GRBM_GUI_ACTIVE"] / xcds * simds)
            out.append(f"  mfma_busy_frac = {frac:.4f}")
    return "\n".join(out) + "\n"


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("trace_csv")
    s.add_argument("--command", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_csv")
    t.add_argument("write_csv")
    t.add_argument("--kernel", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--source", required=True)
    t.add_argument("--bytes-per-launch", type=int, required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--grid", type=int, default=None, help="only dispatches of this grid size")
    t.add_argument("--copy-kernel", default="probe_copy",
                   help="substring naming the calibration copy kernel")
    c = sub.add_parser("counters")
    c.add_argument("csv")
    c.add_argument("--kernel", action="append", required=True, help="substring; repeatable")
    c.add_argument("--command", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        sys.stdout.write(stats(a.trace_csv, a.command))
    elif a.cmd == "counters":
        sys.stdout.write(counters(a.csv, a.kernel, a.command))
    else:
        sys.stdout.write(traffic(a.fetch_csv, a.write_csv, a.kernel, a.copy_bytes, a.source,
                                 a.bytes_per_launch, a.command, a.grid, a.copy_kernel))
    return 0


if __name__ == "__main__":
    sys.exit(main())
