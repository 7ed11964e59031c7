"""Turn rocprofv3 output into the short summaries kept under profiles/.

    python -m nested_integer_weight_amd.profiling summary STATS_CSV [--trace TRACE_CSV] --title T --cmd C
        markdown table of a `--kernel-trace --stats --output-format csv` run;
        with the kernel-trace CSV it also gives each kernel's median dispatch
        duration, and per grid size for the kernels named by --split

    python -m nested_integer_weight_amd.profiling traffic --fetch DB --write DB \
        --kernel SUBSTR [--grid N] --copy-bytes N --src FILE --cmd C --out JSON
        HBM bytes per dispatch of one kernel (optionally one grid size) from a
        FETCH_SIZE run and a WRITE_SIZE run (rocpd SQLite databases), each
        scaled by what the same counter reads for the last device copy in the
        run (bench.py's calibration copy of known size, `--copy-bytes`), which
        calibrates the counter's coverage.

    python -m nested_integer_weight_amd.profiling counters DB --kernel SUBSTR [...] --title T --cmd C
        mean value per dispatch of every counter of a `--pmc` run, per kernel
        and grid size, for the kernels matching the substrings

The databases are the `*_results.db` files rocprofv3 writes with `--pmc`.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import sqlite3
import statistics
import sys
from collections import defaultdict


def _trace_durations(trace_csv: str):
    """{kernel_name: [durations in ns]} and {(kernel_name, grid): [...]}."""
    by_name, by_grid = defaultdict(list), defaultdict(list)
    for r in csv.DictReader(open(trace_csv)):
        d = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        name = r["Kernel_Name"]
        grid = int(r.get("Grid_Size_X", r.get("Grid_Size", 0)) or 0)
        by_name[name].append(d)
        by_grid[(name, grid)].append(d)
    return by_name, by_grid


def summary(stats_csv: str, title: str, cmd: str, trace_csv: str | None = None, split=()) -> str:
    rows = list(csv.DictReader(open(stats_csv)))
    med = {}
    by_grid = {}
    if trace_csv:
        by_name, by_grid = _trace_durations(trace_csv)
        med = {k: statistics.median(v) for k, v in by_name.items()}
    out = [f"# {title}", "", "Command (from the repository root, on one MI355X):", "", "```", cmd, "```", "",
           "Source: `rocprofv3 --kernel-trace --stats` kernel_stats.csv (GPU-side dispatch durations)"
           + (" and kernel_trace.csv (medians)." if trace_csv else "."), "",
           "| kernel | calls | avg us | median us | min us | max us | % of GPU time |",
           "|---|---:|---:|---:|---:|---:|---:|"]
    for r in rows:
        m = med.get(r["Name"])
        out.append(f"| `{r['Name'][:100]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{'' if m is None else f'{m / 1e3:.2f}'} | {int(r['MinNs']) / 1e3:.2f} | "
                   f"{int(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
    if split and by_grid:
        out += ["", "Per grid size (work-items) for the kernels named above:", "",
                "| kernel | grid | calls | median us | avg us |", "|---|---:|---:|---:|---:|"]
        for (name, grid), v in sorted(by_grid.items(), key=lambda t: (t[0][0], t[0][1])):
            if any(s in name for s in split):
                out.append(f"| `{name[:80]}` | {grid} | {len(v)} | {statistics.median(v) / 1e3:.2f} | "
                           f"{sum(v) / len(v) / 1e3:.2f} |")
    return "\n".join(out) + "\n"


def _per_dispatch(db: str, counter: str):
    """{(kernel_name, grid_size): (mean counter value per dispatch, dispatches)}"""
    c = sqlite3.connect(db)
    rows = c.execute("""select kernel_name, grid_size, avg(value), count(*) from counters_collection
                        where counter_name = ? group by kernel_name, grid_size""", (counter,)).fetchall()
    return {(r[0], r[1]): (r[2], r[3]) for r in rows}


def _kernel_value(d: dict, substr: str, grid=None):
    vals = [(v, n) for (name, g), (v, n) in d.items() if substr in name and (grid is None or g == grid)]
    if not vals:
        raise SystemExit(f"no dispatch of a kernel matching {substr!r} (grid {grid})")
    tot = sum(v * n for v, n in vals)
    cnt = sum(n for _, n in vals)
    return tot / cnt, cnt


def _last_copy_value(db: str, counter: str):
    """Counter value of the last device-copy dispatch of the run (the
    calibration copy bench.py issues after its timed work)."""
    c = sqlite3.connect(db)
    row = c.execute("""select value from counters_collection where counter_name = ? and kernel_name like '%copyBuffer%'
                       order by start desc limit 1""", (counter,)).fetchone()
    if row is None:
        raise SystemExit("no device copy dispatch found for calibration")
    return row[0]


def traffic(fetch_db, write_db, kernel, copy_bytes, src, cmd, grid=None):
    f = _per_dispatch(fetch_db, "FETCH_SIZE")
    w = _per_dispatch(write_db, "WRITE_SIZE")
    fk, nf = _kernel_value(f, kernel, grid)
    wk, nw = _kernel_value(w, kernel, grid)
    fc = _last_copy_value(fetch_db, "FETCH_SIZE")
    wc = _last_copy_value(write_db, "WRITE_SIZE")
    f_scale = (copy_bytes / 1024.0) / fc if fc > 0 else None
    w_scale = (copy_bytes / 1024.0) / wc if wc > 0 else None
    fetch_bytes = fk * 1024.0 * f_scale if f_scale else None
    write_bytes = wk * 1024.0 * w_scale if w_scale else None
    with open(src, "rb") as fh:
        h = hashlib.sha256(fh.read()).hexdigest()[:16]
    return {
        "kernel_substr": kernel,
        "grid_size": grid,
        "kernel_src": src,
        "kernel_src_sha256_16": h,
        "dispatches": {"fetch_run": nf, "write_run": nw},
        "fetch_kib_per_dispatch_raw": round(fk, 1),
        "write_kib_per_dispatch_raw": round(wk, 1),
        "copy_calibration": {"copy_bytes": copy_bytes, "fetch_kib_raw": round(fc, 1), "write_kib_raw": round(wc, 1),
                             "fetch_scale": f_scale, "write_scale": w_scale},
        "hbm_fetch_bytes_per_launch": round(fetch_bytes) if fetch_bytes is not None else None,
        "hbm_write_bytes_per_launch": round(write_bytes) if write_bytes is not None else None,
        "hbm_bytes_per_launch": round(fetch_bytes + write_bytes) if fetch_bytes is not None and write_bytes is not None else None,
        "command": cmd,
    }


def counters(db: str, kernels, title: str, cmd: str) -> str:
    c = sqlite3.connect(db)
    rows = c.execute("""select kernel_name, grid_size, counter_name, avg(value), count(*) from counters_collection
                        group by kernel_name, grid_size, counter_name""").fetchall()
    table = defaultdict(dict)
    names = set()
    for name, grid, counter, v, n in rows:
        if any(k in name for k in kernels):
            table[(name, grid)][counter] = (v, n)
            names.add(counter)
    cols = sorted(names)
    out = [f"# {title}", "", "Command (from the repository root, on one MI355X):", "", "```", cmd, "```", "",
           "Source: `rocprofv3 --pmc` counters (rocpd database), mean value per dispatch, summed over the device.",
           "", "| kernel | grid (work-items) | dispatches | " + " | ".join(cols) + " |",
           "|---|---:|---:|" + "---:|" * len(cols)]
    for (name, grid), d in sorted(table.items()):
        n = max(v[1] for v in d.values())
        out.append(f"| `{name[:90]}` | {grid} | {n} | " +
                   " | ".join(f"{d[k][0]:.4g}" if k in d else "" for k in cols) + " |")
    return "\n".join(out) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("summary")
    s.add_argument("csv")
    s.add_argument("--trace")
    s.add_argument("--split", action="append", default=[])
    s.add_argument("--title", required=True)
    s.add_argument("--cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--grid", type=int)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--src", required=True)
    t.add_argument("--cmd", required=True)
    t.add_argument("--out", required=True)
    k = sub.add_parser("counters")
    k.add_argument("db")
    k.add_argument("--kernel", action="append", required=True)
    k.add_argument("--title", required=True)
    k.add_argument("--cmd", required=True)
    a = ap.parse_args(argv)
    if a.what == "summary":
        sys.stdout.write(summary(a.csv, a.title, a.cmd, a.trace, a.split))
    elif a.what == "counters":
        sys.stdout.write(counters(a.db, a.kernel, a.title, a.cmd))
    else:
        res = traffic(a.fetch, a.write, a.kernel, a.copy_bytes, a.src, a.cmd, a.grid)
        with open(a.out, "w") as fh:
            json.dump(res, fh, indent=1)
        print(json.dumps(res, indent=1))


if __name__ == "__main__":
    main()
