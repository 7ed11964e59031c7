"""Turn rocprofv3 output into the short summaries kept under profiles/.

    python -m nested_integer_weight_amd.profiling summary STATS_CSV --title T --cmd C
        markdown table of a `--kernel-trace --stats --output-format csv` run

    python -m nested_integer_weight_amd.profiling traffic --fetch DB --write DB \
        --kernel SUBSTR --copy-bytes N --src FILE --cmd C --out JSON
        HBM bytes per dispatch of one kernel from a FETCH_SIZE run and a
        WRITE_SIZE run (rocpd SQLite databases), each scaled by what the same
        counter reads for the last device copy in the run (bench.py's
        calibration copy of known size, `--copy-bytes`), which calibrates the
        counter's coverage.

The databases are the `*_results.db` files rocprofv3 writes with `--pmc`.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import sqlite3
import sys


def summary(stats_csv: str, title: str, cmd: str) -> str:
    rows = list(csv.DictReader(open(stats_csv)))
    out = [f"# {title}", "", "Command (from the repository root, on one MI355X):", "", "```", cmd, "```", "",
           "Source: `rocprofv3 --kernel-trace --stats` kernel_stats.csv (GPU-side dispatch durations).", "",
           "| kernel | calls | avg us | min us | max us | % of GPU time |",
           "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        out.append(f"| `{r['Name'][:100]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{int(r['MinNs']) / 1e3:.2f} | {int(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
    return "\n".join(out) + "\n"


def _per_dispatch(db: str, counter: str):
    """{(kernel_name, grid_size): mean counter value per dispatch}"""
    c = sqlite3.connect(db)
    rows = c.execute("""select kernel_name, grid_size, avg(value), count(*) from counters_collection
                        where counter_name = ? group by kernel_name, grid_size""", (counter,)).fetchall()
    return {(r[0], r[1]): (r[2], r[3]) for r in rows}


def _kernel_value(d: dict, substr: str):
    vals = [(v, n) for (name, _), (v, n) in d.items() if substr in name]
    if not vals:
        raise SystemExit(f"no dispatch of a kernel matching {substr!r}")
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


def traffic(fetch_db, write_db, kernel, copy_bytes, src, cmd):
    f = _per_dispatch(fetch_db, "FETCH_SIZE")
    w = _per_dispatch(write_db, "WRITE_SIZE")
    fk, nf = _kernel_value(f, kernel)
    wk, nw = _kernel_value(w, kernel)
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


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("summary")
    s.add_argument("csv")
    s.add_argument("--title", required=True)
    s.add_argument("--cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--src", required=True)
    t.add_argument("--cmd", required=True)
    t.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.what == "summary":
        sys.stdout.write(summary(a.csv, a.title, a.cmd))
    else:
        res = traffic(a.fetch, a.write, a.kernel, a.copy_bytes, a.src, a.cmd)
        with open(a.out, "w") as fh:
            json.dump(res, fh, indent=1)
        print(json.dumps(res, indent=1))


if __name__ == "__main__":
    main()
