"""Summarises a rocprofv3 results database (SQLite, `*_results.db`).

    python -m eagle_draft_head_step_amd.rocprof_summary RESULTS.db [--match SUBSTR]

Prints, per kernel symbol: dispatches, average and total duration, share of
all kernel time, and (for databases from a --pmc run) the average of each
collected counter per dispatch.
"""
from __future__ import annotations

import argparse
import sqlite3
import sys
from collections import defaultdict


def summarize(db_path: str, match: str = ""):
    db = sqlite3.connect(db_path)
    cur = db.cursor()
    rows = cur.execute("select id, name, start, end from kernels").fetchall()
    stats = defaultdict(lambda: [0, 0.0])
    by_id = {}
    for kid, name, start, end in rows:
        s = stats[name]
        s[0] += 1
        s[1] += (end - start) / 1e3
        by_id[kid] = name
    counters = defaultdict(lambda: defaultdict(list))
    try:
        cols = [c[1] for c in cur.execute("pragma table_info(pmc_events)")]
        if cols:
            id_col = "dispatch_id" if "dispatch_id" in cols else ("kernel_id" if "kernel_id" in cols else None)
            q = "select * from pmc_events"
            for rec in cur.execute(q).fetchall():
                d = dict(zip(cols, rec))
                name = d.get("name") or d.get("kernel_name") or by_id.get(d.get(id_col), "?")
                cname = d.get("counter_name") or d.get("pmc_name") or d.get("counter") or "counter"
                val = d.get("value") if "value" in d else d.get("counter_value")
                key = d.get("kernel_id", d.get(id_col))
                counters[name][cname].append((key, val))
    except sqlite3.Error:
        pass
    total = sum(v[1] for v in stats.values()) or 1.0
    out = []
    out.append(f"{'kernel':70s} {'n':>6s} {'avg_us':>10s} {'total_us':>11s} {'share':>6s}")
    for name, (n, t) in sorted(stats.items(), key=lambda x: -x[1][1]):
        if match and match not in name:
            continue
        out.append(f"{name[:70]:70s} {n:6d} {t / n:10.2f} {t:11.1f} {100 * t / total:5.1f}%")
        for cname, vals in sorted(counters.get(name, {}).items()):
            per = defaultdict(float)
            for key, v in vals:
                per[key] += float(v)
            avg = sum(per.values()) / max(1, len(per))
            out.append(f"{'':8s}{cname}: avg {avg:.1f} per dispatch over {len(per)} dispatches")
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("db")
    ap.add_argument("--match", default="")
    a = ap.parse_args()
    print(summarize(a.db, a.match))


if __name__ == "__main__":
    sys.exit(main())
