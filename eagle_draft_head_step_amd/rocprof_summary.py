"""Summarises a rocprofv3 results database (SQLite, `*_results.db`).

    python -m eagle_draft_head_step_amd.rocprof_summary RESULTS.db [--match SUBSTR]

Prints, per kernel symbol: dispatches, average and total duration, share of
all kernel time, and (for databases from a --pmc run) the average of each
collected counter per dispatch.  Kernels whose name contains `exclude` (the
host-side pacing spin of the bench's per-kernel timing pass) are left out.
"""
from __future__ import annotations

import argparse
import sqlite3
import sys
from collections import defaultdict


def summarize(db_path: str, match: str = "", exclude: str = "spin_kernel"):
    db = sqlite3.connect(db_path)
    cur = db.cursor()
    rows = cur.execute("select id, name, start, end from kernels").fetchall()
    stats = defaultdict(lambda: [0, 0.0])
    by_id = {}
    for kid, name, start, end in rows:
        if exclude and exclude in name:
            continue
        s = stats[name]
        s[0] += 1
        s[1] += (end - start) / 1e3
        by_id[kid] = name
    counters = defaultdict(lambda: defaultdict(list))
    try:
        for name, did, cname, val in cur.execute(
                "select name, dispatch_id, counter_name, counter_value from pmc_events").fetchall():
            counters[name][cname].append((did, val))
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
            v = sorted(per.values())
            avg = sum(v) / max(1, len(v))
            out.append(f"{'':8s}{cname}: avg {avg:.1f}  min {v[0]:.1f}  max {v[-1]:.1f}  "
                       f"per dispatch over {len(v)} dispatches")
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("db")
    ap.add_argument("--match", default="")
    a = ap.parse_args()
    print(summarize(a.db, a.match))


if __name__ == "__main__":
    sys.exit(main())
