"""Summarises rocprofv3 results databases (SQLite, `*_results.db`).

    python -m eagle_draft_head_step_amd.rocprof_summary RESULTS.db [--match SUBSTR]
    python -m eagle_draft_head_step_amd.rocprof_summary --counters FETCH.db WRITE.db

The first form prints, per kernel symbol: dispatches, average and total
duration, share of all kernel time, and (for databases from a --pmc run) the
average of each collected counter per dispatch.  Kernels whose name contains
`exclude` (the host-side pacing spin of the bench's per-kernel timing pass)
are left out.

The second form joins a FETCH_SIZE run and a WRITE_SIZE run of the same
program into one HBM-traffic summary.  Each counter is calibrated against the
largest dispatch of the device copy the bench runs (a 1 GiB copy, which moves
exactly 1 GiB each way): the summary records `# scale <counter> <factor>`, the
factor that turns that counter's KiB into real KiB.

`--header COMMAND` prefixes the output with the command that produced the
databases and a hash of the kernel sources, so a reader can tell whether the
summary still describes the code.
"""
from __future__ import annotations

import argparse
import hashlib
import os
import sqlite3
import sys
from collections import defaultdict

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
# the sources a kernel family's timing and traffic depend on: its own files,
# the shared headers, and for the step's kernels the host planner that picks
# their launches
KERNEL_SOURCES = {
    "step": ["api.cpp", "common.h", "internal.h", "gemm.hip", "rowops.hip", "attn_mha.hip", "attn_mla.hip"],
    "relaxed": ["accept.hip", "common.h"],
}
COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_KIB = 1 << 20                     # the bench's calibration copy: 1 GiB read, 1 GiB written


def sources_hash(family: str = "step") -> str:
    """sha256 of the family's sources and of the compiler options they are
    built with (the options change the code as much as the sources do)."""
    from eagle_draft_head_step_amd.build import SOURCE_FLAGS, flags
    h = hashlib.sha256()
    for f in sorted(KERNEL_SOURCES[family]):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
        h.update(" ".join(flags() + SOURCE_FLAGS.get(f, [])).encode())
    return h.hexdigest()[:16]


def header(command: str, family: str = "step") -> str:
    files = ", ".join(sorted(KERNEL_SOURCES[family]))
    return "\n".join([
        "# command (run from the repository root on one MI355X, TMPDIR=/tmp):",
        *[f"#   {c.strip()}" for c in command.split(";") if c.strip()],
        f"# kernel sources ({files}) and their compiler options, sha256[:16] = {sources_hash(family)}",
    ])


def copy_max(db_path: str, counter: str):
    """Largest per-dispatch value of `counter` over the calibration copy's dispatches."""
    db = sqlite3.connect(db_path)
    per = defaultdict(float)
    for name, did, cname, val in db.execute(
            "select name, dispatch_id, counter_name, counter_value from pmc_events").fetchall():
        if name.startswith(COPY_KERNEL) and cname == counter:
            per[did] += float(val)
    return max(per.values()) if per else None


def counters_report(fetch_db: str, write_db: str) -> str:
    out = ["# FETCH_SIZE / WRITE_SIZE in KiB per dispatch.  Calibration: the 1024 MiB device copy of the",
           f"# bench's copy-bandwidth probe ({COPY_KERNEL}, the max dispatch) reads {COPY_KIB} KiB",
           f"# and writes {COPY_KIB} KiB."]
    for db, cname in ((fetch_db, "FETCH_SIZE"), (write_db, "WRITE_SIZE")):
        m = copy_max(db, cname)
        if m:
            out.append(f"# scale {cname} {COPY_KIB / m:.4f}")
    out.append("")
    out.append(summarize(fetch_db))
    out.append("")
    out.append(summarize(write_db))
    return "\n".join(out)


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
    ap.add_argument("db", nargs="?")
    ap.add_argument("--match", default="")
    ap.add_argument("--counters", nargs=2, metavar=("FETCH_DB", "WRITE_DB"))
    ap.add_argument("--header", default=None, help="command(s) that made the databases, ';'-separated")
    ap.add_argument("--family", default="step", choices=sorted(KERNEL_SOURCES))
    a = ap.parse_args()
    if a.header:
        print(header(a.header, a.family))
        print()
    if a.counters:
        print(counters_report(*a.counters))
    elif a.db:
        print(summarize(a.db, a.match))
    else:
        ap.error("a results database or --counters is required")


if __name__ == "__main__":
    sys.exit(main())
