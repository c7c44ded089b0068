"""The rocprofv3 summary tool and the bench's reading of it (CPU only).

The bench's roofline `traffic` comes from a committed counter summary: each
counter's per-dispatch average over a kernel family, times the calibration
factor the summary records from a device copy of known size.  These tests
build small results databases with the tables rocprofv3 writes (kernels,
pmc_events) and check the numbers end to end."""
import os
import sqlite3

import bench
from eagle_draft_head_step_amd import rocprof_summary as RS

COPY = RS.COPY_KERNEL
GEMM = "void e3::gemm_kernel<2, 1, 8, 1, false, 0>(e3::GemmParams)"
OTHER = "e3::resid_norm_kernel(e3::ResidNormArgs)"


def _db(path, dispatches):
    """dispatches: (id, kernel name, duration ns, {counter: value}); a counter
    value split in two rows (rocprofv3 reports one per shader engine) must be
    summed per dispatch."""
    db = sqlite3.connect(path)
    db.execute("create table kernels (id integer, name text, start integer, end integer)")
    db.execute("create table pmc_events (name text, dispatch_id integer, counter_name text, counter_value real)")
    t = 0
    for did, name, ns, counters in dispatches:
        db.execute("insert into kernels values (?, ?, ?, ?)", (did, name, t, t + ns))
        t += ns + 100
        for cname, val in counters.items():
            db.execute("insert into pmc_events values (?, ?, ?, ?)", (name, did, cname, val / 2))
            db.execute("insert into pmc_events values (?, ?, ?, ?)", (name, did, cname, val / 2))
    db.commit()
    db.close()
    return path


def test_counters_report_scale_and_averages(tmp_path):
    # the copy moves 1 GiB each way; FETCH_SIZE reads half of it on this chip
    fetch = _db(str(tmp_path / "fetch.db"), [
        (1, COPY, 1000, {"FETCH_SIZE": RS.COPY_KIB / 2}),
        (2, COPY, 1000, {"FETCH_SIZE": 10.0}),
        (3, GEMM, 5000, {"FETCH_SIZE": 100.0}),
        (4, GEMM, 7000, {"FETCH_SIZE": 300.0}),
        (5, OTHER, 500, {"FETCH_SIZE": 8.0}),
    ])
    write = _db(str(tmp_path / "write.db"), [
        (1, COPY, 1000, {"WRITE_SIZE": RS.COPY_KIB}),
        (3, GEMM, 5000, {"WRITE_SIZE": 20.0}),
        (4, GEMM, 7000, {"WRITE_SIZE": 40.0}),
    ])
    text = RS.counters_report(fetch, write)
    assert "# scale FETCH_SIZE 2.0000" in text
    assert "# scale WRITE_SIZE 1.0000" in text
    # two dispatches of the GEMM: average 200 KiB fetched, 30 KiB written
    assert "FETCH_SIZE: avg 200.0  min 100.0  max 300.0  per dispatch over 2 dispatches" in text
    assert "WRITE_SIZE: avg 30.0  min 20.0  max 40.0  per dispatch over 2 dispatches" in text
    # durations: 5 and 7 us
    line = next(ln for ln in text.splitlines() if ln.startswith("void e3::gemm_kernel"))
    assert line.split()[-4:-2] == ["2", "6.00"]


def test_bench_reads_the_summary(tmp_path, monkeypatch):
    fetch = _db(str(tmp_path / "fetch.db"), [
        (1, COPY, 1000, {"FETCH_SIZE": RS.COPY_KIB / 2}),
        (3, GEMM, 5000, {"FETCH_SIZE": 100.0}),
        (4, GEMM, 7000, {"FETCH_SIZE": 300.0}),
    ])
    write = _db(str(tmp_path / "write.db"), [
        (1, COPY, 1000, {"WRITE_SIZE": RS.COPY_KIB}),
        (3, GEMM, 5000, {"WRITE_SIZE": 20.0}),
        (4, GEMM, 7000, {"WRITE_SIZE": 40.0}),
    ])
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "wl_hbm_counters.txt").write_text(RS.header("cmd") + "\n\n" + RS.counters_report(fetch, write))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    # (200 KiB x 2 + 30 KiB x 1) per dispatch, in bytes
    assert bench.counter_traffic("wl", "gemm_kernel<", ", false, 0>") == 1024 * (2 * 200 + 30)
    assert bench.counter_traffic("wl", "gemm_big_kernel", "") is None       # no such family
    # a summary taken from other kernel sources is not used
    (prof / "wl_hbm_counters.txt").write_text(RS.header("cmd").replace(RS.sources_hash(), "0" * 16) + "\n\n" +
                                              RS.counters_report(fetch, write))
    assert bench.counter_traffic("wl", "gemm_kernel<", ", false, 0>") is None


def test_committed_summaries_name_their_sources():
    d = os.path.join(bench.ROOT, "profiles")
    for f in sorted(os.listdir(d)):
        text = open(os.path.join(d, f)).read()
        assert text.startswith("# command"), f
        assert "sha256[:16] = " in text, f
        if f.endswith("_hbm_counters.txt"):
            assert "# scale FETCH_SIZE" in text and "# scale WRITE_SIZE" in text, f
