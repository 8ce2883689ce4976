"""The counter-table tool on small hand-made databases in the rocpd schema
(CPU): per-launch averages skip the first dispatch, several pass databases
of one workload combine, and each ratio is the counters' quotient."""

import sqlite3

import pytest

from paged_kv_cache_kvck_amd import rocpd_counters


def _db(path, kernel, counters, durations=None):
    c = sqlite3.connect(path)
    c.execute("create table pmc_events (name text, counter_name text, counter_value real, dispatch_id int)")
    c.execute("create table kernels (name text, duration int, dispatch_id int)")
    for d, values in enumerate(counters):
        c.execute("insert into pmc_events values (?, 'OTHER', 1, ?)", ("plan_kernel", 100 + d))
        for k, v in values.items():
            # a counter reported in two instances adds up per dispatch
            c.execute("insert into pmc_events values (?, ?, ?, ?)", (kernel, k, v / 2, d))
            c.execute("insert into pmc_events values (?, ?, ?, ?)", (kernel, k, v / 2, d))
        if durations:
            c.execute("insert into kernels values (?, ?, ?)", (kernel, durations[d], d))
    c.commit()
    c.close()


def test_counter_table(tmp_path):
    k = "blocks_kernel<16, 4>"
    a, b = str(tmp_path / "a.db"), str(tmp_path / "b.db")
    # first dispatch (skipped) is far off; the next two average to the values below
    _db(a, k, [{"TCC_EA0_RDREQ_LEVEL_sum": 1e9, "TCC_EA0_RDREQ_sum": 1, "TCC_CYCLE_sum": 1},
               {"TCC_EA0_RDREQ_LEVEL_sum": 2000.0, "TCC_EA0_RDREQ_sum": 10.0, "TCC_CYCLE_sum": 5.0},
               {"TCC_EA0_RDREQ_LEVEL_sum": 4000.0, "TCC_EA0_RDREQ_sum": 10.0, "TCC_CYCLE_sum": 15.0}],
        durations=[9e9, 2e6, 4e6])
    _db(b, k, [{"SQ_WAIT_INST_ANY": 0, "SQ_WAVE_CYCLES": 1},
               {"SQ_WAIT_INST_ANY": 30.0, "SQ_WAVE_CYCLES": 100.0},
               {"SQ_WAIT_INST_ANY": 50.0, "SQ_WAVE_CYCLES": 100.0}])
    out = str(tmp_path / "t.md")
    rocpd_counters.main(["--case", "x", "blocks_kernel", a, b, "--command", "cmd", "--out-md", out])
    text = open(out).read()
    row = next(ln for ln in text.splitlines() if ln.startswith("| x |"))
    cells = [c.strip() for c in row.strip("|").split("|")]
    header = next(ln for ln in text.splitlines() if ln.startswith("| case | ms |"))
    cols = [c.strip() for c in header.strip("|").split("|")]
    got = dict(zip(cols, cells))
    assert got["ms"] == "3.000"                                      # (2 + 4) / 2 ms
    assert got["memory read latency (TCC cycles)"] == "300"          # 3000 / 10
    assert got["reads in flight per TCC"] == "300"                   # 3000 / 10
    assert got["waves blocked at issue %"] == "40"                   # 40 / 100
    assert "plan_kernel" not in text


def test_missing_kernel_is_an_error(tmp_path):
    a = str(tmp_path / "a.db")
    _db(a, "copy_kernel", [{"TCC_CYCLE_sum": 1.0}])
    with pytest.raises(SystemExit):
        rocpd_counters.main(["--case", "x", "blocks_kernel", a, "--command", "c", "--out-md", str(tmp_path / "o.md")])
