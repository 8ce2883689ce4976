"""Summarize rocprofv3 rocpd databases of a ``bench.py`` run into the short
text summaries kept under ``profiles/``.

    python -m paged_kv_cache_kvck_amd.rocpd_summary \\
        --trace T.db [--fetch F.db --write W.db --copy-bytes N] [--kernel NAME] \\
        --workload llama3_8b --main-calls 12 --command "..." --out-md profiles/X.md [--out-json profiles/Y.json]

* ``--kernel``: the kernel summarized (a substring of its name; default the
  main pass, ``blocks_kernel``); ``--valid-bytes`` are its algorithmic bytes
  per launch.
* ``--trace``: kernel-trace database; per-kernel calls / average / min / max
  durations.  The first ``--main-calls`` dispatches of the summarized kernel
  are the timed workload (warm-up + steps); later ones (e.g. the TP-shard
  run) are listed separately.
* ``--fetch`` / ``--write``: ``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE``
  databases.  Each counter is scaled by what it reads for the plain device
  copy of ``--copy-bytes`` bytes that ``bench.py --copy-calibration-gib``
  runs, giving HBM bytes per launch of the main pass.
"""

from __future__ import annotations

import argparse
import json
import os
import sqlite3
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MAIN = "blocks_kernel"


def _kernels(db):
    c = sqlite3.connect(db)
    return c.execute("select name, duration, dispatch_id from kernels order by start").fetchall()


def _pmc(db):
    c = sqlite3.connect(db)
    return c.execute("select name, counter_name, counter_value, dispatch_id from pmc_events order by dispatch_id"
                     ).fetchall()


def _short(name):
    n = name.replace("(anonymous namespace)::", "")
    return n.split("(")[0] if "(" in n and "<" not in n.split("(")[0][-3:] else n[:80]


def _stats(durs):
    return len(durs), statistics.mean(durs) / 1e6, min(durs) / 1e6, max(durs) / 1e6


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-bytes", type=int, default=0)
    ap.add_argument("--workload", required=True)
    ap.add_argument("--main-calls", type=int, required=True)
    ap.add_argument("--warmup", type=int, default=2, help="untimed calls at the start of --main-calls")
    ap.add_argument("--valid-bytes", type=int, required=True)
    ap.add_argument("--command", required=True, help="the rocprofv3 commands that made the databases")
    ap.add_argument("--out-md", required=True)
    ap.add_argument("--out-json")
    ap.add_argument("--kernel", default=MAIN, help="substring of the summarized kernel's name")
    ap.add_argument("--copy-kernel", action="store_true",
                    help="the kernel reads and writes --valid-bytes (fused copy): throughput counts both")
    ap.add_argument("--later-label", default="later calls",
                    help="label of the kernel's dispatches after --main-calls")
    ap.add_argument("--label", help="display name of the kernel (default: --kernel)")
    a = ap.parse_args(argv)
    kernel = a.kernel
    label = a.label or kernel

    rows = _kernels(a.trace)
    # the workload's dispatches: the first kernel matching --kernel fixes the
    # variant (template arguments); other variants (a TP-shard run, a small
    # call) are listed on rows of their own
    main_name = next((name for name, _, _ in rows if kernel in name), None)
    if main_name is None:
        raise SystemExit(f"no dispatch of {kernel!r} in {a.trace}")
    groups = {}
    main_durs = []
    for name, dur, _ in rows:
        if name == main_name:
            main_durs.append(dur)
            continue
        groups.setdefault(_short(name), []).append(dur)
    lines = [f"# rocprofv3 summary: {label} on the {a.workload} workload", "", "Commands (run from /tmp with TMPDIR=/tmp; R = repository root):", "",
             "```", a.command.strip(), "```", "", "## Kernel trace (`--kernel-trace --stats`)", "",
             "| kernel | calls | avg ms | min ms | max ms |", "|---|---|---|---|---|"]
    head = main_durs[:a.main_calls]
    rest = main_durs[a.main_calls:]
    n, avg, mn, mx = _stats(head)
    lines.append(f"| {label} (workload: warm-up + timed steps) | {n} | {avg:.4f} | {mn:.4f} | {mx:.4f} |")
    if rest:
        n2, avg2, mn2, mx2 = _stats(rest)
        lines.append(f"| {label} ({a.later_label}) | {n2} | {avg2:.4f} | {mn2:.4f} | {mx2:.4f} |")
    for k, d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        n3, a3, m3, x3 = _stats(d)
        lines.append(f"| {k} | {n3} | {a3:.4f} | {m3:.4f} | {x3:.4f} |")
    timed = head[a.warmup:] or head
    t_avg = statistics.mean(timed) / 1e6
    moved = a.valid_bytes * (2 if a.copy_kernel else 1)
    what = "bytes moved (valid bytes read + written)" if a.copy_kernel else "valid bytes"
    lines += ["", f"{label}, timed calls only: average {t_avg:.4f} ms -> "
                  f"{moved / (t_avg * 1e-3) / 1e9:.1f} GB/s of {what} "
                  f"({moved} B per launch), {moved / (t_avg * 1e-3) / 8e12 * 100:.1f} % of 8 TB/s."]
    traffic = None
    if a.fetch and a.write and a.copy_bytes:
        res = {}
        for which, db, counter in (("fetch", a.fetch, "FETCH_SIZE"), ("write", a.write, "WRITE_SIZE")):
            ev = [r for r in _pmc(db) if r[1] == counter]
            # the calibration copy is the runtime's device-to-device copy, never a kvck kernel
            copy = [r[2] for r in ev if "copyBuffer" in r[0] and "kvck" not in r[0]]
            copy_kib = max(copy)
            factor = a.copy_bytes / (copy_kib * 1024.0)
            pmc_name = next(r[0] for r in ev if kernel in r[0])
            if pmc_name != main_name:
                raise SystemExit(f"{counter}: first {kernel!r} dispatch is {pmc_name!r}, not {main_name!r}")
            main = [r[2] for r in ev if r[0] == main_name][:a.main_calls]
            kib = statistics.mean(main)
            res[which] = dict(counter=counter, copy_kib=copy_kib, factor=factor, main_kib=kib,
                              bytes=kib * 1024.0 * factor, launches=len(main))
        traffic = res["fetch"]["bytes"] + res["write"]["bytes"]
        lines += ["", "## HBM traffic (`--pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`, separate runs)", "",
                  f"| counter | plain copy reads (KiB) | copy bytes | scale | {label} per launch (KiB) | scaled bytes |",
                  "|---|---|---|---|---|---|"]
        for which in ("fetch", "write"):
            r = res[which]
            lines.append(f"| {r['counter']} | {r['copy_kib']:.0f} | {a.copy_bytes} | {r['factor']:.4f} | "
                         f"{r['main_kib']:.0f} | {r['bytes']:.4e} |")
        lines += ["", f"HBM bytes per launch: {traffic:.4e}; algorithmic (valid) bytes read {a.valid_bytes:.4e}; "
                      f"fetched / algorithmic = {res['fetch']['bytes'] / a.valid_bytes:.4f}; "
                      f"written / algorithmic = {res['write']['bytes'] / a.valid_bytes:.4f}."]
        if a.out_json:
            from paged_kv_cache_kvck_amd.sources import kernel_sources_sha
            with open(a.out_json, "w") as f:
                json.dump({"workload": a.workload, "kernel": kernel, "kernel_sources_sha256": kernel_sources_sha(),
                           "fetch_bytes_per_launch": res["fetch"]["bytes"],
                           "write_bytes_per_launch": res["write"]["bytes"],
                           "fetch_scale": res["fetch"]["factor"], "write_scale": res["write"]["factor"],
                           "valid_bytes_per_launch": a.valid_bytes}, f, indent=1)
                f.write("\n")
    with open(a.out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
