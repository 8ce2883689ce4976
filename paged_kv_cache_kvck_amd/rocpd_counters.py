"""Tables of hardware counters per kernel variant from rocprofv3 ``--pmc``
databases, with the ratios that say what limits a streaming kernel.

    python -m paged_kv_cache_kvck_amd.rocpd_counters \\
        --case LABEL KERNEL A.db [B.db ...] [--case ...] --command "..." --out-md profiles/X.md

Each ``--case`` is one workload profiled in one or more passes (a rocprofv3
run allows only a few counters per hardware block, so counters come from
several runs of the same command).  ``KERNEL`` is a substring of the kernel's
name; the first dispatch matching it fixes the variant, and every dispatch of
that variant but the first (``--skip``) is averaged.  Derived ratios:

* memory-side read latency in TCC cycles = TCC_EA0_RDREQ_LEVEL / TCC_EA0_RDREQ
  (the counters' own definition), and reads in flight per TCC instance =
  TCC_EA0_RDREQ_LEVEL / TCC_CYCLE; likewise for writes;
* DRAM-credit stalls: TCC cycles a read (write) waited for memory-controller
  credits, per TCC cycle;
* wave states: blocked at instruction issue (SQ_WAIT_INST_ANY), waiting for
  anything (SQ_WAIT_ANY), executing (SQ_ACTIVE_INST_ANY), executing VALU, each
  per wave cycle (SQ_WAVE_CYCLES); VALU instructions per memory instruction;
* L1-to-L2 read latency = TCP_TCC_READ_REQ_LATENCY / TCP_TCC_READ_REQ;
  address-translation miss rate of the L1 TLB; TA busy cycles stalled by the
  cache; TD busy cycles waiting on the cache.
"""

from __future__ import annotations

import argparse
import sqlite3
import statistics

RATIOS = [
    ("memory read latency (TCC cycles)", "TCC_EA0_RDREQ_LEVEL_sum", "TCC_EA0_RDREQ_sum", 1.0, "{:.0f}"),
    ("reads in flight per TCC", "TCC_EA0_RDREQ_LEVEL_sum", "TCC_CYCLE_sum", 1.0, "{:.0f}"),
    ("read DRAM-credit stall %", "TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum", "TCC_CYCLE_sum", 100.0, "{:.1f}"),
    ("memory write latency (TCC cycles)", "TCC_EA0_WRREQ_LEVEL_sum", "TCC_EA0_WRREQ_sum", 1.0, "{:.0f}"),
    ("writes in flight per TCC", "TCC_EA0_WRREQ_LEVEL_sum", "TCC_CYCLE_sum", 1.0, "{:.0f}"),
    ("write DRAM-credit stall %", "TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum", "TCC_CYCLE_sum", 100.0, "{:.1f}"),
    ("waves blocked at issue %", "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES", 100.0, "{:.0f}"),
    ("waves waiting %", "SQ_WAIT_ANY", "SQ_WAVE_CYCLES", 100.0, "{:.0f}"),
    ("waves executing %", "SQ_ACTIVE_INST_ANY", "SQ_WAVE_CYCLES", 100.0, "{:.0f}"),
    ("waves executing VALU %", "SQ_ACTIVE_INST_VALU", "SQ_WAVE_CYCLES", 100.0, "{:.0f}"),
    ("VALU per memory instruction", "SQ_INSTS_VALU", "SQ_INSTS_VMEM", 1.0, "{:.1f}"),
    ("L1-to-L2 read latency (cycles)", "TCP_TCC_READ_REQ_LATENCY_sum", "TCP_TCC_READ_REQ_sum", 1.0, "{:.0f}"),
    ("TA busy stalled by cache %", "TA_ADDR_STALLED_BY_TC_CYCLES_sum", "TA_TA_BUSY_sum", 100.0, "{:.0f}"),
    ("TD busy waiting on cache %", "TD_TC_STALL_sum", "TD_TD_BUSY_sum", 100.0, "{:.0f}"),
]


def _case_counters(kernel, dbs, skip):
    """Per-launch averages of every counter found for the kernel variant, and
    its average duration (ms) where a kernel trace was taken with it."""
    avgs, durs, variant = {}, [], None
    for db in dbs:
        c = sqlite3.connect(db)
        ev = c.execute("select name, counter_name, counter_value, dispatch_id from pmc_events "
                       "order by dispatch_id").fetchall()
        names = {d: n for n, _, _, d in ev}
        if variant is None:
            variant = next((names[d] for d in sorted(names) if kernel in names[d]), None)
            if variant is None:
                raise SystemExit(f"no dispatch of {kernel!r} in {db}")
        disp = [d for d in sorted(names) if names[d] == variant][skip:]
        per = {}
        for n, cn, v, d in ev:
            if d in disp:
                per.setdefault(cn, {}).setdefault(d, 0.0)
                per[cn][d] += v
        for cn, by in per.items():
            avgs[cn] = statistics.mean(by.values())
        try:
            durs += [dur / 1e6 for name, dur in c.execute("select name, duration from kernels") if name == variant]
        except sqlite3.Error:
            pass
    return variant, avgs, (statistics.mean(durs[skip:]) if len(durs) > skip else None)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--case", nargs="+", action="append", required=True, metavar="LABEL KERNEL DB",
                    help="label, kernel-name substring, then the pass databases of one workload")
    ap.add_argument("--skip", type=int, default=1, help="leading dispatches of each case left out")
    ap.add_argument("--title", default="hardware counters per kernel variant")
    ap.add_argument("--command", required=True, help="the commands that made the databases")
    ap.add_argument("--out-md", required=True)
    a = ap.parse_args(argv)
    cases = []
    for case in a.case:
        if len(case) < 3:
            raise SystemExit("--case needs LABEL KERNEL DB [DB ...]")
        label, kernel, dbs = case[0], case[1], case[2:]
        variant, avgs, dur = _case_counters(kernel, dbs, a.skip)
        cases.append((label, variant, avgs, dur))
    present = [r for r in RATIOS if any(r[1] in c[2] and r[2] in c[2] for c in cases)]
    lines = [f"# rocprofv3 counters: {a.title}", "", "Commands (run from /tmp with TMPDIR=/tmp; R = repository root):",
             "", "```", a.command.strip(), "```", "",
             "Per-launch averages over each variant's dispatches after the first.", "",
             "| case | ms | " + " | ".join(r[0] for r in present) + " |",
             "|---|---|" + "---|" * len(present)]
    for label, variant, avgs, dur in cases:
        cells = []
        for name, num, den, scale, fmt in present:
            cells.append(fmt.format(scale * avgs[num] / avgs[den]) if num in avgs and den in avgs and avgs[den]
                         else "")
        lines.append(f"| {label} | {'' if dur is None else f'{dur:.3f}'} | " + " | ".join(cells) + " |")
    lines += ["", "Kernel variants:", ""]
    lines += [f"* {label}: `{variant}`" for label, variant, _, _ in cases]
    lines += ["", "Raw per-launch averages:", ""]
    counters = sorted({k for _, _, avgs, _ in cases for k in avgs})
    lines += ["| case | " + " | ".join(counters) + " |", "|---|" + "---|" * len(counters)]
    for label, _, avgs, _ in cases:
        lines.append(f"| {label} | " + " | ".join(f"{avgs[k]:.4g}" if k in avgs else "" for k in counters) + " |")
    with open(a.out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
