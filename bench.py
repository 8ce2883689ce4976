#!/usr/bin/env python3
"""Benchmark of the KV-cache block checksum on one MI355X.

One step = one kvck_checksum_blocks call over the whole batch of the
Llama-3-8B-shaped cache (32 layers x 8 KV heads x head 128, bf16 normal(0,1)
values, block 16, HND pool, 256 requests of 512..8192 tokens): plan, main
pass over every valid K/V byte, second pass.  Inputs are resident in HBM
before timing starts.

    python bench.py [--steps K] [--warmup W] [--only NAME[,NAME..]]

Prints one JSON line: throughput in checksummed KV GB/s (valid cache bytes /
step time), the roofline of the main pass (its own HIP events on its stream,
via the library's instrumentation), the CPU oracle's rate on a bounded sample
of the same workload -- one process, then one process per host CPU over
layer subsets of the same bytes, whose partial sums must add up to the
one-process values -- and in ``extra.configs`` one row per other
configuration of the checksum (GPT-2-shaped pool and its re-pagings, fp8,
MLA, the hybrid model's attention and Mamba groups, the TP-shard run): its
main-pass time and fraction of HBM peak, and its values checked against the
oracle at sampled positions.

``--only`` runs just the named configuration rows (one of CONFIG_NAMES) and
prints them; a profiler run of one kernel variant uses it.
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published

HEADLINE_DESC = ("llama3-8b-shaped paged KV cache: 32 layers x 8 KV heads x head 128 bf16 normal(0,1), block 16, "
                 "HND, 256 requests of 512-8192 tokens")


def committed_traffic(workload: str):
    """HBM bytes per launch of the main pass from the committed rocprofv3
    counter summary, or None when the kernel sources changed since."""
    from paged_kv_cache_kvck_amd.sources import kernel_sources_sha
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("kernel_sources_sha256") != kernel_sources_sha():
        return None
    return int(t["fetch_bytes_per_launch"] + t["write_bytes_per_launch"])


def make_workload(name):
    from paged_kv_cache_kvck_amd import workloads as wl
    if name == "llama3_8b":
        return wl.llama3_8b(), HEADLINE_DESC
    raise SystemExit(f"unknown workload {name}")


# ----------------------------------------------------------------- oracle checks

def _host_bits(t):
    """Raw bits of a device tensor as an unsigned numpy array of its shape."""
    import numpy as np
    import torch
    es = t.element_size()
    dt = {1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}[es]
    npdt = {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}[es]
    return t.contiguous().view(dt).cpu().numpy().view(npdt)


def _block_axis(layout):
    return 0 if layout == "MLA" else 1


def sample_positions(req, n, seed):
    """``n`` random listed positions plus every request's last one (its
    partly valid tail), as (r, k) pairs."""
    import numpy as np
    rng = np.random.default_rng(seed)
    allpos = req.listed()
    pick = [allpos[i] for i in rng.choice(len(allpos), min(n, len(allpos)), replace=False)]
    pick += [(r, int(req.num_blocks[r]) - 1) for r in range(req.num_reqs) if req.num_blocks[r] > 0]
    return sorted(set(pick))


def oracle_check(pools, layout, layers, bases, req, got, positions, head_begin=0, head_count=None):
    """The oracle's checksums of ``positions`` (computed from host copies of
    just the blocks they name) against the GPU's ``got`` [num_reqs,
    max_blocks]: (positions checked, mismatches)."""
    import torch
    import oracle
    mismatches = 0
    for i in range(0, len(positions), 64):
        chunk = positions[i:i + 64]
        ids = sorted({int(req.block_table[r, k]) for r, k in chunk})
        remap = {b: n for n, b in enumerate(ids)}
        idx = torch.tensor(ids, dtype=torch.int64, device=pools[0].device)
        mini = [_host_bits(p.index_select(_block_axis(layout), idx)) for p in pools]
        for r, k in chunk:
            v = oracle.kv_checksum.checksum_position(mini, layout, layers, bases, remap[int(req.block_table[r, k])],
                                                     int(req.start_pos[r]) + k, int(req.num_tokens[r]), head_begin,
                                                     head_count)
            mismatches += int(got[r, k]) != v
    return len(positions), mismatches


# ----------------------------------------------------------------- CPU baseline

def _layer_worker(args):
    """One process of the parallel oracle leg: the oracle over this worker's
    subset of layers for every position of a chunk, reading the chunk's
    blocks from the memory-mapped host copy.  numpy only; never touches the
    GPU.  Returns (partial checksums, seconds of oracle time)."""
    path, layout, layer_idx, layers, bases, items, head_begin, head_count = args
    import numpy as np
    import oracle
    arr = np.load(path, mmap_mode="r")
    caches = [arr[i] for i in layer_idx]
    t0 = time.perf_counter()
    vals = [oracle.kv_checksum.checksum_position(caches, layout, [layers[i] for i in layer_idx],
                                                 [bases[i] for i in layer_idx], b, pos, ntok, head_begin, head_count)
            for b, pos, ntok in items]
    dt = time.perf_counter() - t0
    del caches, arr
    return vals, dt


def cpu_baseline(pools, w, seconds, gpu_out, workers, chunk=512, seed=0):
    """The oracle, as it stands, on a bounded random sample of listed
    positions of the workload, in chunks: each chunk's blocks (all layers) are
    copied to a host file in /dev/shm (outside the timed regions); then

    * one process computes every position of the chunk (``value``, cores 1),
      each compared with the GPU's checksum of the timed steps;
    * ``workers`` processes at once each compute the same positions over their
      own subset of the layers -- a PP-style split of the same bytes -- and the
      partials, added mod 2^64, must equal the one-process values
      (``parallel``: wall time around the workers, dispatch included).

    Stops once the one-process leg has run ``seconds``."""
    import multiprocessing as mp
    import numpy as np
    import torch
    import oracle
    from paged_kv_cache_kvck_amd import workloads as wl

    rng = np.random.default_rng(seed)
    allpos = w.req.listed()
    order = rng.permutation(len(allpos))
    L = w.num_layers
    shard = np.array_split(np.arange(L), min(workers, L))
    shard = [[int(i) for i in s] for s in shard if len(s)]
    row = w.heads_used * w.planes * w.head_size * wl.ELEM_BYTES[w.elem] * L
    shape = (L,) + wl.pool_shape(w.layout, chunk, w.req.block_size, w.num_heads, w.head_size)
    bits = wl.HOST_BITS[w.elem]
    shm_dir = "/dev/shm" if os.path.isdir("/dev/shm") else None
    fd, path = tempfile.mkstemp(prefix="kvck_oracle_", suffix=".npy", dir=shm_dir)
    os.close(fd)
    done = nbytes = mismatches = pmis = 0
    single_s = par_wall = par_busy = 0.0
    i = 0
    pool = None
    try:
        host = np.lib.format.open_memmap(path, mode="w+", dtype=bits, shape=shape)
        pool = mp.get_context("spawn").Pool(len(shard))
        # start the workers (imports) before the first timed chunk
        pool.map(abs, range(len(shard)))
        while single_s < seconds and i < len(order):
            sel = [allpos[j] for j in order[i:i + chunk]]
            i += chunk
            ids = sorted({int(w.req.block_table[r, k]) for r, k in sel})
            remap = {b: n for n, b in enumerate(ids)}
            idx = torch.tensor(ids, dtype=torch.int64, device=pools[0].device)
            ax = _block_axis(w.layout)
            for li, p in enumerate(pools):
                dst = host[li][(slice(None),) * ax + (slice(0, len(ids)),)]
                dst[...] = _host_bits(p.index_select(ax, idx))
            host.flush()
            items = [(remap[int(w.req.block_table[r, k])], int(w.req.start_pos[r]) + k, int(w.req.num_tokens[r]))
                     for r, k in sel]
            caches = [host[li] for li in range(L)]
            t0 = time.perf_counter()
            vals = [oracle.kv_checksum.checksum_position(caches, w.layout, w.layer_numbers, w.bases, b, pos, ntok,
                                                         w.head_begin, w.head_count) for b, pos, ntok in items]
            single_s += time.perf_counter() - t0
            mismatches += sum(int(gpu_out[r, k]) != v for (r, k), v in zip(sel, vals))
            args = [(path, w.layout, s, list(w.layer_numbers), list(w.bases), items, w.head_begin, w.head_count)
                    for s in shard]
            t0 = time.perf_counter()
            parts = pool.map(_layer_worker, args)
            par_wall += time.perf_counter() - t0
            par_busy = max(par_busy, max(dt for _, dt in parts))
            with np.errstate(over="ignore"):
                tot = np.zeros(len(items), dtype=np.uint64)
                for pv, _ in parts:
                    tot += np.array(pv, dtype=np.uint64)
            pmis += int(np.sum(tot != np.array(vals, dtype=np.uint64)))
            for r, k in sel:
                pos = int(w.req.start_pos[r]) + k
                nbytes += min(w.req.block_size, max(0, int(w.req.num_tokens[r]) - pos * w.req.block_size)) * row
            done += len(sel)
            del caches
        del host
    finally:
        if pool is not None:
            pool.terminate()
            pool.join()
        if os.path.exists(path):
            os.unlink(path)
    res = {"value": nbytes / single_s / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"{done} random listed positions of the same workload ({nbytes} valid bytes, all layers and "
                     f"heads), in chunks of {chunk}; numpy in one process, {single_s:.1f} s of oracle time; host "
                     f"copies excluded",
           "gpu_checked_positions": done, "gpu_mismatches": mismatches}
    res["parallel"] = {
        "value": nbytes / par_wall / 1e9, "unit": "GB/s", "cores": len(shard), "kind": "oracle",
        "sample": f"the same {done} positions and bytes, each chunk split over {len(shard)} processes by layer "
                  f"(layers {shard[0][0]}-{shard[0][-1]} in the first, ...): {par_wall:.2f} s of wall time around "
                  f"the processes, dispatch included",
        "split": "layer subsets (a PP-style partition); partials added mod 2^64",
        "positions_compared": done, "partial_sum_mismatches": pmis}
    return res


# ----------------------------------------------------------------- configuration rows

CONFIG_NAMES = ("gpt2_nhd_bs16", "gpt2_nhd_bs64", "gpt2_hnd_bs16", "fp8_nhd_bs16", "fp8_nhd_bs64", "mla_bs64",
                "mla_bs16", "hybrid_attn", "hybrid_mamba")


WARMUP_MS = 100.0


def _timed_main_pass(call, calls, warmup_ms=None):
    """Median and minimum main-pass milliseconds over ``calls`` calls, each
    read from the library's own HIP events, after untimed calls: two, then
    more until about ``warmup_ms`` of them have run (the first pass over
    freshly written pools reads several points slower than later ones).
    Also returns the number of untimed calls, so that a kernel trace of the
    run can leave them out."""
    import torch
    import paged_kv_cache_kvck_amd as kvck
    warmup_ms = WARMUP_MS if warmup_ms is None else warmup_ms
    kvck.kvck_instrument(True)
    try:
        call()
        call()
        torch.cuda.synchronize()
        ms, c = kvck.kvck_instrument_read()
        extra = int(warmup_ms / max(ms / max(c, 1), 1e-3)) if warmup_ms > 0 else 0
        for _ in range(extra):
            call()
        torch.cuda.synchronize()
        kvck.kvck_instrument_read()
        ts = []
        for _ in range(calls):
            call()
            torch.cuda.synchronize()
            ms, c = kvck.kvck_instrument_read()
            ts.append(ms / max(c, 1))
    finally:
        kvck.kvck_instrument(False)
    return statistics.median(ts), min(ts), 2 + extra


def _row(name, desc, valid, med, mn, checked, mism, untimed=None):
    gbs = valid / (med * 1e-3) / 1e9
    row = {"config": name, "workload": desc, "valid_bytes": valid, "main_pass_ms": med, "main_pass_ms_min": mn,
           "GB_per_s": gbs, "frac_of_hbm_peak": gbs / HBM_PEAK_GBS, "oracle_checked_positions": checked,
           "oracle_mismatches": mism}
    if untimed is not None:
        row["untimed_calls"] = untimed
    return row


def _blocks_row(dev, name, desc, pools, layout, layers, req, valid, calls, n_check, seed, bases=None, head_begin=0,
                head_count=None):
    import numpy as np
    import torch
    import paged_kv_cache_kvck_amd as kvck
    bt, nb, sp, nt = (torch.from_numpy(x).to(dev) for x in
                      (req.block_table, req.num_blocks, req.start_pos, req.num_tokens))
    out = torch.zeros((req.num_reqs, req.max_blocks), dtype=torch.uint64, device=dev)
    ws = torch.empty(kvck.kvck_blocks_workspace_bytes(len(pools), req.num_reqs, req.max_blocks), dtype=torch.uint8,
                     device=dev)
    bases = [head_begin] * len(pools) if bases is None else list(bases)
    pc = kvck.prepare_caches(pools, layout, layers, global_head_base=bases, head_begin=head_begin,
                             head_count=head_count)
    med, mn, untimed = _timed_main_pass(lambda: kvck.kvck_checksum_blocks(pc, None, None, bt, nb, sp, nt, out=out,
                                                                          workspace=ws), calls)
    got = out.cpu().numpy().view(np.uint64)
    checked, mism = (0, 0)
    if n_check:
        checked, mism = oracle_check(pools, layout, layers, bases, req, got, sample_positions(req, n_check, seed),
                                     head_begin, head_count)
    row = _row(name, desc, valid, med, mn, checked, mism, untimed)
    print(f"[config] {name:14s} {valid / 1e9:7.2f} GB {med:8.3f} ms {row['GB_per_s']:8.1f} GB/s "
          f"{row['frac_of_hbm_peak'] * 100:5.1f} %  oracle {checked} positions, {mism} mismatches",
          file=sys.stderr, flush=True)
    return row


def config_row(name, dev, calls=10, n_check=200):
    """Build one configuration's pools on the device, time its main pass and
    check sampled positions against the oracle; frees the pools on return."""
    import numpy as np
    import torch
    import paged_kv_cache_kvck_amd as kvck
    from paged_kv_cache_kvck_amd import workloads as wl

    def repaged(src_pools, layout, req, block_size, seed, shape_fn, dtype):
        r2, n2 = wl.page_requests(np.random.default_rng(seed), req.num_tokens, block_size, spare_frac=0.05)
        dst = [torch.zeros(shape_fn(n2), dtype=dtype, device=dev) for _ in src_pools]
        for s_, d_ in zip(src_pools, dst):
            wl.repage_torch(s_, layout, req, d_, layout, r2)
        return dst, r2

    if name.startswith("gpt2"):
        g = wl.gpt2()
        p = g.device_pools()
        desc = ("gpt2-shaped paged KV cache: 12 layers x 12 KV heads x head 64 fp16 random bits, 64 requests of "
                "128-2048 tokens (69,569 tokens); ")
        if name == "gpt2_nhd_bs16":
            return _blocks_row(dev, name, desc + "NHD pool (2,18545,16,12,64) per layer, block 16", p, "NHD",
                               g.layer_numbers, g.req, g.valid_bytes(), calls, n_check, 11)
        if name == "gpt2_nhd_bs64":
            p64, r64 = repaged(p, "NHD", g.req, 64, 40, lambda n: wl.pool_shape("NHD", n, 64, 12, 64), p[0].dtype)
            del p
            return _blocks_row(dev, name, desc + "the same tokens re-paged at block 64, NHD", p64, "NHD",
                               g.layer_numbers, r64, g.valid_bytes(), calls, n_check, 12)
        if name == "gpt2_hnd_bs16":
            ph = [x.permute(0, 1, 3, 2, 4).contiguous() for x in p]
            del p
            return _blocks_row(dev, name, desc + "the same pool permuted to HND, block 16", ph, "HND",
                               g.layer_numbers, g.req, g.valid_bytes(), calls, n_check, 13)
    if name.startswith("fp8"):
        f = wl.gpt2(seed=41, elem="fp8")
        f16 = f.device_pools()
        desc = ("fp8 KV bits (P = head/4): 12 layers x 12 KV heads x head 64 (64-byte rows), NHD, the gpt2-shaped "
                "request lengths; ")
        if name == "fp8_nhd_bs16":
            return _blocks_row(dev, name, desc + "block 16", f16, "NHD", f.layer_numbers, f.req, f.valid_bytes(),
                               calls, n_check, 14)
        if name == "fp8_nhd_bs64":
            f64, r64 = repaged(f16, "NHD", f.req, 64, 42, lambda n: wl.pool_shape("NHD", n, 64, 12, 64), torch.uint8)
            del f16
            return _blocks_row(dev, name, desc + "re-paged at block 64", f64, "NHD", f.layer_numbers, r64,
                               f.valid_bytes(), calls, n_check, 15)
    if name.startswith("mla"):
        m = wl.mla()
        m64 = m.device_pools()
        desc = "MLA-style latent cache: 61 layers x 1 head of 576 bf16 bits, 64 requests of 128-2048 tokens; "
        if name == "mla_bs64":
            return _blocks_row(dev, name, desc + "block 64", m64, "MLA", m.layer_numbers, m.req, m.valid_bytes(),
                               calls, n_check, 16)
        if name == "mla_bs16":
            m16, r16 = repaged(m64, "MLA", m.req, 16, 43, lambda n: (n, 16, 576), m64[0].dtype)
            del m64
            return _blocks_row(dev, name, desc + "re-paged at block 16", m16, "MLA", m.layer_numbers, r16,
                               m.valid_bytes(), calls, n_check, 17)
    if name == "hybrid_attn":
        attn, _ = wl.hybrid()
        pa = attn.device_pools()
        return _blocks_row(dev, name, "hybrid model attention group: 24 layers (numbers 0,2,..,46) x 8 KV heads x "
                                      "head 128 bf16, block 16, HND, 128 requests of 512-8192 tokens", pa,
                           attn.layout, attn.layer_numbers, attn.req, attn.valid_bytes(), calls, n_check, 18)
    if name == "hybrid_mamba":
        import oracle
        _, mamba = wl.hybrid()
        states = mamba.device_states()
        sid = torch.from_numpy(mamba.slot_ids).to(dev)
        sout = torch.zeros(len(mamba.slot_ids), dtype=torch.uint64, device=dev)
        sws = torch.empty(max(256, kvck.kvck_states_workspace_bytes(len(mamba.layer_numbers), mamba.rows_used,
                                                                    len(mamba.slot_ids))), dtype=torch.uint8,
                          device=dev)
        med, mn, untimed = _timed_main_pass(lambda: kvck.kvck_checksum_states(states, mamba.layer_numbers, sid,
                                                                              out=sout, workspace=sws), calls)
        got = sout.cpu().numpy().view(np.uint64)
        # every request (its position 0), from host copies of its slot in every state
        mism = 0
        R = len(mamba.slot_ids)
        for r0 in range(0, R, 32):
            rs = list(range(r0, min(R, r0 + 32)))
            idx = torch.from_numpy(mamba.slot_ids[rs].astype(np.int64)).to(dev)
            host = [[_host_bits(s.index_select(0, idx)) for s in lay] for lay in states]
            want = oracle.checksum_states(host, mamba.layer_numbers, mamba.bases, np.arange(len(rs)))
            mism += int(np.sum(got[rs] != want))
        row = _row(name, "hybrid model Mamba group: 24 layers (numbers 1,3,..,47) x 128 requests x 64 rows of fp32 "
                         "SSM [128x16] + fp16 conv [4x256] state, position 0", mamba.valid_bytes(), med, mn, R, mism,
                   untimed)
        print(f"[config] {name:14s} {row['valid_bytes'] / 1e9:7.2f} GB {med:8.3f} ms {row['GB_per_s']:8.1f} GB/s "
              f"{row['frac_of_hbm_peak'] * 100:5.1f} %  oracle {R} requests, {mism} mismatches",
              file=sys.stderr, flush=True)
        return row
    raise SystemExit(f"unknown configuration {name!r}; one of {CONFIG_NAMES}")


def config_rows(names, dev, calls=10, n_check=200):
    import torch
    rows = []
    for n in names:
        rows.append(config_row(n, dev, calls, n_check))
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return rows


def config_rows_isolated(names, calls=10, n_check=200, timeout=300):
    """Each configuration row in a child process of its own (``bench.py
    --only NAME``), before the headline allocates anything.  Pool placement
    follows the allocation history.  The same hybrid attention pools read at
    87.6 % of 8 TB/s as a process's first allocation, and at 81.7-84.8 % after
    other pool sets had come and gone in that process, so every row is
    measured as a first allocation, like the headline.  The device's history
    counts too: right after a process has held the headline's 154 GB, every
    row, and the headline itself, read 1-6 points lower (hybrid attention
    84.6 %, headline 83.4 %).  With the rows run first, the same box read
    87.6 % and 86.9 %.  A row whose child fails is reported with its error."""
    import subprocess
    rows = []
    for n in names:
        cmd = [sys.executable, os.path.abspath(__file__), "--only", n, "--config-calls", str(calls),
               "--oracle-positions", str(n_check), "--config-warmup-ms", str(WARMUP_MS)]
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout)
        except subprocess.TimeoutExpired:
            rows.append({"config": n, "error": f"timed out after {timeout} s"})
            continue
        sys.stderr.write("".join(ln + "\n" for ln in r.stderr.splitlines() if ln.startswith("[config]")))
        sys.stderr.flush()
        lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
        if r.returncode != 0 or not lines:
            rows.append({"config": n, "error": f"exit status {r.returncode}: {r.stderr[-400:]}"})
            continue
        rows += json.loads(lines[-1])["configs"]
    return rows


def copy_calibration(dev, gib):
    """One plain device copy of ``gib`` GiB (the runtime's copy kernel): the
    reference that rocprofv3 counter runs scale FETCH_SIZE / WRITE_SIZE by."""
    import torch
    n = int(gib * (1 << 30))
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty(n, dtype=torch.uint8, device=dev)
    a.fill_(1)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    return n


# ----------------------------------------------------------------- main

def main(argv=None):
    global WARMUP_MS
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3_8b")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="processes of the parallel oracle leg (0: the host's CPUs, at most 16)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-shard", action="store_true", help="skip the TP-shard row")
    ap.add_argument("--no-copy", action="store_true", help="skip the fused copy + checksum timing")
    ap.add_argument("--no-small", action="store_true", help="skip the tiny-call latency timing")
    ap.add_argument("--no-configs", action="store_true", help="skip the other configurations' rows")
    ap.add_argument("--only", default="", help="comma-separated configuration rows to run alone (no headline)")
    ap.add_argument("--configs-after", action="store_true",
                    help="run the configuration rows' child processes after the headline instead of before it")
    ap.add_argument("--config-calls", type=int, default=10, help="timed calls per configuration row")
    ap.add_argument("--config-warmup-ms", type=float, default=WARMUP_MS,
                    help="untimed calls before a row's timed ones: two, then about this many ms more (0: two)")
    ap.add_argument("--oracle-positions", type=int, default=200,
                    help="random positions per configuration checked against the oracle (plus every tail)")
    ap.add_argument("--copy-calibration-gib", type=float, default=0.0,
                    help="after timing, run one plain device copy of this many GiB (counter calibration)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported (the checksum path is "
              f"single-GPU; partial sums of head or layer shards add up across GPUs)", file=sys.stderr)
        return 1

    import torch
    import paged_kv_cache_kvck_amd as kvck

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    WARMUP_MS = args.config_warmup_ms
    if args.only:
        names = [n for n in args.only.split(",") if n]
        rows = config_rows(names, dev, args.config_calls, args.oracle_positions)
        res = {"configs": rows}
        if args.copy_calibration_gib > 0:
            res["copy_calibration_bytes"] = copy_calibration(dev, args.copy_calibration_gib)
        print(json.dumps(res), flush=True)
        return 0

    # The configuration rows run first, each in a child process, before this
    # process allocates anything: see config_rows_isolated.
    early_rows = None
    if not args.configs_after and not args.no_configs:
        early_rows = config_rows_isolated(CONFIG_NAMES, args.config_calls, args.oracle_positions)
    w, desc = make_workload(args.workload)
    print(f"[bench] building {args.workload}: pools {w.shape} x {w.num_layers}", file=sys.stderr, flush=True)
    pools = w.device_pools()
    req = w.req
    bt = torch.from_numpy(req.block_table).to(dev)
    nb = torch.from_numpy(req.num_blocks).to(dev)
    sp = torch.from_numpy(req.start_pos).to(dev)
    nt = torch.from_numpy(req.num_tokens).to(dev)
    out = torch.zeros((req.num_reqs, req.max_blocks), dtype=torch.uint64, device=dev)
    ws = torch.empty(kvck.kvck_blocks_workspace_bytes(w.num_layers, req.num_reqs, req.max_blocks),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    prepared = {}

    def step(head_begin=w.head_begin, head_count=w.head_count, bases=None, o=out):
        key = (head_begin, head_count, None if bases is None else tuple(bases))
        if key not in prepared:
            prepared[key] = kvck.prepare_caches(pools, w.layout, w.layer_numbers, global_head_base=bases,
                                                head_begin=head_begin, head_count=head_count)
        kvck.kvck_checksum_blocks(prepared[key], None, None, bt, nb, sp, nt, out=o, workspace=ws, stream=stream)

    valid = w.valid_bytes()
    kvck.kvck_instrument(True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    kvck.kvck_instrument_read()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        step()
        marks[i].record(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    per_step = [e0.elapsed_time(marks[0])] + [marks[i - 1].elapsed_time(marks[i]) for i in range(1, args.steps)]
    main_ms, calls = kvck.kvck_instrument_read()
    main_avg = main_ms / max(calls, 1)
    out_main = out.cpu().numpy().view("uint64").copy()  # the timed steps' checksums, for the oracle check
    achieved = valid / (main_avg * 1e-3) / 1e9

    extra = {"valid_bytes_per_step": valid, "pct_of_hbm_peak": valid / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS * 100,
             "main_pass_ms": main_avg,
             "step_ms_median": statistics.median(per_step), "step_ms_min": min(per_step),
             "listed_positions": int(req.num_blocks.sum()),
             "metadata_bytes_per_step": int(req.num_blocks.sum()) * (4 + 8 + 32) + req.num_reqs * 20}
    configs = []
    if not args.no_shard:
        # TP = 4 shard over heads {2, 3}, global numbering from 2: every step
        # timed with the headline's instrumentation, then sampled positions of
        # the last step checked against the oracle
        shard_bytes = valid // 4
        sbases = [2] * w.num_layers
        sout = torch.zeros_like(out)
        for _ in range(2):
            step(2, 2, sbases, sout)
        torch.cuda.synchronize()
        kvck.kvck_instrument_read()
        e0.record(stream)
        for _ in range(args.steps):
            step(2, 2, sbases, sout)
        e1.record(stream)
        torch.cuda.synchronize()
        sms = e0.elapsed_time(e1) / args.steps
        smain, sc = kvck.kvck_instrument_read()
        got = sout.cpu().numpy().view("uint64")
        checked, mism = oracle_check(pools, w.layout, w.layer_numbers, sbases, req, got,
                                     sample_positions(req, args.oracle_positions, 10), 2, 2)
        row = _row("llama3_8b_tp4_shard", "the headline pools, TP = 4 shard: local heads {2,3} with global numbering "
                   "from 2", shard_bytes, smain / max(sc, 1), smain / max(sc, 1), checked, mism)
        row["ms_per_step"] = sms
        row["step_GB_per_s"] = shard_bytes / (sms * 1e-3) / 1e9
        configs.append(row)
        print(f"[config] shard: {row['main_pass_ms']:.3f} ms {row['frac_of_hbm_peak'] * 100:.1f} %, oracle "
              f"{checked} positions, {mism} mismatches", file=sys.stderr, flush=True)
        del sout
    # offloaded-checksum check of every listed position: tag, compare, count
    hashes = torch.randint(0, 256, (req.num_reqs * req.max_blocks, 32), dtype=torch.uint8, device=dev)
    stored, _ = kvck.kvck_tag_checksums(out.view(-1), hashes, 0x1234, num_blocks_per_req=nb, stream=stream)
    mism_t = torch.zeros(req.num_reqs * req.max_blocks, dtype=torch.uint8, device=dev)
    cnt = torch.zeros(1, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        kvck.kvck_tag_checksums(out.view(-1), hashes, 0x1234, num_blocks_per_req=nb, tagged=False, stored=stored,
                                mismatch=mism_t, mismatch_count=cnt, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    extra["offload_check"] = {"positions": int(req.num_blocks.sum()),
                              "us_per_call": e0.elapsed_time(e1) / args.steps * 1e3, "mismatches": int(cnt.item())}
    del hashes, stored, mism_t

    if not args.no_copy:
        # connector save / load fused with the checksum, on the first half of the requests
        half = req.num_reqs // 2
        hb_t, hn_t, hs_t, ht_t = (x[:half].contiguous() for x in (bt, nb, sp, nt))
        entries = int(req.num_blocks[:half].sum())
        per = kvck.kvck_staging_bytes(pools[0], w.layout, w.num_layers)
        staging = torch.empty(entries * per, dtype=torch.uint8, device=dev)
        cout = torch.zeros((half, req.max_blocks), dtype=torch.uint64, device=dev)
        cws = torch.empty(kvck.kvck_blocks_workspace_bytes(w.num_layers, half, req.max_blocks), dtype=torch.uint8,
                          device=dev)
        moved = 0
        for r in range(half):
            lo = int(req.start_pos[r]) * req.block_size
            hi = min(int(req.num_tokens[r]), (int(req.start_pos[r]) + int(req.num_blocks[r])) * req.block_size)
            moved += max(0, hi - lo)
        moved *= w.num_layers * w.heads_used * w.planes * w.head_size * 2
        res = {"valid_bytes": moved, "bytes_moved": 2 * moved}
        ncalls = max(2, args.steps // 4)
        for name, direction in (("save", kvck.KVCK_COPY_SAVE), ("load", kvck.KVCK_COPY_LOAD)):
            def cstep():
                kvck.kvck_copy_checksum_blocks(direction, pools, w.layout, w.layer_numbers, hb_t, hn_t, hs_t, ht_t,
                                               staging, out=cout, workspace=cws, stream=stream)
            cstep()
            torch.cuda.synchronize()
            kvck.kvck_instrument_read()
            e0.record(stream)
            for _ in range(ncalls):
                cstep()
            e1.record(stream)
            torch.cuda.synchronize()
            cms = e0.elapsed_time(e1) / ncalls
            cmain, cc = kvck.kvck_instrument_read()
            cmain /= max(cc, 1)
            res[name] = {"ms_per_call": cms, "main_pass_ms": cmain,
                         "read_plus_write_GB_per_s": 2 * moved / (cmain * 1e-3) / 1e9,
                         "frac_of_hbm_peak": 2 * moved / (cmain * 1e-3) / 1e9 / HBM_PEAK_GBS}
        # the load wrote back what the save read: the pool is unchanged, and so are its checksums
        got = cout.cpu().numpy().view("uint64")
        res["load_checksums_equal_timed_steps"] = bool(all(int(got[r, k]) == int(out_main[r, k])
                                                           for r in range(half)
                                                           for k in range(int(req.num_blocks[r]))))
        extra["fused_copy_half_batch"] = res
        del staging
    kvck.kvck_instrument(False)

    cpu = None
    if not args.no_cpu_baseline:
        workers = args.cpu_workers or min(16, os.cpu_count() or 1)
        print(f"[bench] cpu baseline (oracle): one process, then {workers} over layer subsets", file=sys.stderr,
              flush=True)
        cpu = cpu_baseline(pools, w, args.cpu_seconds, out_main, workers)
        cpu["host_cpu"] = _cpu_model()
    del pools, prepared
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    if not args.no_configs:
        configs += early_rows if early_rows is not None else config_rows_isolated(CONFIG_NAMES, args.config_calls,
                                                                                  args.oracle_positions)
    if configs:
        extra["configs"] = configs
    if not args.no_small:
        # the tiny configuration (one 50-token request on 4 blocks, 2 layers x 2 heads): latency-bound,
        # so each call is timed on its own, event to event, with caches prepared as a hot loop would
        from paged_kv_cache_kvck_amd import workloads as wl
        tw = wl.tiny()
        tpools = tw.device_pools()
        tr = tw.req
        tt = [torch.from_numpy(x).to(dev) for x in (tr.block_table, tr.num_blocks, tr.start_pos, tr.num_tokens)]
        tout = torch.zeros((tr.num_reqs, tr.max_blocks), dtype=torch.uint64, device=dev)
        tws = torch.empty(kvck.kvck_blocks_workspace_bytes(tw.num_layers, tr.num_reqs, tr.max_blocks),
                          dtype=torch.uint8, device=dev)
        tpc = kvck.prepare_caches(tpools, tw.layout, tw.layer_numbers)
        lat = []
        for i in range(60):
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record(stream)
            kvck.kvck_checksum_blocks(tpc, None, None, *tt, out=tout, workspace=tws, stream=stream)
            t1.record(stream)
            torch.cuda.synchronize()
            if i >= 10:
                lat.append(t0.elapsed_time(t1) * 1e3)
        got = tout.cpu().numpy().view("uint64")
        checked, mism = oracle_check(tpools, tw.layout, tw.layer_numbers, tw.bases, tr, got, tr.listed())
        # the same call through a PreparedCall (every argument marshalled once)
        pout = torch.zeros_like(tout)
        pcall = kvck.prepare_call(tpc, *tt, pout, tws, stream=stream)
        plat = []
        for i in range(60):
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record(stream)
            pcall()
            t1.record(stream)
            torch.cuda.synchronize()
            if i >= 10:
                plat.append(t0.elapsed_time(t1) * 1e3)
        same = bool(torch.equal(pout.view(torch.int64), tout.view(torch.int64)))
        extra["tiny_call_latency"] = {"workload": "2 layers x 2 KV heads x head 64 bf16, block 16, NHD, one 50-token "
                                                  "request on 4 blocks (51,200 valid bytes)",
                                      "us_median": statistics.median(lat), "us_min": min(lat), "calls": len(lat),
                                      "prepared_call_us_median": statistics.median(plat),
                                      "prepared_call_us_min": min(plat), "prepared_call_equals": same,
                                      "oracle_checked_positions": checked, "oracle_mismatches": mism}
        del tpools, tpc, pcall
    if args.copy_calibration_gib > 0:
        extra["copy_calibration_bytes"] = copy_calibration(dev, args.copy_calibration_gib)

    line = {
        "metric": "checksummed KV GB/s and % of MI355X HBM peak; bit-exact vs CPU oracle",
        "value": valid / (ms_step * 1e-3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u64",
        "data": "synthetic",
        "config": {"workload": desc, "num_layers": w.num_layers, "kv_heads": w.heads_used, "head_size": w.head_size,
                   "block_size": req.block_size, "layout": w.layout, "num_requests": req.num_reqs,
                   "tokens": w.valid_tokens(), "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": committed_traffic(args.workload)},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)
    return 0


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip() + f" ({os.cpu_count()} logical CPUs visible)"
    except OSError:
        pass
    return f"{os.cpu_count()} logical CPUs"


if __name__ == "__main__":
    sys.exit(main())
