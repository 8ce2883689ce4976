#!/usr/bin/env python3
"""Benchmark of the KV-cache block checksum on one MI355X.

One step = one kvck_checksum_blocks call over the whole batch of the
Llama-3-8B-shaped cache (32 layers x 8 KV heads x head 128, bf16 normal(0,1)
values, block 16, HND pool, 256 requests of 512..8192 tokens): plan, main
pass over every valid K/V byte, second pass.  Inputs are resident in HBM
before timing starts.

    python bench.py [--steps K] [--warmup W] [--workload llama3_8b|gpt2|hybrid_attn]

Prints one JSON line: throughput in checksummed KV GB/s (valid cache bytes /
step time), the roofline of the main pass (its own HIP events on its stream,
via the library's instrumentation), and the CPU oracle's rate on a bounded
sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published

from paged_kv_cache_kvck_amd.sources import code_only as _code_only, kernel_sources_sha  # noqa: E402


def committed_traffic(workload: str):
    """HBM bytes per launch of the main pass from the committed rocprofv3
    counter summary, or None when the kernel sources changed since."""
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
        return wl.llama3_8b(), ("llama3-8b-shaped paged KV cache: 32 layers x 8 KV heads x head 128 bf16 "
                                "normal(0,1), block 16, HND, 256 requests of 512-8192 tokens")
    if name == "gpt2":
        return wl.gpt2(), ("gpt2-shaped paged KV cache: 12 layers x 12 KV heads x head 64 fp16 random bits, "
                           "block 16, NHD pool (2,18545,16,12,64) per layer, 64 requests of 128-2048 tokens")
    if name == "hybrid_attn":
        return wl.hybrid()[0], ("hybrid model attention group: 24 layers x 8 KV heads x head 128 bf16, block 16, "
                                "HND, 128 requests of 512-8192 tokens")
    raise SystemExit(f"unknown workload {name}")


def cpu_baseline(pools, w, seconds, gpu_out=None, seed=0):
    """The oracle, as it stands, on a bounded random sample of listed positions
    (host copies of their blocks are made outside the timed region).  Each
    value it computes is also compared with ``gpu_out`` (the GPU's checksums of
    the timed steps, uint64 [num_reqs, max_blocks]) when given."""
    import numpy as np
    import torch
    import oracle
    from paged_kv_cache_kvck_amd import workloads as wl

    rng = np.random.default_rng(seed)
    allpos = w.req.listed()
    order = rng.permutation(len(allpos))
    done, nbytes, elapsed, i, mismatches = 0, 0, 0.0, 0, 0
    row = w.heads_used * w.planes * w.head_size * wl.ELEM_BYTES[w.elem] * w.num_layers
    while elapsed < seconds and i < len(order):
        chunk = [allpos[j] for j in order[i:i + 32]]
        i += 32
        ids = sorted({int(w.req.block_table[r, k]) for r, k in chunk})
        remap = {b: n for n, b in enumerate(ids)}
        idx = torch.tensor(ids, dtype=torch.int64, device=pools[0].device)
        mini = []
        for p in pools:
            sub = p.index_select(0 if w.layout == "MLA" else 1, idx).contiguous()
            mini.append(sub.view(torch.int16).cpu().numpy().view(np.uint16))
        t0 = time.perf_counter()
        vals = [oracle.kv_checksum.checksum_position(mini, w.layout, w.layer_numbers, w.bases,
                                                     remap[int(w.req.block_table[r, k])],
                                                     int(w.req.start_pos[r]) + k, int(w.req.num_tokens[r]),
                                                     w.head_begin, w.head_count) for r, k in chunk]
        elapsed += time.perf_counter() - t0
        if gpu_out is not None:
            mismatches += sum(int(gpu_out[r, k]) != v for (r, k), v in zip(chunk, vals))
        for r, k in chunk:
            pos = int(w.req.start_pos[r]) + k
            v = min(w.req.block_size, max(0, int(w.req.num_tokens[r]) - pos * w.req.block_size))
            nbytes += v * row
        done += len(chunk)
    res = {"value": nbytes / elapsed / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"{done} random listed positions of the same workload ({nbytes} valid bytes, all layers and "
                     f"heads), numpy single-threaded, {elapsed:.1f} s of oracle time; host copies excluded"}
    if gpu_out is not None:
        # the same positions of the timed GPU steps, compared bit for bit
        res["gpu_checked_positions"] = done
        res["gpu_mismatches"] = mismatches
    return res


def _oracle_worker(args):
    """One process of the parallel CPU baseline: the oracle on host pools of
    the workload's shapes (random bits), full blocks at random positions, for
    about ``seconds``.  Uses numpy only; never touches the GPU."""
    seed, seconds, layout, nb, bs, nh, d, elem, layers, bases, head_begin, head_count = args
    import numpy as np
    import oracle
    from paged_kv_cache_kvck_amd import workloads as wl
    rng = np.random.default_rng(seed)
    pools = [wl.host_random_bits(rng, wl.pool_shape(layout, nb, bs, nh, d), elem) for _ in layers]
    n = nh - head_begin if head_count is None else head_count
    per_block = bs * n * 2 * d * wl.ELEM_BYTES[elem] * len(layers)
    done, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        b, pos = int(rng.integers(0, nb)), int(rng.integers(0, 512))
        oracle.kv_checksum.checksum_position(pools, layout, layers, bases, b, pos, (pos + 1) * bs, head_begin,
                                             head_count)
        done += 1
    return done * per_block, time.perf_counter() - t0


def cpu_baseline_parallel(w, seconds, workers):
    """The oracle in ``workers`` fresh processes at once (spawned: numpy only),
    each on its own host pools of the workload's shapes: aggregate GB/s."""
    import multiprocessing as mp
    args = [(1000 + i, seconds, w.layout, 64, w.req.block_size, w.num_heads, w.head_size, w.elem,
             list(w.layer_numbers), list(w.bases), w.head_begin, w.head_count) for i in range(workers)]
    pool = mp.get_context("spawn").Pool(workers)
    try:
        # bounded: workers that cannot start (no importable main module) would be respawned forever
        res = pool.map_async(_oracle_worker, args).get(timeout=seconds + 120)
    except Exception as e:  # timeout or a worker error: no parallel figure
        print(f"[bench] parallel cpu baseline skipped: {e!r}", file=sys.stderr, flush=True)
        return None
    finally:
        pool.terminate()
        pool.join()
    nbytes = sum(r[0] for r in res)
    wall = max(r[1] for r in res)
    return {"value": nbytes / wall / 1e9, "unit": "GB/s", "cores": workers,
            "sample": f"{workers} processes x {seconds:.0f} s, each the oracle on its own host pools of the "
                      f"workload's shapes (64 blocks per layer, random bits), full blocks at random positions"}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3_8b")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="processes of the parallel CPU baseline (0: the host's CPUs, at most 16)")
    ap.add_argument("--cpu-parallel-seconds", type=float, default=5.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-shard", action="store_true", help="skip the TP-shard timing")
    ap.add_argument("--no-states", action="store_true", help="skip the Mamba-state timing")
    ap.add_argument("--no-copy", action="store_true", help="skip the fused copy + checksum timing")
    ap.add_argument("--no-small", action="store_true", help="skip the tiny-call latency timing")
    ap.add_argument("--survey", action="store_true",
                    help="after the headline, time the main pass of every other configuration (extra.survey)")
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

    def step(head_begin=w.head_begin, head_count=w.head_count, bases=None):
        key = (head_begin, head_count, None if bases is None else tuple(bases))
        if key not in prepared:
            prepared[key] = kvck.prepare_caches(pools, w.layout, w.layer_numbers, global_head_base=bases,
                                                head_begin=head_begin, head_count=head_count)
        kvck.kvck_checksum_blocks(prepared[key], None, None, bt, nb, sp, nt, out=out, workspace=ws, stream=stream)

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
    if not args.no_shard and w.layout == "HND" and w.num_heads == 8:
        # TP = 4 shard over heads {2, 3}, global numbering from 2
        shard_bytes = valid // 4
        for _ in range(2):
            step(2, 2, [2] * w.num_layers)
        torch.cuda.synchronize()
        kvck.kvck_instrument_read()
        e0.record(stream)
        for _ in range(args.steps):
            step(2, 2, [2] * w.num_layers)
        e1.record(stream)
        torch.cuda.synchronize()
        sms = e0.elapsed_time(e1) / args.steps
        smain, sc = kvck.kvck_instrument_read()
        extra["tp4_shard_heads_2_3"] = {"valid_bytes": shard_bytes, "ms_per_step": sms,
                                        "GB_per_s": shard_bytes / (sms * 1e-3) / 1e9,
                                        "main_pass_ms": smain / max(sc, 1),
                                        "main_pass_GB_per_s": shard_bytes / (smain / max(sc, 1) * 1e-3) / 1e9}
    # offloaded-checksum check of every listed position: tag, compare, count
    hashes = torch.randint(0, 256, (req.num_reqs * req.max_blocks, 32), dtype=torch.uint8, device=dev)
    stored, _ = kvck.kvck_tag_checksums(out.view(-1), hashes, 0x1234, num_blocks_per_req=nb, stream=stream)
    mism = torch.zeros(req.num_reqs * req.max_blocks, dtype=torch.uint8, device=dev)
    cnt = torch.zeros(1, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        kvck.kvck_tag_checksums(out.view(-1), hashes, 0x1234, num_blocks_per_req=nb, tagged=False, stored=stored,
                                mismatch=mism, mismatch_count=cnt, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    extra["offload_check"] = {"positions": int(req.num_blocks.sum()), "us_per_call": e0.elapsed_time(e1) / args.steps * 1e3,
                              "mismatches": int(cnt.item())}
    del hashes, stored, mism

    if not args.no_copy and w.layout == "HND":
        # connector save / load fused with the checksum, on the first half of the requests
        half = req.num_reqs // 2
        hb_t, hn_t, hs_t, ht_t = bt[:half].contiguous(), nb[:half].contiguous(), sp[:half].contiguous(), nt[:half].contiguous()
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
        for name, direction in (("save", kvck.KVCK_COPY_SAVE), ("load", kvck.KVCK_COPY_LOAD)):
            def cstep():
                kvck.kvck_copy_checksum_blocks(direction, pools, w.layout, w.layer_numbers, hb_t, hn_t, hs_t, ht_t,
                                               staging, out=cout, workspace=cws, stream=stream)
            cstep()
            torch.cuda.synchronize()
            kvck.kvck_instrument_read()
            e0.record(stream)
            for _ in range(max(2, args.steps // 4)):
                cstep()
            e1.record(stream)
            torch.cuda.synchronize()
            cms = e0.elapsed_time(e1) / max(2, args.steps // 4)
            cmain, cc = kvck.kvck_instrument_read()
            cmain /= max(cc, 1)
            res[name] = {"ms_per_call": cms, "main_pass_ms": cmain,
                         "read_plus_write_GB_per_s": 2 * moved / (cmain * 1e-3) / 1e9,
                         "frac_of_hbm_peak": 2 * moved / (cmain * 1e-3) / 1e9 / HBM_PEAK_GBS}
        extra["fused_copy_half_batch"] = res
        del staging

    if not args.no_states:
        # Mamba running-state rows: the hybrid workload's 24 Mamba layers
        from paged_kv_cache_kvck_amd import workloads as wl
        mamba = wl.hybrid()[1]
        states = mamba.device_states()
        sid = torch.from_numpy(mamba.slot_ids).to(dev)
        sout = torch.zeros(len(mamba.slot_ids), dtype=torch.uint64, device=dev)
        sws = torch.empty(max(256, kvck.kvck_states_workspace_bytes(len(mamba.layer_numbers), mamba.rows_used,
                                                                    len(mamba.slot_ids))), dtype=torch.uint8,
                          device=dev)

        def sstep():
            kvck.kvck_checksum_states(states, mamba.layer_numbers, sid, out=sout, workspace=sws, stream=stream)

        for _ in range(2):
            sstep()
        torch.cuda.synchronize()
        kvck.kvck_instrument_read()
        e0.record(stream)
        for _ in range(args.steps):
            sstep()
        e1.record(stream)
        torch.cuda.synchronize()
        sms = e0.elapsed_time(e1) / args.steps
        smain, sc = kvck.kvck_instrument_read()
        sb = mamba.valid_bytes()
        extra["mamba_states"] = {"workload": "24 Mamba layers x 128 requests x 64 rows of fp32 SSM [128x16] + fp16 "
                                             "conv [4x256] state", "valid_bytes": sb, "ms_per_step": sms,
                                 "GB_per_s": sb / (sms * 1e-3) / 1e9, "main_pass_ms": smain / max(sc, 1),
                                 "main_pass_GB_per_s": sb / (smain / max(sc, 1) * 1e-3) / 1e9}
        del states
    kvck.kvck_instrument(False)
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
        extra["tiny_call_latency"] = {"workload": "2 layers x 2 KV heads x head 64 bf16, block 16, NHD, one 50-token "
                                                  "request on 4 blocks (51,200 valid bytes)",
                                      "us_median": statistics.median(lat), "us_min": min(lat), "calls": len(lat)}
        del tpools, tpc
    if args.copy_calibration_gib > 0:
        n = int(args.copy_calibration_gib * (1 << 30))
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty(n, dtype=torch.uint8, device=dev)
        a.fill_(1)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        extra["copy_calibration_bytes"] = n
        del a, b

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(pools, w, args.cpu_seconds, gpu_out=out_main)
        cpu["host_cpu"] = _cpu_model()
        workers = args.cpu_workers or min(16, os.cpu_count() or 1)
        print(f"[bench] cpu baseline, {workers} processes", file=sys.stderr, flush=True)
        cpu["parallel"] = cpu_baseline_parallel(w, args.cpu_parallel_seconds, workers)

    if args.survey:
        del pools
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        extra["survey"] = config_survey(dev)

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


def config_survey(dev, calls=10):
    """Main-pass time of each other configuration (median of `calls` calls,
    HIP events around the main pass), one after another in this process: the
    GPT-2-shaped pool and its re-pagings (block 64, HND, fp8 bits at blocks 16
    and 64), the 61-layer MLA latent at blocks 64 and 16, and the hybrid
    model's attention group and Mamba states.  Rows are printed to stderr as
    they finish."""
    import numpy as np
    import torch
    import paged_kv_cache_kvck_amd as kvck
    from paged_kv_cache_kvck_amd import workloads as wl

    rows = []

    def timed(call):
        kvck.kvck_instrument(True)
        call()
        call()
        torch.cuda.synchronize()
        kvck.kvck_instrument_read()
        ts = []
        for _ in range(calls):
            call()
            torch.cuda.synchronize()
            ms, c = kvck.kvck_instrument_read()
            ts.append(ms / c)
        kvck.kvck_instrument(False)
        return statistics.median(ts)

    def report(name, valid, ms):
        gbs = valid / (ms * 1e-3) / 1e9
        rows.append({"config": name, "valid_bytes": valid, "main_pass_ms": ms, "GB_per_s": gbs,
                     "pct_of_hbm_peak": gbs / HBM_PEAK_GBS * 100})
        print(f"[survey] {name:52s} {valid / 1e9:7.2f} GB {ms:8.3f} ms {gbs:8.1f} GB/s "
              f"{gbs / HBM_PEAK_GBS * 100:5.1f} %", file=sys.stderr, flush=True)

    def blocks(name, pools, layout, layers, req, valid):
        bt, nb, sp, nt = (torch.from_numpy(x).to(dev) for x in
                          (req.block_table, req.num_blocks, req.start_pos, req.num_tokens))
        out = torch.zeros((req.num_reqs, req.max_blocks), dtype=torch.uint64, device=dev)
        ws = torch.empty(kvck.kvck_blocks_workspace_bytes(len(pools), req.num_reqs, req.max_blocks),
                         dtype=torch.uint8, device=dev)
        pc = kvck.prepare_caches(pools, layout, layers)
        report(name, valid, timed(lambda: kvck.kvck_checksum_blocks(pc, None, None, bt, nb, sp, nt, out=out,
                                                                    workspace=ws)))

    def free():
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

    g = wl.gpt2()
    p = g.device_pools()
    blocks("gpt2 NHD fp16, block 16", p, "NHD", g.layer_numbers, g.req, g.valid_bytes())
    r64, n64 = wl.page_requests(np.random.default_rng(40), g.req.num_tokens, 64, spare_frac=0.05)
    p64 = [torch.zeros(wl.pool_shape("NHD", n64, 64, 12, 64), dtype=p[0].dtype, device=dev) for _ in p]
    for s_, d_ in zip(p, p64):
        wl.repage_torch(s_, "NHD", g.req, d_, "NHD", r64)
    blocks("gpt2 tokens re-paged at block 64 (NHD)", p64, "NHD", g.layer_numbers, r64, g.valid_bytes())
    del p64
    free()
    ph = [x.permute(0, 1, 3, 2, 4).contiguous() for x in p]
    blocks("gpt2 pool as HND, block 16", ph, "HND", g.layer_numbers, g.req, g.valid_bytes())
    del ph, p
    free()
    f = wl.gpt2(seed=41, elem="fp8")
    f16 = f.device_pools()
    blocks("fp8 bits 12 x 64 (64-byte rows) NHD, block 16", f16, "NHD", f.layer_numbers, f.req, f.valid_bytes())
    rf64, nf64 = wl.page_requests(np.random.default_rng(42), f.req.num_tokens, 64, spare_frac=0.05)
    f64 = [torch.zeros(wl.pool_shape("NHD", nf64, 64, 12, 64), dtype=torch.uint8, device=dev) for _ in f16]
    for s_, d_ in zip(f16, f64):
        wl.repage_torch(s_, "NHD", f.req, d_, "NHD", rf64)
    blocks("fp8 bits NHD, block 64", f64, "NHD", f.layer_numbers, rf64, f.valid_bytes())
    del f16, f64
    free()
    m = wl.mla()
    m64 = m.device_pools()
    blocks("MLA 61 x 576 bf16, block 64", m64, "MLA", m.layer_numbers, m.req, m.valid_bytes())
    rm16, nm16 = wl.page_requests(np.random.default_rng(43), m.req.num_tokens, 16, spare_frac=0.05)
    m16 = [torch.zeros((nm16, 16, 576), dtype=m64[0].dtype, device=dev) for _ in m64]
    for s_, d_ in zip(m64, m16):
        wl.repage_torch(s_, "MLA", m.req, d_, "MLA", rm16)
    blocks("MLA, block 16", m16, "MLA", m.layer_numbers, rm16, m.valid_bytes())
    del m64, m16
    free()
    attn, mamba = wl.hybrid()
    pa = attn.device_pools()
    blocks("hybrid attention group (24 x 8 x 128 bf16 HND)", pa, attn.layout, attn.layer_numbers, attn.req,
           attn.valid_bytes())
    del pa
    free()
    states = mamba.device_states()
    sid = torch.from_numpy(mamba.slot_ids).to(dev)
    sout = torch.zeros(len(mamba.slot_ids), dtype=torch.uint64, device=dev)
    sws = torch.empty(max(256, kvck.kvck_states_workspace_bytes(len(mamba.layer_numbers), mamba.rows_used,
                                                                len(mamba.slot_ids))), dtype=torch.uint8, device=dev)
    report("hybrid Mamba states (24 layers x 128 requests)", mamba.valid_bytes(),
           timed(lambda: kvck.kvck_checksum_states(states, mamba.layer_numbers, sid, out=sout, workspace=sws)))
    del states
    free()
    return rows


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
