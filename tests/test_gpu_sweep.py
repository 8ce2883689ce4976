"""Seeded sweep of small random configurations: HIP path == oracle at every
listed position (GPU).

Each case draws a layout (NHD, HND, FlashInfer-style, MLA, x-split K + V,
K + element-transposed V), an element type, head count and size, block size,
layer numbers up to the largest allowed, requests with start offsets, past-end
positions and empty requests, an optional head subset, a forced schedule or
merge setting, and sometimes the listed plan in place of planning in place --
the corners where lane-table shapes and schedules change.
The cases are fixed by the seed, so a failure names a reproducible case.
"""

import zlib

import numpy as np
import pytest

import oracle
from paged_kv_cache_kvck_amd import workloads as wl
from gpu_helpers import gpu_blocks, log, to_device_bits

pytestmark = pytest.mark.gpu

LAYOUTS = ["NHD", "HND", "FI_NHD", "FI_HND", "MLA", "XSPLIT_PAIR", "TRANS_PAIR"]



def _spread(x):
    """A drawn layer number x < 2^15 moved up by 0..16 bits (x mod 17), so the
    cases cover layer numbers up to 2^31 - 1 (64-bit slice factors) without
    changing the random stream that draws the rest of each case."""
    return int(x) << (int(x) % 17)

def _case(i):
    rng = np.random.default_rng(zlib.crc32(f"sweep{i}".encode()))
    layout = LAYOUTS[i % len(LAYOUTS)]
    elem = ["fp8", "bf16", "fp16", "fp32"][int(rng.integers(0, 4))]
    es = wl.ELEM_BYTES[elem]
    heads = 1 if layout == "MLA" else int(rng.integers(1, 13))
    # head size: a whole number of 8-byte pieces per row (16-byte runs for x-split)
    unit = 16 // es if layout == "XSPLIT_PAIR" else 8 // es
    d = unit * int(rng.integers(1, max(2, 320 // unit // (4 if layout == "MLA" else 1)) + 1))
    bs_choices = [1, 2, 3, 4, 8, 16, 32, 64]
    if layout == "TRANS_PAIR":
        bs_choices = [b for b in bs_choices if (b * es) % 8 == 0]
    bs = int(rng.choice(bs_choices))
    n_layers = int(rng.integers(1, 5))
    layers = sorted(_spread(x) for x in rng.choice(32768, size=n_layers, replace=False))
    n_req = int(rng.integers(1, 6))
    lengths = [int(x) for x in rng.integers(0, 4 * bs + 40, size=n_req)]
    start = [int(x) for x in rng.integers(0, 3, size=n_req)]
    extra = [int(x) for x in rng.integers(0, 2, size=n_req)]
    hb = int(rng.integers(0, heads))
    hc = int(rng.integers(1, heads - hb + 1))
    if rng.random() < 0.4:
        hb, hc = 0, None
    base = int(rng.integers(0, 65536 - heads))
    env = [{}, {"KVCK_SCHEDULE": "simple"}, {"KVCK_SCHEDULE": "pipelined"}, {"KVCK_MERGE_HEADS": "1"},
           {"KVCK_MERGE_HEADS": "0"}][int(rng.integers(0, 5))]
    if rng.random() < 0.3:
        env = dict(env, KVCK_PLAN="compact")   # positions listed by the plan launch, not planned in place
    return dict(i=i, layout=layout, elem=elem, heads=heads, d=d, bs=bs, layers=layers, lengths=lengths,
                start=start, extra=extra, hb=hb, hc=hc, base=base, env=env)


CASES = [_case(i) for i in range(480)]


def _ids(c):
    return f"{c['i']}-{c['layout']}-{c['elem']}-h{c['heads']}-d{c['d']}-bs{c['bs']}"


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_sweep_case(case, monkeypatch):
    for k, v in case["env"].items():
        monkeypatch.setenv(k, v)
    log(f"[sweep] {_ids(case)} env={case['env']} heads {case['hb']}+{case['hc']} layers {case['layers']}")
    rng = np.random.default_rng(1000 + case["i"])
    layout, bs, nh, d = case["layout"], case["bs"], case["heads"], case["d"]
    req, nb = wl.page_requests(rng, case["lengths"], bs, start_pos=case["start"], extra_blocks=case["extra"],
                               spare_frac=0.3)
    pool_layout = {"XSPLIT_PAIR": "HND", "TRANS_PAIR": "HND"}.get(layout, layout)
    hp = [wl.host_random_bits(rng, wl.pool_shape(pool_layout, nb, bs, nh, d), case["elem"])
          for _ in case["layers"]]
    n = nh - case["hb"] if case["hc"] is None else case["hc"]
    bases = [case["base"] + 3 * j for j in range(len(hp))]
    bases = [min(b, 65536 - n) for b in bases]
    want = oracle.checksum_blocks(hp, pool_layout, case["layers"], bases, req.block_table, req.num_blocks,
                                  req.start_pos, req.num_tokens, head_begin=case["hb"], head_count=n)
    kw = dict(bases=bases, head_begin=case["hb"], head_count=case["hc"])
    if layout == "XSPLIT_PAIR":
        x = 16 // wl.ELEM_BYTES[case["elem"]]
        k = [to_device_bits(np.ascontiguousarray(p[0].reshape(nb, nh, bs, d // x, x).transpose(0, 1, 3, 2, 4)))
             for p in hp]
        v = [to_device_bits(np.ascontiguousarray(p[1])) for p in hp]
        got = gpu_blocks(k, "K_XSPLIT", case["layers"], req, **kw)
        with np.errstate(over="ignore"):
            got = got + gpu_blocks(v, "V_HND", case["layers"], req, **kw)
    elif layout == "TRANS_PAIR":
        k = [to_device_bits(np.ascontiguousarray(p[0])) for p in hp]
        v = [to_device_bits(np.ascontiguousarray(p[1].transpose(0, 1, 3, 2))) for p in hp]
        got = gpu_blocks(k, "K_HND", case["layers"], req, **kw)
        with np.errstate(over="ignore"):
            got = got + gpu_blocks(v, "V_TRANS", case["layers"], req, **kw)
    else:
        got = gpu_blocks([to_device_bits(p) for p in hp], layout, case["layers"], req, **kw)
    for r, kk in req.listed():
        assert int(got[r, kk]) == int(want[r, kk]), (r, kk)


def _states_case(i):
    rng = np.random.default_rng(zlib.crc32(f"states{i}".encode()))
    nstates = int(rng.integers(1, 5))
    rows = int(rng.integers(1, 40))
    states = []
    for _ in range(nstates):
        elem = ["fp16", "fp32"][int(rng.integers(0, 2))]
        per16 = 16 // wl.ELEM_BYTES[elem]                       # row bytes are whole 16-byte chunks
        inner = per16 * int(rng.integers(1, 70))
        states.append((elem, inner))
    layers = sorted(_spread(x) for x in rng.choice(32768, size=int(rng.integers(1, 5)), replace=False))
    slots = int(rng.integers(2, 12))
    n_req = int(rng.integers(1, 8))
    row_begin = int(rng.integers(0, rows))
    row_count = int(rng.integers(1, rows - row_begin + 1))
    base = int(rng.integers(0, 65536 - row_count))
    return dict(i=i, states=states, rows=rows, layers=layers, slots=slots, n_req=n_req, row_begin=row_begin,
                row_count=row_count, base=base)


STATE_CASES = [_states_case(i) for i in range(120)]


@pytest.mark.parametrize("case", STATE_CASES, ids=lambda c: f"{c['i']}-s{len(c['states'])}-r{c['rows']}")
def test_states_sweep_case(case):
    import torch
    import paged_kv_cache_kvck_amd as kvck
    from gpu_helpers import DEV
    log(f"[states sweep] {case}")
    rng = np.random.default_rng(4000 + case["i"])
    hs = [[wl.host_random_bits(rng, (case["slots"], case["rows"], inner), elem) for elem, inner in case["states"]]
          for _ in case["layers"]]
    slot_ids = rng.integers(0, case["slots"], size=case["n_req"]).astype(np.int32)   # repeats allowed
    bases = [case["base"]] * len(case["layers"])
    got = kvck.kvck_checksum_states([[to_device_bits(a) for a in l] for l in hs], case["layers"],
                                    torch.from_numpy(slot_ids).to(DEV), global_row_base=bases,
                                    row_begin=case["row_begin"], row_count=case["row_count"], check=True)
    want = oracle.checksum_states(hs, case["layers"], bases, slot_ids, row_begin=case["row_begin"],
                                  row_count=case["row_count"])
    assert np.array_equal(got.cpu().numpy(), want)
