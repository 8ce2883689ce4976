"""Writes tests/golden/tiny_oracle.json: the oracle's checksums of the tiny
workload (2 layers x 2 KV heads, head 64 bf16 bits, block 16, NHD pool of 16
blocks, one 50-token request).  Calls only ``oracle`` and the seeded input
generator; it is a regression guard for the oracle, not an independent pin.

    python tests/golden/make_golden.py
"""

import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import kv_checksum as o  # noqa: E402
from paged_kv_cache_kvck_amd import workloads as wl  # noqa: E402


def main():
    w = wl.tiny()
    pools = w.host_pools()
    out = o.checksum_blocks(pools, w.layout, w.layer_numbers, w.bases, w.req.block_table,
                            w.req.num_blocks, w.req.start_pos, w.req.num_tokens)
    doc = {
        "_about": "oracle checksums of workloads.tiny(seed=1) with host pools; written by make_golden.py",
        "block_table": w.req.block_table[0].tolist(),
        "num_tokens": int(w.req.num_tokens[0]),
        "checksums": [str(int(x)) for x in out[0, :int(w.req.num_blocks[0])]],
        "pool_sha256": __import__("hashlib").sha256(b"".join(p.tobytes() for p in pools)).hexdigest(),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    print(path)


if __name__ == "__main__":
    main()
