"""Identity of the kernel sources that committed HBM counters were taken on.

A rocprofv3 counter summary under ``profiles/`` records a hash of the sources
that decide what the measured kernel reads; a reader of that summary (the
benchmark's ``roofline.traffic``) treats it as stale once the hash differs.
Only code counts: comments and whitespace are removed before hashing.
"""

from __future__ import annotations

import hashlib
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)

# The sources that decide what the checksum main pass reads: its own file,
# the device helpers and argument structs it is built from, the host code
# that picks its schedule, and the public header.
MAIN_PASS_SOURCES = ("paged_kv_cache_kvck_amd/csrc/kvck_blocks.hip", "paged_kv_cache_kvck_amd/csrc/kvck_device.h",
                     "paged_kv_cache_kvck_amd/csrc/kvck_internal.h", "paged_kv_cache_kvck_amd/csrc/kvck_api.hip",
                     "include/kvck.h")


def code_only(text: str) -> str:
    """C/C++ source without comments and whitespace: what the compiler sees."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return re.sub(r"\s+", "", text)


def kernel_sources_sha(files=MAIN_PASS_SOURCES) -> str:
    """sha256 over the code of ``files`` (paths relative to the repository root)."""
    h = hashlib.sha256()
    for p in (os.path.join(ROOT, f) for f in files):
        with open(p, encoding="utf-8") as f:
            h.update(os.path.basename(p).encode())
            h.update(code_only(f.read()).encode())
    return h.hexdigest()
