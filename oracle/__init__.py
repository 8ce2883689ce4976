"""CPU oracle of the connector-agnostic KV-cache block checksum.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The HIP library and
its Python binding never import it, and it imports nothing from them: the two
share no code, headers, tables or helpers.

What it computes is defined on the vLLM API page
"vllm.distributed.kv_transfer.kv_checksum.checksum" (module docstring):

* slice checksum: the pieces x_j of one (layer, head) slice, each times the
  odd weight 2j+1, summed modulo 2^64                          (docstring item 1)
* block checksum: the slices' checksums s(L, h), each times the odd factor
  m(L, h) = 2(L*H + h) + 1 with H = MAX_KV_HEADS_PER_LAYER, summed modulo
  2^64                                                          (item 2)
* Mamba running states: every global row of a layer's states is a slice
                                                               (Mamba paragraph)

``tags`` holds the offloaded-checksum tags (page function
``block_checksum_tags``) and the load-time comparison.

Two independent implementations of the checksum live here:

``kv_checksum``  numpy, vectorised per (position, cache); the oracle proper.
``brute``        pure-Python integers, one piece at a time; for tiny inputs,
                 used to pin the numpy oracle.

Pins (tests/test_oracle_*.py): brute force on tiny inputs, closed forms
(single nonzero piece, all-ones pieces, zero cache, single-byte probes of the
byte -> piece mapping), and the invariants the page states (additivity over
block sizes, layout independence, TP/PP partial sums, single-piece detection,
exclusion of slots at or past ``num_tokens``).

Parity unpinned: the Mamba slice contents (which rows of which states form a
slice, and in which order) follow this package's reading of the Mamba
paragraph; no value printed on the pages fixes it, so only closed forms and
brute force of the same reading pin it.
"""

from .kv_checksum import (  # noqa: F401
    BLOCK_CHECKSUM_BYTES,
    MAX_KV_HEADS_PER_LAYER,
    LAYOUTS,
    num_valid_tokens,
    slice_factor,
    checksum_blocks,
    checksum_states,
)
from . import brute  # noqa: F401
from . import tags  # noqa: F401
