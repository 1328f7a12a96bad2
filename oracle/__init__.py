"""CPU oracle for paged KV-cache decode attention.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import anything from this package.  The HIP library never calls it, and it
imports nothing from ``paged_kv_cache_334_amd``: the two sides share no code,
only the seeded inputs that the tests hand to both.

What it computes, and where the pages state it:

* ``paged_decode`` -- one decode step of attention for every (sequence, query
  head), with the sequence's keys and values resolved through its block table
  into contiguous arrays first ("PagedAttention Explained", agentechip.com,
  sections "Block Tables and Non-Contiguous Storage" and "Implementing a
  Simplified Paged KV Cache", method ``get_keys_values``), then plain two-pass
  softmax attention in float64.
* ``paged_attend_causal`` -- several new tokens per sequence, each attending
  causally over the cached prefix up to itself (speculative verify, a prompt
  chunk); the same single-query attention over each token's visible prefix.
* ``partitioned_decode`` -- the same result reached through per-partition
  (max, sum, acc) partials and a max-rescaled merge (the split-K form).
* ``reshape_and_cache`` / ``copy_blocks`` -- the cache write of the newest
  token at ``position_in_block = length % block_size`` of the last block of
  the table (same page, ``append_token``) and the copy-on-write block copy
  ("Master Paged Attention for LLM Inference", krapton.com, section "How Paged
  Attention Works: The Mechanics", item 4; "PagedAttention Explained",
  section "Shared Prefix Caching").
* ``swap_blocks`` -- whole blocks between two pools of the same shape (the CPU
  swap space; "PagedAttention Explained", "Programmatic Control Over KV Cache").

Every function here is pinned by ``tests/test_oracle.py`` to values that do not
come from the oracle itself (closed forms, a library attention routine, brute
force on tiny inputs, invariants the pages state, the worked example the pages
print).  No function is "parity unpinned".
"""

from .layout import PoolDesc, k_offset, v_offset, decode_bits, chunk_elems
from .attention import (
    resolve_sequence,
    paged_decode,
    paged_decode_bruteforce,
    partitioned_decode,
    paged_attend_causal,
)
from .cache_ops import reshape_and_cache, copy_blocks, new_pools, swap_blocks

__all__ = [
    "PoolDesc",
    "k_offset",
    "v_offset",
    "decode_bits",
    "chunk_elems",
    "resolve_sequence",
    "paged_decode",
    "paged_decode_bruteforce",
    "partitioned_decode",
    "paged_attend_causal",
    "reshape_and_cache",
    "copy_blocks",
    "new_pools",
    "swap_blocks",
]
