"""KV-cache memory accounting: paged blocks against contiguous reservations.

Integer bookkeeping on the host, over block tables and context lengths (no
attention arithmetic).  Two layouts hold the same tokens:

* paged: whole blocks taken on demand, so a sequence leaves at most
  ``block_size - 1`` rows of its last block unused, and sequences sharing a
  prefix reference the same physical blocks ("PagedAttention Explained",
  sections "Block Tables and Non-Contiguous Storage" and "Shared Prefix
  Caching");
* contiguous: every sequence reserves ``reserve_len`` token rows up front and
  keeps its own copy of every token; what it does not fill is wasted (same
  page, "The Memory Fragmentation Problem", internal fragmentation).

The block size trades these against table size: smaller blocks leave less of
the last block empty but take more table entries (lookups) per token ("PagedAttention
Explained", "Best Practices", "Choose the Right Block Size").
"""

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class MemoryReport:
    block_size: int
    num_seqs: int
    tokens: int            # token rows the sequences hold (shared ones counted per sequence)
    unique_tokens: int     # token rows of distinct physical blocks (each block: its longest referencing sequence)
    paged_blocks: int      # distinct physical blocks referenced
    table_entries: int     # block-table entries the decode follows (one per block per sequence)
    reserve_len: int       # contiguous reservation per sequence, in tokens
    bytes_per_token: int   # key + value bytes of one token row

    @property
    def paged_slots(self) -> int:
        return self.paged_blocks * self.block_size

    @property
    def paged_tail_waste(self) -> int:
        """Allocated but unused token rows of the referenced blocks."""
        return self.paged_slots - self.unique_tokens

    @property
    def paged_waste_fraction(self) -> float:
        return self.paged_tail_waste / self.paged_slots if self.paged_slots else 0.0

    @property
    def reserved_slots(self) -> int:
        return self.num_seqs * self.reserve_len

    @property
    def reserved_waste(self) -> int:
        """Reserved but unused token rows of the contiguous layout."""
        return self.reserved_slots - self.tokens

    @property
    def reserved_waste_fraction(self) -> float:
        return self.reserved_waste / self.reserved_slots if self.reserved_slots else 0.0

    @property
    def saving_fraction(self) -> float:
        """Share of the contiguous layout's memory the paged one does not need."""
        return 1.0 - self.paged_slots / self.reserved_slots if self.reserved_slots else 0.0

    def as_dict(self) -> dict:
        bpt = self.bytes_per_token
        return {
            "block_size": self.block_size,
            "paged_bytes": self.paged_slots * bpt,
            "paged_tail_waste_fraction": round(self.paged_waste_fraction, 6),
            "contiguous_reserve_len": self.reserve_len,
            "contiguous_bytes": self.reserved_slots * bpt,
            "contiguous_waste_fraction": round(self.reserved_waste_fraction, 6),
            "paged_saving_fraction": round(self.saving_fraction, 6),
            "table_entries_per_token": round(self.table_entries / self.tokens, 6) if self.tokens else 0.0,
        }


def memory_report(block_tables, context_lens, block_size: int, reserve_len: int = None,
                  bytes_per_token: int = 1) -> MemoryReport:
    """Account the memory of sequences ``b`` holding ``context_lens[b]`` tokens
    in the blocks ``block_tables[b, :ceil(len / block_size)]``.  ``reserve_len``
    (default: the longest context) is the contiguous layout's reservation."""
    tables = np.asarray(block_tables)
    lens = np.asarray(context_lens, dtype=np.int64)
    if len(tables) != len(lens):
        raise ValueError("block_tables and context_lens disagree on the number of sequences")
    if (lens < 0).any():
        raise ValueError("negative context length")
    nblocks = -(-lens // block_size)
    if len(lens) and nblocks.max() > tables.shape[1]:
        raise ValueError("a context needs more blocks than its table row holds")
    rows = {}
    for b, (n, k) in enumerate(zip(lens.tolist(), nblocks.tolist())):
        for j in range(k):
            blk = int(tables[b, j])
            rows[blk] = max(rows.get(blk, 0), min(block_size, n - j * block_size))
    reserve = int(lens.max()) if reserve_len is None and len(lens) else int(reserve_len or 0)
    if len(lens) and reserve < lens.max():
        raise ValueError("the contiguous reservation is shorter than a context")
    return MemoryReport(block_size=block_size, num_seqs=len(lens), tokens=int(lens.sum()),
                        unique_tokens=int(sum(rows.values())), paged_blocks=len(rows),
                        table_entries=int(nblocks.sum()), reserve_len=reserve, bytes_per_token=bytes_per_token)
