"""Seeded synthetic decode workloads and the host-side block bookkeeping that
produces their block tables, slots and copy-on-write pairs.

This module holds no attention arithmetic and no pool-layout arithmetic.  It
only draws random inputs and does the integer bookkeeping the host does above
the library: a free list of physical block ids, per-sequence block tables,
reference counts, the slot of each appended token, and copy-on-write when a
sequence appends into a block it shares.  Both the HIP path and the CPU oracle
are fed from what it returns.

Bookkeeping rules ("PagedAttention Explained", agentechip.com, section
"Implementing a Simplified Paged KV Cache"):

* a new block is taken from the front of the free list when a sequence's
  length is a multiple of ``block_size``; an empty free list raises
  an error (CacheExhausted);
* the token goes to row ``length % block_size`` of the last block of the
  sequence's table; here that becomes its slot ``block * block_size + row``;
* freeing a sequence decrements each block's reference count and returns the
  block to the free list at zero;
* sequences that fork share blocks (reference count > 1); appending into a
  shared last block first copies it to a fresh block ("Master Paged Attention
  for LLM Inference", "How Paged Attention Works: The Mechanics", item 4).

Random inputs: NumPy PCG64 with one independent stream per purpose,
``default_rng([seed, purpose])``; values are float32 N(0, 1), rounded to
bfloat16 by round-to-nearest-even on the bits.
"""

from collections import deque
from dataclasses import dataclass, field, replace
from typing import List, Optional, Sequence, Tuple, Union

import numpy as np

BF16 = "bf16"
F32 = "f32"

_ELT = {BF16: 2, F32: 4}

# purposes of the random streams
_CTX, _PERM, _Q, _K, _V, _OUTLIER, _COW, _QLEN = 1, 2, 3, 4, 5, 6, 7, 8


class CacheExhausted(RuntimeError):
    pass


class BlockManager:
    """Free list, block tables, reference counts and slots of a paged KV cache."""

    def __init__(self, num_blocks: int, block_size: int, free_order: Optional[Sequence[int]] = None):
        self.num_blocks = num_blocks
        self.block_size = block_size
        order = range(num_blocks) if free_order is None else free_order
        self.free = deque(int(b) for b in order)
        self.ref = [0] * num_blocks
        self.tables = {}
        self.lengths = {}
        self.pending_copies: List[Tuple[int, int]] = []

    def _take(self) -> int:
        if not self.free:
            raise CacheExhausted("block pool is empty: cannot give the sequence a new block")
        blk = self.free.popleft()
        self.ref[blk] += 1
        return blk

    def allocate_sequence(self, seq_id) -> None:
        self.tables[seq_id] = []
        self.lengths[seq_id] = 0

    def fork(self, parent, child) -> None:
        """``child`` starts with ``parent``'s tokens, sharing its blocks."""
        self.tables[child] = list(self.tables[parent])
        self.lengths[child] = self.lengths[parent]
        for blk in self.tables[child]:
            self.ref[blk] += 1

    def append_slot(self, seq_id) -> int:
        """Reserve the slot of the sequence's next token and return it."""
        length = self.lengths[seq_id]
        row = length % self.block_size
        table = self.tables[seq_id]
        if row == 0:
            table.append(self._take())
        elif self.ref[table[-1]] > 1:
            src = table[-1]
            dst = self._take()
            self.ref[src] -= 1
            table[-1] = dst
            self.pending_copies.append((src, dst))
        self.lengths[seq_id] = length + 1
        return table[-1] * self.block_size + row

    def free_sequence(self, seq_id) -> None:
        for blk in self.tables[seq_id]:
            self.ref[blk] -= 1
            if self.ref[blk] == 0:
                self.free.append(blk)
        del self.tables[seq_id]
        del self.lengths[seq_id]

    def take_copies(self) -> List[Tuple[int, int]]:
        pairs, self.pending_copies = self.pending_copies, []
        return pairs


def f32_to_bf16_bits(values: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits, round to nearest, ties to even (finite input)."""
    u = np.ascontiguousarray(values, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass(frozen=True)
class WorkloadSpec:
    name: str
    dtype: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    ctx: Union[Tuple[int, int], Tuple[int, ...]]  # (lo, hi) inclusive uniform, or explicit lengths
    ctx_is_list: bool = False
    shared_prefix: int = 0  # tokens every sequence of a prefix group shares (block aligned)
    tree_prefix: int = 0  # of those, tokens every prefix group shares with the others (block aligned)
    prefix_groups: int = 1  # sequence b < num_seqs - unshared_seqs joins group b % prefix_groups
    unshared_seqs: int = 0  # trailing sequences with no shared prefix
    cow_fraction: float = 0.0  # fraction of sequences whose last block was just forked
    outlier_fraction: float = 0.0  # key rows scaled by ``outlier_scale``
    outlier_scale: float = 8.0
    pool_factor: float = 1.5
    num_blocks: Optional[int] = None  # fixed pool size instead of pool_factor
    scale: Optional[float] = None  # default 1/sqrt(head_dim)
    seed: int = 0
    # new tokens per sequence in the step (their keys/values are written, then
    # each attends causally): an int, or (lo, hi) inclusive uniform; at most
    # the context length
    query_len: Union[int, Tuple[int, int]] = 1

    @property
    def group(self) -> int:
        return self.num_heads // self.num_kv_heads


# The five workloads: a tiny float32 case, a 7B-shaped MHA layer, a 70B-shaped
# GQA layer, a long-context case and a shared-prefix case with copy-on-write.
SPECS = {
    "tiny-f32": WorkloadSpec("tiny-f32", F32, 4, 2, 2, 64, 16, (5, 16, 17, 33), ctx_is_list=True,
                             num_blocks=16, scale=0.125, seed=1001),
    "mha-7b": WorkloadSpec("mha-7b", BF16, 64, 32, 32, 128, 16, (128, 2048), seed=1002),
    "gqa-70b": WorkloadSpec("gqa-70b", BF16, 128, 64, 8, 128, 16, (512, 4096), seed=1003),
    "long-32k": WorkloadSpec("long-32k", BF16, 8, 32, 8, 128, 32, (32768, 32768),
                             outlier_fraction=0.01, seed=1004),
    "shared-prefix": WorkloadSpec("shared-prefix", BF16, 200, 32, 8, 128, 16, (16, 512),
                                  shared_prefix=30000, cow_fraction=0.10, seed=1005),
}
# Nested sharing, as beam search leaves it: 8 requests x 16 beams under one
# 4096-token system prompt, each request's 2048-token prompt shared by its
# beams, U[16, 256] tokens of each beam's own, 10% of the beams just forked.
TREE_SPECS = {
    "beam-tree": WorkloadSpec("beam-tree", BF16, 128, 32, 8, 128, 16, (16, 256), shared_prefix=6144,
                              tree_prefix=4096, prefix_groups=8, cow_fraction=0.10, seed=1008),
}
SPECS.update(TREE_SPECS)
ORDER = ["tiny-f32", "mha-7b", "gqa-70b", "long-32k", "shared-prefix"]

# Several new tokens per sequence: the 70B-shaped GQA batch verifying 4 tokens
# per sequence (3 drafted + 1), as a speculative-decoding step does; and 8
# sequences each appending a 512-token chunk of their prompt (chunked prefill
# over the paged cache).
MULTI_SPECS = {
    "verify-gqa-70b": WorkloadSpec("verify-gqa-70b", BF16, 128, 64, 8, 128, 16, (512, 4096), seed=1006,
                                   query_len=4),
    "prefill-gqa-70b": WorkloadSpec("prefill-gqa-70b", BF16, 8, 64, 8, 128, 16, (1024, 4096), seed=1007,
                                    query_len=512),
}


@dataclass
class Workload:
    spec: WorkloadSpec
    num_blocks: int
    scale: float
    context_lens: np.ndarray  # [B] int32
    block_tables: np.ndarray  # [B, max_blocks] int32, tables as the decode sees them
    table_pad: int  # value in table entries past each sequence's blocks
    q: np.ndarray  # [B, Hq, D] element bits
    init_k: np.ndarray  # [T0, Hkv, D] bits of every token written before the step
    init_v: np.ndarray
    init_slots: np.ndarray  # [T0] int32
    new_k: np.ndarray  # [T, Hkv, D] bits of the step's new tokens (T = B with one per sequence)
    new_v: np.ndarray
    new_slots: np.ndarray  # [T] int32
    cow_pairs: np.ndarray  # [P, 2] int32 (src, dst) copied before the new tokens are written
    outlier_positions: dict = field(default_factory=dict)
    # new tokens of sequence b: rows query_start[b] .. query_start[b+1]-1 of q and new_k/new_v
    query_start: Optional[np.ndarray] = None

    @property
    def query_lens(self) -> np.ndarray:
        return np.diff(self.query_start).astype(np.int32)

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max()) if len(self.query_lens) else 0

    @property
    def dtype(self) -> str:
        return self.spec.dtype

    @property
    def max_blocks(self) -> int:
        return self.block_tables.shape[1]

    @property
    def max_context(self) -> int:
        return int(self.context_lens.max()) if len(self.context_lens) else 0

    def unique_kv_bytes(self) -> int:
        """Key+value bytes of every physical block row the decode must read:
        each referenced block counted once, with as many rows as the longest
        referencing sequence keeps valid in it."""
        bs = self.spec.block_size
        rows = {}
        for b, n in enumerate(self.context_lens.tolist()):
            for j in range(-(-n // bs)):
                blk = int(self.block_tables[b, j])
                rows[blk] = max(rows.get(blk, 0), min(bs, n - j * bs))
        return 2 * self.spec.num_kv_heads * self.spec.head_dim * _ELT[self.dtype] * sum(rows.values())

    def logical_kv_bytes(self) -> int:
        """Key+value bytes summed over sequences (shared blocks counted per reader)."""
        return 2 * self.spec.num_kv_heads * self.spec.head_dim * _ELT[self.dtype] * int(self.context_lens.sum())


def _normal_bits(rng, shape, dtype, chunk_rows: int = 1 << 14, scale_rows=None):
    """Seeded N(0,1) float32 values as element bits, drawn in row chunks."""
    rows = shape[0]
    per_row = int(np.prod(shape[1:]))
    out = np.empty((rows, per_row), dtype=np.uint16 if dtype == BF16 else np.uint32)
    for lo in range(0, rows, chunk_rows):
        hi = min(rows, lo + chunk_rows)
        vals = rng.standard_normal((hi - lo, per_row), dtype=np.float32)
        if scale_rows is not None:
            factor = scale_rows[lo:hi]
            vals *= factor[:, None]
        out[lo:hi] = f32_to_bf16_bits(vals) if dtype == BF16 else vals.view(np.uint32)
    return out.reshape(shape)


def prefix_group_of(spec: WorkloadSpec, b: int) -> int:
    """Prefix group of sequence b, or -1 when it shares no prefix."""
    if not spec.shared_prefix or b >= spec.num_seqs - spec.unshared_seqs:
        return -1
    return b % spec.prefix_groups


def context_lengths(spec: WorkloadSpec) -> np.ndarray:
    """Context length of every sequence (shared prefix and newest token included)."""
    if spec.ctx_is_list:
        ctx = np.asarray(spec.ctx, dtype=np.int64)
        if len(ctx) != spec.num_seqs:
            raise ValueError("explicit context list does not match num_seqs")
    else:
        lo, hi = spec.ctx
        ctx = np.random.default_rng([spec.seed, _CTX]).integers(lo, hi, size=spec.num_seqs, endpoint=True)
        ctx = ctx.astype(np.int64)
    shared = np.array([prefix_group_of(spec, b) >= 0 for b in range(spec.num_seqs)], dtype=bool)
    return ctx + np.where(shared, spec.shared_prefix, 0)


def query_lengths(spec: WorkloadSpec, ctx: np.ndarray) -> np.ndarray:
    """New tokens per sequence this step (at least 1, at most the context)."""
    if isinstance(spec.query_len, int):
        qlen = np.full(spec.num_seqs, spec.query_len, dtype=np.int64)
    else:
        lo, hi = spec.query_len
        qlen = np.random.default_rng([spec.seed, _QLEN]).integers(lo, hi, size=spec.num_seqs, endpoint=True)
    return np.minimum(np.maximum(qlen, 1), ctx).astype(np.int64)


def generate(spec: Union[str, WorkloadSpec], table_pad: str = "unused", **overrides) -> Workload:
    """Build a workload: context lengths, block tables, the bits of every
    cached token, the step's new tokens, copy-on-write pairs and queries.

    ``table_pad`` chooses what fills table entries past each sequence's blocks:
    ``"unused"`` (a physical block nothing ever writes, so it keeps its NaN
    poison) or ``"minus1"``.
    """
    if isinstance(spec, str):
        spec = SPECS[spec]
    if overrides:
        spec = replace(spec, **overrides)
    bs = spec.block_size
    nseq = spec.num_seqs
    if spec.shared_prefix % bs or spec.tree_prefix % bs:
        raise ValueError("the shared prefixes must be whole numbers of blocks")
    if spec.tree_prefix > spec.shared_prefix:
        raise ValueError("the prefix common to all groups cannot exceed a group's")

    rng = lambda purpose: np.random.default_rng([spec.seed, purpose])  # noqa: E731
    ctx = context_lengths(spec)
    qlen = query_lengths(spec, ctx)
    # new tokens never reach back into a shared prefix
    own_ctx = ctx - np.array([spec.shared_prefix if prefix_group_of(spec, b) >= 0 else 0 for b in range(nseq)])
    qlen = np.minimum(qlen, np.maximum(own_ctx, 1))
    query_start = np.concatenate([[0], np.cumsum(qlen)]).astype(np.int32)

    # copy-on-write choice: sequences whose first new token lands inside a block
    # that already holds rows, i.e. the block they would share with a sibling
    cow_seqs = []
    if spec.cow_fraction > 0:
        candidates = np.nonzero(((ctx - qlen) % bs) != 0)[0]
        k = int(round(spec.cow_fraction * nseq))
        cow_seqs = sorted(rng(_COW).choice(candidates, size=min(k, len(candidates)), replace=False).tolist())

    # pool size
    prefix_blocks = spec.shared_prefix // bs
    groups = spec.prefix_groups if spec.shared_prefix else 0
    own = [int(n) - (spec.shared_prefix if prefix_group_of(spec, b) >= 0 else 0) for b, n in enumerate(ctx)]
    tree_blocks = spec.tree_prefix // bs if groups else 0
    needed = tree_blocks + (prefix_blocks - tree_blocks) * groups + int(sum(-(-o // bs) for o in own)) + len(cow_seqs)
    num_blocks = spec.num_blocks if spec.num_blocks is not None else int(np.ceil(spec.pool_factor * needed))
    if num_blocks < needed + 1:
        raise ValueError("pool too small")
    free_order = rng(_PERM).permutation(num_blocks)
    mgr = BlockManager(num_blocks, bs, free_order)

    # token order: the prefix common to all groups, the rest of each group's
    # prefix (forked from it), then each sequence's own tokens
    init_slots = []
    init_owner = []  # (seq, or -1 - group for a prefix token, -1 - groups for a common one, position)
    if tree_blocks:
        mgr.allocate_sequence(("tree",))
        for pos in range(spec.tree_prefix):
            init_slots.append(mgr.append_slot(("tree",)))
            init_owner.append((-1 - groups, pos))
    for gi in range(groups):
        if tree_blocks:
            mgr.fork(("tree",), ("prefix", gi))
        else:
            mgr.allocate_sequence(("prefix", gi))
        for pos in range(spec.tree_prefix if tree_blocks else 0, spec.shared_prefix):
            init_slots.append(mgr.append_slot(("prefix", gi)))
            init_owner.append((-1 - gi, pos))
    if tree_blocks:
        mgr.free_sequence(("tree",))
    for b in range(nseq):
        gi = prefix_group_of(spec, b)
        if gi >= 0:
            mgr.fork(("prefix", gi), b)
        else:
            mgr.allocate_sequence(b)
        first = spec.shared_prefix if gi >= 0 else 0
        for pos in range(first, int(ctx[b] - qlen[b])):
            init_slots.append(mgr.append_slot(b))
            init_owner.append((b, pos))
    for gi in range(groups):
        mgr.free_sequence(("prefix", gi))
    for b in cow_seqs:  # an implicit sibling keeps referencing every block of b
        mgr.fork(b, ("sibling", b))
    # the step: each sequence's new tokens (copy-on-write happens at the first)
    new_slots = [mgr.append_slot(b) for b in range(nseq) for _ in range(int(qlen[b]))]
    cow_pairs = np.asarray(mgr.take_copies(), dtype=np.int32).reshape(-1, 2)

    # block tables as the decode sees them
    max_blocks = max(len(mgr.tables[b]) for b in range(nseq))
    if table_pad == "unused":
        pad = int(mgr.free[0])
    elif table_pad == "minus1":
        pad = -1
    else:
        raise ValueError(table_pad)
    tables = np.full((nseq, max_blocks), pad, dtype=np.int32)
    for b in range(nseq):
        tables[b, : len(mgr.tables[b])] = mgr.tables[b]

    # token values, in the token order above, the new tokens last
    hkv, hd = spec.num_kv_heads, spec.head_dim
    total = len(init_slots) + len(new_slots)
    key_scale = None
    outliers = {}
    if spec.outlier_fraction > 0:
        key_scale = np.ones(total, dtype=np.float32)
        orng = rng(_OUTLIER)
        index_of = {}
        for i, (b, pos) in enumerate(init_owner):
            index_of[(b, pos)] = i
        for b in range(nseq):
            for i in range(int(qlen[b])):
                index_of[(b, int(ctx[b] - qlen[b]) + i)] = len(init_slots) + int(query_start[b]) + i
        for b in range(nseq):
            first = spec.shared_prefix if prefix_group_of(spec, b) >= 0 else 0
            n_out = int(np.floor(spec.outlier_fraction * (int(ctx[b]) - first)))
            pos = np.sort(orng.choice(np.arange(first, int(ctx[b])), size=n_out, replace=False))
            outliers[b] = pos
            for p in pos.tolist():
                key_scale[index_of[(b, p)]] = spec.outlier_scale
    keys = _normal_bits(rng(_K), (total, hkv, hd), spec.dtype, scale_rows=key_scale)
    values = _normal_bits(rng(_V), (total, hkv, hd), spec.dtype)
    q = _normal_bits(rng(_Q), (len(new_slots), spec.num_heads, hd), spec.dtype)
    t0 = len(init_slots)
    return Workload(
        spec=spec,
        num_blocks=num_blocks,
        scale=float(spec.scale if spec.scale is not None else 1.0 / np.sqrt(hd)),
        context_lens=ctx.astype(np.int32),
        block_tables=tables,
        table_pad=pad,
        q=q,
        init_k=keys[:t0],
        init_v=values[:t0],
        init_slots=np.asarray(init_slots, dtype=np.int32),
        new_k=keys[t0:],
        new_v=values[t0:],
        new_slots=np.asarray(new_slots, dtype=np.int32),
        cow_pairs=cow_pairs,
        outlier_positions=outliers,
        query_start=query_start,
    )
