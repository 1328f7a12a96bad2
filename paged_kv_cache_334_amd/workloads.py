"""Seeded synthetic decode workloads and the host-side block bookkeeping that
produces their block tables, slots and copy-on-write pairs.

This module holds no attention arithmetic and no pool-layout arithmetic.  It
only draws random inputs and does the integer bookkeeping the host does above
the library: a free list of physical block ids, per-sequence block tables,
reference counts, the slot of each appended token, and copy-on-write when a
sequence appends into a block it shares.  Both the HIP path and the CPU oracle
are fed from what it returns.

The bookkeeping lives in ``BlockPool`` (its docstring gives the rules and
the passages they come from): whole runs of tokens are placed at once, so a
workload of hundreds of thousands of cached tokens is laid out in a few
array operations per sequence.

Random inputs: NumPy PCG64 with one independent stream per purpose,
``default_rng([seed, purpose])``; values are float32 N(0, 1), rounded to
bfloat16 by round-to-nearest-even on the bits.
"""

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


class BlockPool:
    """Physical block ids of one paged cache and who holds them.

    State: a FIFO of free ids (a ring over an int32 array: ids are taken from
    its front and returned to its back), a holder count per id, and per
    sequence its held ids in logical order plus its token count.  Requests are
    served whole: ``extend`` reserves every slot of a run of tokens at once, or
    raises ``CacheExhausted`` and changes nothing.

    Rules (the slot rule is what ``reshape_and_cache`` consumes): the run's
    tokens take rows ``position % block_size`` of the sequence's blocks, a new
    block is taken each time a position is a multiple of ``block_size``
    ("PagedAttention Explained", "Implementing a Simplified Paged KV Cache");
    a run that starts inside a last block held by others first moves the
    sequence to a private copy, queued as a (source, destination) pair
    (copy-on-write: "Master Paged Attention for LLM Inference", "How Paged
    Attention Works: The Mechanics", item 4); releasing a sequence drops its
    hold on each block, and ids left with no holder go to the back of the FIFO
    in the sequence's logical order.
    """

    def __init__(self, num_blocks: int, block_size: int, free_order: Optional[Sequence[int]] = None):
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        ring = np.arange(self.num_blocks, dtype=np.int32) if free_order is None else np.asarray(free_order, np.int32)
        if ring.shape != (self.num_blocks,):
            raise ValueError("free_order must list every block once")
        self._ring = ring.copy()
        self._head = 0
        self._nfree = self.num_blocks
        self.holders = np.zeros(self.num_blocks, dtype=np.int32)
        self._held = {}  # sequence -> list of block ids, logical order
        self._tokens = {}  # sequence -> token count
        self._copies: List[Tuple[int, int]] = []

    # -- the free FIFO ----------------------------------------------------------
    @property
    def free_count(self) -> int:
        return self._nfree

    def free_ids(self) -> np.ndarray:
        """Free ids, front of the FIFO first."""
        return self._ring[(self._head + np.arange(self._nfree)) % self.num_blocks]

    def _pop_front(self, k: int) -> np.ndarray:
        ids = self._ring[(self._head + np.arange(k)) % self.num_blocks]
        self._head = (self._head + k) % self.num_blocks
        self._nfree -= k
        self.holders[ids] += 1
        return ids

    def _push_back(self, ids: np.ndarray) -> None:
        pos = (self._head + self._nfree + np.arange(len(ids))) % self.num_blocks
        self._ring[pos] = ids
        self._nfree += len(ids)

    # -- sequences --------------------------------------------------------------
    def new_sequence(self, seq) -> None:
        self._held[seq] = []
        self._tokens[seq] = 0

    def share_sequence(self, parent, child) -> None:
        """``child`` holds every block of ``parent`` (its tokens so far)."""
        held = list(self._held[parent])
        self._held[child] = held
        self._tokens[child] = self._tokens[parent]
        self.holders[np.asarray(held, dtype=np.int64)] += 1

    def extend(self, seq, n: int) -> np.ndarray:
        """Slots (``block * block_size + row``) of the sequence's next ``n`` tokens."""
        bs = self.block_size
        held = self._held[seq]
        first = self._tokens[seq]
        grow = -(-(first + n) // bs) - len(held)  # blocks the run adds past the held ones
        private = first % bs != 0 and n > 0 and self.holders[held[-1]] > 1
        if grow + int(private) > self._nfree:
            raise CacheExhausted(f"block pool is empty: {grow + int(private)} blocks wanted, {self._nfree} free")
        if private:
            src = held[-1]
            dst = int(self._pop_front(1)[0])
            self.holders[src] -= 1
            held[-1] = dst
            self._copies.append((int(src), dst))
        if grow > 0:
            held.extend(self._pop_front(grow).tolist())
        self._tokens[seq] = first + n
        pos = np.arange(first, first + n, dtype=np.int64)
        return (np.asarray(held, dtype=np.int64)[pos // bs] * bs + pos % bs).astype(np.int32)

    def release(self, seq) -> None:
        ids = np.asarray(self._held.pop(seq), dtype=np.int64)
        del self._tokens[seq]
        self.holders[ids] -= 1
        self._push_back(ids[self.holders[ids] == 0].astype(np.int32))

    def table(self, seq) -> List[int]:
        return list(self._held[seq])

    def tokens(self, seq) -> int:
        return self._tokens[seq]

    def drain_copies(self) -> List[Tuple[int, int]]:
        """Copy-on-write pairs queued since the last call, oldest first."""
        pairs, self._copies = self._copies, []
        return pairs


def f32_to_bf16_bits(values: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits, round to nearest, ties to even (finite input).

    Adds 0x7FFF plus the lowest kept bit to the float32 bits and keeps the top
    16 bits; done in place on one uint32 copy, the top halves read through a
    uint16 view (little-endian: the high half of element i is half 2i+1)."""
    u = np.array(values, dtype=np.float32, copy=True, order="C").view(np.uint32)
    lsb = u >> np.uint32(16)
    lsb &= np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    return u.view(np.uint16)[..., 1::2].copy()


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
    # token positions [lo, hi) the outliers are drawn from (None: the sequence's own tokens)
    outlier_window: Optional[Tuple[int, int]] = None
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
    pool = BlockPool(num_blocks, bs, free_order)

    # token order: the prefix common to all groups, the rest of each group's
    # prefix (its holder shares the common part), then each sequence's own
    # tokens; each sequence's run of own tokens is one contiguous range of it
    runs = []  # slot arrays, in token order
    own_start = np.zeros(nseq, dtype=np.int64)  # token index of sequence b's first own token
    count = 0
    if tree_blocks:
        pool.new_sequence(("tree",))
        runs.append(pool.extend(("tree",), spec.tree_prefix))
        count += spec.tree_prefix
    for gi in range(groups):
        if tree_blocks:
            pool.share_sequence(("tree",), ("prefix", gi))
        else:
            pool.new_sequence(("prefix", gi))
        n = spec.shared_prefix - (spec.tree_prefix if tree_blocks else 0)
        runs.append(pool.extend(("prefix", gi), n))
        count += n
    if tree_blocks:
        pool.release(("tree",))
    for b in range(nseq):
        gi = prefix_group_of(spec, b)
        if gi >= 0:
            pool.share_sequence(("prefix", gi), b)
        else:
            pool.new_sequence(b)
        n = int(ctx[b] - qlen[b]) - (spec.shared_prefix if gi >= 0 else 0)
        own_start[b] = count
        runs.append(pool.extend(b, n))
        count += n
    for gi in range(groups):
        pool.release(("prefix", gi))
    for b in cow_seqs:  # an implicit sibling keeps holding every block of b
        pool.share_sequence(b, ("sibling", b))
    init_slots = np.concatenate(runs).astype(np.int32) if runs else np.zeros(0, np.int32)
    # the step: each sequence's new tokens (copy-on-write happens at the first)
    new_slots = np.concatenate([pool.extend(b, int(qlen[b])) for b in range(nseq)]).astype(np.int32)
    cow_pairs = np.asarray(pool.drain_copies(), dtype=np.int32).reshape(-1, 2)

    # block tables as the decode sees them
    max_blocks = max(len(pool.table(b)) for b in range(nseq))
    if table_pad == "unused":
        pad = int(pool.free_ids()[0])
    elif table_pad == "minus1":
        pad = -1
    else:
        raise ValueError(table_pad)
    tables = np.full((nseq, max_blocks), pad, dtype=np.int32)
    for b in range(nseq):
        held = pool.table(b)
        tables[b, : len(held)] = held

    # token values, in the token order above, the new tokens last
    hkv, hd = spec.num_kv_heads, spec.head_dim
    total = len(init_slots) + len(new_slots)
    key_scale = None
    outliers = {}
    if spec.outlier_fraction > 0:
        key_scale = np.ones(total, dtype=np.float32)
        orng = rng(_OUTLIER)
        for b in range(nseq):
            first = spec.shared_prefix if prefix_group_of(spec, b) >= 0 else 0
            n_out = int(np.floor(spec.outlier_fraction * (int(ctx[b]) - first)))
            lo, hi = first, int(ctx[b])
            if spec.outlier_window is not None:
                lo, hi = max(lo, spec.outlier_window[0]), min(hi, spec.outlier_window[1])
                if n_out > hi - lo:
                    raise ValueError("outlier window holds fewer tokens than outliers")
            pos = np.sort(orng.choice(np.arange(lo, hi), size=n_out, replace=False))
            outliers[b] = pos
            # a cached own token's index follows its sequence's run; a new token's
            # follows every cached one, in query-row order
            cached = int(ctx[b] - qlen[b])
            idx = np.where(pos < cached, own_start[b] + (pos - first),
                           len(init_slots) + int(query_start[b]) + (pos - cached))
            key_scale[idx] = spec.outlier_scale
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
        init_slots=init_slots,
        new_k=keys[t0:],
        new_v=values[t0:],
        new_slots=new_slots,
        cow_pairs=cow_pairs,
        outlier_positions=outliers,
        query_start=query_start,
    )
