"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each ``pin_*`` function raises ``AssertionError`` when the oracle disagrees.
``test_oracle.py`` runs them on seeded workloads; ``test_oracle_mutations.py``
plants plausible mistakes in the oracle and checks that some pin fails.

Sources of the pinned facts:
* closed forms and special cases of softmax attention (a single token, zero
  scale, equal values, a dominant logit);
* a library routine: PyTorch's scaled-dot-product attention on the contiguous
  keys/values of each sequence, taken from a slot map with no pool layout;
* invariants the pages state: paging changes where blocks live, not the
  result ("What is PagedAttention", aitechboss.com, "Step 3: Use Page Tables
  Instead of Continuous Memory"); a sequence's blocks need not be contiguous
  ("PagedAttention Explained", "Block Tables and Non-Contiguous Storage");
  shared-prefix sequences reference the same physical blocks ("PagedAttention
  Explained", "Shared Prefix Caching");
* brute force with Python scalars on tiny inputs;
* for several new tokens per step: token-by-token decoding (the result a
  verify pass must reproduce), torch's own causal mask when a whole prompt is
  one chunk, and that no row depends on the tokens after it.
"""

import numpy as np

import oracle
from logical_model import (
    contiguous_kv,
    desc_of,
    oracle_causal,
    oracle_decode,
    oracle_pools,
    sdpa_causal_prompt,
    sdpa_reference,
    slot_map,
    to_f64,
)
from paged_kv_cache_334_amd.workloads import BlockPool, Workload


def pin_single_token(wl):
    """context_len 1: the only weight is exactly 1, so out = that value row exactly."""
    assert (wl.context_lens == 1).all()
    out = oracle_decode(wl)
    g = wl.spec.group
    for b in range(wl.spec.num_seqs):
        _, v = contiguous_kv(wl, b)
        expect = np.repeat(to_f64(v[0], wl.dtype), g, axis=0)
        assert np.array_equal(out[b], expect), f"seq {b}"


def pin_zero_scale(wl):
    """scale 0: all logits equal, so out = the plain mean of the value rows."""
    assert wl.scale == 0.0
    out = oracle_decode(wl)
    g = wl.spec.group
    for b in range(wl.spec.num_seqs):
        _, v = contiguous_kv(wl, b)
        expect = np.repeat(to_f64(v, wl.dtype).mean(axis=0), g, axis=0)
        assert np.allclose(out[b], expect, rtol=0, atol=1e-12), f"seq {b}"


def with_equal_values(wl):
    """Copy of ``wl`` whose every value row of kv head h equals row 0 of head h."""
    c = wl.init_v[:1] if len(wl.init_v) else wl.new_v[:1]
    return Workload(**{**wl.__dict__, "init_v": np.broadcast_to(c, wl.init_v.shape).copy(),
                       "new_v": np.broadcast_to(c, wl.new_v.shape).copy()})


def pin_equal_values(wl):
    """All value rows equal c: the weights sum to one, so out = c."""
    out = oracle_decode(wl)
    c = to_f64(wl.init_v[0] if len(wl.init_v) else wl.new_v[0], wl.dtype)  # [Hkv, D]
    expect = np.repeat(c, wl.spec.group, axis=0)
    for b in range(wl.spec.num_seqs):
        assert np.allclose(out[b], expect, rtol=0, atol=1e-13), f"seq {b}"


def pin_dominant_logit(wl, winner_of):
    """One key per sequence has a logit at least 800 above every other: the
    other weights underflow to exactly 0 in float64, so out = that value row."""
    out = oracle_decode(wl)
    g = wl.spec.group
    for b in range(wl.spec.num_seqs):
        _, v = contiguous_kv(wl, b)
        expect = np.repeat(to_f64(v[winner_of[b]], wl.dtype), g, axis=0)
        assert np.array_equal(out[b], expect), f"seq {b}"


def relabel_blocks(wl, seed):
    """The same logical cache with every physical block id renamed by a random
    permutation (tables, slots and copy pairs renamed alike)."""
    perm = np.random.default_rng(seed).permutation(wl.num_blocks).astype(np.int64)
    bs = wl.spec.block_size

    def slots(s):
        s = np.asarray(s, dtype=np.int64)
        return np.where(s >= 0, perm[s // bs] * bs + s % bs, s).astype(np.int32)

    tables = np.where(wl.block_tables >= 0, perm[np.maximum(wl.block_tables, 0)], wl.block_tables).astype(np.int32)
    pairs = perm[wl.cow_pairs.astype(np.int64)].astype(np.int32).reshape(-1, 2)
    return Workload(**{**wl.__dict__, "block_tables": tables, "init_slots": slots(wl.init_slots),
                       "new_slots": slots(wl.new_slots), "cow_pairs": pairs,
                       "table_pad": int(perm[wl.table_pad]) if wl.table_pad >= 0 else wl.table_pad})


def pin_placement_invariance(wl, seeds=(1, 2)):
    """Re-placing the physical blocks leaves the output bit-identical."""
    base = oracle_decode(wl)
    for s in seeds:
        other = oracle_decode(relabel_blocks(wl, s))
        assert np.array_equal(base, other), f"relabel seed {s}"


def pin_unpaged_reference(wl, atol=1e-12):
    """Equals torch's attention on each sequence's contiguous keys/values."""
    out = oracle_decode(wl)
    smap = slot_map(wl)
    for b in range(wl.spec.num_seqs):
        ref = sdpa_reference(wl, b, smap)
        err = np.abs(out[b] - ref).max() if ref.size else 0.0
        assert err <= atol, f"seq {b}: max abs {err}"


def pin_weights(wl):
    """Softmax weights are non-negative and sum to one."""
    _, weights = oracle_decode(wl, return_weights=True)
    for (b, h), w in weights.items():
        assert len(w) == int(wl.context_lens[b])
        assert (w >= 0).all()
        assert abs(w.sum() - 1.0) <= 1e-10, (b, h, w.sum())


def pin_bruteforce(wl, atol=1e-12):
    """Vectorized oracle = Python-scalar brute force."""
    desc, k_pool, v_pool = oracle_pools(wl)
    fast = oracle.paged_decode(wl.q, k_pool, v_pool, desc, wl.block_tables, wl.context_lens, wl.scale)
    slow = oracle.paged_decode_bruteforce(wl.q, k_pool, v_pool, desc, wl.block_tables, wl.context_lens, wl.scale)
    assert np.abs(fast - slow).max() <= atol


def private_copy(wl):
    """The same sequences with every block private: each sequence gets fresh
    blocks holding its own copy of every token (shared prefix included)."""
    bs = wl.spec.block_size
    smap = slot_map(wl)
    keys = np.concatenate([wl.init_k, wl.new_k])
    values = np.concatenate([wl.init_v, wl.new_v])
    nseq = wl.spec.num_seqs
    total_blocks = int(sum(-(-int(n) // bs) for n in wl.context_lens)) + 1
    pool = BlockPool(total_blocks, bs)
    rows, slots = [], []
    for b in range(nseq):
        pool.new_sequence(b)
        for p in range(int(wl.context_lens[b])):
            rows.append(smap[int(wl.block_tables[b, p // bs]) * bs + p % bs])
        slots.extend(pool.extend(b, int(wl.context_lens[b])).tolist())
    max_blocks = max(len(pool.table(b)) for b in range(nseq))
    pad = int(pool.free_ids()[0])
    tables = np.full((nseq, max_blocks), pad, dtype=np.int32)
    for b in range(nseq):
        tables[b, : len(pool.table(b))] = pool.table(b)
    rows = np.asarray(rows, dtype=np.int64)
    empty = keys[:0]
    return Workload(**{**wl.__dict__, "num_blocks": total_blocks, "block_tables": tables, "table_pad": pad,
                       "init_k": keys[rows], "init_v": values[rows], "init_slots": np.asarray(slots, np.int32),
                       "new_k": empty, "new_v": empty, "new_slots": np.zeros(0, np.int32),
                       "cow_pairs": np.zeros((0, 2), np.int32)})


def pin_shared_equals_private(wl):
    """Sequences pointing at shared physical blocks = the same sequences with private copies."""
    assert np.array_equal(oracle_decode(wl), oracle_decode(private_copy(wl)))


def as_mha(wl):
    """GQA workload -> MHA workload whose kv head h*g+i is a copy of kv head h."""
    g = wl.spec.group
    rep = lambda a: np.repeat(a, g, axis=1)  # noqa: E731
    from dataclasses import replace

    spec = replace(wl.spec, num_kv_heads=wl.spec.num_heads)
    return Workload(**{**wl.__dict__, "spec": spec, "init_k": rep(wl.init_k), "init_v": rep(wl.init_v),
                       "new_k": rep(wl.new_k), "new_v": rep(wl.new_v)})


def pin_gqa_is_replicated_mha(wl):
    """Grouped heads = multi-head attention with each kv head replicated g times."""
    assert wl.spec.group > 1
    a = oracle_decode(wl)
    b = oracle_decode(as_mha(wl))
    # the grouped product is one matrix product per kv head, the replicated one
    # a product per head, so the summation order may differ in the last bits
    assert np.abs(a - b).max() <= 1e-13


def pin_partitions(wl, sizes, atol=1e-12):
    """Partial (max, sum, acc) per partition merged with max rescaling = single pass."""
    desc, k_pool, v_pool = oracle_pools(wl)
    single = oracle.paged_decode(wl.q, k_pool, v_pool, desc, wl.block_tables, wl.context_lens, wl.scale)
    for tp in sizes:
        part = oracle.partitioned_decode(wl.q, k_pool, v_pool, desc, wl.block_tables, wl.context_lens, wl.scale,
                                         tokens_per_partition=tp)
        assert np.abs(part - single).max() <= atol, f"partition {tp}"


def pin_poison_independence(wl):
    """Unwritten slots (tails of last blocks, unused blocks) never reach the output."""
    base = oracle_decode(wl)
    assert np.isfinite(base).all()
    for fill in (0x0000, 0x7F80 if wl.dtype == "bf16" else 0x7F800000, 0x3F80 if wl.dtype == "bf16" else 0x3F800000):
        other = oracle_decode(wl, pools=oracle_pools(wl, fill=fill))
        assert np.array_equal(base, other), hex(fill)


def pin_layout_bruteforce(desc, seed=0):
    """Tokens written by the oracle's cache write land exactly where the scalar
    layout formulas say, read back through the tile views, and nothing else changes."""
    rng = np.random.default_rng(seed)
    bits_t = np.uint16 if desc.dtype == "bf16" else np.uint32
    total = desc.num_blocks * desc.block_size
    t = max(1, total // 3)
    slots = rng.choice(total, size=t, replace=False).astype(np.int32)
    k = rng.integers(1, 1 << 15, size=(t, desc.num_kv_heads, desc.head_dim)).astype(bits_t)
    v = rng.integers(1, 1 << 15, size=(t, desc.num_kv_heads, desc.head_dim)).astype(bits_t)
    k_pool, v_pool = oracle.new_pools(desc, fill=0)
    oracle.reshape_and_cache(k_pool, v_pool, desc, k, v, slots)
    expect_k = np.zeros_like(k_pool)
    expect_v = np.zeros_like(v_pool)
    for i, s in enumerate(slots.tolist()):
        p, r = divmod(s, desc.block_size)
        for h in range(desc.num_kv_heads):
            for d in range(desc.head_dim):
                expect_k[oracle.k_offset(desc, p, h, r, d)] = k[i, h, d]
                expect_v[oracle.v_offset(desc, p, h, r, d)] = v[i, h, d]
    assert np.array_equal(k_pool, expect_k)
    assert np.array_equal(v_pool, expect_v)
    # the tile views read the same elements back
    from oracle.layout import key_tiles, value_tiles

    ids = np.arange(desc.num_blocks)
    for h in range(desc.num_kv_heads):
        kt = key_tiles(k_pool, desc, ids, h)
        vt = value_tiles(v_pool, desc, ids, h)
        for p in range(desc.num_blocks):
            for r in range(desc.block_size):
                for d in range(0, desc.head_dim, 3):
                    assert kt[p, r, d] == k_pool[oracle.k_offset(desc, p, h, r, d)]
                    assert vt[p, r, d] == v_pool[oracle.v_offset(desc, p, h, r, d)]


def pin_copy_blocks(desc, pairs, seed=0):
    """Each destination becomes what its source held before the call; every
    other element keeps its bits."""
    rng = np.random.default_rng(seed)
    bits_t = np.uint16 if desc.dtype == "bf16" else np.uint32
    k_pool = rng.integers(0, 1 << 16, size=desc.elems).astype(bits_t)
    v_pool = rng.integers(0, 1 << 16, size=desc.elems).astype(bits_t)
    k0, v0 = k_pool.copy(), v_pool.copy()
    oracle.copy_blocks(k_pool, v_pool, desc, pairs)
    per = desc.num_kv_heads * desc.block_size * desc.head_dim
    dsts = {d for _, d in pairs}
    for blk in range(desc.num_blocks):
        sl = slice(blk * per, (blk + 1) * per)
        if blk in dsts:
            src = [s for s, d in pairs if d == blk][0]
            ssl = slice(src * per, (src + 1) * per)
            assert np.array_equal(k_pool[sl], k0[ssl]) and np.array_equal(v_pool[sl], v0[ssl])
        else:
            assert np.array_equal(k_pool[sl], k0[sl]) and np.array_equal(v_pool[sl], v0[sl])


# ---- several new tokens per step (causal) -------------------------------------------

def pin_causal_one_token_is_decode(wl):
    """With one new token per sequence the causal form is the decode itself."""
    assert (wl.query_lens == 1).all()
    pools = oracle_pools(wl)
    assert np.array_equal(oracle_causal(wl, pools), oracle_decode(wl, pools))


def pin_causal_is_sequential_decode(wl):
    """New token i of sequence b gets what a decode step computes for the same
    sequence with its cache ending at that token (context_len cut to the
    token's position + 1): a verify pass over draft tokens must reproduce
    token-by-token decoding."""
    pools = oracle_pools(wl)
    desc, k_pool, v_pool = pools
    out = oracle_causal(wl, pools)
    for b in range(wl.spec.num_seqs):
        first, last = int(wl.query_start[b]), int(wl.query_start[b + 1])
        n, ctx = last - first, int(wl.context_lens[b])
        for i in range(n):
            cut = np.array([ctx - n + i + 1], dtype=np.int32)
            one = oracle.paged_decode(wl.q[first + i][None], k_pool, v_pool, desc, wl.block_tables[b][None], cut,
                                      wl.scale)
            assert np.array_equal(out[first + i], one[0]), f"seq {b} token {i}"


def pin_causal_whole_prompt(wl, atol=1e-12):
    """Sequences whose every token is new: torch's attention with its own
    causal mask on the contiguous keys/values."""
    out = oracle_causal(wl)
    smap = slot_map(wl)
    whole = [b for b in range(wl.spec.num_seqs) if wl.query_lens[b] == wl.context_lens[b]]
    assert whole, "no whole-prompt sequence in the workload"
    for b in whole:
        ref = sdpa_causal_prompt(wl, b, smap)
        got = out[wl.query_start[b]:wl.query_start[b + 1]]
        err = np.abs(got - ref).max()
        assert err <= atol, f"seq {b}: max abs {err}"


def pin_causal_future_invariance(wl, seed=0):
    """Changing the key and value of each sequence's last new token changes
    only that token's rows: nothing before a token sees it."""
    rng = np.random.default_rng(seed)
    last = wl.query_start[1:] - 1
    new_k, new_v = wl.new_k.copy(), wl.new_v.copy()
    new_k[last] = rng.permutation(new_k[last].reshape(-1)).reshape(new_k[last].shape) ^ new_k.dtype.type(1 << 3)
    new_v[last] = new_v[last] ^ new_v.dtype.type(1 << 4)
    other = Workload(**{**wl.__dict__, "new_k": new_k, "new_v": new_v})
    a, b_out = oracle_causal(wl), oracle_causal(other)
    before = np.ones(len(a), dtype=bool)
    before[last] = False
    assert np.array_equal(a[before], b_out[before]), "a row saw a later token"
    assert not np.array_equal(a[last], b_out[last]), "the last token did not see itself"
