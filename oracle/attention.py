"""Paged decode attention, the plain way (float64, two passes).

Definition followed.  At a decode step the model produces one token per
sequence and attends over every token the sequence already holds ("PagedAttention
Explained", section "What Is the KV Cache?").  The attention kernel follows the
block table, reads each block it names and attends over all of those keys and
values joined in logical order (same page, "Block Tables and Non-Contiguous
Storage"), and
paging changes only where the cache lives, not what attention returns ("What is
PagedAttention", aitechboss.com, "Step 3: Use Page Tables Instead of Continuous
Memory"; "Master Paged Attention for LLM Inference", FAQ "Does Paged Attention
affect model accuracy?").  So the oracle:

1. resolves the block table into contiguous keys and values -- stack the
   sequence's blocks in table order and keep the first ``context_len`` rows,
   as ``get_keys_values`` does in the page's simplified cache;
2. computes standard scaled-dot-product attention of the one query row per
   head over those rows: logits ``s_t = scale * <q, k_t>``, ``m = max s``,
   ``e_t = exp(s_t - m)``, ``w_t = e_t / sum e``, ``out = sum_t w_t v_t``.

Readings where the pages are silent: the attention formula itself (standard
softmax attention, ``scale`` passed in); no mask beyond the context length (the
query is the newest token and its key/value were written before attention);
query head ``h`` reads kv head ``h // (Hq/Hkv)`` (contiguous groups); a
sequence with ``context_len == 0`` yields an all-zero output row.
"""

import math
import struct

import numpy as np

from .layout import BF16, F32, PoolDesc, decode_bits, k_offset, key_tiles, v_offset, value_tiles


def _check_heads(num_heads: int, desc: PoolDesc) -> int:
    if num_heads % desc.num_kv_heads:
        raise ValueError("query heads must be a multiple of kv heads")
    return num_heads // desc.num_kv_heads


def resolve_sequence(k_pool, v_pool, desc: PoolDesc, table_row, context_len: int, kv_head: int):
    """Keys and values of one sequence and kv head as contiguous float64
    ``[context_len, D]`` arrays, in logical token order."""
    bs = desc.block_size
    nblocks = -(-int(context_len) // bs)
    ids = np.asarray(table_row[:nblocks], dtype=np.int64)
    if nblocks and (ids.min() < 0 or ids.max() >= desc.num_blocks):
        raise ValueError("block table entry outside the pool")
    keys = key_tiles(k_pool, desc, ids, kv_head).reshape(nblocks * bs, desc.head_dim)[:context_len]
    values = value_tiles(v_pool, desc, ids, kv_head).reshape(nblocks * bs, desc.head_dim)[:context_len]
    return decode_bits(keys, desc.dtype), decode_bits(values, desc.dtype)


def _attend(qg: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float):
    """Two-pass softmax attention of ``qg [g, D]`` over ``keys/values [n, D]``.
    Returns ``out [g, D]`` and the weights ``w [g, n]``."""
    logits = scale * (keys @ qg.T)  # [n, g]
    m = logits.max(axis=0)  # pass 1: the maximum logit per head
    e = np.exp(logits - m)  # pass 2: shifted exponentials, their sum, weights
    w = e / e.sum(axis=0)
    return w.T @ values, w.T


def paged_decode(q_bits, k_pool, v_pool, desc: PoolDesc, block_tables, context_lens, scale: float,
                 pairs=None, return_weights: bool = False):
    """Decode attention for every (sequence, query head), or for the listed
    ``pairs`` of (sequence, query head) only.

    ``q_bits`` is ``[B, Hq, D]`` raw element bits; ``block_tables`` is
    ``[B, max_blocks]``; ``context_lens`` is ``[B]``.  Returns float64
    ``out [B, Hq, D]`` (or ``[len(pairs), D]``), and with ``return_weights`` a
    dict mapping (b, h) to the softmax weights over that sequence's tokens.
    """
    q = decode_bits(np.asarray(q_bits), desc.dtype)
    nseq, num_heads, hd = q.shape
    g = _check_heads(num_heads, desc)
    want = None
    if pairs is not None:
        want = {}
        for b, h in pairs:
            want.setdefault((int(b), int(h) // g), []).append(int(h))
    out = np.zeros((nseq, num_heads, hd), dtype=np.float64)
    weights = {}
    todo = want.keys() if want is not None else [(b, kvh) for b in range(nseq) for kvh in range(desc.num_kv_heads)]
    for b, kvh in todo:
        n = int(context_lens[b])
        if n == 0:
            continue
        keys, values = resolve_sequence(k_pool, v_pool, desc, block_tables[b], n, kvh)
        heads = np.arange(kvh * g, (kvh + 1) * g)
        o, w = _attend(q[b, heads], keys, values, scale)
        out[b, heads] = o
        if return_weights:
            for i, h in enumerate(heads):
                weights[(b, int(h))] = w[i]
    if pairs is not None:
        out = np.stack([out[int(b), int(h)] for b, h in pairs]) if len(pairs) else np.zeros((0, hd))
    return (out, weights) if return_weights else out


def _scalar(bits: int, dtype: str) -> float:
    """One element's bits -> Python float, by re-packing the bytes."""
    if dtype == BF16:
        return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]
    if dtype == F32:
        return struct.unpack("<f", struct.pack("<I", int(bits) & 0xFFFFFFFF))[0]
    raise ValueError(dtype)


def paged_decode_bruteforce(q_bits, k_pool, v_pool, desc: PoolDesc, block_tables, context_lens, scale: float):
    """The same result with Python scalars and loops only: every key and value
    element is located with the scalar layout formulas, one at a time.  For
    tiny inputs (a few thousand multiply-adds)."""
    nseq, num_heads, hd = np.asarray(q_bits).shape
    g = _check_heads(num_heads, desc)
    bs = desc.block_size
    out = [[[0.0] * hd for _ in range(num_heads)] for _ in range(nseq)]
    for b in range(nseq):
        n = int(context_lens[b])
        for h in range(num_heads):
            kvh = h // g
            qv = [_scalar(q_bits[b][h][d], desc.dtype) for d in range(hd)]
            logits = []
            for t in range(n):
                p = int(block_tables[b][t // bs])
                acc = 0.0
                for d in range(hd):
                    acc += qv[d] * _scalar(k_pool[k_offset(desc, p, kvh, t % bs, d)], desc.dtype)
                logits.append(scale * acc)
            if n == 0:
                continue
            m = max(logits)
            e = [math.exp(s - m) for s in logits]
            z = sum(e)
            for d in range(hd):
                acc = 0.0
                for t in range(n):
                    p = int(block_tables[b][t // bs])
                    acc += (e[t] / z) * _scalar(v_pool[v_offset(desc, p, kvh, t % bs, d)], desc.dtype)
                out[b][h][d] = acc
    return np.array(out, dtype=np.float64)


def partitioned_decode(q_bits, k_pool, v_pool, desc: PoolDesc, block_tables, context_lens, scale: float,
                       tokens_per_partition: int = None, split_points=None):
    """Decode through partials: cut each sequence's tokens into partitions,
    keep per partition the maximum logit ``m_p``, the shifted sum
    ``l_p = sum exp(s - m_p)`` and ``acc_p = sum exp(s - m_p) v``, then merge
    with ``M = max m_p``: ``out = sum_p e^(m_p - M) acc_p / sum_p e^(m_p - M) l_p``.

    Partitions are either every ``tokens_per_partition`` tokens, or cut at the
    per-sequence token offsets ``split_points[b]`` (e.g. the end of a shared
    prefix).  The merge is exact algebra, so the result equals
    ``paged_decode`` up to rounding.
    """
    q = decode_bits(np.asarray(q_bits), desc.dtype)
    nseq, num_heads, hd = q.shape
    g = _check_heads(num_heads, desc)
    out = np.zeros((nseq, num_heads, hd), dtype=np.float64)
    for b in range(nseq):
        n = int(context_lens[b])
        if n == 0:
            continue
        if split_points is not None:
            cuts = sorted({0, n, *[int(c) for c in split_points[b] if 0 < int(c) < n]})
        else:
            cuts = list(range(0, n, tokens_per_partition)) + [n]
        for kvh in range(desc.num_kv_heads):
            keys, values = resolve_sequence(k_pool, v_pool, desc, block_tables[b], n, kvh)
            heads = np.arange(kvh * g, (kvh + 1) * g)
            logits = scale * (keys @ q[b, heads].T)  # [n, g]
            ms, ls, accs = [], [], []
            for lo, hi in zip(cuts[:-1], cuts[1:]):
                s = logits[lo:hi]
                m_p = s.max(axis=0)
                e = np.exp(s - m_p)
                ms.append(m_p)
                ls.append(e.sum(axis=0))
                accs.append(e.T @ values[lo:hi])
            ms, ls, accs = np.stack(ms), np.stack(ls), np.stack(accs)  # [P, g], [P, g], [P, g, D]
            big_m = ms.max(axis=0)
            f = np.exp(ms - big_m)
            out[b, heads] = (f[:, :, None] * accs).sum(axis=0) / (f * ls).sum(axis=0)[:, None]
    return out


def paged_attend_causal(q_bits, k_pool, v_pool, desc: PoolDesc, block_tables, context_lens, query_start,
                        scale: float):
    """Attention of several new tokens per sequence (a verify step of
    speculative decoding, a chunk of a prompt) over the paged cache, causal
    among the new tokens.

    Sequence ``b`` holds ``context_lens[b]`` tokens, the last
    ``n_b = query_start[b+1] - query_start[b]`` of them written this step; row
    ``query_start[b] + i`` of ``q_bits [T, Hq, D]`` is the query of new token
    ``i``, which sits at position ``context_lens[b] - n_b + i`` and attends to
    the tokens at positions ``0 .. context_lens[b] - n_b + i`` (itself and
    everything before it, nothing after).  Returns float64 ``out [T, Hq, D]``.

    The pages name speculative decoding and forked sequences as users of the
    shared paged cache ("Master Paged Attention for LLM Inference", "How Paged
    Attention Works: The Mechanics", item 4; "What is PagedAttention",
    "PagedAttention vs Speculative Decoding") and a prompt's prefill that
    fills it ("PagedAttention Explained", "Enabling Automatic Prefix
    Caching"), but give no formula: the reading here is the standard causal
    mask of a decoder, each new token seeing the prefix up to itself.  Each
    row is computed as the single-query attention above over its visible
    prefix.
    """
    q = decode_bits(np.asarray(q_bits), desc.dtype)
    total, num_heads, hd = q.shape
    g = _check_heads(num_heads, desc)
    starts = np.asarray(query_start, dtype=np.int64)
    nseq = len(starts) - 1
    if starts[0] < 0 or starts[-1] > total or (np.diff(starts) < 0).any():
        raise ValueError("query_start must be non-decreasing within [0, T]")
    out = np.zeros((total, num_heads, hd), dtype=np.float64)
    for b in range(nseq):
        first, n_new = int(starts[b]), int(starts[b + 1] - starts[b])
        ctx = int(context_lens[b])
        if n_new == 0:
            continue
        if n_new > ctx:
            raise ValueError(f"sequence {b}: more new tokens than context")
        for kvh in range(desc.num_kv_heads):
            keys, values = resolve_sequence(k_pool, v_pool, desc, block_tables[b], ctx, kvh)
            heads = np.arange(kvh * g, (kvh + 1) * g)
            for i in range(n_new):
                visible = ctx - n_new + i + 1
                o, _ = _attend(q[first + i, heads], keys[:visible], values[:visible], scale)
                out[first + i, heads] = o
    return out
