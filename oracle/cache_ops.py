"""Cache write and copy-on-write block copy, as plain NumPy assignments.

``reshape_and_cache`` stores token ``t``'s key and value for every kv head at
its slot ``s = block * block_size + position_in_block``.  This is the page's
append rule: the token lands in the last block of the sequence's table at
``position_in_block = length % block_size`` ("PagedAttention Explained",
section "Implementing a Simplified Paged KV Cache", ``append_token``).  A
negative slot means "skip this token".

``copy_blocks`` gives a forked sequence its own copy of a block it shared, so
that the write that follows leaves the other owner's copy untouched -- the
copy-on-write behaviour that lets several sequences start from shared KV state
("Master Paged Attention for LLM Inference", "How Paged Attention Works: The
Mechanics", item 4; "PagedAttention Explained", "Shared Prefix Caching").
Every destination block receives the contents its source held before the call.

``swap_blocks`` moves whole blocks between two pools of the same shape, the
CPU swap space that holds blocks of preempted sequences ("PagedAttention
Explained", section "Programmatic Control Over KV Cache", engine argument
``swap_space``): destination block = bit copy of the source block.

All work on the flat raw-bit pools and write through the oracle's own layout
formulas (``oracle.layout``); results are compared bit for bit.
"""

import numpy as np

from .layout import BF16, F32, PoolDesc, bits_dtype

POISON = {BF16: 0x7FC0, F32: 0x7FC00000}  # quiet-NaN bit patterns


def new_pools(desc: PoolDesc, fill=None):
    """Fresh flat key and value pools.  By default every element holds a quiet
    NaN: blocks handed back to the free pool are reused without being cleared,
    so untouched slots hold arbitrary bits and the output must not depend on
    them."""
    value = POISON[desc.dtype] if fill is None else fill
    k_pool = np.full(desc.elems, value, dtype=bits_dtype(desc.dtype))
    return k_pool, k_pool.copy()


def reshape_and_cache(k_pool, v_pool, desc: PoolDesc, k_bits, v_bits, slot_mapping):
    """Write ``k_bits/v_bits [T, Hkv, D]`` into the pools at ``slot_mapping [T]``
    (in place).  Slots must be distinct; negative slots are skipped."""
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = slots >= 0
    slots = slots[keep]
    if slots.size == 0:
        return k_pool, v_pool
    if slots.max() >= desc.num_blocks * desc.block_size:
        raise ValueError("slot outside the pool")
    if np.unique(slots).size != slots.size:
        raise ValueError("slots must be distinct")
    k = np.asarray(k_bits)[keep]
    v = np.asarray(v_bits)[keep]
    blk, pos = slots // desc.block_size, slots % desc.block_size
    n, hkv, hd, bs, x = desc.num_blocks, desc.num_kv_heads, desc.head_dim, desc.block_size, desc.x
    kview = k_pool.reshape(n, hkv, hd // x, bs, x)
    vview = v_pool.reshape(n, hkv, hd, bs)
    # advanced indices on axes 0 and 3 put the token axis first: [T, Hkv, D/x, x]
    kview[blk, :, :, pos, :] = k.reshape(len(slots), hkv, hd // x, x)
    # advanced indices on axes 0 and 3 put the token axis first: [T, Hkv, D]
    vview[blk, :, :, pos] = v
    return k_pool, v_pool


def copy_blocks(k_pool, v_pool, desc: PoolDesc, pairs):
    """For every ``(src, dst)`` row of ``pairs``, make block ``dst`` of both
    pools (all kv heads) a bit copy of what block ``src`` held before the
    call (in place).  Destinations must be distinct."""
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    if pairs.size == 0:
        return k_pool, v_pool
    src, dst = pairs[:, 0], pairs[:, 1]
    if min(src.min(), dst.min()) < 0 or max(src.max(), dst.max()) >= desc.num_blocks:
        raise ValueError("block id outside the pool")
    if np.unique(dst).size != dst.size:
        raise ValueError("destinations must be distinct")
    per_block = desc.num_kv_heads * desc.block_size * desc.head_dim
    for pool in (k_pool, v_pool):
        view = pool.reshape(desc.num_blocks, per_block)
        snapshot = view[src].copy()
        view[dst] = snapshot
    return k_pool, v_pool


def swap_blocks(src_k, src_v, src_desc: PoolDesc, dst_k, dst_v, dst_desc: PoolDesc, pairs):
    """For every ``(src, dst)`` row of ``pairs``, block ``dst`` of the destination
    pools becomes a bit copy of block ``src`` of the source pools (in place).
    Both descriptors must agree in everything but the block count; destinations
    must be distinct."""
    shape = (src_desc.num_kv_heads, src_desc.block_size, src_desc.head_dim, src_desc.dtype)
    if shape != (dst_desc.num_kv_heads, dst_desc.block_size, dst_desc.head_dim, dst_desc.dtype):
        raise ValueError("pools differ in shape or dtype")
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    if pairs.size == 0:
        return dst_k, dst_v
    src, dst = pairs[:, 0], pairs[:, 1]
    if src.min() < 0 or src.max() >= src_desc.num_blocks or dst.min() < 0 or dst.max() >= dst_desc.num_blocks:
        raise ValueError("block id outside its pool")
    if np.unique(dst).size != dst.size:
        raise ValueError("destinations must be distinct")
    per_block = src_desc.num_kv_heads * src_desc.block_size * src_desc.head_dim
    for s_pool, d_pool in ((src_k, dst_k), (src_v, dst_v)):
        s_view = s_pool.reshape(src_desc.num_blocks, per_block)
        d_view = d_pool.reshape(dst_desc.num_blocks, per_block)
        d_view[dst] = s_view[src]
    return dst_k, dst_v
