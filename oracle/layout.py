"""Pool layout and element decoding, written out for the oracle alone.

The pages fix the logical content of a block -- ``block_size`` tokens, each with
a key and a value vector per kv head ("PagedAttention Explained", section
"Implementing a Simplified Paged KV Cache", class ``Block``) -- but not how a
real kernel lays it out in device memory.  The library's documented layout is:

* key pool, elements ``[N, Hkv, D/x, bs, x]`` with ``x = 16 / element_bytes``
  (8 for bfloat16, 4 for float32): key element (block p, head h, token t,
  dim d) sits at ``((p*Hkv + h)*(D/x) + d//x)*(bs*x) + t*x + d%x``;
* value pool, elements ``[N, Hkv, D, bs]``: value element (p, h, t, d) sits at
  ``((p*Hkv + h)*D + d)*bs + t``.

This module is the oracle's own copy of those two formulas (``k_offset`` and
``v_offset``), plus a NumPy view that reads whole tiles through the same
formulas.  ``tests/test_oracle.py`` checks the view against the scalar
formulas element by element.

bfloat16 values are carried as raw ``uint16`` bits and float32 values as raw
``uint32`` bits, so that cache writes and copies can be compared bit for bit.
A bfloat16 is the top 16 bits of the float32 with the same sign, exponent and
leading 7 mantissa bits, so it decodes exactly by a 16-bit left shift.
"""

from dataclasses import dataclass

import numpy as np

BF16 = "bf16"
F32 = "f32"

_ELT_BYTES = {BF16: 2, F32: 4}
_BITS_DTYPE = {BF16: np.uint16, F32: np.uint32}


def chunk_elems(dtype: str) -> int:
    """Elements in one 16-byte chunk of the key layout (the ``x`` above)."""
    return 16 // _ELT_BYTES[dtype]


def bits_dtype(dtype: str):
    return _BITS_DTYPE[dtype]


@dataclass(frozen=True)
class PoolDesc:
    """Shapes shared by both pools: ``num_blocks`` physical blocks, each holding
    ``block_size`` tokens of ``num_kv_heads`` heads of ``head_dim`` elements."""

    num_blocks: int
    num_kv_heads: int
    block_size: int
    head_dim: int
    dtype: str

    @property
    def x(self) -> int:
        return chunk_elems(self.dtype)

    @property
    def elems(self) -> int:
        return self.num_blocks * self.num_kv_heads * self.block_size * self.head_dim


def k_offset(desc: PoolDesc, p: int, h: int, t: int, d: int) -> int:
    """Element offset of key (block p, kv head h, token-in-block t, dim d)."""
    x = desc.x
    hd = desc.head_dim
    return ((p * desc.num_kv_heads + h) * (hd // x) + d // x) * (desc.block_size * x) + t * x + d % x


def v_offset(desc: PoolDesc, p: int, h: int, t: int, d: int) -> int:
    """Element offset of value (block p, kv head h, token-in-block t, dim d)."""
    return ((p * desc.num_kv_heads + h) * desc.head_dim + d) * desc.block_size + t


def decode_bits(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Raw element bits -> float64 values (exact for both element types)."""
    if dtype == BF16:
        as_f32 = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    elif dtype == F32:
        as_f32 = np.ascontiguousarray(bits, dtype=np.uint32).view(np.float32)
    else:
        raise ValueError(f"unknown element type {dtype!r}")
    return as_f32.astype(np.float64)


def key_tiles(k_pool: np.ndarray, desc: PoolDesc, block_ids: np.ndarray, kv_head: int) -> np.ndarray:
    """Key bits of the given physical blocks for one kv head, as ``[n, bs, D]``.

    Reads the flat pool through the layout ``[N, Hkv, D/x, bs, x]``: the token
    axis is the fourth one, so it is moved in front of the chunk axis.
    """
    x = desc.x
    view = k_pool.reshape(desc.num_blocks, desc.num_kv_heads, desc.head_dim // x, desc.block_size, x)
    tiles = view[block_ids, kv_head]  # [n, D/x, bs, x]
    return tiles.transpose(0, 2, 1, 3).reshape(len(block_ids), desc.block_size, desc.head_dim)


def value_tiles(v_pool: np.ndarray, desc: PoolDesc, block_ids: np.ndarray, kv_head: int) -> np.ndarray:
    """Value bits of the given physical blocks for one kv head, as ``[n, bs, D]``
    (the pool holds each tile dim-major, ``[D, bs]``)."""
    view = v_pool.reshape(desc.num_blocks, desc.num_kv_heads, desc.head_dim, desc.block_size)
    tiles = view[block_ids, kv_head]  # [n, D, bs]
    return tiles.transpose(0, 2, 1)
