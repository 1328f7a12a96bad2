"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch each one.  A pin set that let one of these through would not be
pinning the oracle."""

import numpy as np
import pytest

import oracle
import oracle.cache_ops as oco
import oracle.layout as olay
import oracle.attention as opd
import oracle_pins as pins
from test_oracle import _dominant, small


@pytest.fixture(scope="module")
def wls():
    return {
        "tiny": small("tiny-f32"),
        "gqa": small("gqa-70b", num_seqs=3, ctx=(1, 70), num_heads=8, num_kv_heads=2, head_dim=64),
        "prefix": small("shared-prefix", num_seqs=6, shared_prefix=32, ctx=(2, 40), num_heads=4,
                        num_kv_heads=2, head_dim=16, cow_fraction=0.34),
        "causal": small("gqa-70b", num_seqs=3, ctx=(1, 40), num_heads=4, num_kv_heads=2, head_dim=16,
                        query_len=(2, 6)),
        "prompt": small("mha-7b", num_seqs=2, ctx=(3, 20), num_heads=2, num_kv_heads=2, head_dim=16,
                        query_len=64),
    }


def caught(check) -> bool:
    try:
        with np.errstate(all="ignore"):
            check()
    except (AssertionError, ValueError, IndexError, KeyError):
        return True
    return False


def all_pins(w):
    wl_dom, winner = _dominant(w["tiny"])
    return [
        lambda: pins.pin_unpaged_reference(w["tiny"]),
        lambda: pins.pin_unpaged_reference(w["gqa"]),
        lambda: pins.pin_unpaged_reference(w["prefix"]),
        lambda: pins.pin_equal_values(pins.with_equal_values(w["gqa"])),
        lambda: pins.pin_dominant_logit(wl_dom, winner),
        lambda: pins.pin_partitions(w["gqa"], sizes=[7, 16]),
        lambda: pins.pin_layout_bruteforce(oracle.PoolDesc(4, 2, 16, 16, "bf16")),
        lambda: pins.pin_copy_blocks(oracle.PoolDesc(6, 2, 16, 16, "bf16"), [(1, 4), (0, 2)]),
        lambda: pins.pin_causal_is_sequential_decode(w["causal"]),
        lambda: pins.pin_causal_whole_prompt(w["prompt"]),
        lambda: pins.pin_causal_future_invariance(w["causal"]),
    ]


def _attend_no_shift(qg, keys, values, scale):
    e = np.exp(scale * (keys @ qg.T))
    w = e / e.sum(axis=0)
    return w.T @ values, w.T


def _attend_no_normalise(qg, keys, values, scale):
    s = scale * (keys @ qg.T)
    e = np.exp(s - s.max(axis=0))
    return e.T @ values, e.T


def _attend_no_scale(qg, keys, values, scale):
    s = keys @ qg.T
    e = np.exp(s - s.max(axis=0))
    w = e / e.sum(axis=0)
    return w.T @ values, w.T


def _key_tiles_untransposed(k_pool, desc, block_ids, kv_head):
    x = desc.x
    view = k_pool.reshape(desc.num_blocks, desc.num_kv_heads, desc.head_dim // x, desc.block_size, x)
    return view[block_ids, kv_head].reshape(len(block_ids), desc.block_size, desc.head_dim)


def _value_tiles_untransposed(v_pool, desc, block_ids, kv_head):
    view = v_pool.reshape(desc.num_blocks, desc.num_kv_heads, desc.head_dim, desc.block_size)
    return view[block_ids, kv_head].reshape(len(block_ids), desc.block_size, desc.head_dim)


_real_resolve = opd.resolve_sequence


def _resolve_extra_row(k_pool, v_pool, desc, row, n, kvh):
    return _real_resolve(k_pool, v_pool, desc, row, n + 1, kvh)


def _resolve_wrong_head(k_pool, v_pool, desc, row, n, kvh):
    return _real_resolve(k_pool, v_pool, desc, row, n, (kvh + 1) % desc.num_kv_heads)


def _decode_bits_bad_shift(bits, dtype):
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)
    return np.ascontiguousarray(bits, dtype=np.uint32).view(np.float32).astype(np.float64)


_real_write = oco.reshape_and_cache


def _write_next_row(k_pool, v_pool, desc, k, v, slots):
    s = np.asarray(slots, dtype=np.int64)
    shifted = np.where(s >= 0, (s // desc.block_size) * desc.block_size + (s + 1) % desc.block_size, s)
    return _real_write(k_pool, v_pool, desc, k, v, shifted)


def _copy_reversed(k_pool, v_pool, desc, pairs):
    pairs = np.asarray(pairs).reshape(-1, 2)[:, ::-1]
    per = desc.num_kv_heads * desc.block_size * desc.head_dim
    for pool in (k_pool, v_pool):
        view = pool.reshape(desc.num_blocks, per)
        view[pairs[:, 1]] = view[pairs[:, 0]].copy()
    return k_pool, v_pool


def _partitioned_no_rescale(q_bits, k_pool, v_pool, desc, tables, ctx, scale, tokens_per_partition=None,
                            split_points=None):
    q = olay.decode_bits(np.asarray(q_bits), desc.dtype)
    nseq, nh, hd = q.shape
    g = nh // desc.num_kv_heads
    out = np.zeros((nseq, nh, hd))
    for b in range(nseq):
        n = int(ctx[b])
        for kvh in range(desc.num_kv_heads):
            keys, values = _real_resolve(k_pool, v_pool, desc, tables[b], n, kvh)
            heads = np.arange(kvh * g, (kvh + 1) * g)
            s = scale * (keys @ q[b, heads].T)
            accs, ls = 0.0, 0.0
            for lo in range(0, n, tokens_per_partition):
                part = s[lo:lo + tokens_per_partition]
                e = np.exp(part - part.max(axis=0))
                accs = accs + e.T @ values[lo:lo + tokens_per_partition]
                ls = ls + e.sum(axis=0)
            out[b, heads] = accs / ls[:, None]
    return out


def _causal_variant(visible_of, row_of=lambda first, n, i: first + i):
    """The causal oracle with its visible-prefix length or its query row replaced."""
    def fn(q_bits, k_pool, v_pool, desc, tables, ctx, query_start, scale):
        q = olay.decode_bits(np.asarray(q_bits), desc.dtype)
        g = q.shape[1] // desc.num_kv_heads
        out = np.zeros(q.shape, dtype=np.float64)
        for b in range(len(query_start) - 1):
            first, n, c = int(query_start[b]), int(query_start[b + 1] - query_start[b]), int(ctx[b])
            for kvh in range(desc.num_kv_heads):
                keys, values = opd.resolve_sequence(k_pool, v_pool, desc, tables[b], c, kvh)
                heads = np.arange(kvh * g, (kvh + 1) * g)
                for i in range(n):
                    vis = max(1, min(c, visible_of(c, n, i)))
                    o, _ = opd._attend(q[row_of(first, n, i), heads], keys[:vis], values[:vis], scale)
                    out[first + i, heads] = o
        return out
    return fn


MUTATIONS = {
    "softmax without max shift": [(opd, "_attend", _attend_no_shift)],
    "softmax without normalisation": [(opd, "_attend", _attend_no_normalise)],
    "scale dropped": [(opd, "_attend", _attend_no_scale)],
    "key tile not transposed": [(opd, "key_tiles", _key_tiles_untransposed), (olay, "key_tiles",
                                                                             _key_tiles_untransposed)],
    "value tile not transposed": [(opd, "value_tiles", _value_tiles_untransposed),
                                  (olay, "value_tiles", _value_tiles_untransposed)],
    "one row past the context": [(opd, "resolve_sequence", _resolve_extra_row)],
    "wrong kv head": [(opd, "resolve_sequence", _resolve_wrong_head)],
    "bf16 decoded with a 15-bit shift": [(opd, "decode_bits", _decode_bits_bad_shift)],
    "cache write one row off": [(oracle, "reshape_and_cache", _write_next_row),
                                (oco, "reshape_and_cache", _write_next_row)],
    "block copy reversed": [(oracle, "copy_blocks", _copy_reversed), (oco, "copy_blocks", _copy_reversed)],
    "partials merged without rescale": [(oracle, "partitioned_decode", _partitioned_no_rescale)],
    "causal: token does not see itself": [(oracle, "paged_attend_causal", _causal_variant(lambda c, n, i: c - n + i))],
    "causal: one token past itself": [(oracle, "paged_attend_causal", _causal_variant(lambda c, n, i: c - n + i + 2))],
    "causal: no mask among new tokens": [(oracle, "paged_attend_causal", _causal_variant(lambda c, n, i: c))],
    "causal: mask from the sequence start": [(oracle, "paged_attend_causal", _causal_variant(lambda c, n, i: i + 1))],
    "causal: query rows reversed": [(oracle, "paged_attend_causal",
                                     _causal_variant(lambda c, n, i: c - n + i + 1, lambda f, n, i: f + n - 1 - i))],
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, wls, monkeypatch):
    for mod, attr, fn in MUTATIONS[name]:
        monkeypatch.setattr(mod, attr, fn)
    assert any(caught(c) for c in all_pins(wls)), f"no pin caught: {name}"


def test_pins_pass_unmutated(wls):
    for check in all_pins(wls):
        assert not caught(check)
