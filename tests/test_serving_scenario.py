"""The serving scenario on the CPU: the block manager's bookkeeping, and the
oracle over the shared paged pool equal to attention over each sequence's
private recomputed keys/values."""

import numpy as np

import oracle
import serving_scenario as ss


def _oracle_pools(sc):
    desc = oracle.PoolDesc(sc.num_blocks, ss.HKV, ss.BS, ss.HD, "bf16")
    k, v = oracle.new_pools(desc)
    for st in sc.steps:
        oracle.copy_blocks(k, v, desc, st.copies)
        oracle.reshape_and_cache(k, v, desc, st.keys(), st.values(), np.asarray(st.slots, np.int32))
    return desc, k, v


def _private_causal(sc, q):
    """Attention of the verify tokens over private contiguous keys/values (float64)."""
    from logical_model import to_f64

    g = ss.HQ // ss.HKV
    qf = to_f64(q, "bf16")
    out = np.zeros(qf.shape)
    scale = 1 / np.sqrt(ss.HD)
    for b, seq in enumerate(sc.seqs):
        keys, values = ss.contiguous_kv(sc, seq)
        n = len(keys)
        for i in range(sc.verify_len):
            vis = n - sc.verify_len + i + 1
            for h in range(ss.HQ):
                s = scale * keys[:vis, h // g] @ qf[b * sc.verify_len + i, h]
                w = np.exp(s - s.max())
                out[b * sc.verify_len + i, h] = (w / w.sum()) @ values[:vis, h // g]
    return out


def test_bookkeeping():
    sc = ss.build()
    assert all(sc.cached[r] == 64 for r in range(1, 6)) and sc.cached[0] == 0
    assert len(sc.steps[0].copies) == 0 and len(sc.steps[1].copies) == 1
    # every request shares the system prompt's first four blocks
    assert (sc.tables[:, :4] == sc.tables[0, :4]).all()
    assert sc.lens.tolist() == [len(sc.tokens[s]) for s in sc.seqs]
    # the prefix cache saved 5 x 64 token writes
    assert sum(len(st.slots) for st in sc.steps) == sum(sc.lens) - 5 * 64 - (sc.lens[6] - sc.verify_len - 2)


def test_shared_pool_equals_private_recompute():
    sc = ss.build()
    desc, k, v = _oracle_pools(sc)
    q, starts = ss.queries(sc)
    got = oracle.paged_attend_causal(q, k, v, desc, sc.tables, sc.lens, starts, 1 / np.sqrt(ss.HD))
    ref = _private_causal(sc, q)
    assert np.abs(got - ref).max() <= 1e-12
