"""The serving scenario on the GPU: the library's cache writes and block copies
replayed in server order give the oracle's pools bit for bit, and the
multi-token, decode and cascade attention calls over the shared pool match the
oracle."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from paged_kv_cache_334_amd import ops  # noqa: F401  (fails loudly when the library is missing)

import oracle
import serving_scenario as ss
from gpu_harness import check_attention, out_to_f64, to_bits, to_device
from test_serving_scenario import _oracle_pools


@pytest.fixture(scope="module")
def served():
    print("[serving] building scenario", flush=True)
    sc = ss.build()
    k, v = ops.new_pools(sc.num_blocks, ss.HKV, ss.BS, ss.HD, torch.bfloat16, "cuda", fill=0x7FC0)
    for st in sc.steps:
        if len(st.copies):
            ops.copy_blocks(k, v, torch.from_numpy(np.ascontiguousarray(st.copies)).cuda())
        ops.reshape_and_cache(to_device(st.keys(), "bf16"), to_device(st.values(), "bf16"),
                              torch.from_numpy(np.asarray(st.slots, np.int32)).cuda(), k, v)
    torch.cuda.synchronize()
    return sc, k, v, _oracle_pools(sc)


def test_pools_bit_exact(served):
    sc, k, v, (desc, k_ref, v_ref) = served
    assert np.array_equal(to_bits(k), k_ref) and np.array_equal(to_bits(v), v_ref)


def test_verify_step(served):
    sc, k, v, (desc, k_ref, v_ref) = served
    q, starts = ss.queries(sc)
    scale = 1 / np.sqrt(ss.HD)
    ref = oracle.paged_attend_causal(q, k_ref, v_ref, desc, sc.tables, sc.lens, starts, scale)
    tables = torch.from_numpy(sc.tables).cuda()
    lens = torch.from_numpy(sc.lens).cuda()
    for kernel in ("mfma", "vector"):
        print(f"[serving] verify step, {kernel}", flush=True)
        out = ops.paged_attn_multi_token(to_device(q, "bf16"), k, v, tables, lens, torch.from_numpy(starts).cuda(),
                                         scale, sc.verify_len, max_context_len=int(sc.lens.max()), kernel=kernel,
                                         out_dtype=torch.float32)
        check_attention(out_to_f64(out), ref, "bf16", "f32", f"serving/verify/{kernel}")


def test_decode_and_cascade(served):
    sc, k, v, (desc, k_ref, v_ref) = served
    q_all, _ = ss.queries(sc)
    q = np.ascontiguousarray(q_all[sc.verify_len - 1::sc.verify_len])  # the last verify token of each request
    scale = 1 / np.sqrt(ss.HD)
    ref = oracle.paged_decode(q, k_ref, v_ref, desc, sc.tables, sc.lens, scale)
    tables = torch.from_numpy(sc.tables).cuda()
    lens = torch.from_numpy(sc.lens).cuda()
    qd = to_device(q, "bf16")
    plan = ops.plan_shared_prefix(sc.tables, sc.lens, ss.BS, min_group_seqs=4, min_prefix_blocks=4)
    assert plan.groups == 1 and (plan.prefix_blocks() >= 4).sum() == len(sc.seqs)
    for name, kw in [("decode", {}), ("cascade", {"prefix_plan": plan})]:
        print(f"[serving] {name}", flush=True)
        out = ops.paged_attn_decode(qd, k, v, tables, lens, scale, max_context_len=int(sc.lens.max()),
                                    out_dtype=torch.float32, **kw)
        check_attention(out_to_f64(out), ref, "bf16", "f32", f"serving/{name}")
