"""Several new tokens per sequence, causal among them (pkv_paged_attn_multi_token),
on the GPU against the oracle's paged_attend_causal: small ragged cases on
every kernel (vector, 32-row MFMA tiles, 128-row LDS-staged tiles with and
without the workspace's fp16 value copy) and
partitioning, the broken-length paths, values at the fp16 limit for the tile
kernel, and the verify and prompt-chunk workloads at full size."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from paged_kv_cache_334_amd import ops  # noqa: F401  (fails loudly when the library is missing)

import oracle
from gpu_harness import GpuWorkload, check_attention, check_fp16_path, out_to_f64, to_bits
from logical_model import oracle_pools
from paged_kv_cache_334_amd.workloads import MULTI_SPECS, WorkloadSpec, bf16_bits_to_f32, f32_to_bf16_bits, generate


def _say(msg):
    print(msg, flush=True)


SMALL = {
    # group 8, up to 5 new tokens: 40 rows per kv head, two 32-row tiles
    "g8": lambda: generate("gqa-70b", num_seqs=4, ctx=(1, 300), num_heads=16, num_kv_heads=2, query_len=(1, 5)),
    # group 4, block 32, outlier keys, 2..4 new tokens: one 16-row tile
    "g4-bs32": lambda: generate("long-32k", num_seqs=3, ctx=(100, 700), num_heads=8, num_kv_heads=2,
                                query_len=(2, 4), outlier_fraction=0.01),
    # one query head per kv head, up to 20 new tokens
    "g1": lambda: generate("mha-7b", num_seqs=3, ctx=(1, 200), num_heads=4, num_kv_heads=4, query_len=(1, 20)),
    # head_dim 64 (vector kernel), group 2
    "g2-d64": lambda: generate("mha-7b", num_seqs=3, ctx=(1, 200), num_heads=4, num_kv_heads=2, head_dim=64,
                               query_len=(1, 7)),
    # float32 (vector kernel), group 4, block 32
    "f32-g4-bs32": lambda: generate(WorkloadSpec("f32-g4", "f32", 3, 8, 2, 128, 32, (1, 150), seed=7,
                                                 query_len=(1, 5))),
    # whole prompts as one chunk: up to 130 tokens x group 4 = 520 rows, 17 row tiles
    "prompt": lambda: generate("gqa-70b", num_seqs=2, ctx=(40, 130), num_heads=8, num_kv_heads=2, query_len=512),
    # 8-token blocks (block pairs on the matrix-core kernel), group 4, up to 6 new tokens
    "g4-bs8": lambda: generate("gqa-70b", num_seqs=3, ctx=(1, 250), num_heads=8, num_kv_heads=2, block_size=8,
                               query_len=(1, 6)),
    # 8-token blocks, group 8, up to 5 new tokens: 32-row tiles over block pairs
    "g8-bs8": lambda: generate("gqa-70b", num_seqs=4, ctx=(1, 300), num_heads=16, num_kv_heads=2, block_size=8,
                               query_len=(1, 5)),
    # shared prefix with copy-on-write at the first new token
    "prefix-cow": lambda: generate("shared-prefix", num_seqs=8, shared_prefix=256, ctx=(16, 100), num_heads=8,
                                   num_kv_heads=2, cow_fraction=0.25, query_len=(1, 4)),
}

VARIANTS = [  # (kernel, partition tokens, blocks in flight)
    ("auto", 0, 0),
    ("mfma", 1 << 30, 1),
    ("mfma", 32, 0),
    ("mfma", 96, 1),
    # odd block counts per partition at 8-token blocks: the last pair of a
    # partition has no second block, and its repeated first block must stay out
    # of the softmax sum
    ("mfma", 24, 1),
    ("mfma", 40, 0),
    ("vector", 1 << 30, 0),
    ("vector", 48, 0),
    # 128-row causal tiles: one partition (rows written directly), and
    # partitions of one and of three 64-token stages (partials + merge)
    ("tile", 0, 0),
    ("tile", 1 << 30, 0),
    ("tile", 64, 0),
    ("tile", 192, 0),
]


def _mfma_ok(wl):
    return wl.dtype == "bf16" and wl.spec.head_dim == 128


@pytest.fixture(scope="module", params=sorted(SMALL))
def small_case(request):
    name = request.param
    _say(f"[multi] building {name}")
    wl = SMALL[name]()
    gw = GpuWorkload(wl)
    desc, k_pool, v_pool = oracle_pools(wl)
    ref = oracle.paged_attend_causal(wl.q, k_pool, v_pool, desc, wl.block_tables, wl.context_lens, wl.query_start,
                                     wl.scale)
    return name, wl, gw, (desc, k_pool, v_pool), ref


def test_small_cache_ops_bit_exact(small_case):
    name, wl, gw, (desc, k_ref, v_ref), _ = small_case
    assert np.array_equal(to_bits(gw.k_pool), k_ref) and np.array_equal(to_bits(gw.v_pool), v_ref), name


@pytest.mark.parametrize("kernel,ptoks,inflight", VARIANTS)
@pytest.mark.parametrize("out_dtype", ["same", "f32"])
def test_small_multi(small_case, kernel, ptoks, inflight, out_dtype):
    name, wl, gw, _, ref = small_case
    if kernel in ("mfma", "tile") and not _mfma_ok(wl):
        pytest.skip("matrix-core kernels: bf16, head_dim 128")
    if out_dtype == "f32" and wl.dtype == "f32":
        pytest.skip("same")
    if kernel == "mfma" and inflight == 0 and wl.max_query_len * wl.spec.group > 16:
        inflight = 1
    _say(f"[multi] {name} kernel={kernel} ptoks={ptoks} inflight={inflight} out={out_dtype}")
    odt = torch.float32 if out_dtype == "f32" else None
    out = out_to_f64(gw.multi(kernel=kernel, partition_tokens=ptoks, blocks_in_flight=inflight, out_dtype=odt))
    torch.cuda.synchronize()
    check_attention(out, ref, wl.dtype, "f32" if (odt is not None or wl.dtype == "f32") else "bf16",
                    f"{name}/{kernel}/{ptoks}")


@pytest.mark.parametrize("copy", [0, -1])
@pytest.mark.parametrize("ptoks", [0, 64])
def test_small_multi_tile_fp16_path(small_case, ptoks, copy):
    """The tiles' fp16 path wherever the values fit (min_eff_tokens 1: no walk
    goes back to the exact path for having few effective tokens), against its
    own error bound; with the default (128) the small rows here would take the
    exact path.  Values from the workspace's fp16 copy (copy 0) or converted
    in LDS by each tile (copy -1): the same bits either way."""
    name, wl, gw, _, ref = small_case
    if not _mfma_ok(wl):
        pytest.skip("matrix-core kernels: bf16, head_dim 128")
    _say(f"[multi] {name} tile fp16 path ptoks={ptoks} copy={copy}")
    out = gw.multi(kernel="tile", partition_tokens=ptoks, min_eff_tokens=1.0, out_dtype=torch.float32,
                   tile_value_copy=copy)
    check_fp16_path(out_to_f64(out), ref, wl, f"{name}/tile-fp16/{ptoks}/{copy}")
    if copy == -1:
        other = gw.multi(kernel="tile", partition_tokens=ptoks, min_eff_tokens=1.0, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(out, other), f"{name}: the value copy changed the result"


@pytest.mark.parametrize("ptoks", [0, 64, 192])
def test_small_multi_tile_without_value_copy(small_case, ptoks):
    """The tiles converting their values in LDS (tile_value_copy -1), on the
    default effective-token floor, against the oracle in both output forms."""
    name, wl, gw, _, ref = small_case
    if not _mfma_ok(wl):
        pytest.skip("matrix-core kernels: bf16, head_dim 128")
    for odt in (None, torch.float32):
        _say(f"[multi] {name} tile without value copy ptoks={ptoks} out={odt}")
        out = out_to_f64(gw.multi(kernel="tile", partition_tokens=ptoks, out_dtype=odt, tile_value_copy=-1))
        check_attention(out, ref, "bf16", "f32" if odt is not None else "bf16", f"{name}/tile-nocopy/{ptoks}")


def test_small_multi_deterministic(small_case):
    name, wl, gw, _, _ = small_case
    a = gw.multi(partition_tokens=32)
    b = gw.multi(partition_tokens=32)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), name


def test_one_new_token_matches_decode_oracle():
    """One new token per sequence through the multi-token path is the decode step."""
    wl = generate("gqa-70b", num_seqs=5, ctx=(1, 400), num_heads=16, num_kv_heads=2)
    gw = GpuWorkload(wl)
    desc, k_pool, v_pool = oracle_pools(wl)
    ref = oracle.paged_decode(wl.q, k_pool, v_pool, desc, wl.block_tables, wl.context_lens, wl.scale)
    for kernel in ("mfma", "vector"):
        _say(f"[multi] one token per sequence, {kernel}")
        out = out_to_f64(gw.multi(kernel=kernel, out_dtype=torch.float32))
        check_attention(out, ref, wl.dtype, "f32", f"one-token/{kernel}")


def test_zero_scale_gives_mean_of_visible_values():
    """scale 0: every visible token weighs the same (also checks that masked
    logits never reach the exponent as -inf * 0)."""
    wl = generate("gqa-70b", num_seqs=3, ctx=(1, 100), num_heads=8, num_kv_heads=2, query_len=(1, 6), scale=0.0)
    gw = GpuWorkload(wl)
    desc, k_pool, v_pool = oracle_pools(wl)
    ref = oracle.paged_attend_causal(wl.q, k_pool, v_pool, desc, wl.block_tables, wl.context_lens, wl.query_start,
                                     0.0)
    for kernel in ("mfma", "vector", "tile"):
        _say(f"[multi] zero scale, {kernel}")
        out = out_to_f64(gw.multi(kernel=kernel, partition_tokens=32, out_dtype=torch.float32))
        check_attention(out, ref, wl.dtype, "f32", f"zero-scale/{kernel}")
    one = generate("gqa-70b", num_seqs=3, ctx=(1, 100), num_heads=8, num_kv_heads=2, scale=0.0)
    gw1 = GpuWorkload(one)
    pools = oracle_pools(one)
    ref1 = oracle.paged_decode(one.q, pools[1], pools[2], pools[0], one.block_tables, one.context_lens, 0.0)
    for kernel in ("mfma", "vector"):
        _say(f"[decode] zero scale, {kernel}")
        out = out_to_f64(gw1.decode(kernel=kernel, out_dtype=torch.float32))
        check_attention(out, ref1, one.dtype, "f32", f"decode-zero-scale/{kernel}")


def test_broken_lengths():
    """More new tokens than context, or than max_query_len: the covered rows
    become NaN.  Query starts running past q: that sequence's rows stay untouched."""
    wl = generate("gqa-70b", num_seqs=4, ctx=(20, 100), num_heads=8, num_kv_heads=2, query_len=(2, 4))
    gw = GpuWorkload(wl)
    desc, k_pool, v_pool = oracle_pools(wl)
    ref = oracle.paged_attend_causal(wl.q, k_pool, v_pool, desc, wl.block_tables, wl.context_lens, wl.query_start,
                                     wl.scale)
    qs = wl.query_start
    for kernel in ("mfma", "vector", "tile"):
        _say(f"[multi] broken lengths, {kernel}")
        ctx = gw.context_lens.clone()
        ctx[1] = int(wl.query_lens[1]) - 1  # fewer tokens than new ones
        out = torch.full((len(wl.q), wl.spec.num_heads, wl.spec.head_dim), 7.0, device="cuda")
        ops.paged_attn_multi_token(gw.q, gw.k_pool, gw.v_pool, gw.block_tables, ctx, gw.query_start, wl.scale,
                                   max_query_len=wl.max_query_len, max_context_len=wl.max_context, out=out,
                                   kernel=kernel, partition_tokens=32)
        got = out_to_f64(out)
        assert np.isnan(got[qs[1]:qs[2]]).all()
        keep = np.r_[qs[0]:qs[1], qs[2]:qs[4]]
        check_attention(got[keep], ref[keep], wl.dtype, "f32", f"broken-ctx/{kernel}")

        starts = gw.query_start.clone()
        starts[-1] = len(wl.q) + 5  # the last sequence's rows run past q
        out.fill_(7.0)
        ops.paged_attn_multi_token(gw.q, gw.k_pool, gw.v_pool, gw.block_tables, gw.context_lens, starts, wl.scale,
                                   max_query_len=wl.max_query_len, max_context_len=wl.max_context, out=out,
                                   kernel=kernel, partition_tokens=32)
        got = out_to_f64(out)
        assert (got[qs[3]:] == 7.0).all(), "rows of a sequence with bad query starts were written"
        check_attention(got[:qs[3]], ref[:qs[3]], wl.dtype, "f32", f"broken-start/{kernel}")

        short = int(wl.query_lens.max()) - 1  # a host bound below the longest
        longest = int(np.argmax(wl.query_lens))
        out.fill_(7.0)
        ops.paged_attn_multi_token(gw.q, gw.k_pool, gw.v_pool, gw.block_tables, gw.context_lens, gw.query_start,
                                   wl.scale, max_query_len=short, max_context_len=wl.max_context, out=out,
                                   kernel=kernel, partition_tokens=32)
        got = out_to_f64(out)
        first = int(qs[longest])
        assert np.isnan(got[first:first + short]).all()
        assert (got[first + short:qs[longest + 1]] == 7.0).all()


# ---- full size ----------------------------------------------------------------------

def _sub_batch(wl, seqs):
    """Query rows, tables, lengths and query starts of the listed sequences only."""
    rows = np.concatenate([np.arange(wl.query_start[b], wl.query_start[b + 1]) for b in seqs])
    lens = wl.query_lens[seqs]
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return rows, wl.q[rows], wl.block_tables[seqs], wl.context_lens[seqs], starts


@pytest.mark.parametrize("kernel", ["auto", "mfma"])
@pytest.mark.parametrize("out_dtype", ["same", "f32"])
@pytest.mark.parametrize("name", sorted(MULTI_SPECS))
def test_full_multi(name, out_dtype, kernel):
    """Full-size workloads in the benchmark's launch configuration (automatic
    plan: 32-row MFMA tiles for verify, 128-row tiles for the prompt chunks),
    and the prompt chunks on the 32-row kernel too.  The verify workload is
    compared on every row; the prompt chunks (512 new tokens per sequence, one
    oracle attention per token) on their longest and shortest sequences, which
    keeps the oracle within seconds."""
    if kernel == "mfma" and name.startswith("verify"):
        pytest.skip("the automatic plan is this one")
    _say(f"[multi-full] building {name} ({kernel})")
    wl = generate(MULTI_SPECS[name])
    gw = GpuWorkload(wl)
    odt = torch.float32 if out_dtype == "f32" else None
    out = out_to_f64(gw.multi(out_dtype=odt, kernel=kernel))
    assert np.isfinite(out).all()
    desc, k_pool, v_pool = oracle_pools(wl)
    if wl.max_query_len <= 64:
        seqs = list(range(wl.spec.num_seqs))
    else:
        seqs = sorted({int(np.argmax(wl.context_lens)), int(np.argmin(wl.context_lens))})
    rows, q, tables, lens, starts = _sub_batch(wl, seqs)
    _say(f"[multi-full] oracle on {len(seqs)} sequences, {len(rows)} query rows")
    ref = oracle.paged_attend_causal(q, k_pool, v_pool, desc, tables, lens, starts, wl.scale)
    check_attention(out[rows], ref, wl.dtype, "f32" if odt is not None else "bf16", f"{name}/full/{out_dtype}")


@pytest.mark.parametrize("num_seqs", [256, 300])
def test_more_sequences_than_the_ranking_takes(num_seqs):
    """256 sequences of 1-4 new tokens (the most the longest-first ranking of
    the matrix-core kernel and the 128-row tiles takes, many lengths tied) and
    300 (natural order), on both kernels."""
    wl = generate("gqa-70b", num_seqs=num_seqs, ctx=(1, 60), num_heads=16, num_kv_heads=2, query_len=(1, 4))
    gw = GpuWorkload(wl)
    desc, k_pool, v_pool = oracle_pools(wl)
    ref = oracle.paged_attend_causal(wl.q, k_pool, v_pool, desc, wl.block_tables, wl.context_lens, wl.query_start,
                                     wl.scale)
    for kernel in ("mfma", "tile"):
        for ptoks in (1 << 30, 32):
            _say(f"[multi] {num_seqs} sequences, {kernel}, partition {ptoks}")
            inflight = 1 if kernel == "mfma" else 0
            out = out_to_f64(gw.multi(kernel=kernel, partition_tokens=ptoks, blocks_in_flight=inflight,
                                      out_dtype=torch.float32))
            torch.cuda.synchronize()
            check_attention(out, ref, wl.dtype, "f32", f"{num_seqs}-seqs/{kernel}/{ptoks}")


@pytest.mark.parametrize("min_eff", [0.0, 1.0])
@pytest.mark.parametrize("bits,label", [(0x477F, "65280-in-fp16-range"), (0x4780, "65536-beyond-fp16"),
                                        (0xC780, "minus-65536-beyond-fp16")])
def test_tile_values_near_the_fp16_limit(bits, label, min_eff):
    """Large values through the 128-row tiles: 65280 (the largest bf16 within
    fp16's range) stays on the fp16 path, +-65536 beyond it sends its tile back
    over its walk on the exact path (bf16 values, weights as bf16 hi + lo).
    With the default effective-token floor and with none (1), and with one
    partition and with several."""
    wl = generate("gqa-70b", num_seqs=3, ctx=(300, 700), num_heads=16, num_kv_heads=2, query_len=(40, 80))
    v = wl.init_v.copy()
    for tok, h, d in ((5, 0, 3), (150, 1, 77), (290, 0, 127)):  # cached tokens (the first sequences come first)
        v[tok, h, d] = bits
    wl.init_v = v
    gw = GpuWorkload(wl)
    desc, kp, vp = oracle_pools(wl)
    ref = oracle.paged_attend_causal(wl.q, kp, vp, desc, wl.block_tables, wl.context_lens, wl.query_start,
                                     wl.scale)
    assert np.abs(ref).max() > 10.0  # the large values reach the output
    for ptoks in (0, 128):
        _say(f"[multi] tile, value {label}, partition {ptoks}, min_eff {min_eff}")
        out = out_to_f64(gw.multi(kernel="tile", partition_tokens=ptoks, out_dtype=torch.float32,
                                  min_eff_tokens=min_eff))
        assert np.isfinite(out).all(), label
        err = np.abs(out - ref)
        assert (err <= 2e-3 + 2e-3 * np.abs(ref)).all(), f"{label}/{ptoks}: max abs {err.max():.3g}"
        b = out_to_f64(gw.multi(kernel="tile", partition_tokens=ptoks, min_eff_tokens=min_eff))
        check_attention(b, ref, "bf16", "bf16", f"tile/{label}/{ptoks}")


def test_tile_bad_block_id_gives_nan_rows():
    """A block id outside the pool in a sequence's table: that sequence's rows
    (all kv heads) are NaN on the tile kernel, the other sequences unchanged."""
    wl = generate("gqa-70b", num_seqs=3, ctx=(200, 400), num_heads=16, num_kv_heads=2, query_len=(20, 40))
    gw = GpuWorkload(wl)
    good = out_to_f64(gw.multi(kernel="tile"))
    bad = gw.block_tables.clone()
    bad[1, 2] = wl.num_blocks + 3
    gw.block_tables = bad
    out = out_to_f64(gw.multi(kernel="tile"))
    qs = wl.query_start
    assert np.isnan(out[qs[1]:qs[2]]).all()
    keep = np.r_[qs[0]:qs[1], qs[2]:qs[3]]
    assert np.array_equal(out[keep], good[keep])


@pytest.mark.parametrize("min_eff", [0.0, 1.0])
@pytest.mark.parametrize("ptoks", [0, 128])
def test_tile_logit_far_above_the_first_stage(ptoks, min_eff):
    """Causal tiles on the fp16 path take their softmax reference from the
    first 64 tokens of their walk; keys past them whose logits lie 16 or more
    (base 2) above overflow an fp16 weight, and the walk must come out right
    through the exact path.  Cached keys past the first stage of each sequence
    are scaled by 40.  With the default effective-token floor the rows those
    keys dominate take the exact path anyway (strict bound); with the floor at
    1 the rows they dominate without overflowing stay on the fp16 path, whose
    own bound applies."""
    wl = generate("gqa-70b", num_seqs=3, ctx=(400, 700), num_heads=16, num_kv_heads=2, query_len=(40, 80))
    k = bf16_bits_to_f32(wl.init_k).copy()
    starts = np.concatenate([[0], np.cumsum(wl.context_lens - wl.query_lens)])
    for b in range(3):
        k[starts[b] + np.array([150, 151, 290])] *= 40.0  # cached tokens, sequence by sequence
    wl.init_k = f32_to_bf16_bits(k)
    gw = GpuWorkload(wl)
    desc, kp, vp = oracle_pools(wl)
    ref = oracle.paged_attend_causal(wl.q, kp, vp, desc, wl.block_tables, wl.context_lens, wl.query_start,
                                     wl.scale)
    _say(f"[multi] tile, large logits, partition {ptoks}, min_eff {min_eff}")
    out = out_to_f64(gw.multi(kernel="tile", partition_tokens=ptoks, min_eff_tokens=min_eff,
                              out_dtype=torch.float32))
    if min_eff == 1.0:
        check_fp16_path(out, ref, wl, f"tile/large-logits/{ptoks}")
    else:
        check_attention(out, ref, "bf16", "f32", f"tile/large-logits/{ptoks}")


def test_tile_long_context_many_partitions():
    """One sequence with a 12000-token context and 96 new tokens (group 4: 384
    rows, three 128-row tiles): the automatic plan splits the walk into many
    64-token-stage partitions whose partials the multi-token merge combines;
    every row against the oracle, both output forms, and against one
    partition per walk."""
    wl = generate("long-32k", num_seqs=1, ctx=(12000, 12000), num_heads=8, num_kv_heads=2, query_len=96,
                  outlier_fraction=0.0)
    gw = GpuWorkload(wl)
    desc, kp, vp = oracle_pools(wl)
    ref = oracle.paged_attend_causal(wl.q, kp, vp, desc, wl.block_tables, wl.context_lens, wl.query_start,
                                     wl.scale)
    for ptoks, odt in ((0, torch.float32), (0, None), (1 << 30, torch.float32)):
        _say(f"[multi] tile, 12000-token context, partition {ptoks}, out {odt}")
        out = out_to_f64(gw.multi(kernel="tile", partition_tokens=ptoks, out_dtype=odt))
        check_attention(out, ref, "bf16", "f32" if odt is not None else "bf16", f"tile/long/{ptoks}/{odt}")
