"""The C ABI library, without a GPU: it loads, exports every entry point the
header declares, and rejects bad host-side arguments before launching
anything (these paths return before the first HIP call)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]
LIB = os.path.join(ROOT, "paged_kv_cache_334_amd", "libpkv.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libpkv.so not built")


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("pkv_paged_attn_decode", "pkv_reshape_and_cache", "pkv_copy_blocks"):
        assert n in names


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(LIB)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


@pytest.fixture(scope="module")
def ops():
    from paged_kv_cache_334_amd import ops

    return ops


def test_status_strings(ops):
    assert ops.status_string(0) == "ok"
    assert ops.status_string(3) == "workspace missing or too small"
    assert ops.lib.pkv_version() >= 100


def _desc(ops, **kw):
    base = dict(num_blocks=64, num_kv_heads=8, block_size=16, head_dim=128, dtype=ops.PKV_BF16)
    base.update(kw)
    return ops.PoolDesc(**base)


def _decode(ops, desc, num_heads=32, max_ctx=256, ptr=16, opts=None, out_dtype=None, ws=0, ws_bytes=0,
            max_blocks=16, scale=0.1):
    p = ctypes.c_void_p(ptr) if ptr else None
    od = desc.dtype if out_dtype is None else out_dtype
    return ops.lib.pkv_paged_attn_decode(p, p, p, p, p, 4, num_heads, max_blocks, max_ctx, ctypes.byref(desc), scale,
                                         od, p, ctypes.c_void_p(ws) if ws else None, ws_bytes,
                                         ctypes.byref(opts) if opts else None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(block_size=4), 2),
    (dict(block_size=64), 2),
    (dict(head_dim=96), 2),
    (dict(dtype=7), 2),
    (dict(num_blocks=0), 1),
    (dict(num_blocks=(1 << 31) // 16), 1),
])
def test_bad_pool_is_rejected(ops, kw, status):
    assert _decode(ops, _desc(ops, **kw)) == status
    assert ops.lib.pkv_last_error().decode()


@pytest.mark.parametrize("heads,dtype", [(1 << 19, "PKV_BF16"), (1 << 18, "PKV_F32")])
def test_block_bytes_bound(ops, heads, dtype):
    """One block of every kv head must stay below 2^31 bytes (the kernels form
    block offsets as a 32 x 32 -> 64-bit product); the pool check says so
    before anything else is looked at."""
    d = _desc(ops, num_kv_heads=heads, dtype=getattr(ops, dtype))
    assert _decode(ops, d, num_heads=heads) == 1
    assert "element size must stay below 2^31" in ops.lib.pkv_last_error().decode()
    # half as many heads passes the pool check: a split plan then sizes its workspace
    ok = _desc(ops, num_kv_heads=heads // 2, dtype=getattr(ops, dtype))
    split = ops.DecodeOpts(64, 0, 0)
    assert ops.lib.pkv_paged_attn_workspace_bytes(ctypes.byref(ok), 4, heads // 2, 256, ctypes.byref(split)) > 0


def test_bad_decode_arguments(ops):
    d = _desc(ops)
    assert _decode(ops, d, num_heads=12) == 1            # not a multiple of kv heads
    assert _decode(ops, d, num_heads=8 * 3) == 2         # group of 3 is not built
    assert _decode(ops, d, ptr=0) == 1                   # NULL pointers
    assert _decode(ops, d, ptr=8) == 1                   # misaligned
    assert _decode(ops, d, max_ctx=16 * 16 + 1) == 1     # beyond max_blocks * block_size
    assert _decode(ops, d, scale=float("inf")) == 1
    assert _decode(ops, d, scale=-0.5) == 1              # the kernels take the max of unscaled logits
    assert _decode(ops, _desc(ops, dtype=ops.PKV_F32), out_dtype=ops.PKV_BF16) == 2
    assert _decode(ops, d, opts=ops.DecodeOpts(0, 9, 0)) == 1
    assert _decode(ops, _desc(ops, num_kv_heads=32), opts=ops.DecodeOpts(0, 2, 0)) == 2  # MFMA needs a group of 4/8


def test_workspace_is_required_for_split(ops):
    d = _desc(ops)
    opts = ops.DecodeOpts(64, 0, 0)
    need = ops.lib.pkv_paged_attn_workspace_bytes(ctypes.byref(d), 4, 32, 256, ctypes.byref(opts))
    assert need == 4 * 32 * 4 * (128 + 2) * 4  # 4 partitions of 64 tokens
    assert _decode(ops, d, opts=opts) == 3
    assert _decode(ops, d, opts=opts, ws=16, ws_bytes=need - 4) == 3
    single = ops.DecodeOpts(1 << 30, 0, 0)
    assert ops.lib.pkv_paged_attn_workspace_bytes(ctypes.byref(d), 4, 32, 256, ctypes.byref(single)) == 0


def test_zero_sequences_is_a_no_op(ops):
    d = _desc(ops)
    st = ops.lib.pkv_paged_attn_decode(None, None, None, None, None, 0, 32, 16, 256, ctypes.byref(d), 0.1, 1, None,
                                       None, 0, None, None)
    assert st == 0


def test_cache_op_arguments(ops):
    d = _desc(ops)
    p = ctypes.c_void_p(16)
    assert ops.lib.pkv_reshape_and_cache(p, p, 0, 0, p, -1, p, p, ctypes.byref(d), None) == 1
    assert ops.lib.pkv_reshape_and_cache(p, p, 100, 0, p, 4, p, p, ctypes.byref(d), None) == 1  # stride too small
    assert ops.lib.pkv_reshape_and_cache(None, p, 0, 0, p, 4, p, p, ctypes.byref(d), None) == 1
    assert ops.lib.pkv_reshape_and_cache(p, p, 0, 0, p, 0, p, p, ctypes.byref(d), None) == 0  # nothing to do
    assert ops.lib.pkv_copy_blocks(p, p, None, 3, ctypes.byref(d), None) == 1
    assert ops.lib.pkv_copy_blocks(p, p, p, -2, ctypes.byref(d), None) == 1
    assert ops.lib.pkv_copy_blocks(p, p, None, 0, ctypes.byref(d), None) == 0


def test_min_eff_tokens_range(ops):
    d = _desc(ops)
    bad = [-1.0, float("nan"), float("-inf")]
    for v in bad:
        assert _decode(ops, d, opts=ops.DecodeOpts(0, 0, 0, 0, None, None, 0, v)) == 1, v
        assert "min_eff_tokens" in ops.lib.pkv_last_error().decode()
    # accepted: +inf (exact path only), 1, and 0 (the library's value); the
    # workspace does not depend on it
    split = [ops.DecodeOpts(64, 0, 0, 0, None, None, 0, v) for v in (float("inf"), 1.0, 0.0)]
    sizes = {ops.lib.pkv_paged_attn_workspace_bytes(ctypes.byref(d), 4, 32, 256, ctypes.byref(o)) for o in split}
    assert sizes == {4 * 32 * 4 * (128 + 2) * 4}


def test_blocks_in_flight_range(ops):
    d = _desc(ops)
    assert _decode(ops, d, opts=ops.DecodeOpts(0, 0, 3)) == 1
    assert _decode(ops, d, opts=ops.DecodeOpts(0, 0, -1)) == 1


def test_heads_per_workgroup_checks(ops):
    mha = _desc(ops, num_kv_heads=32)
    assert _decode(ops, mha, opts=ops.DecodeOpts(0, 0, 0, 3)) == 1                   # out of range
    assert _decode(ops, _desc(ops), opts=ops.DecodeOpts(0, 0, 0, 2)) == 2            # group of 4
    assert _decode(ops, _desc(ops, num_kv_heads=31), num_heads=31, opts=ops.DecodeOpts(0, 0, 0, 2)) == 2  # odd
    assert _decode(ops, mha, opts=ops.DecodeOpts(0, 0, 2, 2)) == 2                   # two blocks in flight


def test_probe_arguments_rejected_without_launch():
    lib = ctypes.CDLL(LIB)
    lib.pkv_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    lib.pkv_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p]
    lib.pkv_probe_gather.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    p = ctypes.c_void_p(16)
    assert lib.pkv_probe_read(None, 1024, p, 8, None) == 1
    assert lib.pkv_probe_read(p, 1000, p, 8, None) == 1       # not a multiple of 16
    assert lib.pkv_probe_copy(p, ctypes.c_void_p(24), 1024, 8, None) == 1  # misaligned
    assert lib.pkv_probe_gather(p, p, 4, 100, p, 8, None) == 1  # tile size not a multiple of 16
    assert lib.pkv_probe_gather(p, p, 0, 4096, p, 8, None) == 1


def test_prefix_plan_is_checked_before_launch(ops):
    import numpy as np

    d = _desc(ops)
    tables = np.tile(np.arange(16, dtype=np.int32), (4, 1))  # 4 sequences sharing every block
    ctx = np.full(4, 256, dtype=np.int32)
    plan = ops.plan_shared_prefix(tables, ctx, 16, 2, 1, device=None)
    assert plan.groups == 1
    words = plan.host

    def call(w, dev=16, desc=d, nwords=None):
        opts = ops.DecodeOpts(0, 0, 0, 0, w.ctypes.data, dev, w.size if nwords is None else nwords)
        return _decode(ops, desc, opts=opts, ws=16, ws_bytes=1 << 30)

    bad = words.copy()
    bad[0] = 0
    assert call(bad) == 1                                   # magic
    assert call(words, nwords=5) == 1                       # truncated
    assert call(words, dev=0) == 1                          # no device copy
    bad = words.copy()
    bad[1] = 5
    assert call(bad) == 1                                   # other batch size
    g0 = 6 + 2 * 4  # words of group 0 (after prefix_of[4] and group_of[4])
    bad = words.copy()
    bad[g0 + 3] = 9
    assert call(bad) == 1                                   # leader outside the batch
    bad = words.copy()
    bad[6 + 2] = 3
    assert call(bad) == 1                                   # member with another prefix
    bad = words.copy()
    bad[6 + 4 + 2] = -1
    assert call(bad) == 1                                   # member without a group
    bad = words.copy()
    bad[g0 + 5] = 0
    assert call(bad) == 1                                   # group as its own parent
    bad = words.copy()
    bad[g0 + 4] = 4
    assert call(bad) == 1                                   # root not starting at block 0
    # a nested plan (root over all four, children over the first and last two) whose
    # child names itself as parent: rejected, no endless walk up the tree
    t2 = tables.copy()
    t2[2:, 8:] += 100
    nested = ops.plan_shared_prefix(t2, ctx, 16, 2, 1, device=None).host
    assert int(nested[3]) == 3
    nopts = ops.DecodeOpts(0, 0, 0, 0, nested.ctypes.data, 16, nested.size)
    assert _decode(ops, d, opts=nopts, ws=16, ws_bytes=16) == 3  # plan accepted, stops at the workspace check
    bad = nested.copy()
    bad[g0 + 6 + 5] = 1
    assert call(bad) == 1                                   # child as its own parent
    bad = nested.copy()
    bad[g0 + 6 + 5] = 7
    assert call(bad) == 1                                   # parent outside the plan
    mem = g0 + 3 * 6  # member lists: root [0 1 2 3], then [0 1], then [2 3]
    assert nested[mem:].tolist() == [0, 1, 2, 3, 0, 1, 2, 3]
    bad = nested.copy()
    bad[mem + 4:mem + 6] = [1, 0]
    assert call(bad) == 1                                   # member list not increasing
    bad = nested.copy()
    bad[g0 + 1:g0 + 3] = [1, 3]                             # root lists [1 2 3]: sequence 0 missing
    assert call(bad) == 1
    assert "missing from a group on its path" in ops.lib.pkv_last_error().decode()
    assert call(words, desc=_desc(ops, dtype=ops.PKV_F32)) == 2  # cascade needs bf16
    opts = ops.DecodeOpts(0, 0, 0, 0, words.ctypes.data, 16, words.size)
    ws = ops.lib.pkv_paged_attn_workspace_bytes(ctypes.byref(d), 4, 32, 256, ctypes.byref(opts))
    assert ws > 0  # the prefix partials live in the workspace
    assert _decode(ops, d, opts=opts, ws=16, ws_bytes=ws - 16) == 3


def test_prefix_values_f16_checks(ops):
    """Size of the fp16 copy of a plan's prefix values (pass blocks of every
    group, every kv head), and the argument checks of its maker and of the
    decode option, all before anything is launched."""
    import numpy as np

    d = _desc(ops)
    tables = np.tile(np.arange(16, dtype=np.int32), (4, 1))  # 4 sequences sharing 16 blocks (4 pass iterations)
    ctx = np.full(4, 256, dtype=np.int32)
    words = ops.plan_shared_prefix(tables, ctx, 16, 2, 1, device=None).host
    tile = 16 * 128 * 2  # one block of one kv head, fp16
    size = lambda w, desc=d: ops.lib.pkv_prefix_values_f16_bytes(ctypes.byref(desc), w.ctypes.data, w.size)
    assert size(words) == 16 * 8 * tile
    # nested: root over the first 8 blocks, two children over blocks 8..15 each
    t2 = tables.copy()
    t2[2:, 8:] += 100
    nested = ops.plan_shared_prefix(t2, ctx, 16, 2, 1, device=None).host
    assert size(nested) == (8 + 8 + 8) * 8 * tile
    assert size(words, _desc(ops, dtype=ops.PKV_F32)) == 0
    assert size(words, _desc(ops, head_dim=64)) == 0
    bad = words.copy()
    bad[0] = 0
    assert size(bad) == 0

    p = ctypes.c_void_p(16)
    need = 16 * 8 * tile

    def make(v=p, plan_dev=p, desc=d, out=p, out_bytes=need, w=words):
        return ops.lib.pkv_prefix_values_f16(v, p, 4, 16, ctypes.byref(desc), w.ctypes.data, plan_dev, w.size,
                                             out, out_bytes, None)
    assert make(plan_dev=None) == 1
    assert make(desc=_desc(ops, dtype=ops.PKV_F32)) == 2
    assert make(w=bad) == 1
    assert make(v=None) == 1
    assert make(out=ctypes.c_void_p(8)) == 1                 # misaligned
    assert make(out_bytes=need - 1) == 1
    assert "smaller than pkv_prefix_values_f16_bytes" in ops.lib.pkv_last_error().decode()

    def decode(vals, vbytes):
        opts = ops.DecodeOpts(0, 0, 0, 0, words.ctypes.data, 16, words.size, 0.0, 0, vals, vbytes)
        return _decode(ops, d, opts=opts, ws=16, ws_bytes=1 << 30)
    assert decode(16, need - 16) == 1                        # smaller than the plan's copy
    assert decode(8, need) == 1                              # misaligned
    assert "prefix_values_f16" in ops.lib.pkv_last_error().decode()


def test_swap_arguments(ops):
    d = _desc(ops)
    p = ctypes.c_void_p(16)
    other = _desc(ops, block_size=32)
    assert ops.lib.pkv_swap_blocks(p, p, ctypes.byref(d), p, p, ctypes.byref(other), p, 2, None) == 1  # shapes
    assert ops.lib.pkv_swap_blocks(p, p, ctypes.byref(d), p, p, ctypes.byref(d), p, -1, None) == 1
    assert ops.lib.pkv_swap_blocks(p, None, ctypes.byref(d), p, p, ctypes.byref(d), p, 2, None) == 1
    assert ops.lib.pkv_swap_blocks(p, p, ctypes.byref(d), p, p, ctypes.byref(d), p, 0, None) == 0


def _multi(ops, desc, num_heads=32, max_ctx=256, ptr=16, opts=None, out_dtype=None, ws=0, ws_bytes=0,
           max_blocks=16, scale=0.1, nseq=4, ntok=12, max_q=4):
    p = ctypes.c_void_p(ptr) if ptr else None
    od = desc.dtype if out_dtype is None else out_dtype
    return ops.lib.pkv_paged_attn_multi_token(p, p, p, p, p, p, nseq, num_heads, ntok, max_q, max_blocks, max_ctx,
                                              ctypes.byref(desc), scale, od, p, ctypes.c_void_p(ws) if ws else None,
                                              ws_bytes, ctypes.byref(opts) if opts else None, None)


def test_multi_token_arguments(ops):
    d = _desc(ops)
    single = ops.DecodeOpts(1 << 30, 0, 0)
    assert _multi(ops, d, num_heads=12, opts=single) == 1
    assert _multi(ops, d, ptr=0, opts=single) == 1
    assert _multi(ops, d, ptr=8, opts=single) == 1
    assert _multi(ops, d, scale=-1.0, opts=single) == 1
    assert _multi(ops, d, max_q=-1, opts=single) == 1
    assert _multi(ops, d, max_q=70000, opts=single) == 2
    assert _multi(ops, d, max_ctx=16 * 16 + 1, opts=single) == 1
    # the matrix-core kernel takes bf16 / head_dim 128; f32 runs on the vector kernel
    assert _multi(ops, _desc(ops, dtype=ops.PKV_F32), opts=ops.DecodeOpts(1 << 30, 2, 0)) == 2
    assert _multi(ops, _desc(ops, head_dim=64), opts=ops.DecodeOpts(1 << 30, 2, 0)) == 2
    # no shared-prefix plan, one kv head per workgroup, one block in flight for 32-row tiles
    plan = (ctypes.c_int32 * 8)()
    assert _multi(ops, d, opts=ops.DecodeOpts(1 << 30, 0, 0, 0, ctypes.addressof(plan), 16, 8)) == 2
    assert _multi(ops, d, opts=ops.DecodeOpts(1 << 30, 0, 0, 2)) == 2
    assert _multi(ops, d, max_q=5, opts=ops.DecodeOpts(1 << 30, 2, 2)) == 2  # 5 tokens x group 4 = 20 rows: 32-row tiles
    # vector kernel: one workgroup per (sequence, new token) within the grid's z range
    assert _multi(ops, d, nseq=300, max_q=300, opts=ops.DecodeOpts(1 << 30, 1, 0)) == 2
    # nothing to do
    assert _multi(ops, d, ntok=0, opts=single) == 0
    assert _multi(ops, d, nseq=0, opts=single) == 0


def test_multi_token_workspace(ops):
    d = _desc(ops)  # 8 kv heads, group 4
    opts = ops.DecodeOpts(64, 0, 0)
    # 3 new tokens x 4 heads = 12 rows: one 16-row tile; 4 partitions of 64 tokens
    need = ops.lib.pkv_paged_attn_multi_token_workspace_bytes(ctypes.byref(d), 4, 32, 12, 3, 256, ctypes.byref(opts))
    assert need == 12 * 32 * 4 * (128 + 2) * 4
    assert _multi(ops, d, opts=opts, max_q=3) == 3
    assert _multi(ops, d, opts=opts, max_q=3, ws=16, ws_bytes=need - 4) == 3
    single = ops.DecodeOpts(1 << 30, 0, 0)
    assert ops.lib.pkv_paged_attn_multi_token_workspace_bytes(ctypes.byref(d), 4, 32, 12, 3, 256,
                                                              ctypes.byref(single)) == 0


def test_tile_value_copy(ops):
    """The causal tiles' fp16 value copy is counted in the multi-token
    workspace: whole 64-token stages of every sequence's blocks, after the
    split-K partials at a 256-byte boundary.  tile_value_copy = -1 drops it;
    other values are rejected before any launch."""
    d = _desc(ops)  # 8 kv heads, group 4, 16-token blocks, head_dim 128

    def need(opts):
        return ops.lib.pkv_paged_attn_multi_token_workspace_bytes(ctypes.byref(d), 4, 32, 128, 32, 256,
                                                                  ctypes.byref(opts))

    # 4 sequences x 32 new tokens x group 4 = 128 rows per sequence: the tile kernel
    copy = 4 * 16 * 8 * (16 * 128 * 2)  # sequences x blocks (256 / 16, whole stages) x kv heads x tile bytes
    assert need(ops.DecodeOpts(1 << 30, 0, 0)) == copy
    assert need(ops.DecodeOpts(1 << 30, 3, 0, 0, None, None, 0, 0.0, -1)) == 0
    partials = 128 * 32 * 4 * (128 + 2) * 4  # 4 partitions of 64 tokens
    assert need(ops.DecodeOpts(64, 3, 0)) == (partials + 255) // 256 * 256 + copy
    assert need(ops.DecodeOpts(64, 3, 0, 0, None, None, 0, 0.0, -1)) == partials
    # fewer rows than the tile kernel's threshold: no tiles, no copy
    assert ops.lib.pkv_paged_attn_multi_token_workspace_bytes(ctypes.byref(d), 4, 32, 12, 3, 256,
                                                              ctypes.byref(ops.DecodeOpts(1 << 30, 0, 0))) == 0
    for v in (1, 2, -2):
        bad = ops.DecodeOpts(1 << 30, 3, 0, 0, None, None, 0, 0.0, v)
        assert need(bad) == 0
        assert _multi(ops, d, nseq=4, ntok=128, max_q=32, opts=bad) == 1
        assert "tile_value_copy" in ops.lib.pkv_last_error().decode()


def test_block_size_8(ops):
    """8-token blocks are accepted by the decode and multi-token kernels (the
    matrix-core ones walk them in pairs) and by the shared-prefix pass."""
    d = _desc(ops, block_size=8)
    single = ops.DecodeOpts(1 << 30, 0, 0)
    assert ops.lib.pkv_paged_attn_workspace_bytes(ctypes.byref(d), 4, 32, 256, ctypes.byref(single)) == 0
    # an explicit matrix-core request plans (a split makes the workspace nonzero)
    assert ops.lib.pkv_paged_attn_workspace_bytes(ctypes.byref(d), 4, 32, 256, ctypes.byref(ops.DecodeOpts(64, 2, 0))) > 0
    need = ops.lib.pkv_paged_attn_multi_token_workspace_bytes(ctypes.byref(d), 4, 32, 12, 3, 256,
                                                              ctypes.byref(ops.DecodeOpts(64, 2, 0)))
    assert need > 0
    plan = (ctypes.c_int32 * 22)(0x32564b50, 4, 8, 1, 16, 2, 16, 16, 0, 0, 0, 0, -1, -1, 16, 0, 2, 0, 0, -1, 0, 1)
    opts = ops.DecodeOpts(0, 0, 0, 0, ctypes.addressof(plan), 16, 22)
    assert _decode(ops, d, opts=opts, max_blocks=32) == 3  # plan accepted, stops at the workspace check
    assert "workspace" in ops.lib.pkv_last_error().decode()
