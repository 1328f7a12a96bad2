"""ctypes binding of libpkv (C ABI in include/pkv.h), same entry-point names.

Argument marshalling only: tensors become device pointers, shapes become the
pool descriptor, and the current HIP stream of torch is passed through.  Every
step of the computation runs in the library's kernels.  Importing this module
raises ImportError when libpkv.so has not been built (``python -m
paged_kv_cache_334_amd.build``); there is no fallback.

Pool tensors use the library layout: keys ``[N, Hkv, D/x, bs, x]`` and values
``[N, Hkv, D, bs]`` with ``x = 16 / element bytes`` (see ``new_pools``).
"""

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m paged_kv_cache_334_amd.build`")
lib = ctypes.CDLL(_LIB_PATH)

PKV_F32, PKV_BF16 = 0, 1
KERNELS = {"auto": 0, "vector": 1, "mfma": 2, "tile": 3}
STATUS = {0: "PKV_OK", 1: "PKV_EINVAL", 2: "PKV_EUNSUPPORTED", 3: "PKV_EWORKSPACE", 4: "PKV_EHIP", 5: "PKV_ENOSPACE"}


class PoolDesc(ctypes.Structure):
    _fields_ = [
        ("num_blocks", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


class DecodeOpts(ctypes.Structure):
    _fields_ = [
        ("partition_tokens", ctypes.c_int32),
        ("kernel", ctypes.c_int32),
        ("blocks_in_flight", ctypes.c_int32),
        ("heads_per_workgroup", ctypes.c_int32),
        ("prefix_plan", ctypes.c_void_p),
        ("prefix_plan_dev", ctypes.c_void_p),
        ("prefix_plan_words", ctypes.c_size_t),
        ("min_eff_tokens", ctypes.c_float),
        ("tile_value_copy", ctypes.c_int32),
        ("prefix_values_f16", ctypes.c_void_p),
        ("prefix_values_f16_bytes", ctypes.c_size_t),
    ]


_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
lib.pkv_paged_attn_workspace_bytes.restype = _sz
lib.pkv_paged_attn_workspace_bytes.argtypes = [ctypes.POINTER(PoolDesc), _i32, _i32, _i32, ctypes.POINTER(DecodeOpts)]
lib.pkv_prefix_values_f16_bytes.restype = _sz
lib.pkv_prefix_values_f16_bytes.argtypes = [ctypes.POINTER(PoolDesc), _vp, _sz]
lib.pkv_prefix_values_f16.restype = _i32
lib.pkv_prefix_values_f16.argtypes = [_vp, _vp, _i32, _i32, ctypes.POINTER(PoolDesc), _vp, _vp, _sz, _vp, _sz, _vp]
lib.pkv_paged_attn_decode.restype = _i32
lib.pkv_paged_attn_decode.argtypes = [
    _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, ctypes.POINTER(PoolDesc), ctypes.c_float, _i32, _vp, _vp, _sz,
    ctypes.POINTER(DecodeOpts), _vp,
]
lib.pkv_paged_attn_decode_noalloc.restype = _i32
lib.pkv_paged_attn_decode_noalloc.argtypes = [
    _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, ctypes.POINTER(PoolDesc), ctypes.c_float, _i32, _vp,
    ctypes.POINTER(DecodeOpts), _vp,
]
lib.pkv_paged_attn_decode_scratch_limit.restype = _sz
lib.pkv_paged_attn_decode_scratch_limit.argtypes = []
lib.pkv_paged_attn_multi_token_workspace_bytes.restype = _sz
lib.pkv_paged_attn_multi_token_workspace_bytes.argtypes = [ctypes.POINTER(PoolDesc), _i32, _i32, _i32, _i32, _i32,
                                                           ctypes.POINTER(DecodeOpts)]
lib.pkv_paged_attn_multi_token.restype = _i32
lib.pkv_paged_attn_multi_token.argtypes = [
    _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(PoolDesc), ctypes.c_float, _i32,
    _vp, _vp, _sz, ctypes.POINTER(DecodeOpts), _vp,
]
lib.pkv_reshape_and_cache.restype = _i32
lib.pkv_reshape_and_cache.argtypes = [_vp, _vp, _i64, _i64, _vp, _i32, _vp, _vp, ctypes.POINTER(PoolDesc), _vp]
lib.pkv_copy_blocks.restype = _i32
lib.pkv_copy_blocks.argtypes = [_vp, _vp, _vp, _i32, ctypes.POINTER(PoolDesc), _vp]
lib.pkv_swap_blocks.restype = _i32
lib.pkv_swap_blocks.argtypes = [_vp, _vp, ctypes.POINTER(PoolDesc), _vp, _vp, ctypes.POINTER(PoolDesc), _vp, _i32, _vp]
lib.pkv_plan_shared_prefix.restype = _sz
lib.pkv_plan_shared_prefix.argtypes = [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _sz]
_bm = ctypes.c_void_p
_i32p = ctypes.POINTER(ctypes.c_int32)
for _name, _res, _args in [
    ("pkv_bm_create", _bm, [_i32, _i32, _vp]),
    ("pkv_bm_destroy", None, [_bm]),
    ("pkv_bm_last_error", ctypes.c_char_p, [_bm]),
    ("pkv_bm_num_free", _i32, [_bm]),
    ("pkv_bm_ref_count", _i32, [_bm, _i32]),
    ("pkv_bm_num_cached", _i32, [_bm]),
    ("pkv_bm_add_sequence", _i32, [_bm, _i64]),
    ("pkv_bm_add_sequence_cached", _i32, [_bm, _i64, _vp, _i32, _i32p]),
    ("pkv_bm_fork", _i32, [_bm, _i64, _i64]),
    ("pkv_bm_append_tokens", _i32, [_bm, _i64, _i32, _vp, _vp]),
    ("pkv_bm_take_copies", _i32, [_bm, _vp, _i32]),
    ("pkv_bm_free_sequence", _i32, [_bm, _i64]),
    ("pkv_bm_sequence_length", _i32, [_bm, _i64]),
    ("pkv_bm_block_table", _i32, [_bm, _i64, _vp, _i32]),
    ("pkv_bm_export_batch", _i32, [_bm, _vp, _i32, _i32, _i32, _vp, _vp]),
]:
    getattr(lib, _name).restype = _res
    getattr(lib, _name).argtypes = _args
lib.pkv_status_string.restype = ctypes.c_char_p
lib.pkv_status_string.argtypes = [_i32]
lib.pkv_last_error.restype = ctypes.c_char_p
lib.pkv_last_error.argtypes = []
lib.pkv_version.restype = _i32
lib.pkv_version.argtypes = []


class PkvError(RuntimeError):
    def __init__(self, status: int, where: str):
        detail = lib.pkv_last_error().decode()
        super().__init__(f"{where}: {STATUS.get(status, status)} ({detail})")
        self.status = status


def status_string(status: int) -> str:
    return lib.pkv_status_string(status).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise PkvError(status, where)


def _elem(t: torch.Tensor) -> int:
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return PKV_BF16
    if t.dtype in (torch.float32, torch.int32):
        return PKV_F32
    raise TypeError(f"unsupported element type {t.dtype}")


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t):
    return None if t is None else t.data_ptr()


def pool_desc(k_pool: torch.Tensor, v_pool: torch.Tensor) -> PoolDesc:
    """Descriptor from pool tensors shaped ``[N, Hkv, D/x, bs, x]`` and ``[N, Hkv, D, bs]``."""
    if k_pool.dim() != 5 or v_pool.dim() != 4:
        raise ValueError("k_pool must be [N, Hkv, D/x, bs, x] and v_pool [N, Hkv, D, bs]")
    n, hkv, dx, bs, x = k_pool.shape
    if tuple(v_pool.shape) != (n, hkv, dx * x, bs) or k_pool.dtype != v_pool.dtype:
        raise ValueError("key and value pools disagree")
    if not (k_pool.is_contiguous() and v_pool.is_contiguous()):
        raise ValueError("pools must be contiguous")
    dt = _elem(k_pool)
    if x * (2 if dt == PKV_BF16 else 4) != 16:
        raise ValueError("last key-pool axis must hold 16 bytes")
    return PoolDesc(n, hkv, bs, dx * x, dt)


def new_pools(num_blocks, num_kv_heads, block_size, head_dim, dtype=torch.bfloat16, device="cuda", fill=None):
    """Allocate key/value pools in the library layout (torch allocates; the
    library never does).  ``fill`` is an optional raw bit pattern."""
    x = 16 // torch.tensor([], dtype=dtype).element_size()
    k = torch.empty((num_blocks, num_kv_heads, head_dim // x, block_size, x), dtype=dtype, device=device)
    v = torch.empty((num_blocks, num_kv_heads, head_dim, block_size), dtype=dtype, device=device)
    if fill is not None:
        bits = torch.int16 if dtype == torch.bfloat16 else torch.int32
        val = fill - (1 << 16) if (bits == torch.int16 and fill >= 1 << 15) else fill
        k.view(bits).fill_(val)
        v.view(bits).fill_(val)
    return k, v


class PrefixPlan:
    """Plan words of pkv_plan_shared_prefix: ``host`` (a NumPy int32 array the
    library reads during each call) and ``dev`` (their device copy, read by the
    kernels).  ``groups`` is the number of shared-prefix groups found."""

    def __init__(self, host, dev):
        self.host = host
        self.dev = dev

    @property
    def groups(self) -> int:
        return int(self.host[3])

    def prefix_blocks(self):
        """Blocks of each sequence covered by a shared prefix (its deepest
        group's, 0 = none)."""
        n = int(self.host[1])
        return self.host[6:6 + n]

    def group_of(self):
        """Deepest shared-prefix group of each sequence (-1 = none)."""
        n = int(self.host[1])
        return self.host[6 + n:6 + 2 * n]


def plan_shared_prefix(block_tables, context_lens, block_size, min_group_seqs=4, min_prefix_blocks=8,
                       device="cuda") -> PrefixPlan:
    """Find sequences sharing a block-table prefix.  ``block_tables`` and
    ``context_lens`` are host (NumPy or CPU tensor) int32 arrays."""
    import numpy as np

    bt = np.ascontiguousarray(np.asarray(block_tables.cpu() if hasattr(block_tables, "cpu") else block_tables),
                              dtype=np.int32)
    cl = np.ascontiguousarray(np.asarray(context_lens.cpu() if hasattr(context_lens, "cpu") else context_lens),
                              dtype=np.int32)
    nseq, mb = bt.shape
    if cl.shape != (nseq,):
        raise ValueError("context_lens does not match block_tables")
    args = (bt.ctypes.data, cl.ctypes.data, nseq, mb, block_size, min_group_seqs, min_prefix_blocks)
    need = int(lib.pkv_plan_shared_prefix(*args, None, 0))
    if need == 0:
        raise ValueError("pkv_plan_shared_prefix rejected its arguments")
    host = np.zeros(need, dtype=np.int32)
    got = int(lib.pkv_plan_shared_prefix(*args, host.ctypes.data, need))
    if got != need:
        raise RuntimeError("plan size changed between calls")
    dev = torch.from_numpy(host).to(device) if device is not None else None
    return PrefixPlan(host, dev)


def _opts(partition_tokens, kernel, blocks_in_flight, prefix_plan, heads_per_workgroup=0, min_eff_tokens=0.0,
          tile_value_copy=0, prefix_values=None):
    base = (int(partition_tokens), KERNELS[kernel], int(blocks_in_flight), int(heads_per_workgroup))
    vals = (None, 0) if prefix_values is None else (_ptr(prefix_values),
                                                     prefix_values.numel() * prefix_values.element_size())
    if prefix_plan is None:
        return DecodeOpts(*base, None, None, 0, float(min_eff_tokens), int(tile_value_copy), *vals)
    return DecodeOpts(*base, prefix_plan.host.ctypes.data, _ptr(prefix_plan.dev), prefix_plan.host.size,
                      float(min_eff_tokens), int(tile_value_copy), *vals)


def prefix_values_f16_bytes(k_pool, v_pool, prefix_plan) -> int:
    """Bytes of the fp16 copy of the plan's shared-prefix values (0: none)."""
    desc = pool_desc(k_pool, v_pool)
    return int(lib.pkv_prefix_values_f16_bytes(ctypes.byref(desc), prefix_plan.host.ctypes.data,
                                               prefix_plan.host.size))


def prefix_values_f16(k_pool, v_pool, block_tables, prefix_plan, out=None, stream=None):
    """The fp16 copy of the plan's shared-prefix values (pkv_prefix_values_f16),
    for ``prefix_values=`` of the decode calls: made once per plan and reused
    while the plan and the prefix blocks do not change.  Returns the uint8
    device tensor, or None when the plan has no pass blocks."""
    desc = pool_desc(k_pool, v_pool)
    if block_tables.dtype != torch.int32 or not block_tables.is_contiguous():
        raise TypeError("block_tables must be contiguous int32")
    need = prefix_values_f16_bytes(k_pool, v_pool, prefix_plan)
    if need == 0:
        return None
    if out is None:
        out = torch.empty(need, dtype=torch.uint8, device=v_pool.device)
    nseq, mb = block_tables.shape
    st = lib.pkv_prefix_values_f16(_ptr(v_pool), _ptr(block_tables), nseq, mb, ctypes.byref(desc),
                                   prefix_plan.host.ctypes.data, _ptr(prefix_plan.dev), prefix_plan.host.size,
                                   _ptr(out), out.numel() * out.element_size(), _stream(stream))
    _check(st, "pkv_prefix_values_f16")
    return out


def paged_attn_workspace_bytes(k_pool, v_pool, num_seqs, num_heads, max_context_len, partition_tokens=0,
                               kernel="auto", blocks_in_flight=0, prefix_plan=None, heads_per_workgroup=0,
                               min_eff_tokens=0.0) -> int:
    desc = pool_desc(k_pool, v_pool)
    opts = _opts(partition_tokens, kernel, blocks_in_flight, prefix_plan, heads_per_workgroup, min_eff_tokens)
    return int(lib.pkv_paged_attn_workspace_bytes(ctypes.byref(desc), num_seqs, num_heads, max_context_len,
                                                  ctypes.byref(opts)))


def paged_attn_decode(q, k_pool, v_pool, block_tables, context_lens, scale, out=None, max_context_len=None,
                      workspace=None, partition_tokens=0, kernel="auto", out_dtype=None, stream=None,
                      blocks_in_flight=0, prefix_plan=None, heads_per_workgroup=0, min_eff_tokens=0.0,
                      prefix_values=None):
    """``out[b, h] = softmax(scale * q[b, h] . K^T) . V`` over sequence b's
    paged keys/values.  ``q`` is ``[B, Hq, D]``; ``block_tables`` ``[B, max_blocks]``
    int32; ``context_lens`` ``[B]`` int32.  ``max_context_len`` is a host-side
    upper bound (default ``max_blocks * block_size``).  Allocates ``out`` and the
    workspace with torch when they are not given."""
    desc = pool_desc(k_pool, v_pool)
    nseq, nh, hd = q.shape
    if hd != desc.head_dim or _elem(q) != desc.dtype:
        raise ValueError("q does not match the pools")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    if not (q.is_contiguous() and block_tables.is_contiguous() and context_lens.is_contiguous()):
        raise ValueError("q, block_tables and context_lens must be contiguous")
    max_blocks = block_tables.shape[1]
    if max_context_len is None:
        max_context_len = max_blocks * desc.block_size
    if out is None:
        odt = q.dtype if out_dtype is None else out_dtype
        out = torch.empty((nseq, nh, hd), dtype=odt, device=q.device)
    odt_code = PKV_BF16 if out.dtype == torch.bfloat16 else PKV_F32
    opts = _opts(partition_tokens, kernel, blocks_in_flight, prefix_plan, heads_per_workgroup, min_eff_tokens,
                 prefix_values=prefix_values)
    need = int(lib.pkv_paged_attn_workspace_bytes(ctypes.byref(desc), nseq, nh, int(max_context_len),
                                                  ctypes.byref(opts)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.pkv_paged_attn_decode(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), _ptr(context_lens), nseq,
                                   nh, max_blocks, int(max_context_len), ctypes.byref(desc), float(scale), odt_code,
                                   _ptr(out), _ptr(workspace), ws_bytes, ctypes.byref(opts), _stream(stream))
    _check(st, "pkv_paged_attn_decode")
    return out


def paged_attn_decode_noalloc(q, k_pool, v_pool, block_tables, context_lens, scale, out, max_context_len=None,
                              partition_tokens=0, kernel="auto", stream=None, blocks_in_flight=0, prefix_plan=None,
                              heads_per_workgroup=0, min_eff_tokens=0.0, prefix_values=None):
    """``paged_attn_decode`` through pkv_paged_attn_decode_noalloc: no workspace
    argument, nothing allocated (``out`` must be given); the partials go to the
    library's per-GPU scratch array.  Calls must not overlap on one GPU."""
    desc = pool_desc(k_pool, v_pool)
    nseq, nh, hd = q.shape
    if hd != desc.head_dim or _elem(q) != desc.dtype:
        raise ValueError("q does not match the pools")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    if not (q.is_contiguous() and block_tables.is_contiguous() and context_lens.is_contiguous()):
        raise ValueError("q, block_tables and context_lens must be contiguous")
    if tuple(out.shape) != (nseq, nh, hd) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, Hq, D] tensor")
    max_blocks = block_tables.shape[1]
    if max_context_len is None:
        max_context_len = max_blocks * desc.block_size
    odt_code = PKV_BF16 if out.dtype == torch.bfloat16 else PKV_F32
    opts = _opts(partition_tokens, kernel, blocks_in_flight, prefix_plan, heads_per_workgroup, min_eff_tokens,
                 prefix_values=prefix_values)
    st = lib.pkv_paged_attn_decode_noalloc(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
                                           _ptr(context_lens), nseq, nh, max_blocks, int(max_context_len),
                                           ctypes.byref(desc), float(scale), odt_code, _ptr(out), ctypes.byref(opts),
                                           _stream(stream))
    _check(st, "pkv_paged_attn_decode_noalloc")
    return out


def paged_attn_decode_scratch_limit() -> int:
    return int(lib.pkv_paged_attn_decode_scratch_limit())


def paged_attn_multi_token_workspace_bytes(k_pool, v_pool, num_seqs, num_heads, num_query_tokens, max_query_len,
                                           max_context_len, partition_tokens=0, kernel="auto",
                                           blocks_in_flight=0, min_eff_tokens=0.0, tile_value_copy=0) -> int:
    desc = pool_desc(k_pool, v_pool)
    opts = _opts(partition_tokens, kernel, blocks_in_flight, None, 0, min_eff_tokens, tile_value_copy)
    return int(lib.pkv_paged_attn_multi_token_workspace_bytes(ctypes.byref(desc), num_seqs, num_heads,
                                                              num_query_tokens, max_query_len, max_context_len,
                                                              ctypes.byref(opts)))


def paged_attn_multi_token(q, k_pool, v_pool, block_tables, context_lens, query_start, scale, max_query_len,
                           out=None, max_context_len=None, workspace=None, partition_tokens=0, kernel="auto",
                           out_dtype=None, stream=None, blocks_in_flight=0, min_eff_tokens=0.0, tile_value_copy=0):
    """Several new tokens per sequence, causal among them: row
    ``query_start[b] + i`` of ``q [T, Hq, D]`` (new token i of sequence b, at
    position ``context_lens[b] - n_b + i``) attends over the sequence's tokens up
    to and including itself.  ``query_start [B+1]`` int32 on the device;
    ``max_query_len`` is the host bound of ``n_b``."""
    desc = pool_desc(k_pool, v_pool)
    ntok, nh, hd = q.shape
    nseq = query_start.shape[0] - 1
    if hd != desc.head_dim or _elem(q) != desc.dtype:
        raise ValueError("q does not match the pools")
    for t in (block_tables, context_lens, query_start):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise TypeError("block_tables, context_lens and query_start must be contiguous int32")
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    if block_tables.shape[0] != nseq or context_lens.shape[0] != nseq:
        raise ValueError("block_tables, context_lens and query_start disagree on the number of sequences")
    max_blocks = block_tables.shape[1]
    if max_context_len is None:
        max_context_len = max_blocks * desc.block_size
    if out is None:
        odt = q.dtype if out_dtype is None else out_dtype
        out = torch.empty((ntok, nh, hd), dtype=odt, device=q.device)
    odt_code = PKV_BF16 if out.dtype == torch.bfloat16 else PKV_F32
    opts = _opts(partition_tokens, kernel, blocks_in_flight, None, 0, min_eff_tokens, tile_value_copy)
    need = int(lib.pkv_paged_attn_multi_token_workspace_bytes(ctypes.byref(desc), nseq, nh, ntok, int(max_query_len),
                                                              int(max_context_len), ctypes.byref(opts)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.pkv_paged_attn_multi_token(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), _ptr(context_lens),
                                        _ptr(query_start), nseq, nh, ntok, int(max_query_len), max_blocks,
                                        int(max_context_len), ctypes.byref(desc), float(scale), odt_code, _ptr(out),
                                        _ptr(workspace), ws_bytes, ctypes.byref(opts), _stream(stream))
    _check(st, "pkv_paged_attn_multi_token")
    return out


def reshape_and_cache(k, v, slot_mapping, k_pool, v_pool, stream=None):
    """Write ``k, v [T, Hkv, D]`` (token axis may be strided) into the pools at
    ``slot_mapping [T]`` int32 (negative = skip)."""
    desc = pool_desc(k_pool, v_pool)
    if slot_mapping.dtype != torch.int32 or not slot_mapping.is_contiguous():
        raise TypeError("slot_mapping must be contiguous int32")
    t = k.shape[0]
    for x in (k, v):
        if x.dim() != 3 or x.shape[1:] != (desc.num_kv_heads, desc.head_dim) or _elem(x) != desc.dtype:
            raise ValueError("k/v must be [T, Hkv, D] of the pool's element type")
        if x.stride(2) != 1 or x.stride(1) != desc.head_dim:
            raise ValueError("k/v rows must be dense within a token")
    if v.shape[0] != t or slot_mapping.shape[0] != t:
        raise ValueError("k, v and slot_mapping lengths differ")
    st = lib.pkv_reshape_and_cache(_ptr(k), _ptr(v), k.stride(0), v.stride(0), _ptr(slot_mapping), t, _ptr(k_pool),
                                   _ptr(v_pool), ctypes.byref(desc), _stream(stream))
    _check(st, "pkv_reshape_and_cache")


def copy_blocks(k_pool, v_pool, src_dst_pairs, stream=None):
    """Copy whole blocks of both pools: ``src_dst_pairs [P, 2]`` int32 on the device."""
    desc = pool_desc(k_pool, v_pool)
    if src_dst_pairs.dtype != torch.int32 or not src_dst_pairs.is_contiguous():
        raise TypeError("src_dst_pairs must be contiguous int32")
    p = src_dst_pairs.shape[0] if src_dst_pairs.numel() else 0
    st = lib.pkv_copy_blocks(_ptr(k_pool), _ptr(v_pool), _ptr(src_dst_pairs) if p else None, p, ctypes.byref(desc),
                             _stream(stream))
    _check(st, "pkv_copy_blocks")


def swap_blocks(src_k_pool, src_v_pool, dst_k_pool, dst_v_pool, src_dst_pairs, stream=None):
    """Copy whole blocks from one pool to another of the same shape (e.g. a
    device pool and a pool in pinned host memory): ``src_dst_pairs [P, 2]`` int32,
    device or pinned host."""
    src = pool_desc(src_k_pool, src_v_pool)
    dst = pool_desc(dst_k_pool, dst_v_pool)
    for t in (src_k_pool, src_v_pool, dst_k_pool, dst_v_pool, src_dst_pairs):
        if not t.is_cuda and not t.is_pinned():
            raise ValueError("host-side pools and pairs must be pinned (pin_memory=True) so the device can reach them")
    if src_dst_pairs.dtype != torch.int32 or not src_dst_pairs.is_contiguous():
        raise TypeError("src_dst_pairs must be contiguous int32")
    p = src_dst_pairs.shape[0] if src_dst_pairs.numel() else 0
    st = lib.pkv_swap_blocks(_ptr(src_k_pool), _ptr(src_v_pool), ctypes.byref(src), _ptr(dst_k_pool),
                             _ptr(dst_v_pool), ctypes.byref(dst), _ptr(src_dst_pairs) if p else None, p,
                             _stream(stream))
    _check(st, "pkv_swap_blocks")


# measurement kernels (include/pkv_probe.h)
lib.pkv_probe_read.restype = _i32
lib.pkv_probe_read.argtypes = [_vp, _sz, _vp, _i32, _vp]
lib.pkv_probe_gather.restype = _i32
lib.pkv_probe_gather.argtypes = [_vp, _vp, _i32, _i32, _vp, _i32, _vp]
lib.pkv_probe_copy.restype = _i32
lib.pkv_probe_copy.argtypes = [_vp, _vp, _sz, _i32, _vp]


def _probe_check(st, where):
    if st != 0:
        raise RuntimeError(f"{where} returned {st}")


def probe_read(buf, sink, num_workgroups, stream=None):
    """Stream ``buf`` (any contiguous device tensor) once; ``sink`` holds
    ``num_workgroups`` 32-bit words."""
    _probe_check(lib.pkv_probe_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), num_workgroups,
                                    _stream(stream)), "pkv_probe_read")


def probe_gather(pool, tile_ids, tile_bytes, sink, num_workgroups, stream=None):
    """Read ``tile_ids.numel()`` tiles of ``tile_bytes`` from ``pool``."""
    _probe_check(lib.pkv_probe_gather(_ptr(pool), _ptr(tile_ids), tile_ids.numel(), tile_bytes, _ptr(sink),
                                      num_workgroups, _stream(stream)), "pkv_probe_gather")


def probe_copy(src, dst, num_workgroups, stream=None):
    """Copy ``src`` into ``dst`` (same byte size)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst sizes differ")
    _probe_check(lib.pkv_probe_copy(_ptr(src), _ptr(dst), nbytes, num_workgroups, _stream(stream)), "pkv_probe_copy")


class BlockManagerError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {STATUS.get(status, status)} ({detail})")
        self.status = status


class BlockManager:
    """Native host block manager (pkv_bm_* in include/pkv.h): free list,
    block tables, reference counts, copy-on-write and the prefix cache.  Host
    memory only; sequence ids are Python ints."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        import numpy as np

        self.num_blocks, self.block_size = int(num_blocks), int(block_size)
        order = None
        if free_order is not None:
            order = np.ascontiguousarray(np.asarray(free_order, dtype=np.int32))
        self._destroy = lib.pkv_bm_destroy  # kept: module globals may be gone when __del__ runs at exit
        self._h = lib.pkv_bm_create(self.num_blocks, self.block_size, None if order is None else order.ctypes.data)
        if not self._h:
            raise ValueError("pkv_bm_create rejected its arguments")

    def close(self):
        if getattr(self, "_h", None):
            self._destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def _check(self, st, where):
        if st != 0:
            raise BlockManagerError(st, where, lib.pkv_bm_last_error(self._h).decode())

    @property
    def num_free(self) -> int:
        return int(lib.pkv_bm_num_free(self._h))

    @property
    def num_cached(self) -> int:
        return int(lib.pkv_bm_num_cached(self._h))

    def ref_count(self, block: int) -> int:
        return int(lib.pkv_bm_ref_count(self._h, int(block)))

    def allocate_sequence(self, seq: int) -> None:
        self._check(lib.pkv_bm_add_sequence(self._h, int(seq)), "pkv_bm_add_sequence")

    def allocate_sequence_cached(self, seq: int, prompt_tokens) -> int:
        """Start ``seq`` from a prompt, sharing cached full blocks; returns the
        number of leading prompt tokens they cover."""
        import numpy as np

        toks = np.ascontiguousarray(np.asarray(prompt_tokens, dtype=np.int32))
        cached = ctypes.c_int32(0)
        self._check(lib.pkv_bm_add_sequence_cached(self._h, int(seq), toks.ctypes.data if toks.size else None,
                                                   toks.size, ctypes.byref(cached)), "pkv_bm_add_sequence_cached")
        return int(cached.value)

    def fork(self, parent: int, child: int) -> None:
        self._check(lib.pkv_bm_fork(self._h, int(parent), int(child)), "pkv_bm_fork")

    def append_slots(self, seq: int, num_tokens: int = None, token_ids=None):
        """Slots of the next tokens of ``seq`` (int32 array)."""
        import numpy as np

        ids = None
        if token_ids is not None:
            ids = np.ascontiguousarray(np.asarray(token_ids, dtype=np.int32))
            num_tokens = ids.size if num_tokens is None else num_tokens
            if ids.size != num_tokens:
                raise ValueError("token_ids length differs from num_tokens")
        slots = np.empty(int(num_tokens), dtype=np.int32)
        self._check(lib.pkv_bm_append_tokens(self._h, int(seq), int(num_tokens),
                                             None if ids is None or ids.size == 0 else ids.ctypes.data,
                                             slots.ctypes.data if slots.size else None), "pkv_bm_append_tokens")
        return slots

    def append_slot(self, seq: int) -> int:
        return int(self.append_slots(seq, 1)[0])

    def take_copies(self):
        """Queued copy-on-write pairs as an int32 array [P, 2] (clears the queue)."""
        import numpy as np

        n = int(lib.pkv_bm_take_copies(self._h, None, 0))
        pairs = np.empty((n, 2), dtype=np.int32)
        if n:
            got = int(lib.pkv_bm_take_copies(self._h, pairs.ctypes.data, n))
            if got != n:
                raise RuntimeError("copy queue changed during take_copies")
        else:
            lib.pkv_bm_take_copies(self._h, pairs.ctypes.data, 0)
        return pairs

    def free_sequence(self, seq: int) -> None:
        self._check(lib.pkv_bm_free_sequence(self._h, int(seq)), "pkv_bm_free_sequence")

    def length(self, seq: int) -> int:
        n = int(lib.pkv_bm_sequence_length(self._h, int(seq)))
        if n < 0:
            raise KeyError(seq)
        return n

    def block_table(self, seq: int):
        import numpy as np

        n = int(lib.pkv_bm_block_table(self._h, int(seq), None, 0))
        if n < 0:
            raise KeyError(seq)
        out = np.empty(n, dtype=np.int32)
        if n:
            lib.pkv_bm_block_table(self._h, int(seq), out.ctypes.data, n)
        return out

    def export_batch(self, seqs, max_blocks_per_seq: int = None, pad: int = -1):
        """(block_tables [B, max_blocks], context_lens [B]) int32 host arrays."""
        import numpy as np

        ids = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        if max_blocks_per_seq is None:
            max_blocks_per_seq = max([1] + [len(self.block_table(s)) for s in ids.tolist()])
        tables = np.empty((ids.size, int(max_blocks_per_seq)), dtype=np.int32)
        lens = np.empty(ids.size, dtype=np.int32)
        self._check(lib.pkv_bm_export_batch(self._h, ids.ctypes.data if ids.size else None, ids.size,
                                            int(max_blocks_per_seq), int(pad),
                                            tables.ctypes.data if ids.size else None,
                                            lens.ctypes.data if ids.size else None), "pkv_bm_export_batch")
        return tables, lens
