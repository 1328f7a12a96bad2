"""GPU-side test helpers: upload a workload through the library's own cache ops,
download pools as raw bits, and the attention tolerance checks."""

import numpy as np
import torch

from paged_kv_cache_334_amd import ops
from paged_kv_cache_334_amd.workloads import BF16

POISON = {BF16: 0x7FC0, "f32": 0x7FC00000}


def to_device(bits, dtype, device="cuda"):
    bits = np.ascontiguousarray(bits)
    if dtype == BF16:
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(bits.view(np.float32)).to(device)


def to_bits(t):
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).reshape(-1)
    return t.view(torch.int32).numpy().view(np.uint32).reshape(-1)


class GpuWorkload:
    """Device copies of a workload's step: pools filled with NaN bits, then the
    cached tokens written, copy-on-write pairs copied and the new tokens written,
    all by the library (pkv_reshape_and_cache, pkv_copy_blocks)."""

    def __init__(self, wl, device="cuda"):
        s = wl.spec
        self.wl = wl
        tdt = torch.bfloat16 if s.dtype == BF16 else torch.float32
        self.k_pool, self.v_pool = ops.new_pools(wl.num_blocks, s.num_kv_heads, s.block_size, s.head_dim, tdt,
                                                 device, fill=POISON[s.dtype])
        self.q = to_device(wl.q, s.dtype, device)
        self.block_tables = torch.from_numpy(wl.block_tables).to(device)
        self.context_lens = torch.from_numpy(wl.context_lens).to(device)
        self.init_k = to_device(wl.init_k, s.dtype, device)
        self.init_v = to_device(wl.init_v, s.dtype, device)
        self.init_slots = torch.from_numpy(wl.init_slots).to(device)
        self.new_k = to_device(wl.new_k, s.dtype, device)
        self.new_v = to_device(wl.new_v, s.dtype, device)
        self.new_slots = torch.from_numpy(wl.new_slots).to(device)
        self.cow_pairs = torch.from_numpy(wl.cow_pairs.reshape(-1, 2)).to(device)
        self.query_start = torch.from_numpy(wl.query_start).to(device)
        if len(wl.init_slots):
            ops.reshape_and_cache(self.init_k, self.init_v, self.init_slots, self.k_pool, self.v_pool)
        self.step_cache_ops()
        torch.cuda.synchronize()

    def step_cache_ops(self):
        ops.copy_blocks(self.k_pool, self.v_pool, self.cow_pairs)
        if len(self.wl.new_slots):
            ops.reshape_and_cache(self.new_k, self.new_v, self.new_slots, self.k_pool, self.v_pool)

    def decode(self, **kw):
        kw.setdefault("max_context_len", self.wl.max_context)
        return ops.paged_attn_decode(self.q, self.k_pool, self.v_pool, self.block_tables, self.context_lens,
                                     self.wl.scale, **kw)


    def multi(self, **kw):
        kw.setdefault("max_context_len", self.wl.max_context)
        kw.setdefault("max_query_len", self.wl.max_query_len)
        return ops.paged_attn_multi_token(self.q, self.k_pool, self.v_pool, self.block_tables, self.context_lens,
                                          self.query_start, self.wl.scale, **kw)


def out_to_f64(out):
    return out.detach().float().cpu().numpy().astype(np.float64)


def check_attention(got, ref, dtype_in, dtype_out, label=""):
    """Tolerances for attention outputs against the float64 oracle.

    * float32 inputs: max abs error <= 1e-5.
    * bfloat16 inputs, float32 output: max abs <= 2e-3, and elementwise
      relative error <= 1e-2 wherever |ref| >= 1e-2.
    * bfloat16 inputs, bfloat16 output: |got - ref| <= 2e-3 + 1e-2 * |ref|
      elementwise (the output's own rounding costs up to 2^-9 relative).
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{label}: non-finite output"
    err = np.abs(got - ref)
    if dtype_in == "f32":
        assert err.max() <= 1e-5, f"{label}: max abs {err.max():.3g}"
        return float(err.max())
    if dtype_out == "f32":
        assert err.max() <= 2e-3, f"{label}: max abs {err.max():.3g}"
        big = np.abs(ref) >= 1e-2
        if big.any():
            rel = (err[big] / np.abs(ref[big])).max()
            assert rel <= 1e-2, f"{label}: max rel {rel:.3g}"
        return float(err.max())
    bound = 2e-3 + 1e-2 * np.abs(ref)
    worst = (err / bound).max()
    assert worst <= 1.0, f"{label}: error/bound {worst:.3g} (max abs {err.max():.3g})"
    return float(err.max())


def value_max(wl):
    """Largest |value| of the workload's finite cached and new values."""
    if wl.dtype != BF16:
        vals = [np.abs(np.asarray(a, np.float64)) for a in (wl.init_v, wl.new_v) if np.size(a)]
    else:
        vals = [np.abs((np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64))
                for a in (wl.init_v, wl.new_v) if np.size(a)]
    return max(float(np.nanmax(np.where(np.isfinite(v), v, 0.0))) for v in vals)


def check_fp16_path(got, ref, wl, label=""):
    """Bound for the fp16 path of the LDS-staged matrix-core kernel, float32
    output: each weight rounded to fp16 is off by at most 2^-11 of itself, or by
    2^-25 below fp16's normal range, and numerator and denominator use the same
    rounded weights, so an output element moves by at most that fraction of the
    weighted mean of |v - out|, itself at most max|v| + |out| (the weight sum
    is at least 1).  Plus 1e-5 for float32 accumulation and the merges."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.isfinite(got).all(), f"{label}: non-finite output"
    ntok = int(wl.context_lens.max())
    bound = (2.0 ** -11 * 1.001 + ntok * 2.0 ** -25) * (value_max(wl) + np.abs(ref)) + 1e-5
    worst = (np.abs(got - ref) / bound).max()
    assert worst <= 1.0, f"{label}: error/bound {worst:.3g} (max abs {np.abs(got - ref).max():.3g})"
    return float(worst)
