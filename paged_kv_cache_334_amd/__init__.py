"""Paged KV-cache decode attention for AMD MI355X (gfx950).

The compute path lives in the HIP library ``libpkv.so`` (C ABI declared in
``include/pkv.h``).  ``paged_kv_cache_334_amd.ops`` is a thin ctypes binding
over it with the same entry-point names; it only marshals pointers, sizes and
the current HIP stream.  Importing the binding fails loudly when the library
has not been built.  ``paged_kv_cache_334_amd.workloads`` holds the seeded
synthetic inputs and host-side block bookkeeping.
"""

_OPS = {
    "paged_attn_decode",
    "paged_attn_workspace_bytes",
    "reshape_and_cache",
    "copy_blocks",
    "status_string",
    "lib",
}


def __getattr__(name):
    if name in _OPS:
        from . import ops

        return getattr(ops, name)
    raise AttributeError(name)
