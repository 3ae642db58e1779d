"""MI355X-native attention over a block-paged KV cache.

The compute path is the C-ABI library ``libpkv.so`` (hand-written HIP for
gfx950, declared in ``include/pkv.h``).  ``paged_kv_cache_274_amd.ops`` is a
thin ctypes binding with the same call names; torch tensors supply device
memory and the current stream.  ``workloads`` builds seeded synthetic inputs.
"""

__all__ = ["kv_append", "paged_decode_attention", "paged_prefill_attention",
           "decode_workspace_bytes", "decode_num_splits"]


def __getattr__(name):
    if name in __all__:
        from . import ops
        return getattr(ops, name)
    raise AttributeError(name)
