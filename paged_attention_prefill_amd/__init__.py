"""MI355X-native paged attention over a block-table KV cache.

The compute path lives in ``libpagedattn.so`` (hand-written HIP for gfx950,
C ABI declared in ``include/pagedattn.h``); ``paged_attention_prefill_amd.ops``
is the thin ctypes binding over it.  Importing this package loads nothing;
``ops`` loads the shared library on first use and raises if it is missing.
"""

__all__ = ["ops", "inputs", "workload"]
