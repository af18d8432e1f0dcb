"""Paged KV-cache attention for AMD MI355X (gfx950).

The compute path is the HIP library ``libpa.so`` (sources in ``csrc/``,
C ABI declared in ``include/pa.h``).  ``paged_kv_cache_275_amd.ops`` is a thin
ctypes binding over it; importing this package does not load the library, the
first call into ``ops`` does, and fails loudly if it is missing.
"""
__all__ = ["ops", "workloads"]
