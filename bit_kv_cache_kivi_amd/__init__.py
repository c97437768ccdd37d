"""Low-bit KV-cache quantization and fused decode attention for MI355X (gfx950).

The compute path is the HIP library ``libkvq.so`` (C-ABI in ``include/kvq.h``);
``bit_kv_cache_kivi_amd.kvq`` is its ctypes binding.  ``inputs`` draws the
seeded synthetic workloads.  Importing the package loads nothing native.
"""
__all__ = ["kvq", "inputs"]
