"""HARD-KV decode-time cascade-cache step on one AMD MI355X (gfx950).

The compute lives in ``libhardkv.so`` (HIP kernels behind a C ABI declared in
``include/hardkv.h``); ``decode_kv_cache_02_amd.hardkv`` is its ctypes binding.
"""

__all__ = ["hardkv"]
