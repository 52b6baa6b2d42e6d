"""MI355X-native hot path of Forcing-KV hybrid head-wise KV-cache compression.

The compute lives in ``libfkv.so`` (HIP kernels for gfx950 behind a C ABI,
declared in ``include/fkv.h``).  ``hybrid_kv_cache_amd.fkv`` is the thin
ctypes binding; importing this package itself loads nothing.
"""
