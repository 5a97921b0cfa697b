"""MI355X-native CSA2 decode over an FP4 global KV cache.

The compute path is the HIP library ``libcsa2.so`` (C ABI declared in
``include/csa2.h``); ``fp4_kv_cache_decode_amd.csa2`` is its thin ctypes
binding.  Nothing is loaded at import time.
"""
