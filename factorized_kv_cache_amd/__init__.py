"""Tensor Product Attention with a factorised KV cache, native to MI355X (gfx950).

The compute lives in libtpa.so (hand-written HIP kernels behind a C ABI,
declared in include/tpa.h); ``factorized_kv_cache_amd.tpa`` is its ctypes
binding.  Importing the binding requires the built library.
"""
