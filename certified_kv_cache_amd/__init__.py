"""WitCert hot path on MI355X: HIP kernels behind the C ABI in include/witcert.h.

``certified_kv_cache_amd._lib`` is the ctypes binding of libwitcert.so (built by
``python -m certified_kv_cache_amd.build``); ``inputs`` synthesizes workloads.
Importing the binding fails loudly when the library has not been built.
"""
__all__ = ["inputs"]
