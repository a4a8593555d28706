"""TurboQuant compressed KV cache for AMD Instinct MI355X.

The work happens in libtq.so (hand-written HIP for gfx950) behind a C ABI
(include/tq.h); ``kv_cache_vector_07_amd.tq`` is its ctypes binding and
``kv_cache_vector_07_amd.inputs`` the seeded synthetic workloads. Importing the
package does not load the library; the first binding call does, and fails
loudly if it has not been built (``python -m kv_cache_vector_07_amd.build``).
"""

__all__ = ["tq", "inputs"]
