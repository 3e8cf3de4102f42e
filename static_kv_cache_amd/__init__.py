"""Static KV-cache decode for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libkvc.so`` (hand-written HIP
kernels, declared in ``include/kvc.h``); ``static_kv_cache_amd.kvc`` is a
thin ctypes binding over it (argument marshalling only). Importing this
package loads nothing; the library is opened on first use and the binding
raises if it has not been built.

``static_kv_cache_amd.synthetic`` holds the seeded input generators shared
by the tests and the benchmark; it contains none of the method's arithmetic.
"""

__all__ = ["kvc", "synthetic"]
