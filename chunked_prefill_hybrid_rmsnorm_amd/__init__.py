"""MI355X-native hybrid-batch decoder layer (chunked prefill + piggybacked decodes).

The compute lives in ``libhybrid_layer.so`` (hand-written HIP for gfx950,
C ABI declared in ``include/hybrid_layer.h``); ``binding`` is a thin ctypes
layer over it.  Importing this package does not load the library; the
binding loads it on first use and raises if it is missing.
"""

__all__ = ["inputs", "roofline", "binding"]
