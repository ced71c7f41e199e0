"""MI355X-native hot path of Decode Context Parallelism (DCP).

The computation lives in ``libdcp.so`` (C ABI, ``include/dcp.h``), built from
the HIP sources in ``csrc/``.  ``kv_cache_context_amd.dcp`` is the ctypes
binding with the same names; ``kv_cache_context_amd.ops`` adds tensor-level
argument checking on top of it.
"""
from . import dcp  # noqa: F401
