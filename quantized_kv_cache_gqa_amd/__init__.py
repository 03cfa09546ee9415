"""Quantized-KV grouped-query decode attention with a fused risk meter (gfx950).

The compute path is the HIP library libkvq.so (include/kvq.h); ``kvq`` is its
ctypes binding.  Importing this package does not load the library; the first
call does, and fails loudly if it was not built.
"""
from . import kvq  # noqa: F401
