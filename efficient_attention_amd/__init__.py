"""MI355X-native (gfx950) Orthros attention hot path.

The compute lives in ``liborthros.so`` (hand-written HIP kernels behind a C ABI, declared in
``include/orthros.h``). ``efficient_attention_amd.orthros`` is a thin ctypes binding that
takes torch tensors for device memory and streams. Importing this package does not load the
library; the binding loads it on first use and raises if it is missing.
"""
__all__ = ["orthros", "synthetic"]
