"""MI355X-native MLRA decode attention over a paged latent KV cache.

The compute lives in ``libmlra.so`` (HIP kernels for gfx950 behind a C ABI,
declared in ``include/mlra.h``); ``api`` marshals torch tensors into that ABI.
Importing this package does not load the library: the first call does, and
raises if the library has not been built.
"""
__all__ = ["configs", "inputs", "api"]
