"""FP8 (e4m3) paged decode attention for MI355X (gfx950).

The compute lives in ``libpafp8.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/pafp8.h``); ``paged_attention_fp8_amd.ops`` is a thin
ctypes binding that passes torch tensors' device pointers and the current
stream through.  Importing this package does not load the library; the first
call does, and fails loudly if it has not been built.
"""
__all__ = ["inputs", "ops"]
