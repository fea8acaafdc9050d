"""HARD-KV decode-step compression + attention for MI355X (gfx950).

The hot path lives in libhardkv.so (hand-written HIP kernels behind the C
ABI in include/hardkv.h); ``hardkv`` is its ctypes binding and ``synth``
draws seeded synthetic inputs.  Importing this package loads nothing.
"""
__all__ = ["hardkv", "synth"]
