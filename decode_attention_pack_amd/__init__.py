"""KIVI packed-KV decode attention for AMD Instinct MI355X (gfx950).

The compute lives in ``libkivi.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/kivi.h``).  ``decode_attention_pack_amd.kivi`` is the thin
ctypes binding over it; importing this package does not load the library.
"""
__all__ = ["kivi", "synth"]
