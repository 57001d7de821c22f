"""MI355X-native low-rank compressed-KV decode (S4R-style).

The compute path is the C-ABI library ``libkvlr.so`` (hand-written HIP for
gfx950) declared in ``include/kvlr.h``; ``kvlr`` is its thin ctypes binding.
Importing this package does not load the library; ``kvlr.load()`` does, and
fails loudly when it has not been built.
"""
__all__ = ["configs", "synth", "kvlr"]
