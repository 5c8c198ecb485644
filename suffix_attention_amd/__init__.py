"""Replay attention over a captured, paged prompt KV cache on AMD MI355X (gfx950).

Every step runs in liblongstraw.so (hand-written HIP); `api` is the thin binding, `driver`
the serial group replay.  Importing this package does not load the library; the first
call does, and fails loudly if it has not been built.
"""
__all__ = ["api", "driver", "configs", "datagen"]
