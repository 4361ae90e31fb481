"""libds4attn: one layer's compressed sparse attention step on MI355X (gfx950).

The compute lives in libds4attn.so (hand-written HIP); `ops` is a thin ctypes
binding.  Importing this package loads nothing; `ops.lib()` loads the library.
"""
__all__ = ["ops"]
