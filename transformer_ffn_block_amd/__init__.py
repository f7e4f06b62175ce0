"""MI355X-native pre-norm SwiGLU FFN block.

The compute lives in a C-ABI HIP library (libffn.so, declared in
include/ffn.h); `ffn` is its thin ctypes binding and `inputs` the seeded
synthetic-input generator.  Importing the package loads nothing native:
`ffn.lib()` loads the library on first use and raises if it is missing.
"""
__all__ = ["ffn", "inputs"]
