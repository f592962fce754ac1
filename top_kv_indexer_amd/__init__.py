"""MI355X (gfx950) HiSA hierarchical sparse selection, flat top-k indexer and
sparse local+pooled attention.

The compute lives in libhisa.so (HIP kernels behind the C ABI of
include/hisa.h); `hisa` is its Python binding and `synth` draws seeded
synthetic inputs.  Importing the package loads nothing.
"""
__all__ = ["hisa", "synth", "build"]
