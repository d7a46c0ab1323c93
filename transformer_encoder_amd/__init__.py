"""MI355X (gfx950) ModernBERT-base encoder forward.

The compute lives in libmbert.so (hand-written HIP kernels behind the C ABI of
include/mbert.h); ``binding`` marshals arguments to it and ``model`` uploads weights and calls
the whole forward. Importing this package does not load the library; the first call does, and
raises if it has not been built.
"""
from . import binding  # noqa: F401

__all__ = ["binding"]
