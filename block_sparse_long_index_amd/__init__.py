"""MiniMax Sparse Attention (MSA) forward path for AMD MI355X (gfx950).

The compute lives in ``libmsa.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/msa.h``).  ``ops`` is a thin ctypes binding over it
that marshals torch tensors (device pointers and the current HIP stream) and
nothing else.  Importing this package does not load the library; the first
op call does, and raises if it was not built.
"""
from . import accounting  # noqa: F401

__all__ = ["accounting", "ops"]


def __getattr__(name):
    if name == "ops":
        from . import ops
        return ops
    raise AttributeError(name)
