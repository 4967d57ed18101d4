"""MiniMax Sparse Attention (MSA) forward path for AMD MI355X (gfx950).

The compute lives in ``libmsa.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/msa.h``).  ``ops`` is a thin ctypes binding over it
that marshals torch tensors (device pointers and the current HIP stream) and
nothing else; the library is loaded on the first op call, which raises if it
was not built.  ``accounting`` holds the algorithmic work counts.
"""
__all__ = ["accounting", "ops"]
