"""Chunkwise gated delta-rule attention (DeltaNet, Gated DeltaNet, KDA) for AMD MI355X.

The operator lives in a C-ABI shared library of hand-written HIP kernels for
gfx950 (``libdn.so``, declared in ``include/dn.h``).  ``binding`` is a thin
ctypes layer over it (argument marshalling only); ``workloads`` draws the
seeded synthetic inputs.  Importing this package loads nothing: the library is
opened on first use, and a missing or unbuilt library is an error, never a
fallback.
"""

__all__ = ["binding", "workloads"]
