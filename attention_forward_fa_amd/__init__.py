"""Fused attention forward pass for AMD Instinct MI355X (gfx950).

The computation runs in hand-written HIP kernels behind a C-ABI shared library
(``libfa_mi355x.so``, declared in ``include/fa_mi355x.h``).  ``fwd`` is the thin
Python binding; it marshals torch device tensors and the current stream into
that library and does no arithmetic of its own.
"""
from .inputs import AttnInputs  # noqa: F401

__all__ = ["AttnInputs", "fwd", "fwd_fp8", "load_library"]


def __getattr__(name):
    # The binding is imported lazily so that the input generator and the
    # accounting helpers work on machines without the ROCm runtime.
    if name in ("fwd", "fwd_fp8", "load_library", "FAError"):
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
