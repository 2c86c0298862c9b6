"""Windowed grouped-query attention on AMD Instinct MI355X (gfx950).

The compute lives in a C-ABI shared library of hand-written HIP kernels
(``libgqa_mi355x.so``, built from ``csrc/``; declarations in ``include/gqa.h``
at the repository root).  ``binding`` marshals torch device tensors into that
ABI; it performs no arithmetic of its own, loads the library on first use and
raises if it is missing.
"""

from . import binding, inputs, work  # noqa: F401

__all__ = ["binding", "inputs", "work"]
