"""Windowed grouped-query attention on AMD Instinct MI355X (gfx950).

The compute lives in a C-ABI shared library of hand-written HIP kernels
(``libgqa_mi355x.so``, built from ``csrc/``; declarations in ``include/gqa.h``
at the repository root).  ``binding`` marshals torch device tensors into that
ABI; it performs no arithmetic of its own and raises if the library is
missing.
"""

from . import inputs, work  # noqa: F401  (pure host helpers, no device code)

__all__ = ["inputs", "work", "binding"]


def __getattr__(name):
    if name == "binding":
        from . import binding
        return binding
    raise AttributeError(name)
