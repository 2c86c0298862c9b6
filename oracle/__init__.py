"""Oracle for windowed grouped-query attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the ``smoke()`` check of ``__graft_entry__`` and the
CPU-baseline leg of ``bench.py`` may import anything from this package.  The
product path (the ``windowed_gqa_kv_amd`` binding, the C-ABI library and its
HIP kernels) never imports, calls or links it, and this package imports
nothing from the product path.

``attention``  plain materialized float64 attention (NumPy), the definition.
``brute``      the same definition with scalar Python loops, for tiny shapes.
``rotary``     rotary position embedding of Q and of K before it enters the cache.
``rolling``    the rolling (ring-buffer) KV cache of a windowed layer.
``fp8``        an FP8 (E4M3) KV cache with per-tensor scales.
``int8``       an INT8 KV cache with per-KV-head scales.
"""

from .materialized import (  # noqa: F401
    allowed,
    attention,
    prefill,
    decode,
    append_kv,
    sink_logits,
    softcap_fn,
)
from . import brute  # noqa: F401
from . import rotary  # noqa: F401
from . import rolling  # noqa: F401
from . import fp8  # noqa: F401
from . import int8  # noqa: F401
