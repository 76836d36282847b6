"""CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, the ``smoke()`` check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its Python
binding) never imports, calls or falls back to it.

Everything here is plain float64 numpy that materialises the score matrix, as
the pages define "standard attention"; it shares no code, tables or helpers
with the GPU kernels.
"""
from .sdpa_fp64 import (  # noqa: F401
    attention,
    attention_head,
    attention_probs_head,
    attention_parallel,
    dequantize_e4m3,
    kv_head_of,
    visible,
)
from .sdpa_bwd_fp64 import attention_backward, attention_backward_head  # noqa: F401
