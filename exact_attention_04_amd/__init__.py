"""MI355X-native exact attention, forward and backward (HIP kernels for gfx950 behind a C ABI).

    from exact_attention_04_amd import attention
    o, lse = attention(q, k, v, causal=True)          # q, k, v: [B, S, H, D] on the GPU
    dq, dk, dv, delta = attention_backward(q, k, v, o, do, lse, causal=True)

The compute runs in libea_attn.so (built by ``python -m
exact_attention_04_amd.build``); importing this package does not load it, and
calling without it raises.
"""
from .attention import attention, attention_backward, make_args, plan  # noqa: F401

__all__ = ["attention", "attention_backward", "make_args", "plan"]
