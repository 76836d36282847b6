"""The product path has no CPU fallback: without the built HIP library every
call raises, and CPU tensors are refused rather than computed on the host."""
import subprocess
import sys
import textwrap

import pytest


def test_missing_library_raises():
    code = textwrap.dedent("""
        import torch
        from exact_attention_04_amd import _lib, attention
        _lib.LIB_PATH = "/nonexistent/libea_attn.so"
        _lib._lib = None
        try:
            _lib.lib()
        except RuntimeError as e:
            assert "missing" in str(e), e
        else:
            raise SystemExit("no error without the library")
        print("ok")
    """)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr


def test_cpu_tensors_are_refused():
    import torch
    from exact_attention_04_amd import attention, attention_backward
    x = torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        attention(x, x, x)
    l = torch.zeros(1, 2, 8, dtype=torch.float32)
    with pytest.raises(ValueError):
        attention_backward(x, x, x, x, x, l)
