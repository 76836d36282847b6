"""Python entry point over the C ABI: argument marshalling only.

``attention(q, k, v, causal=..., window_size=..., softmax_scale=...)`` mirrors
the call the "Flash Attention | Hermes Skill" page shows for the flash-attn
library (Workflow 2, Step 2: q, k, v as [batch, seqlen, nheads, headdim],
``causal``, ``window_size=(left, right)`` with -1 for no limit,
``softmax_scale=None`` for 1/sqrt(headdim)) and accepts the SDPA layout
[batch, heads, seq, dim] of its Quick start with ``layout="bhsd"``.

Every step of the computation runs in the HIP library; torch provides device
memory (``torch.empty``), pointers, strides and the current stream.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import torch

from . import _lib

_DTYPES = {
    torch.float16: _lib.EA_F16,
    torch.bfloat16: _lib.EA_BF16,
    torch.float8_e4m3fn: _lib.EA_FP8_E4M3,
    torch.float32: _lib.EA_F32,
}


def _dims(x: torch.Tensor, layout: str):
    """(B, S, H, D) and the element strides (b, s, h) of a 4-D tensor."""
    if x.dim() != 4:
        raise ValueError(f"expected a 4-D tensor, got shape {tuple(x.shape)}")
    if x.stride(3) != 1 and x.shape[3] > 1:
        raise ValueError("the head dimension must be contiguous (stride 1)")
    st = x.stride()
    if layout == "bshd":
        return (x.shape[0], x.shape[1], x.shape[2], x.shape[3]), (st[0], st[1], st[2])
    if layout == "bhsd":
        return (x.shape[0], x.shape[2], x.shape[1], x.shape[3]), (st[0], st[2], st[1])
    raise ValueError(f"layout must be 'bshd' or 'bhsd', got {layout!r}")


def _check_buffer(name: str, t: torch.Tensor, shape, dtype: torch.dtype, device: torch.device) -> None:
    """A caller-supplied output: the kernels write it in full, so its shape,
    dtype and device must be the ones the call produces."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device:
        raise ValueError(f"{name} must be a {dtype} tensor of shape {tuple(shape)} on {device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


def _check_rows(name: str, t: torch.Tensor, B: int, H: int, N: int, device: torch.device) -> None:
    """A float32 [B, H, N] per-row array (LSE, delta) with contiguous rows."""
    _check_buffer(name, t, (B, H, N), torch.float32, device)
    if N > 1 and t.stride(2) != 1:
        raise ValueError(f"{name} rows must be contiguous (stride 1 along the sequence)")


_INT32_MAX = 2 ** 31 - 1


def _window(window_size) -> Tuple[int, int]:
    """The window bounds as C int32 values.  -1 means unbounded; a bound past
    int32 reaches beyond any sequence the library accepts, so it is passed as
    the largest int32 (the library treats a bound >= N as unbounded too)."""
    out = []
    for w in window_size:
        w = int(w)
        if w < -1:
            raise ValueError(f"window bounds must be >= -1, got {tuple(window_size)}")
        out.append(min(w, _INT32_MAX))
    return out[0], out[1]


def make_args(q, k, v, o, lse, *, causal=False, window_size=(-1, -1), softmax_scale=None,
              layout="bshd", descale=None, pv_dtype=None) -> _lib.AttnArgs:
    """Fill an ``ea_attn_args`` for the given tensors (no checks beyond shapes)."""
    (B, N, H, D), (qb, qs, qh) = _dims(q, layout)
    (Bk, Nk, Hk, Dk), (kb, ks, kh) = _dims(k, layout)
    (_, _, _, _), (vb, vs, vh) = _dims(v, layout)
    (_, _, _, _), (ob, os_, oh) = _dims(o, layout)
    if Bk != B or Dk != D or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError(f"unsupported dtypes q={q.dtype} k={k.dtype} v={v.dtype}")
    a = _lib.AttnArgs()
    a.struct_size = _lib.ctypes.sizeof(_lib.AttnArgs)
    a.in_dtype = _DTYPES[q.dtype]
    a.out_dtype = _DTYPES.get(o.dtype, 0)
    a.causal = 1 if causal else 0
    a.window_left, a.window_right = _window(window_size)
    a.softmax_scale = float(1.0 / math.sqrt(D) if softmax_scale is None else softmax_scale)
    dq, dk, dv = (1.0, 1.0, 1.0) if descale is None else descale
    a.q_descale, a.k_descale, a.v_descale = float(dq), float(dk), float(dv)
    a.batch, a.seqlen_q, a.seqlen_k, a.nheads_q, a.nheads_k, a.headdim = B, N, Nk, H, Hk, D
    a.q, a.k, a.v, a.o = q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr()
    a.q_stride_b, a.q_stride_s, a.q_stride_h = qb, qs, qh
    a.k_stride_b, a.k_stride_s, a.k_stride_h = kb, ks, kh
    a.v_stride_b, a.v_stride_s, a.v_stride_h = vb, vs, vh
    a.o_stride_b, a.o_stride_s, a.o_stride_h = ob, os_, oh
    if lse is not None:
        a.lse = lse.data_ptr()
        a.lse_stride_b, a.lse_stride_h = lse.stride(0), lse.stride(1)
    if pv_dtype is not None:
        if pv_dtype not in _DTYPES:
            raise ValueError(f"unsupported pv_dtype {pv_dtype}")
        a.pv_dtype = _DTYPES[pv_dtype]
    return a


# Workspace bytes wanted by the library, per argument signature (ea_attn_plan).
_ws_bytes = {}


def _workspace_bytes(a: _lib.AttnArgs) -> int:
    key = bytes(a)[:_lib.AttnArgs.q.offset] + bytes(a)[_lib.AttnArgs.q_stride_b.offset:_lib.AttnArgs.workspace.offset]
    n = _ws_bytes.get(key)
    if n is None:
        n = int(_lib.plan(a).workspace_bytes)
        _ws_bytes[key] = n
    return n


def out_dtype_for(dtype: torch.dtype) -> torch.dtype:
    return torch.bfloat16 if dtype == torch.float8_e4m3fn else dtype


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
              window_size: Tuple[int, int] = (-1, -1), softmax_scale: Optional[float] = None,
              layout: str = "bshd", descale: Optional[Tuple[float, float, float]] = None,
              return_lse: bool = True, out: Optional[torch.Tensor] = None,
              lse: Optional[torch.Tensor] = None, split_kv: bool = True,
              pv_dtype: Optional[torch.dtype] = None):
    """Exact attention forward on the current HIP stream.

    Returns ``(o, lse)``: o in q's layout and shape (bf16 for fp8 inputs, else
    q's dtype), lse as float32 [B, H, N] (None when ``return_lse`` is False).
    ``descale`` gives the per-tensor fp8 scales (stored value * descale = real
    value).  ``split_kv`` lets the call use a workspace from torch's
    allocator, as large as ``plan`` reports: a launch with too few query
    tiles to fill the GPU splits each tile's keys into chunks (merged by a
    second kernel), and fp8 inputs with bf16 P.V read a bf16 copy of V
    widened once by a first kernel (bitwise the same results); False passes
    no workspace (no split, V widened per tile inside the kernel).
    ``pv_dtype`` (fp8 inputs only): ``torch.float8_e4m3fn`` runs P.V with P
    and V in e4m3 on the 8-bit matrix instructions; None or ``torch.bfloat16``
    keeps P in bf16 (the default).  Raises ValueError for arguments the
    library rejects.
    """
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor (this library has no CPU path)")
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
    (B, N, H, _), _ = _dims(q, layout)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype_for(q.dtype), device=q.device)
    else:
        _check_buffer("out", out, q.shape, out_dtype_for(q.dtype), q.device)
    if not return_lse:
        lse = None
    elif lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        _check_rows("lse", lse, B, H, N, q.device)
    a = make_args(q, k, v, out, lse, causal=causal, window_size=window_size, softmax_scale=softmax_scale,
                  layout=layout, descale=descale, pv_dtype=pv_dtype)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    ws = None
    if split_kv and B > 0 and N > 0:
        nbytes = _workspace_bytes(a)
        if nbytes > 0:
            ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
            a.workspace, a.workspace_bytes = ws.data_ptr(), nbytes
    _lib.check(_lib.fwd(a, stream))
    return out, lse


def plan(q, k, v, o, lse=None, **kw) -> _lib.PlanInfo:
    """The tile configuration ``attention`` would launch (no device work)."""
    return _lib.plan(make_args(q, k, v, o, lse, **kw))


def attention_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, dout: torch.Tensor,
                       lse: torch.Tensor, *, causal: bool = False, window_size: Tuple[int, int] = (-1, -1),
                       softmax_scale: Optional[float] = None, layout: str = "bshd",
                       dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                       dv: Optional[torch.Tensor] = None, delta: Optional[torch.Tensor] = None):
    """Gradients of attention on the current HIP stream (16-bit inputs).

    ``o`` and ``lse`` are the forward's outputs for the same arguments and
    ``dout`` the gradient with respect to ``o``.  Returns ``(dq, dk, dv,
    delta)``: dq, dk, dv shaped like q, k, v; delta = rowsum(dout * o) as
    float32 [B, H, N].  Raises ValueError for arguments the library rejects.
    """
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("lse", lse)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor (this library has no CPU path)")
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
    if q.dtype not in (torch.float16, torch.bfloat16) or any(t.dtype != q.dtype for t in (k, v, o, dout)):
        raise ValueError("the backward takes float16 or bfloat16 q, k, v, o, dout of one dtype")
    (B, N, H, D), (qb, qs, qh) = _dims(q, layout)
    (Bk, Nk, Hk, Dk), (kb, ks, kh) = _dims(k, layout)
    if Bk != B or Nk != N or Dk != D or tuple(v.shape) != tuple(k.shape) or tuple(o.shape) != tuple(q.shape) \
            or tuple(dout.shape) != tuple(q.shape):
        raise ValueError("shape mismatch between q, k, v, o, dout")
    _check_rows("lse", lse, B, H, N, q.device)
    for name, t, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t is not None:
            _check_buffer(name, t, like.shape, like.dtype, q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if delta is None:
        delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        _check_rows("delta", delta, B, H, N, q.device)
    a = _lib.BwdArgs()
    a.struct_size = _lib.ctypes.sizeof(_lib.BwdArgs)
    a.dtype = _DTYPES[q.dtype]
    a.causal = 1 if causal else 0
    a.window_left, a.window_right = _window(window_size)
    a.softmax_scale = float(1.0 / math.sqrt(D) if softmax_scale is None else softmax_scale)
    a.batch, a.seqlen, a.nheads_q, a.nheads_k, a.headdim = B, N, H, Hk, D
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        _, (sb, ss, sh) = _dims(t, layout)
        setattr(a, f"{name}_stride_b", sb)
        setattr(a, f"{name}_stride_s", ss)
        setattr(a, f"{name}_stride_h", sh)
    a.q, a.k, a.v, a.o, a.dout = q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr()
    a.dq, a.dk, a.dv = dq.data_ptr(), dk.data_ptr(), dv.data_ptr()
    a.lse, a.delta = lse.data_ptr(), delta.data_ptr()
    a.lse_stride_b, a.lse_stride_h = lse.stride(0), lse.stride(1)
    a.delta_stride_b, a.delta_stride_h = delta.stride(0), delta.stride(1)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    _lib.check(_lib.bwd(a, stream))
    return dq, dk, dv, delta
