"""GPU check of the allocation-free forward, ea_attn_fwd_noalloc, through the
C ABI: its output against ea_attn_fwd's on the same inputs (the same kernels
and key split, so the same bits), two calls in a row with the second on a
smaller problem (the static scratch keeps the first call's contents), and the
float64 oracle's tolerance on the second.  The split launches are fp8 ones:
16-bit launches with few query tiles split their keys inside the workgroup
and need no scratch."""
import numpy as np
import pytest
import torch

from exact_attention_04_amd import _lib, attention, plan
from exact_attention_04_amd.attention import make_args
from exact_attention_04_amd.workloads import small_case
from parity_helpers import compare, stored_f64

import oracle

pytestmark = pytest.mark.gpu


def _gpu(inp):
    return tuple(t.cuda() for t in (inp.q, inp.k, inp.v))


def _noalloc(q, k, v, **kw):
    (B, N, H) = (q.shape[0], q.shape[1], q.shape[2]) if kw.get("layout", "bshd") == "bshd" else (q.shape[0], q.shape[2], q.shape[1])
    o = torch.empty(q.shape, dtype=torch.bfloat16 if q.dtype == torch.float8_e4m3fn else q.dtype, device=q.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    a = make_args(q, k, v, o, lse, **kw)
    st = _lib.fwd_noalloc(a, torch.cuda.current_stream().cuda_stream)
    assert st == _lib.EA_OK, _lib.status_string(st)
    return o, lse


@pytest.mark.parametrize("order", ["large_then_small", "small_then_large"])
def test_noalloc_equals_the_workspace_entry_point(order):
    # fp8 launches with few query tiles split their keys among workgroups
    # (16-bit ones use key streams inside the workgroup and need no scratch)
    cases = [
        (small_case(1, 8, 2048, 128, "fp8", "bhsd", 31), dict(causal=True, layout="bhsd", softmax_scale=0.125)),
        (small_case(1, 2, 1000, 128, "fp8", "bshd", 32), dict(causal=True, window_size=(700, -1))),
    ]
    for inp, kw in cases:
        kw["descale"] = inp.descale
    if order == "small_then_large":
        cases = cases[::-1]
    for inp, kw in cases:
        q, k, v = _gpu(inp)
        o = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
        info = plan(q, k, v, o, **kw)
        splits, nbytes = info.splits, info.workspace_bytes
        assert splits > 1 and 0 < nbytes <= 32 << 20, (splits, nbytes)
        o_ref, l_ref = attention(q, k, v, **kw)            # caller workspace from torch
        o_na, l_na = _noalloc(q, k, v, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o_na, o_ref) and torch.equal(l_na, l_ref)
    # the last call against the oracle as well
    inp, kw = cases[-1]
    qf, kf, vf = (stored_f64(t, s) for t, s in zip((inp.q, inp.k, inp.v), inp.descale))
    o_exp, l_exp = oracle.attention(qf, kf, vf, scale=kw.get("softmax_scale", 1.0 / np.sqrt(qf.shape[-1])),
                                    causal=kw["causal"], window=kw.get("window_size", (-1, -1)),
                                    layout=kw.get("layout", "bshd"))
    compare(o_na.float().cpu().double().numpy(), o_exp, l_na.cpu().double().numpy(), l_exp, "fp8", "noalloc")


def test_noalloc_without_a_split_and_refusals():
    # a launch that fills the GPU needs no split, hence no scratch
    q, k, v = _gpu(small_case(2, 32, 1024, 128, "bf16", "bshd", 33))
    o = torch.empty_like(q)
    splits = plan(q, k, v, o, causal=True).splits   # 512 query tiles x heads: two per CU
    assert splits == 1
    o_ref, l_ref = attention(q, k, v, causal=True)
    o_na, l_na = _noalloc(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o_na, o_ref) and torch.equal(l_na, l_ref)
    # a caller workspace is refused (this entry point uses the library's own)
    lse = torch.empty(2, 32, 1024, dtype=torch.float32, device="cuda")
    ws = torch.empty(4096, dtype=torch.uint8, device="cuda")
    a = make_args(q, k, v, o, lse, causal=True)
    a.workspace, a.workspace_bytes = ws.data_ptr(), 4096
    assert _lib.fwd_noalloc(a, torch.cuda.current_stream().cuda_stream) == _lib.EA_EINVAL
    # a 16-bit launch with few query tiles runs key streams: no scratch either
    q, k, v = _gpu(small_case(1, 2, 1000, 128, "bf16", "bshd", 34))
    o = torch.empty_like(q)
    info = plan(q, k, v, o, causal=True)
    kernel, splits = info.kernel.decode(), info.splits
    assert ",ks" in kernel and splits == 1
    o_ref, l_ref = attention(q, k, v, causal=True)
    o_na, l_na = _noalloc(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o_na, o_ref) and torch.equal(l_na, l_ref)
    # a split that would need more than the 32 MiB scratch is refused
    big = torch.zeros(1, 32768, 1, 128, dtype=torch.float8_e4m3fn, device="cuda")
    o = torch.empty(big.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(1, 1, 32768, dtype=torch.float32, device="cuda")
    a = make_args(big, big, big, o, lse, causal=True, descale=(1.0, 1.0, 1.0))
    assert _lib.fwd_noalloc(a, torch.cuda.current_stream().cuda_stream) == _lib.EA_ESCRATCH
