"""fp8 inputs with P.V in bf16: V widened once into the caller's workspace
gives bitwise the same O and LSE as V widened tile by tile inside the
attention kernel (every e4m3 value is a bf16 value, so both feed the matrix
instruction the same operands), for each way the workspace can be sized."""
import pytest
import torch

from exact_attention_04_amd import _lib, plan
from exact_attention_04_amd.attention import make_args
from exact_attention_04_amd.workloads import small_case
from parity_helpers import upload

pytestmark = pytest.mark.gpu


def run(q, k, v, ws_bytes, layout, **kw):
    B, N, H = (q.shape[0], q.shape[1], q.shape[2]) if layout == "bshd" else (q.shape[0], q.shape[2], q.shape[1])
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    a = make_args(q, k, v, o, lse, layout=layout, **kw)
    ws = None
    if ws_bytes > 0:
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
        ws.fill_(0xFF)   # stale contents must not matter
        a.workspace, a.workspace_bytes = ws.data_ptr(), ws_bytes
    _lib.check(_lib.fwd(a, torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    return o, lse


CASES = [
    # (B, H, Hk, N, layout, causal, window): the first splits its keys
    (1, 8, 8, 2048, "bshd", True, (-1, -1)),
    (2, 4, 2, 700, "bhsd", False, (-1, -1)),
    (1, 2, 2, 1000, "bshd", False, (300, 20)),
    (2, 32, 32, 1024, "bshd", True, (-1, -1)),
    (3, 6, 1, 333, "bhsd", True, (100, -1)),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}h{}k{}n{}_{}_c{}_w{}_{}".format(
    c[0], c[1], c[2], c[3], c[4], int(c[5]), *c[6]))
def test_widened_copy_is_bitwise_the_in_kernel_widening(case):
    B, H, Hk, N, layout, causal, window = case
    inp = small_case(B, H, N, 128, "fp8", layout, 8800 + N, heads_kv=Hk)
    q, k, v = upload(inp)
    kw = dict(causal=causal, window_size=window, descale=inp.descale)
    vcopy = (B * Hk * N * 128 * 2 + 255) // 256 * 256
    info = plan(q, k, v, torch.empty(q.shape, dtype=torch.bfloat16, device=q.device), layout=layout, **kw)
    split_bytes = info.workspace_bytes - vcopy
    assert split_bytes >= 0, (info.workspace_bytes, vcopy)
    none = run(q, k, v, 0, layout, **kw)
    copy_only = run(q, k, v, vcopy if split_bytes == 0 or vcopy < split_bytes else 0, layout, **kw)
    assert torch.equal(copy_only[0], none[0]) and torch.equal(copy_only[1], none[1])
    if info.splits > 1:
        full = run(q, k, v, info.workspace_bytes, layout, **kw)        # copy + split
        split_only = run(q, k, v, split_bytes, layout, **kw)            # split, V widened in the kernel
        assert torch.equal(full[0], split_only[0]) and torch.equal(full[1], split_only[1])
    else:
        full = run(q, k, v, info.workspace_bytes, layout, **kw)
        assert torch.equal(full[0], none[0]) and torch.equal(full[1], none[1])


def test_widened_copy_of_a_strided_v_view():
    # V as a view into wider rows (row stride 256 elements, starting 64 bytes in)
    inp = small_case(2, 4, 500, 128, "fp8", "bshd", 8899)
    q, k, v = upload(inp)
    wide = torch.zeros((2, 500, 4, 256), dtype=torch.uint8, device=q.device)
    wide[..., 64:192] = v.view(torch.uint8)
    vs = wide[..., 64:192].view(torch.float8_e4m3fn)
    assert vs.stride() == (500 * 4 * 256, 4 * 256, 256, 1)
    kw = dict(causal=True, window_size=(-1, -1), descale=inp.descale)
    info = plan(q, k, vs, torch.empty(q.shape, dtype=torch.bfloat16, device=q.device), **kw)
    vcopy = 2 * 4 * 500 * 128 * 2
    assert info.workspace_bytes >= vcopy
    # the reference: contiguous V widened in the kernel, with the same key
    # split as the copy run (the split reorders the sums)
    ref = run(q, k, v, info.workspace_bytes - vcopy, "bshd", **kw)
    got = run(q, k, vs, info.workspace_bytes, "bshd", **kw)
    assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])
