"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and its argument checks and planner behave as documented.

No call here launches work: ea_attn_plan touches no device memory, and the
ea_attn_fwd calls below all fail validation before any device is queried.
"""
import ctypes
import math
import os
import re
import subprocess

import pytest

from exact_attention_04_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ea_attn.h")

# The library under test: the in-tree build, or a host-only build of the same
# C ABI layer (HIP calls and launches stubbed) named by EA_ABI_TEST_LIB, which
# tests/test_abi_host.py uses to run these tests under AddressSanitizer and
# UndefinedBehaviorSanitizer.
HOST_LIB = os.environ.get("EA_ABI_TEST_LIB")
_handle = None


def abi():
    global _handle
    if _handle is None:
        _handle = _lib.bind(ctypes.CDLL(HOST_LIB)) if HOST_LIB else _lib.lib()
    return _handle


def status(code):
    return abi().ea_status_string(code).decode()


pytestmark = pytest.mark.skipif(not HOST_LIB and not os.path.exists(_lib.LIB_PATH), reason="libea_attn.so not built")
product_only = pytest.mark.skipif(bool(HOST_LIB), reason="checks the in-tree GPU library itself")

FAKE = 0x7F0000000000   # never dereferenced: plan() and failing fwd() calls do not touch memory


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(ea_\w+)\s*\(", text, re.M)))


def test_header_declares_exactly_the_exports():
    assert header_functions() == sorted(_lib.EXPORTS)


@product_only
def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True, check=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in header_functions():
        assert name in syms, f"{name} not exported"
        assert hasattr(abi(), name)


@product_only
def test_library_embeds_gpu_code():
    from exact_attention_04_amd.build import elf_section_names
    assert ".hip_fatbin" in elf_section_names(_lib.LIB_PATH)


def test_abi_version_and_status_strings():
    assert abi().ea_abi_version() == _lib.EA_ABI_VERSION
    for code in range(6):
        assert status(code)
    assert status(99) == "unknown status"
    assert abi().ea_last_hip_error() == 0


def test_struct_sizes_match_c():
    # same layout rules as the C compiler on x86-64 / amdgcn
    assert ctypes.sizeof(_lib.AttnArgs) == 4 + 5 * 4 + 4 * 4 + 6 * 8 + 5 * 8 + 14 * 8 + 2 * 8 + 2 * 4
    assert ctypes.sizeof(_lib.PlanInfo) == 4 + 4 * 4 + 4 + 3 * 8 + 64 + 8 + 2 * 4
    assert ctypes.sizeof(_lib.BwdArgs) == 4 + 4 * 4 + 4 + 5 * 8 + 10 * 8 + 24 * 8 + 4 * 8


def make(B=2, N=300, H=3, D=128, dtype=_lib.EA_BF16, layout="bshd", **kw):
    a = _lib.AttnArgs()
    a.struct_size = ctypes.sizeof(_lib.AttnArgs)
    a.in_dtype = dtype
    a.out_dtype = _lib.EA_BF16 if dtype == _lib.EA_FP8_E4M3 else dtype
    a.softmax_scale = 1.0 / math.sqrt(D)
    a.q_descale = a.k_descale = a.v_descale = 1.0
    a.window_left = a.window_right = -1
    a.batch, a.seqlen_q, a.seqlen_k, a.nheads_q, a.nheads_k, a.headdim = B, N, N, H, H, D
    size = B * N * H * D * 4 + 4096
    a.q, a.k, a.v, a.o = FAKE, FAKE + size, FAKE + 2 * size, FAKE + 3 * size
    if layout == "bshd":
        sb, ss, sh = N * H * D, H * D, D
    else:
        sb, ss, sh = N * H * D, D, N * D
    for t in "qkvo":
        setattr(a, f"{t}_stride_b", sb)
        setattr(a, f"{t}_stride_s", ss)
        setattr(a, f"{t}_stride_h", sh)
    a.lse = FAKE + 4 * size
    a.lse_stride_b, a.lse_stride_h = H * N, N
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


SIZE = 2 * 300 * 3 * 128 * 4 + 4096   # make()'s spacing of the fake tensors


def plan_status(a):
    info = _lib.PlanInfo()
    info.struct_size = ctypes.sizeof(_lib.PlanInfo)
    return abi().ea_attn_plan(ctypes.byref(a), ctypes.byref(info)), info


def test_plan_valid_configs():
    # B2 H3 N300 has few query tiles (18 items of 128 rows): 16-bit inputs run
    # key streams (4 x 32 rows at d = 64, 2 x 128 rows at d = 128), fp8 the
    # plain 128-row configuration
    for dtype, D, bm, waves, name in ((_lib.EA_F16, 64, 32, 4, "attn_fwd<f16,d64,bm32,bn64,ks4>"),
                                      (_lib.EA_BF16, 128, 128, 8, "attn_fwd<bf16,d128,bm128,bn64,ks2>"),
                                      (_lib.EA_FP8_E4M3, 128, 128, 4, "attn_fwd<fp8,d128,bm128,bn64>")):
        for layout in ("bshd", "bhsd"):
            st, info = plan_status(make(dtype=dtype, D=D, layout=layout))
            assert st == _lib.EA_OK, status(st)
            assert (info.block_m, info.block_n, info.waves) == (bm, 64, waves)
            assert info.grid == 2 * 3 * math.ceil(300 / bm)
            assert info.kernel.decode() == name
            assert info.lds_bytes <= 160 * 1024


def test_plan_configuration_by_launch_size():
    # 16-bit: two workgroups of 128 rows per CU (512 items) keep the plain
    # configuration; fewer items take key streams: at d = 64, four streams
    # of 32 rows for under 128 items, two streams of 64 rows where the
    # query tiles' key work is unbalanced (causal), else two of 128 rows
    for (B, N, H, D, causal), name, waves in (
            ((4, 4096, 32, 128, 1), "attn_fwd<bf16,d128,bm128,bn64>", 4),
            ((2, 1024, 32, 128, 1), "attn_fwd<bf16,d128,bm128,bn64>", 4),
            ((2, 1024, 16, 128, 1), "attn_fwd<bf16,d128,bm128,bn64,ks2>", 8),
            ((1, 512, 8, 128, 1), "attn_fwd<bf16,d128,bm128,bn64,ks2>", 8),
            ((2, 2048, 8, 64, 1), "attn_fwd<bf16,d64,bm64,bn64,ks2>", 4),
            ((2, 2048, 8, 64, 0), "attn_fwd<bf16,d64,bm128,bn64,ks2>", 8),
            ((1, 1920, 8, 64, 1), "attn_fwd<bf16,d64,bm32,bn64,ks4>", 4),
            ((1, 512, 8, 64, 1), "attn_fwd<bf16,d64,bm32,bn64,ks4>", 4),
            ((1, 512, 8, 64, 0), "attn_fwd<bf16,d64,bm32,bn64,ks4>", 4)):
        a = make(B=B, N=N, H=H, D=D, causal=causal)
        for t in "qkvo":
            setattr(a, f"{t}_stride_b", N * H * D)
            setattr(a, f"{t}_stride_s", H * D)
            setattr(a, f"{t}_stride_h", D)
        for t, i in zip("qkvo", range(4)):
            setattr(a, t, FAKE + i * (B * N * H * D * 2 + 4096))
        a.lse = FAKE + 4 * (B * N * H * D * 2 + 4096)
        a.lse_stride_b, a.lse_stride_h = H * N, N
        st, info = plan_status(a)
        assert st == 0, ((B, N, H, D, causal), status(st))
        assert info.kernel.decode() == name, ((B, N, H, D, causal), info.kernel)
        assert info.waves == waves and info.splits == 1 and info.workspace_bytes == 0, (name, info.waves)


def test_plan_window_balance_picks_the_configuration():
    # at d = 64 with 128-511 items: a window that leaves the query tiles'
    # key work balanced keeps 128 rows; one that unbalances it takes 64 rows
    for wl, wr, name in ((200, 200, "attn_fwd<f16,d64,bm128,bn64,ks2>"),
                         (1500, -1, "attn_fwd<f16,d64,bm128,bn64,ks2>"),
                         (-1, 0, "attn_fwd<f16,d64,bm64,bn64,ks2>"),
                         (100, -1, "attn_fwd<f16,d64,bm64,bn64,ks2>")):
        a = make(B=2, N=2048, H=8, D=64, dtype=_lib.EA_F16, causal=0, window_left=wl, window_right=wr)
        st, info = plan_status(a)
        assert st == 0 and info.kernel.decode() == name, (wl, wr, info.kernel)


def test_plan_headline_shape():
    st, info = plan_status(make(B=4, N=4096, H=32, causal=1))
    assert st == 0 and info.waves == 4 and info.block_m == 128
    assert info.grid == 4 * 32 * 32
    # causal: query tile t (128 rows) visits 2t+2 key tiles of 64, 2 of them on the diagonal
    assert info.kv_tiles == 128 * sum(2 * t + 2 for t in range(32))
    assert info.masked_tiles == 128 * 32 * 2


def test_plan_tile_counts_causal_and_window():
    # causal N=4096: query tile t (128 rows) visits 2t+2 key tiles of 64
    st, info = plan_status(make(B=1, N=4096, H=1, causal=1))
    assert st == 0
    assert info.kv_tiles == sum(2 * t + 2 for t in range(32))
    assert info.masked_tiles == 32 * 2
    st, info = plan_status(make(B=1, N=4096, H=1))
    assert info.kv_tiles == 32 * 64 and info.masked_tiles == 0
    # window [i-4095, i] at N=16384: at most 66 key tiles per query tile
    st, info = plan_status(make(B=1, N=16384, H=1, causal=1, window_left=4095, window_right=0))
    assert st == 0
    assert info.kv_tiles <= 128 * 66


@pytest.mark.parametrize("field,value,code", [
    ("struct_size", 8, _lib.EA_EINVAL),
    ("batch", -1, _lib.EA_EINVAL),
    ("nheads_q", 0, _lib.EA_EINVAL),
    ("in_dtype", 9, _lib.EA_EINVAL),
    ("softmax_scale", float("nan"), _lib.EA_EINVAL),
    ("softmax_scale", float("inf"), _lib.EA_EINVAL),
    ("q_descale", 2.0, _lib.EA_EINVAL),            # descale != 1 on 16-bit input
    ("window_left", -2, _lib.EA_EINVAL),
    ("q", 0, _lib.EA_EINVAL),
    ("o", FAKE, _lib.EA_EINVAL),                    # o aliases q
    ("in_dtype", _lib.EA_F32, _lib.EA_EUNSUPPORTED),  # fp32 input
    ("headdim", 96, _lib.EA_EUNSUPPORTED),
    ("seqlen_k", 299, _lib.EA_EUNSUPPORTED),
    ("nheads_k", 2, _lib.EA_EUNSUPPORTED),         # 3 query heads cannot share 2 K/V heads
    ("out_dtype", _lib.EA_F16, _lib.EA_EUNSUPPORTED),
    ("softmax_scale", -0.5, _lib.EA_EUNSUPPORTED),
    ("q", FAKE + 8, _lib.EA_EUNSUPPORTED),          # not 16-byte aligned
    ("k_stride_s", 128 * 3 + 4, _lib.EA_EUNSUPPORTED),  # row stride not a 16-byte multiple
    ("v_stride_h", -128, _lib.EA_EUNSUPPORTED),
    ("lse", FAKE + 2, _lib.EA_EUNSUPPORTED),
    ("lse", FAKE + 16, _lib.EA_EINVAL),             # lse inside q
    ("lse", FAKE + 3 * SIZE + 64, _lib.EA_EINVAL),  # lse inside o
    # an absurd row stride is refused before any product with it can wrap
    ("k_stride_s", 1 << 62, _lib.EA_EUNSUPPORTED),
    # so are batch and head strides and LSE strides whose extents overflow
    ("q_stride_b", 1 << 62, _lib.EA_EUNSUPPORTED),
    ("v_stride_h", (1 << 62) + 8, _lib.EA_EUNSUPPORTED),
    ("o_stride_b", (1 << 46) // 2 * 8, _lib.EA_EUNSUPPORTED),   # fits int64, extent past 2^47 bytes
    ("lse_stride_b", 1 << 61, _lib.EA_EUNSUPPORTED),
    ("lse_stride_h", 1 << 62, _lib.EA_EUNSUPPORTED),
    ("batch", 1 << 40, _lib.EA_EUNSUPPORTED),
])
def test_validation_errors(field, value, code):
    a = make()
    setattr(a, field, value)
    st, _ = plan_status(a)
    assert st == code, (field, value, status(st))
    # the launch entry points apply the same checks before touching a device
    assert abi().ea_attn_fwd(ctypes.byref(a), None) == code
    assert abi().ea_attn_fwd_noalloc(ctypes.byref(a), None) == code


def test_shared_kv_heads():
    # query heads sharing K/V heads: any Hk that divides Hq
    for hk in (1, 2, 4, 8):
        a = make(H=8, nheads_k=hk)
        for t in "kv":   # K/V tensors with hk heads (BSHD strides)
            setattr(a, f"{t}_stride_b", 300 * hk * 128)
            setattr(a, f"{t}_stride_s", hk * 128)
        st, info = plan_status(a)
        assert st == _lib.EA_OK, (hk, status(st))
        assert info.grid == 2 * 8 * math.ceil(300 / 128)
    assert plan_status(make(H=8, nheads_k=3))[0] == _lib.EA_EUNSUPPORTED


def test_key_split_plan_and_workspace_rules():
    fp8 = _lib.EA_FP8_E4M3
    # 16-bit launches with few query tiles split their keys inside the
    # workgroup (key streams): no workspace
    st, info = plan_status(make(B=2, N=2048, H=8, D=64, dtype=_lib.EA_F16, causal=1))
    assert st == 0 and info.splits == 1 and info.workspace_bytes == 0 and "ks2" in info.kernel.decode()
    # fp8: balanced work (no mask) is not split, however few the query tiles;
    # with P.V in bf16 the workspace wanted is the bf16 copy of V
    # (B x Hk x N x D x 2 bytes), with e4m3 P.V nothing
    st, info = plan_status(make(B=1, N=512, H=8, D=128, dtype=fp8))
    assert st == 0 and info.splits == 1 and info.workspace_bytes == 8 * 512 * 128 * 2
    st, info = plan_status(make(B=1, N=512, H=8, D=128, dtype=fp8, pv_dtype=fp8))
    assert st == 0 and info.splits == 1 and info.workspace_bytes == 0
    # shared K/V heads: the copy holds the K/V heads only
    st, info = plan_status(make(B=2, N=100, H=8, D=128, dtype=fp8, nheads_k=2))
    assert st == 0 and info.workspace_bytes == (2 * 2 * 100 * 128 * 2 + 255) // 256 * 256
    # causal fp8 B1 H8 N2048: 128 items, the heaviest tile sees 32 key tiles
    # against 17 on average -> 2 chunks; the workspace holds the copy of V,
    # then the chunks' partial results
    st, info = plan_status(make(B=1, N=2048, H=8, D=128, dtype=fp8, causal=1))
    assert st == 0 and info.splits == 2
    assert info.workspace_bytes == 8 * 2048 * 128 * 2 + 2 * 8 * 2048 * (128 + 1) * 4
    # causal fp8 B1 H2 N1000: 16 items -> up to 8 chunks, capped by the balance rule
    st, info = plan_status(make(B=1, N=1000, H=2, D=128, causal=1, dtype=fp8))
    assert st == 0 and info.splits == 2
    # the headline shape fills the GPU: no split, no workspace
    st, info = plan_status(make(B=4, N=4096, H=32, causal=1))
    assert st == 0 and info.splits == 1 and info.workspace_bytes == 0
    # a workspace must be 16-byte aligned and overlap no tensor
    a = make(workspace=FAKE + 5 * SIZE + 8, workspace_bytes=4096)
    assert plan_status(a)[0] == _lib.EA_EUNSUPPORTED
    a = make(workspace=FAKE + 3 * SIZE, workspace_bytes=4096)           # inside o
    assert plan_status(a)[0] == _lib.EA_EINVAL
    a = make(workspace=FAKE + 4 * SIZE, workspace_bytes=4096)           # inside lse
    assert plan_status(a)[0] == _lib.EA_EINVAL
    assert plan_status(make(workspace=FAKE + 5 * SIZE, workspace_bytes=4096))[0] == _lib.EA_OK


def test_version1_structs_are_accepted():
    # callers built against the first ABI pass the structs without the
    # workspace fields; the library then neither reads nor writes them
    a = make(workspace=FAKE, workspace_bytes=64)   # would alias q if read
    assert plan_status(a)[0] == _lib.EA_EINVAL
    a.struct_size = _lib.AttnArgs.workspace.offset
    assert plan_status(a)[0] == _lib.EA_OK
    a.struct_size -= 8
    assert plan_status(a)[0] == _lib.EA_EINVAL
    info = _lib.PlanInfo()
    info.struct_size = _lib.PlanInfo.workspace_bytes.offset
    info.workspace_bytes = 12345
    info.splits = 7
    assert abi().ea_attn_plan(ctypes.byref(make(B=1, N=512, H=8, D=64, dtype=_lib.EA_F16)), ctypes.byref(info)) == 0
    assert info.workspace_bytes == 12345 and info.splits == 7 and info.block_m == 32


def test_version2_structs_are_accepted():
    # callers built against the second ABI pass the struct without pv_dtype
    a = make(dtype=_lib.EA_FP8_E4M3, pv_dtype=99, reserved=5)   # invalid if read
    assert plan_status(a)[0] == _lib.EA_EINVAL
    a.struct_size = _lib.AttnArgs.pv_dtype.offset
    st, info = plan_status(a)
    assert st == _lib.EA_OK and info.kernel.decode() == "attn_fwd<fp8,d128,bm128,bn64>"


def test_pv_dtype_rules():
    # fp8 inputs: 0 / bf16 keep P in bf16, e4m3 selects the 8-bit P.V kernel
    for pv, name, lds in ((0, "attn_fwd<fp8,d128,bm128,bn64>", 2 * (8192 + 16384)),
                          (_lib.EA_BF16, "attn_fwd<fp8,d128,bm128,bn64>", 2 * (8192 + 16384)),
                          (_lib.EA_FP8_E4M3, "attn_fwd<fp8,pv8,d128,bm128,bn64>", 2 * (8192 + 8192))):
        st, info = plan_status(make(dtype=_lib.EA_FP8_E4M3, pv_dtype=pv))
        assert st == _lib.EA_OK and info.kernel.decode() == name and info.lds_bytes == lds
    assert plan_status(make(dtype=_lib.EA_FP8_E4M3, pv_dtype=_lib.EA_F16))[0] == _lib.EA_EINVAL
    assert plan_status(make(dtype=_lib.EA_FP8_E4M3, pv_dtype=_lib.EA_FP8_E4M3, reserved=1))[0] == _lib.EA_EINVAL
    # 16-bit inputs take no pv_dtype
    assert plan_status(make(pv_dtype=_lib.EA_FP8_E4M3))[0] == _lib.EA_EUNSUPPORTED
    assert plan_status(make(pv_dtype=_lib.EA_BF16))[0] == _lib.EA_EUNSUPPORTED
    assert abi().ea_attn_fwd(ctypes.byref(make(pv_dtype=_lib.EA_FP8_E4M3)), None) == _lib.EA_EUNSUPPORTED


def test_fp8_argument_rules():
    a = make(dtype=_lib.EA_FP8_E4M3, q_descale=0.01, k_descale=0.02, v_descale=0.03)
    assert plan_status(a)[0] == _lib.EA_OK
    assert plan_status(make(dtype=_lib.EA_FP8_E4M3, q_descale=0.0))[0] == _lib.EA_EINVAL
    assert plan_status(make(dtype=_lib.EA_FP8_E4M3, out_dtype=_lib.EA_F16))[0] == _lib.EA_EUNSUPPORTED
    assert plan_status(make(dtype=_lib.EA_FP8_E4M3, D=64))[0] == _lib.EA_EUNSUPPORTED


def test_empty_problem_is_ok_without_pointers():
    a = make(B=0)
    a.q = a.k = a.v = a.o = 0
    st, info = plan_status(a)
    assert st == _lib.EA_OK and info.grid == 0
    assert abi().ea_attn_fwd(ctypes.byref(a), None) == _lib.EA_OK
    a = make(N=0)
    assert abi().ea_attn_fwd(ctypes.byref(a), None) == _lib.EA_OK


def test_plan_rejects_small_info_struct():
    info = _lib.PlanInfo()
    info.struct_size = 4
    assert abi().ea_attn_plan(ctypes.byref(make()), ctypes.byref(info)) == _lib.EA_EINVAL


@product_only
def test_python_wrapper_rejects_cpu_tensors():
    import torch
    from exact_attention_04_amd import attention
    x = torch.zeros(1, 8, 1, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        attention(x, x, x)


def make_bwd(B=2, N=300, H=3, D=128, **kw):
    """Backward arguments over fake, disjoint BSHD tensors."""
    a = _lib.BwdArgs()
    a.struct_size = ctypes.sizeof(_lib.BwdArgs)
    a.dtype = _lib.EA_BF16
    a.window_left = a.window_right = -1
    a.softmax_scale = 1.0 / math.sqrt(D)
    a.batch, a.seqlen, a.nheads_q, a.nheads_k, a.headdim = B, N, H, H, D
    size = B * N * H * D * 4 + 4096
    for i, t in enumerate(("q", "k", "v", "o", "dout", "lse", "delta", "dq", "dk", "dv")):
        setattr(a, t, FAKE + i * size)
    for t in ("q", "k", "v", "o", "do", "dq", "dk", "dv"):
        setattr(a, f"{t}_stride_b", N * H * D)
        setattr(a, f"{t}_stride_s", H * D)
        setattr(a, f"{t}_stride_h", D)
    a.lse_stride_b = a.delta_stride_b = H * N
    a.lse_stride_h = a.delta_stride_h = N
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


BWD_SIZE = 2 * 300 * 3 * 128 * 4 + 4096   # make_bwd()'s spacing of the fake tensors


@pytest.mark.parametrize("field,value,code", [
    ("struct_size", 8, _lib.EA_EINVAL),
    ("seqlen", -1, _lib.EA_EINVAL),
    ("nheads_k", 0, _lib.EA_EINVAL),
    ("softmax_scale", float("nan"), _lib.EA_EINVAL),
    ("window_right", -2, _lib.EA_EINVAL),
    ("dv", 0, _lib.EA_EINVAL),
    ("dq", FAKE + 64, _lib.EA_EINVAL),                  # dq inside q
    ("dk", FAKE + 7 * BWD_SIZE, _lib.EA_EINVAL),        # dk on top of dq
    ("delta", FAKE + 5 * BWD_SIZE, _lib.EA_EINVAL),     # delta on top of lse
    ("dtype", _lib.EA_FP8_E4M3, _lib.EA_EUNSUPPORTED),  # forward only in fp8
    ("dtype", _lib.EA_F32, _lib.EA_EUNSUPPORTED),
    ("headdim", 80, _lib.EA_EUNSUPPORTED),
    ("nheads_k", 2, _lib.EA_EUNSUPPORTED),
    ("softmax_scale", 0.0, _lib.EA_EUNSUPPORTED),
    ("dout", FAKE + 4 * BWD_SIZE + 8, _lib.EA_EUNSUPPORTED),   # not 16-byte aligned
    ("lse", FAKE + 5 * BWD_SIZE + 2, _lib.EA_EUNSUPPORTED),    # not 4-byte aligned
    ("q_stride_s", 3 * 128 + 4, _lib.EA_EUNSUPPORTED),
    ("dk_stride_h", -128, _lib.EA_EUNSUPPORTED),
    ("v_stride_s", 1 << 62, _lib.EA_EUNSUPPORTED),
    ("dq_stride_b", 1 << 62, _lib.EA_EUNSUPPORTED),
    ("k_stride_h", (1 << 62) + 8, _lib.EA_EUNSUPPORTED),
    ("delta_stride_b", 1 << 62, _lib.EA_EUNSUPPORTED),
    ("nheads_q", 3 << 40, _lib.EA_EUNSUPPORTED),
])
def test_bwd_validation_errors(field, value, code):
    # every failing check returns before a device is queried
    a = make_bwd()
    setattr(a, field, value)
    assert abi().ea_attn_bwd(ctypes.byref(a), None) == code, (field, value)


def test_bwd_empty_problem_is_ok_without_pointers():
    for fields in ({"batch": 0}, {"seqlen": 0}):
        a = make_bwd(**fields)
        for t in ("q", "k", "v", "o", "dout", "lse", "delta", "dq", "dk", "dv"):
            setattr(a, t, 0)
        assert abi().ea_attn_bwd(ctypes.byref(a), None) == _lib.EA_OK


@pytest.mark.parametrize("causal", [0, 1])
def test_window_bounds_past_the_sequence_plan_as_unbounded(causal):
    # a window bound >= N reaches past every key: the plan (tile walk, grid,
    # split) is that of -1, also at int32's largest value, where the row +
    # bound sums would otherwise wrap
    big = 2 ** 31 - 1
    for N in (300, 4096):
        st, ref = plan_status(make(B=1, N=N, H=2, causal=causal))
        assert st == 0
        for wl, wr in ((big, big), (big, -1), (-1, big), (N, N), (N, 0 if causal else N)):
            st, info = plan_status(make(B=1, N=N, H=2, causal=causal, window_left=wl, window_right=wr))
            assert st == 0, (wl, wr)
            got = (info.grid, info.kv_tiles, info.masked_tiles, info.splits, info.workspace_bytes)
            want = (ref.grid, ref.kv_tiles, ref.masked_tiles, ref.splits, ref.workspace_bytes)
            assert got == want, (N, wl, wr, got, want)
    # a bound just inside the sequence still bounds
    st, info = plan_status(make(B=1, N=4096, H=2, causal=causal, window_left=4094, window_right=0))
    assert st == 0 and info.kv_tiles < plan_status(make(B=1, N=4096, H=2))[1].kv_tiles


@product_only
def test_python_window_values_are_range_checked():
    import torch
    from exact_attention_04_amd.attention import make_args
    x = torch.zeros(1, 8, 1, 64, dtype=torch.float16)
    # past int32: the largest int32 (unbounded, as any bound >= N), never a wrapped value
    a = make_args(x, x, x, x, None, window_size=(2 ** 40, 2 ** 33 + 5))
    assert (a.window_left, a.window_right) == (2 ** 31 - 1, 2 ** 31 - 1)
    for bad in ((-2, 0), (0, -(2 ** 32) + 5), (-(2 ** 40), -1)):
        with pytest.raises(ValueError):
            make_args(x, x, x, x, None, window_size=bad)


def test_noalloc_scratch_limit_and_workspace_rules():
    # the allocation-free forward keeps the key split's partial results in a
    # 32 MiB static array: a plan that wants more is refused before any
    # device call, with its own status
    a = make(B=1, N=32768, H=1, D=128, causal=1, dtype=_lib.EA_FP8_E4M3)
    st, info = plan_status(a)
    assert st == 0 and info.splits == 2
    assert info.workspace_bytes == 32768 * 128 * 2 + 2 * 32768 * 129 * 4   # V copy + split
    assert 2 * 32768 * 129 * 4 > 32 << 20
    assert abi().ea_attn_fwd_noalloc(ctypes.byref(a), None) == _lib.EA_ESCRATCH
    assert "scratch" in status(_lib.EA_ESCRATCH)
    with pytest.raises(ValueError):
        _lib.check(_lib.EA_ESCRATCH)
    # it takes no caller workspace
    a = make(workspace=FAKE + 5 * SIZE, workspace_bytes=4096, q_stride_s=-1)   # invalid stride checked first
    assert abi().ea_attn_fwd_noalloc(ctypes.byref(a), None) == _lib.EA_EUNSUPPORTED
    a = make(workspace=FAKE + 5 * SIZE, workspace_bytes=4096)
    assert abi().ea_attn_fwd_noalloc(ctypes.byref(a), None) == _lib.EA_EINVAL
    # an empty problem is fine without pointers
    e = make(B=0)
    e.q = e.k = e.v = e.o = 0
    assert abi().ea_attn_fwd_noalloc(ctypes.byref(e), None) == _lib.EA_OK
