"""GPU parity: the HIP path against the float64 oracle on the same seeded inputs.

Small shapes are compared element by element over whole tensors (several
query tiles and key tiles, ragged tails, every mask kind).  The named
workloads run at full size in the launch configuration the benchmark times,
and are compared on sampled heads and rows that the oracle computes one by
one.
"""
import numpy as np
import pytest
import torch

from exact_attention_04_amd.workloads import WORKLOADS, make_inputs, small_case
from parity_helpers import full_check, run_gpu, sample_rows, sampled_check

pytestmark = pytest.mark.gpu

MASKS = {
    "none": (False, (-1, -1)),
    "causal": (True, (-1, -1)),
    "causal_w3": (True, (3, 0)),
    "w17_5": (False, (17, 5)),
    "diag": (False, (0, 0)),
    "right0": (False, (-1, 0)),
    "causal_w100": (True, (100, -1)),
}


@pytest.mark.parametrize("mask", list(MASKS))
@pytest.mark.parametrize("n", [1, 7, 63, 64, 65, 127, 129, 200, 1000])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_small_sweep(dtype, d, n, mask):
    causal, window = MASKS[mask]
    seed = 1000 * d + n + 7 * list(MASKS).index(mask) + (0 if dtype == "f16" else 500000)
    inp = small_case(2, 3, n, d, dtype, "bshd", seed)
    full_check(inp, dtype, causal=causal, window=window, what=f"{dtype} d{d} n{n} {mask}")


@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
@pytest.mark.parametrize("mask", ["none", "causal", "w17_5"])
def test_layouts(layout, mask):
    causal, window = MASKS[mask]
    inp = small_case(2, 4, 333, 64, "f16", layout, 77)
    full_check(inp, "f16", causal=causal, window=window, layout=layout, what=f"{layout} {mask}")


@pytest.mark.parametrize("mask", ["none", "causal", "causal_w100", "w17_5"])
@pytest.mark.parametrize("n", [1, 65, 300, 1000])
def test_fp8_small(n, mask):
    causal, window = MASKS[mask]
    inp = small_case(1, 3, n, 128, "fp8", "bshd", 9000 + n)
    full_check(inp, "fp8", causal=causal, window=window, what=f"fp8 n{n} {mask}")


def test_explicit_scale():
    inp = small_case(1, 2, 257, 64, "f16", "bhsd", 5)
    full_check(inp, "f16", causal=True, scale=1.0 / 8.0, layout="bhsd", what="scale 1/8")
    full_check(inp, "f16", causal=False, scale=0.37, layout="bhsd", what="scale 0.37")


# ---------------------------------------------------------------------------
# The named workloads at full size
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["sdpa_b1h8n512d64_f16", "sdpa_b2h8n2048d64_f16", "sdpa_b2h8n2048d64_f16_causal"])
def test_workload_full(name):
    w = WORKLOADS[name]
    inp = make_inputs(w)
    r = full_check(inp, w.dtype, causal=w.causal, window=(w.window_left, w.window_right), scale=w.softmax_scale,
                   layout=w.layout, what=name)
    print(name, r)


@pytest.mark.parametrize("name", ["sdpa_b4h32n4096d128_bf16_causal", "swa_b1h32n16384d128_bf16_w4095",
                                  "fp8_b1h16n65536d128_causal"])
def test_workload_sampled(name):
    w = WORKLOADS[name]
    inp = make_inputs(w)
    window = (w.window_left, w.window_right)
    o, lse = run_gpu(inp, causal=w.causal, window=window, scale=w.softmax_scale, layout=w.layout)
    assert torch.isfinite(o.float()).all().item()
    assert torch.isfinite(lse).all().item()
    rng = np.random.default_rng(w.seed)
    heads = [(0, 0), (w.batch - 1, w.heads - 1)]
    heads += [(int(rng.integers(w.batch)), int(rng.integers(w.heads))) for _ in range(2)]
    rows = sample_rows(w.seqlen, w.seed)
    r = sampled_check(inp, w.dtype, o, lse, heads, rows, causal=w.causal, window=window, scale=w.softmax_scale,
                      layout=w.layout, what=name)
    print(name, r)


# ---------------------------------------------------------------------------
# K/V heads shared by groups of query heads
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("heads,heads_kv", [(8, 2), (6, 3), (4, 1), (16, 4)])
@pytest.mark.parametrize("mask", ["none", "causal", "w17_5"])
@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
def test_shared_kv_heads(heads, heads_kv, mask, layout):
    causal, window = MASKS[mask]
    inp = small_case(2, heads, 333, 128, "bf16", layout, 60 + heads + heads_kv, heads_kv=heads_kv)
    full_check(inp, "bf16", causal=causal, window=window, layout=layout,
               what=f"H{heads}/Hk{heads_kv} {mask} {layout}")


@pytest.mark.parametrize("batch,heads,heads_kv", [(1, 64, 8), (2, 64, 8), (1, 72, 24), (2, 32, 4)])
def test_shared_kv_heads_xcd_groups(batch, heads, heads_kv):
    # (batch, K/V head) counts of 8, 16, 24 and 8: the work order puts the
    # query heads of one K/V head (8, 24) or of two (16) on an XCD at a time;
    # at least 512 query tiles x heads (N = 1100), so the plain configuration
    # runs
    from exact_attention_04_amd import plan
    from parity_helpers import upload
    inp = small_case(batch, heads, 1100, 128, "bf16", "bshd", 9900 + batch * 10 + heads_kv, heads_kv=heads_kv)
    q, k, v = upload(inp)
    info = plan(q, k, v, torch.empty_like(q), causal=True)
    assert ",ks" not in info.kernel.decode() and info.splits == 1, info.kernel
    full_check(inp, "bf16", causal=True, what=f"xcd groups B{batch} H{heads}/Hk{heads_kv}")


@pytest.mark.parametrize("dtype,d", [("f16", 64), ("fp8", 128)])
def test_shared_kv_heads_other_types(dtype, d):
    inp = small_case(1, 8, 300, d, dtype, "bshd", 71, heads_kv=2)
    full_check(inp, dtype, causal=True, what=f"{dtype} d{d} H8/Hk2")


@pytest.mark.parametrize("name", ["gqa_b4h32kv8n4096d128_bf16_causal", "mqa_b4h32kv1n4096d128_bf16_causal"])
def test_shared_kv_workload_sampled(name):
    w = WORKLOADS[name]
    inp = make_inputs(w)
    o, lse = run_gpu(inp, causal=w.causal, scale=w.softmax_scale, layout=w.layout)
    assert torch.isfinite(o.float()).all().item()
    rng = np.random.default_rng(w.seed)
    heads = [(0, 0), (w.batch - 1, w.heads - 1), (1, 5), (2, 30)]
    heads += [(int(rng.integers(w.batch)), int(rng.integers(w.heads))) for _ in range(2)]
    r = sampled_check(inp, w.dtype, o, lse, heads, sample_rows(w.seqlen, w.seed), causal=w.causal,
                      scale=w.softmax_scale, layout=w.layout, what=name)
    print(name, r)


# ---------------------------------------------------------------------------
# Key split for launches with few query tiles: both paths against the oracle
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("split", [True, False])
@pytest.mark.parametrize("name", ["sdpa_b1h8n512d64_f16", "sdpa_b2h8n2048d64_f16", "sdpa_b2h8n2048d64_f16_causal"])
def test_key_split_workloads(name, split):
    w = WORKLOADS[name]
    inp = make_inputs(w)
    r = full_check(inp, w.dtype, causal=w.causal, window=(w.window_left, w.window_right), scale=w.softmax_scale,
                   layout=w.layout, what=f"{name} split={split}", split_kv=split)
    print(name, split, r)


@pytest.mark.parametrize("mask", ["none", "causal", "w17_5", "causal_w100"])
@pytest.mark.parametrize("n,d,dtype", [(1000, 128, "bf16"), (777, 64, "f16"), (1500, 128, "fp8")])
def test_key_split_masks(n, d, dtype, mask):
    causal, window = MASKS[mask]
    inp = small_case(1, 2, n, d, dtype, "bshd", 7000 + n + d)
    full_check(inp, dtype, causal=causal, window=window, what=f"split {dtype} n{n} {mask}", split_kv=True)


@pytest.mark.parametrize("window", [(-1, -1), (1000, -1)])
@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
@pytest.mark.parametrize("dtype,d,heads,heads_kv", [("bf16", 128, 8, 2), ("f16", 64, 4, 1), ("fp8", 128, 8, 2)])
def test_key_split_with_shared_kv_heads(dtype, d, heads, heads_kv, layout, window):
    # causal launches with few query tiles, plain and with a window of 1000
    # keys that still leaves the tiles unbalanced, with query heads sharing
    # K/V heads: 16-bit inputs split the keys among key streams inside the
    # workgroup, fp8 among workgroups (chunks merged by a second kernel)
    from exact_attention_04_amd import plan
    from parity_helpers import upload
    causal = True
    inp = small_case(1, heads, 1100, d, dtype, layout, 8100 + heads + d, heads_kv=heads_kv)
    q, k, v = upload(inp)
    o = torch.empty(q.shape, dtype=torch.bfloat16 if dtype == "fp8" else q.dtype, device=q.device)
    (B, N, H) = (1, 1100, heads)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    info = plan(q, k, v, o, lse, causal=causal, window_size=window, layout=layout,
                descale=inp.descale if dtype == "fp8" else None)
    kernel, splits = info.kernel.decode(), info.splits
    if dtype == "fp8":
        assert splits > 1, kernel
    else:
        assert ",ks" in kernel and splits == 1, kernel
    full_check(inp, dtype, causal=causal, window=window, layout=layout, split_kv=True,
               what=f"split {dtype} H{heads}/Hk{heads_kv} {layout} window {window}")


@pytest.mark.parametrize("mask", list(MASKS))
@pytest.mark.parametrize("n", [1, 63, 129, 333])
@pytest.mark.parametrize("dtype,d", [("f16", 64), ("bf16", 128)])
def test_plain_configuration_small_shapes(dtype, d, n, mask):
    # enough (batch, head) pairs that the launch keeps the plain 128-row
    # configuration (at least 512 query tiles x heads), with ragged tails and
    # every mask kind; the small sweeps above run with key streams
    from exact_attention_04_amd import plan
    from parity_helpers import upload
    causal, window = MASKS[mask]
    B, H = (8, 32) if n > 128 else (16, 32)
    inp = small_case(B, H, n, d, dtype, "bshd", 9300 + n + d + 3 * list(MASKS).index(mask))
    q, k, v = upload(inp)
    kernel = plan(q, k, v, torch.empty_like(q), causal=causal, window_size=window).kernel.decode()
    assert ",ks" not in kernel, kernel
    full_check(inp, dtype, causal=causal, window=window, what=f"plain {dtype} d{d} n{n} {mask}")


@pytest.mark.parametrize("n", [65, 200, 330, 1000])
@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (-1, -1)), (True, (130, 0)), (False, (70, 70))])
@pytest.mark.parametrize("dtype,d", [("f16", 64), ("bf16", 128)])
def test_key_streams_uneven_tiles(dtype, d, n, causal, window):
    # key tile counts that do not divide among the streams (a stream's last
    # tile past the range is loaded as zeros and skipped), query tiles whose
    # visible keys fit in fewer tiles than there are streams
    from exact_attention_04_amd import plan
    from parity_helpers import upload
    inp = small_case(1, 2, n, d, dtype, "bshd", 9500 + n + d)
    q, k, v = upload(inp)
    kernel = plan(q, k, v, torch.empty_like(q), causal=causal, window_size=window).kernel.decode()
    assert (",ks4" if d == 64 else ",ks2") in kernel, kernel
    full_check(inp, dtype, causal=causal, window=window, what=f"streams {dtype} d{d} n{n} {causal} {window}")


@pytest.mark.parametrize("n,causal,window", [(700, True, (-1, -1)), (1000, True, (-1, -1)),
                                             (1500, False, (100, -1)), (1500, False, (-1, 0))])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_two_streams_of_64_rows(dtype, n, causal, window):
    # d = 64 launches with 128-511 query tiles of 128 rows whose key work is
    # unbalanced run with 64-row workgroups and two key streams; ragged
    # tails (N not a multiple of 64) and every kind of mask edge
    from exact_attention_04_amd import plan
    from parity_helpers import upload
    B, H = 4, 8
    inp = small_case(B, H, n, 64, dtype, "bshd", 9700 + n + (7 if causal else 0))
    q, k, v = upload(inp)
    kernel = plan(q, k, v, torch.empty_like(q), causal=causal, window_size=window).kernel.decode()
    assert "bm64" in kernel and ",ks2" in kernel, kernel
    full_check(inp, dtype, causal=causal, window=window, what=f"64-row streams {dtype} n{n} {causal} {window}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale", [1.0, 2.0])
def test_scores_outgrowing_the_first_tile(dtype, causal, scale):
    # Keys grow along the sequence, so late scores exceed the first tile's
    # maximum by far: by about 2^86 (scale 1) or 2^172 (scale 2) in p.  The
    # first exceeds fp16 P's range but not bf16's, the second overflows fp32
    # exp2 too; either way the kernel must detect it and redo the row block
    # with the exact row maximum as reference.
    import torch as _t
    from exact_attention_04_amd.workloads import Inputs, torch_dtype
    n, d = 700, 64
    rng = np.random.default_rng(31)
    q = np.ones((1, n, 2, d), dtype=np.float32) + 0.1 * rng.standard_normal((1, n, 2, d)).astype(np.float32)
    ramp = (np.arange(n, dtype=np.float32) / n)[None, :, None, None]
    k = ramp * (1.0 + 0.1 * rng.standard_normal((1, n, 2, d)).astype(np.float32))
    v = rng.standard_normal((1, n, 2, d)).astype(np.float32)
    td = torch_dtype(dtype)
    inp = Inputs(*(_t.from_numpy(x).to(td) for x in (q, k, v)), (1.0, 1.0, 1.0))
    full_check(inp, dtype, causal=causal, scale=scale, what=f"growing scores {dtype} causal={causal} scale={scale}")


# ---------------------------------------------------------------------------
# A long sequence: the last query tiles loop over 4096 key tiles
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal,window", [(True, (-1, -1)), (True, (4095, 0))])
def test_long_sequence_sampled(causal, window):
    n = 262144
    inp = small_case(1, 2, n, 128, "bf16", "bshd", 8800 + window[0])
    o, lse = run_gpu(inp, causal=causal, window=window)
    assert torch.isfinite(o.float()).all().item()
    rows = sorted(set(range(0, 40)) | {4095, 4096, 65535, 131072, n // 2 + 7} | set(range(n - 40, n)))
    r = sampled_check(inp, "bf16", o, lse, [(0, 0), (0, 1)], rows, causal=causal, window=window,
                      what=f"N={n} window={window}")
    print(r)
