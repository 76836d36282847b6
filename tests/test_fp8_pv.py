"""GPU parity of the e4m3 P.V variant (pv_dtype=float8_e4m3fn, fp8 inputs).

P is rounded to e4m3 (3 mantissa bits) before the P.V product, V stays as
stored; tiles that carry more than 1/8 of a row's running sum also multiply
P's e4m3 rounding residual.  Every case is held to the fp8 bound of the
other fp8 tests: max |O - O_ref| <= 3e-2 against the oracle on the
dequantised inputs, LSE within 1e-3, over every row (whole tensors on small
shapes; at full size the first 64 rows, tile edges, the end and random rows).
"""
import numpy as np
import pytest
import torch

from exact_attention_04_amd.workloads import WORKLOADS, Inputs, make_inputs, quantize_e4m3_per_tensor, small_case
from parity_helpers import full_check, run_gpu, sample_rows, sampled_check

pytestmark = pytest.mark.gpu

E4M3 = torch.float8_e4m3fn
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
@pytest.mark.parametrize("n", [1, 7, 63, 64, 65, 129, 300, 1000, 2000])
def test_pv8_small_sweep(n, mask):
    causal, window = MASKS[mask]
    inp = small_case(1, 3, n, 128, "fp8", "bshd", 12000 + n + 11 * list(MASKS).index(mask))
    r = full_check(inp, "fp8", causal=causal, window=window, what=f"pv8 n{n} {mask}", pv_dtype=E4M3)
    print(n, mask, r)


@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
@pytest.mark.parametrize("split", [True, False])
def test_pv8_layouts_and_split(layout, split):
    inp = small_case(2, 4, 1500, 128, "fp8", layout, 12500 + (layout == "bhsd"))
    full_check(inp, "fp8", causal=True, layout=layout, split_kv=split, what=f"pv8 {layout} split={split}",
               pv_dtype=E4M3)


def test_pv8_shared_kv_heads():
    inp = small_case(1, 8, 700, 128, "fp8", "bshd", 12600, heads_kv=2)
    full_check(inp, "fp8", causal=True, what="pv8 H8/Hk2", pv_dtype=E4M3)


def test_pv8_same_as_default_where_p_is_exact():
    # one visible key per row (diagonal window): p = 1 exactly in e4m3 and
    # bf16, so both P formats give O = v_i exactly
    inp = small_case(1, 2, 333, 128, "fp8", "bshd", 12700)
    o8, l8 = run_gpu(inp, window=(0, 0), pv_dtype=E4M3)
    o16, l16 = run_gpu(inp, window=(0, 0))
    assert torch.equal(o8, o16)
    assert torch.allclose(l8, l16, rtol=0, atol=1e-6)


def test_pv8_workload_sampled():
    w = WORKLOADS["fp8_b1h16n65536d128_causal"]
    inp = make_inputs(w)
    o, lse = run_gpu(inp, causal=w.causal, scale=w.softmax_scale, layout=w.layout, pv_dtype=E4M3)
    assert torch.isfinite(o.float()).all().item()
    assert torch.isfinite(lse).all().item()
    rng = np.random.default_rng(w.seed)
    heads = [(0, 0), (0, w.heads - 1)] + [(0, int(rng.integers(w.heads))) for _ in range(2)]
    r = sampled_check(inp, w.dtype, o, lse, heads, sample_rows(w.seqlen, w.seed), causal=w.causal,
                      scale=w.softmax_scale, layout=w.layout, what="pv8 " + w.name)
    print(w.name, r)


def _fp8_inputs(q, k, v):
    qs = [quantize_e4m3_per_tensor(x) for x in (q, k, v)]
    return Inputs(qs[0][0], qs[1][0], qs[2][0], tuple(s for _, s in qs))


@pytest.mark.parametrize("causal", [False, True])
def test_pv8_dominant_keys(causal):
    # Query 2j and key j share a large component, so each even row puts a
    # sizeable share of its weight (about a sixth) on one key in the middle of
    # its range, about 2 above the first tile's maximum in the exponent (p 2^3
    # near 60, where e4m3 steps by 8): that entry's rounding does not average
    # out, and the tile holding it must take the residual pass.
    n, d, a = 900, 128, 7.8
    rng = np.random.default_rng(41)
    q = rng.standard_normal((1, n, 2, d)).astype(np.float32)
    k = rng.standard_normal((1, n, 2, d)).astype(np.float32)
    v = rng.standard_normal((1, n, 2, d)).astype(np.float32)
    basis = rng.standard_normal((n, d)).astype(np.float32)
    basis /= np.linalg.norm(basis, axis=1, keepdims=True)
    q[0] += a * basis[:, None, :]
    for j in range(n // 2):
        k[0, j] += a * basis[2 * j][None, :]
    inp = _fp8_inputs(q, k, v)
    full_check(inp, "fp8", causal=causal, what=f"pv8 dominant keys causal={causal}", pv_dtype=E4M3)


@pytest.mark.parametrize("causal", [False, True])
def test_pv8_scores_outgrowing_the_first_tile(causal):
    # Keys grow along the sequence, so later scores pass the first tile's
    # maximum by far more than e4m3 P can hold (p 2^3 >= 480 turns NaN): the
    # kernel must detect it and redo the row block with the exact maximum.
    n, d = 700, 128
    rng = np.random.default_rng(43)
    q = np.ones((1, n, 2, d), dtype=np.float32) + 0.1 * rng.standard_normal((1, n, 2, d)).astype(np.float32)
    ramp = (np.arange(n, dtype=np.float32) / n)[None, :, None, None]
    k = ramp * (1.0 + 0.1 * rng.standard_normal((1, n, 2, d)).astype(np.float32))
    v = rng.standard_normal((1, n, 2, d)).astype(np.float32)
    inp = _fp8_inputs(q, k, v)
    full_check(inp, "fp8", causal=causal, scale=0.2, what=f"pv8 growing scores causal={causal}", pv_dtype=E4M3)


def test_pv8_rejected_for_16bit_inputs():
    q = torch.zeros(1, 64, 2, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        from exact_attention_04_amd import attention
        attention(q, q, q, pv_dtype=E4M3)


def test_pv8_deterministic():
    # no atomics and no order-dependent sums: repeated calls give identical bits
    inp = small_case(2, 8, 1111, 128, "fp8", "bshd", 12800)
    o1, l1 = run_gpu(inp, causal=True, pv_dtype=E4M3)
    for _ in range(4):
        o2, l2 = run_gpu(inp, causal=True, pv_dtype=E4M3)
        assert torch.equal(o1.view(torch.uint8), o2.view(torch.uint8)) and torch.equal(l1, l2)
