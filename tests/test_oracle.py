"""Pins for the float64 oracle, against things other than the oracle itself.

Each test fixes the oracle to something the pages or mathematics determine:
brute force on tiny inputs, a library routine (torch CPU scaled dot-product
attention, the routine the "Flash Attention | Hermes Skill" page's Quick start
calls), closed forms, invariants, a hand-derived worked example, and the OCP
e4m3 format definition.  The planted-mistake tests at the end check that these
pins do catch plausible errors in the oracle.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import sdpa_fp64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
MASKS = [
    (False, -1, -1),   # no mask
    (True, -1, -1),    # causal
    (False, 2, 1),     # two-sided window
    (True, 3, -1),     # causal + left window
    (True, 0, 0),      # diagonal only
    (False, -1, 0),    # right window 0 without causal == causal
    (False, 1, -1),    # left window only
    (True, 2, 5),      # causal caps the right side
]


def brute_force(q, k, v, scale, causal, wl, wr):
    """Pure-Python loops with math.fsum / math.exp (exact-sum brute force)."""
    nq, nk, dv = len(q), len(k), len(v[0])
    o = [[0.0] * dv for _ in range(nq)]
    lse = [0.0] * nq
    for i in range(nq):
        keys = []
        for j in range(nk):
            ok = True
            if causal and j > i:
                ok = False
            if wl >= 0 and j < i - wl:
                ok = False
            if wr >= 0 and j > i + wr:
                ok = False
            if ok:
                keys.append((j, scale * math.fsum(q[i][t] * k[j][t] for t in range(len(q[i])))))
        if not keys:
            lse[i] = -math.inf
            continue
        m = max(s for _, s in keys)
        w = [(j, math.exp(s - m)) for j, s in keys]
        z = math.fsum(e for _, e in w)
        for c in range(dv):
            o[i][c] = math.fsum(e * v[j][c] for j, e in w) / z
        lse[i] = m + math.log(z)
    return np.array(o), np.array(lse)


def rand_head(rng, n, d, nk=None):
    nk = n if nk is None else nk
    return rng.standard_normal((n, d)), rng.standard_normal((nk, d)), rng.standard_normal((nk, d))


@pytest.mark.parametrize("causal,wl,wr", MASKS)
@pytest.mark.parametrize("n,d", [(1, 1), (5, 3), (9, 8), (16, 4)])
def test_brute_force_tiny(n, d, causal, wl, wr):
    rng = np.random.default_rng(n * 100 + d)
    q, k, v = rand_head(rng, n, d)
    scale = 0.7
    o, lse = oracle.attention_head(q, k, v, scale, causal, wl, wr)
    ob, lb = brute_force(q.tolist(), k.tolist(), v.tolist(), scale, causal, wl, wr)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-13)


def test_brute_force_rectangular_and_large_scores():
    # Nq != Nk (top-left aligned mask) and scores far from zero (tests max subtraction).
    rng = np.random.default_rng(7)
    q, k, v = rand_head(rng, 6, 5, nk=11)
    q *= 30.0
    for causal, wl, wr in MASKS:
        o, lse = oracle.attention_head(q, k, v, 1.3, causal, wl, wr)
        ob, lb = brute_force(q.tolist(), k.tolist(), v.tolist(), 1.3, causal, wl, wr)
        np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, lb, rtol=1e-14, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
def test_matches_torch_sdpa_fp64(causal, layout):
    rng = np.random.default_rng(11)
    B, H, N, D = 2, 3, 70, 16
    qt, kt, vt = (torch.from_numpy(rng.standard_normal((B, H, N, D))) for _ in range(3))
    scale = 0.31
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=scale).numpy()
    args = [x.numpy() for x in (qt, kt, vt)]
    if layout == "bshd":
        args = [np.swapaxes(x, 1, 2) for x in args]
    o, lse = oracle.attention(*args, scale=scale, causal=causal, layout=layout)
    if layout == "bshd":
        o = np.swapaxes(o, 1, 2)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    # LSE against scipy's logsumexp of torch-computed scaled scores
    from scipy.special import logsumexp
    s = (torch.matmul(qt, kt.transpose(-1, -2)) * scale).numpy()
    if causal:
        s = np.where(np.tril(np.ones((N, N), dtype=bool)), s, -np.inf)
    np.testing.assert_allclose(lse, logsumexp(s, axis=-1), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal,wl,wr", MASKS)
def test_probability_rows_sum_to_one(causal, wl, wr):
    rng = np.random.default_rng(3)
    q, k, _ = rand_head(rng, 40, 8)
    p = oracle.attention_probs_head(q, k, 0.5, causal, wl, wr)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-13)
    assert (p >= 0).all()
    vis = oracle.visible(np.arange(40)[:, None], np.arange(40)[None, :], 40, causal, wl, wr)
    assert (p[~vis] == 0).all()


@pytest.mark.parametrize("causal,wl,wr", MASKS)
def test_constant_v_gives_constant_output(causal, wl, wr):
    rng = np.random.default_rng(4)
    q, k, _ = rand_head(rng, 33, 8)
    c = rng.standard_normal(8)
    v = np.tile(c, (33, 1))
    o, _ = oracle.attention_head(q, k, v, 0.4, causal, wl, wr)
    np.testing.assert_allclose(o, np.tile(c, (33, 1)), rtol=0, atol=1e-13)


def test_permutation_equivariance_without_mask():
    rng = np.random.default_rng(5)
    q, k, v = rand_head(rng, 25, 8)
    o, lse = oracle.attention_head(q, k, v, 0.6)
    pk = rng.permutation(25)
    o2, lse2 = oracle.attention_head(q, k[pk], v[pk], 0.6)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-13)
    pq = rng.permutation(25)
    o3, lse3 = oracle.attention_head(q[pq], k, v, 0.6)
    np.testing.assert_allclose(o3, o[pq], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse3, lse[pq], rtol=0, atol=1e-13)


def test_closed_forms():
    rng = np.random.default_rng(6)
    n, d, scale = 20, 8, 0.45
    q, k, v = rand_head(rng, n, d)
    # causal row 0 sees only key 0
    o, lse = oracle.attention_head(q, k, v, scale, causal=True)
    np.testing.assert_allclose(o[0], v[0], rtol=0, atol=1e-15)
    assert abs(lse[0] - scale * float(q[0] @ k[0])) < 1e-14
    # window (0, 0): only the diagonal key -> O = V, LSE = scale * q_i . k_i
    o, lse = oracle.attention_head(q, k, v, scale, False, 0, 0)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, scale * np.einsum("id,id->i", q, k), rtol=0, atol=1e-14)
    # Q = 0: uniform weights over visible keys
    for causal, wl, wr in MASKS:
        o, lse = oracle.attention_head(np.zeros_like(q), k, v, scale, causal, wl, wr)
        for i in range(n):
            js = [j for j in range(n) if (not causal or j <= i) and (wl < 0 or j >= i - wl) and (wr < 0 or j <= i + wr)]
            np.testing.assert_allclose(o[i], v[js].mean(axis=0), rtol=0, atol=1e-14)
            assert abs(lse[i] - math.log(len(js))) < 1e-14
    # N = 1: O = v
    o, lse = oracle.attention_head(q[:1], k[:1], v[:1], scale)
    np.testing.assert_allclose(o, v[:1], rtol=0, atol=1e-15)
    # scaling q by alpha and scale by 1/alpha leaves everything unchanged (alpha a power of two: exact)
    o1, l1 = oracle.attention_head(q, k, v, scale, True)
    o2, l2 = oracle.attention_head(q * 4.0, k, v, scale / 4.0, True)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-15)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-15)


def test_worked_example_golden():
    with open(os.path.join(GOLDEN, "worked_2x2.json")) as f:
        g = json.load(f)
    consts = {"ln3": math.log(3.0), "ln4": math.log(4.0)}
    q, k, v = (np.array(g[x]) for x in ("q", "k", "v"))
    scale = consts[g["scale"]]
    for key, causal in (("non_causal", False), ("causal", True)):
        o, lse = oracle.attention_head(q, k, v, scale, causal)
        np.testing.assert_allclose(o, np.array(g[key]["o"]), rtol=0, atol=1e-15)
        np.testing.assert_allclose(lse, [consts[s] for s in g[key]["lse"]], rtol=0, atol=1e-15)


def test_mask_consistency():
    rng = np.random.default_rng(8)
    n = 37
    q, k, v = rand_head(rng, n, 8)
    base = oracle.attention_head(q, k, v, 0.5, causal=True)
    for args in [(False, -1, 0), (True, -1, 0), (True, n, 0), (True, n + 5, -1), (True, -1, 7)]:
        o, lse = oracle.attention_head(q, k, v, 0.5, *args)
        np.testing.assert_array_equal(o, base[0])
        np.testing.assert_array_equal(lse, base[1])
    full = oracle.attention_head(q, k, v, 0.5)
    o, lse = oracle.attention_head(q, k, v, 0.5, False, n, n)
    np.testing.assert_array_equal(o, full[0])
    np.testing.assert_array_equal(lse, full[1])


def test_row_subset_and_blocking(monkeypatch):
    rng = np.random.default_rng(9)
    q, k, v = rand_head(rng, 300, 8)
    for causal, wl, wr in MASKS:
        o, lse = oracle.attention_head(q, k, v, 0.3, causal, wl, wr)
        rows = [299, 0, 17, 150, 151, 298]
        o2, l2 = oracle.attention_head(q, k, v, 0.3, causal, wl, wr, rows=rows)
        np.testing.assert_allclose(o2, o[rows], rtol=0, atol=1e-14)
        np.testing.assert_allclose(l2, lse[rows], rtol=0, atol=1e-14)
        monkeypatch.setattr(sdpa_fp64, "_MAX_BLOCK_ELEMS", 300 * 7)   # 7-row blocks
        o3, l3 = oracle.attention_head(q, k, v, 0.3, causal, wl, wr)
        monkeypatch.undo()
        np.testing.assert_allclose(o3, o, rtol=0, atol=1e-14)
        np.testing.assert_allclose(l3, lse, rtol=0, atol=1e-14)


def test_layouts_and_default_scale():
    rng = np.random.default_rng(10)
    x = [rng.standard_normal((2, 3, 19, 8)) for _ in range(3)]   # bhsd
    o1, l1 = oracle.attention(*x, causal=True, layout="bhsd")
    o2, l2 = oracle.attention(*[np.swapaxes(a, 1, 2) for a in x], causal=True, layout="bshd")
    np.testing.assert_array_equal(np.swapaxes(o2, 1, 2), o1)
    np.testing.assert_array_equal(l2, l1)
    o3, _ = oracle.attention(*x, scale=1.0 / math.sqrt(8.0), causal=True, layout="bhsd")
    np.testing.assert_array_equal(o3, o1)
    oh, lh = oracle.attention(*x, causal=True, layout="bhsd", heads=[(1, 2), (0, 1)], rows=[3, 18])
    np.testing.assert_allclose(oh[0], o1[1, 2, [3, 18]], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lh[1], l1[0, 1, [3, 18]], rtol=0, atol=1e-15)


def test_fully_masked_row_reading():
    # Nq > Nk with causal leaves no row empty, but a window past the keys does.
    rng = np.random.default_rng(12)
    q, k, v = rand_head(rng, 6, 4, nk=3)
    o, lse = oracle.attention_head(q, k, v, 1.0, False, 0, 0)   # rows 3..5 see nothing
    assert np.all(o[3:] == 0) and np.all(np.isneginf(lse[3:]))
    np.testing.assert_allclose(o[:3], v, atol=1e-15)


def test_e4m3_decoder_against_format_and_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.dequantize_e4m3(codes, 1.0)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    np.testing.assert_array_equal(mine[~nan], ref[~nan])
    # closed forms from the format definition
    assert mine[0x7E] == 448.0 and mine[0xFE] == -448.0
    assert mine[0x01] == 2.0 ** -9 and mine[0x08] == 2.0 ** -6 and mine[0x07] == 7 * 2.0 ** -9
    assert mine[0x38] == 1.0 and mine[0xB8] == -1.0 and mine[0x3C] == 1.5
    assert np.isnan(mine[0x7F]) and np.isnan(mine[0xFF])
    np.testing.assert_array_equal(oracle.dequantize_e4m3(codes[:127], 0.25), mine[:127] * 0.25)


def test_parallel_matches_serial():
    rng = np.random.default_rng(13)
    heads = [rand_head(rng, 64, 8) for _ in range(3)]
    res = oracle.attention_parallel(heads, 0.5, True, (-1, -1), processes=2)
    for (q, k, v), (o, l) in zip(heads, res):
        o2, l2 = oracle.attention_head(q, k, v, 0.5, True)
        np.testing.assert_array_equal(o, o2)
        np.testing.assert_array_equal(l, l2)


# ---------------------------------------------------------------------------
# Fewer K/V heads than query heads (multi-query / grouped-query attention)
# ---------------------------------------------------------------------------

def _gqa_case(rng, B, H, Hk, N, D, layout):
    shp = (B, N, H, D) if layout == "bshd" else (B, H, N, D)
    shk = (B, N, Hk, D) if layout == "bshd" else (B, Hk, N, D)
    return rng.standard_normal(shp), rng.standard_normal(shk), rng.standard_normal(shk)


@pytest.mark.parametrize("hk", [1, 2, 3, 6])
@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
@pytest.mark.parametrize("causal,wl,wr", [(False, -1, -1), (True, -1, -1), (True, 4, 0), (False, 3, 2)])
def test_gqa_matches_mha_on_repeated_kv(hk, layout, causal, wl, wr):
    # sharing a K/V head among a group of query heads is the same as giving
    # every query head its own copy of that K/V head
    rng = np.random.default_rng(40 + hk)
    q, k, v = _gqa_case(rng, 2, 6, hk, 23, 8, layout)
    ax = 2 if layout == "bshd" else 1
    kr, vr = (np.repeat(x, 6 // hk, axis=ax) for x in (k, v))
    o1, l1 = oracle.attention(q, k, v, 0.4, causal, (wl, wr), layout)
    o2, l2 = oracle.attention(q, kr, vr, 0.4, causal, (wl, wr), layout)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


@pytest.mark.parametrize("hk", [1, 2, 4])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_matches_torch_sdpa_fp64(hk, causal):
    # torch's scaled_dot_product_attention with enable_gqa (float64, CPU)
    rng = np.random.default_rng(50 + hk)
    q, k, v = _gqa_case(rng, 2, 8, hk, 31, 16, "bhsd")
    o, lse = oracle.attention(q, k, v, 0.3, causal, (-1, -1), "bhsd")
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x) for x in (q, k, v)), is_causal=causal, scale=0.3, enable_gqa=True).numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_gqa_head_counts():
    assert [oracle.kv_head_of(h, 8, 2) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    assert [oracle.kv_head_of(h, 4, 1) for h in range(4)] == [0, 0, 0, 0]
    with pytest.raises(ValueError):
        oracle.kv_head_of(0, 6, 4)
    rng = np.random.default_rng(3)
    q, k, v = _gqa_case(rng, 1, 6, 4, 5, 4, "bshd")
    with pytest.raises(ValueError):
        oracle.attention(q, k, v, 0.5)


def test_planted_gqa_interleaving_is_caught(monkeypatch):
    # query head h reading K/V head h % Hk (interleaved groups) instead of
    # h // (Hq / Hk) must fail the library pin
    monkeypatch.setattr(sdpa_fp64, "kv_head_of", lambda h, hq, hk: h % hk)
    rng = np.random.default_rng(51)
    q, k, v = _gqa_case(rng, 1, 8, 2, 17, 8, "bhsd")
    o, _ = sdpa_fp64.attention(q, k, v, 0.3, False, (-1, -1), "bhsd")
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x) for x in (q, k, v)), scale=0.3, enable_gqa=True).numpy()
    assert not np.allclose(o, ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Planted mistakes: each variant of the oracle carries one plausible bug; the
# pins above must reject it.  The bugs live only in these test doubles.
# ---------------------------------------------------------------------------

def _buggy_visible_strict(i, j, nk, causal, wl, wr):
    ok = j < nk
    if causal:
        ok = ok & (j < i)          # off by one: drops the diagonal
    if wl >= 0:
        ok = ok & (j >= i - wl)
    if wr >= 0:
        ok = ok & (j <= i + wr)
    return ok


_orig_softmax = sdpa_fp64._softmax_block


def _buggy_softmax_no_norm(s):
    p, m, l = _orig_softmax(s)
    return p * 1.0001, m, l        # slightly mis-normalised rows


@pytest.mark.parametrize("mutation", ["causal_off_by_one", "transposed_kv", "scale_dropped", "unnormalised"])
def test_planted_mistakes_are_caught(monkeypatch, mutation):
    rng = np.random.default_rng(14)
    q, k, v = rand_head(rng, 9, 4)
    scale = 0.8
    ob, lb = brute_force(q.tolist(), k.tolist(), v.tolist(), scale, True, -1, -1)
    if mutation == "causal_off_by_one":
        monkeypatch.setattr(sdpa_fp64, "visible", _buggy_visible_strict)
        o, lse = sdpa_fp64.attention_head(q, k, v, scale, True)
    elif mutation == "transposed_kv":
        o, lse = sdpa_fp64.attention_head(q, v, k, scale, True)
    elif mutation == "scale_dropped":
        o, lse = sdpa_fp64.attention_head(q, k, v, 1.0, True)
    else:
        monkeypatch.setattr(sdpa_fp64, "_softmax_block", _buggy_softmax_no_norm)
        o, lse = sdpa_fp64.attention_head(q, k, v, scale, True)
    caught = not (np.allclose(o, ob, rtol=0, atol=1e-13, equal_nan=True) and np.allclose(lse, lb, rtol=0, atol=1e-13, equal_nan=True))
    assert caught, f"planted mistake {mutation} slipped past the brute-force pin"


# ---------------------------------------------------------------------------
# The probability matrix (the backward tests' error bounds are built from it)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal,wl,wr", MASKS)
@pytest.mark.parametrize("n,nk,d", [(1, 1, 1), (5, 5, 3), (9, 9, 8), (16, 16, 4), (6, 11, 5)])
def test_probabilities_against_brute_force(n, nk, d, causal, wl, wr):
    # With V the identity, the definition's output row i is P's row i
    # (O_ic = sum_j P_ij [j == c]), so the brute force over pure-Python loops
    # gives P element by element.
    rng = np.random.default_rng(100 + 7 * n + nk + d)
    q, k, _ = rand_head(rng, n, d, nk)
    scale = 0.7
    pb, _ = brute_force(q.tolist(), k.tolist(), np.eye(nk).tolist(), scale, causal, wl, wr)
    p = oracle.attention_probs_head(q, k, scale, causal, wl, wr)
    assert p.shape == (n, nk)
    np.testing.assert_allclose(p, pb, rtol=0, atol=1e-14)


def test_probabilities_reproduce_the_output():
    # P V is the oracle's O for an arbitrary V, and P's row i is LSE's softmax
    rng = np.random.default_rng(23)
    q, k, v = rand_head(rng, 37, 6)
    for causal, wl, wr in MASKS:
        p = oracle.attention_probs_head(q, k, 0.45, causal, wl, wr)
        o, lse = oracle.attention_head(q, k, v, 0.45, causal, wl, wr)
        np.testing.assert_allclose(p @ v, o, rtol=0, atol=1e-13)
        s = 0.45 * (q @ k.T)
        vis = p > 0
        np.testing.assert_allclose(p[vis], np.exp(s - lse[:, None])[vis], rtol=1e-13, atol=0)


@pytest.mark.parametrize("mutation", ["scale_dropped", "transposed", "unnormalised"])
def test_planted_probability_mistakes_are_caught(monkeypatch, mutation):
    rng = np.random.default_rng(15)
    q, k, _ = rand_head(rng, 9, 4)
    scale = 0.8
    pb, _ = brute_force(q.tolist(), k.tolist(), np.eye(9).tolist(), scale, True, -1, -1)
    if mutation == "scale_dropped":
        p = sdpa_fp64.attention_probs_head(q, k, 1.0, True)
    elif mutation == "transposed":
        p = sdpa_fp64.attention_probs_head(k, q, scale, True)
    else:
        monkeypatch.setattr(sdpa_fp64, "_softmax_block", _buggy_softmax_no_norm)
        p = sdpa_fp64.attention_probs_head(q, k, scale, True)
    assert not np.allclose(p, pb, rtol=0, atol=1e-14), f"planted mistake {mutation} slipped past the pin"
