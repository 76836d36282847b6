"""GPU parity of the backward kernels against the float64 gradient oracle.

Tolerance, derived from where the kernels round (u = 2^-8 for bf16, 2^-11 for
fp16, the unit roundoff of the 16-bit format):
  * P is rounded to 16 bits before dV = P^T dO; sums run in fp32.
  * D_i = dO_i . O_i is computed from the 16-bit O the forward stored:
    |dD_i| <= u sum_d |dO_id O_id|.
  * dS = P (dP - D) is rounded to 16 bits before dK = scale dS^T Q and
    dQ = scale dS K, so with E_ij = P_ij u sum_d |dO_id O_id| + u |dS_ij|:
        |d dV|  <= 2 u (P^T |dO|) + ulp(dV)
        |d dK|  <= 2 scale (E^T |Q|) + ulp(dK)
        |d dQ|  <= 2 scale (E |K|) + ulp(dQ)
    (factor 2: margin for the fp32 exp, the fp32 sums and the rounding of
    P's own error), plus 1e-6 absolute for fp32 accumulation.
  * delta: |d delta_i| <= 1e-5 (1 + sum_d |dO_id O_id|) (fp32 sum of exact
    products of 16-bit values).
The bound is computed elementwise from the oracle's float64 P, dP, D.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from exact_attention_04_amd import attention, attention_backward
from exact_attention_04_amd.workloads import small_case, torch_dtype

pytestmark = pytest.mark.gpu

U = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
MASKS = {
    "none": (False, (-1, -1)),
    "causal": (True, (-1, -1)),
    "w17_5": (False, (17, 5)),
    "causal_w100": (True, (100, -1)),
    "diag": (False, (0, 0)),
}


def ulp16(x, dtype):
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    if dtype == "bf16":
        return np.ldexp(1.0, (np.maximum(e, -126) - 7).astype(np.int64))
    return np.ldexp(1.0, (np.maximum(e, -14) - 10).astype(np.int64))


def to_bhsd(x, layout):
    return x if layout == "bhsd" else np.swapaxes(x, 1, 2)


def head_bounds(q, k, v, do, o, scale, causal, window, dtype, p=None):
    """Elementwise error bounds of one query head's contributions, all float64
    [N, D] arrays: (dq bound, this head's share of the dk and dv bounds, the
    delta bound)."""
    u = U[dtype]
    if p is None:
        p = oracle.attention_probs_head(q, k, scale, causal, window[0], window[1])
    dp = do @ v.T
    dsum = np.sum(np.abs(do * o), axis=1)
    d_exact = np.sum(do * (p @ v), axis=1)
    e = p * (u * dsum)[:, None] + u * np.abs(p * (dp - d_exact[:, None]))
    return (2 * scale * (e @ np.abs(k)), 2 * scale * (e.T @ np.abs(q)), 2 * u * (p.T @ np.abs(do)),
            1e-5 * (1 + dsum))


def bounds(qf, kf, vf, dof, o16f, scale, causal, window, layout, dtype):
    """Elementwise error bounds for dq, dk, dv (input layout) and delta."""
    q, k, v, do, o = (to_bhsd(x, layout) for x in (qf, kf, vf, dof, o16f))
    B, H, N, D = q.shape
    Hk = k.shape[1]
    bq = np.zeros_like(q)
    bk = np.zeros_like(k)
    bv = np.zeros_like(v)
    bd = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            g = oracle.kv_head_of(h, H, Hk)
            hq, hk, hv, hd = head_bounds(q[b, h], k[b, g], v[b, g], do[b, h], o[b, h], scale, causal, window, dtype)
            bq[b, h] = hq
            bk[b, g] += hk
            bv[b, g] += hv
            bd[b, h] = hd
    back = (lambda x: x) if layout == "bhsd" else (lambda x: np.swapaxes(x, 1, 2))
    return back(bq) + 1e-6, back(bk) + 1e-6, back(bv) + 1e-6, bd


def f64(t):
    return t.to(torch.float64).cpu().numpy()


def check_bwd(B, H, Hk, N, D, dtype, mask, layout, seed, use_gpu_forward=False):
    # mask: a name in MASKS or a (causal, (window_left, window_right)) pair
    causal, window = MASKS[mask] if isinstance(mask, str) else mask
    inp = small_case(B, H, N, D, dtype, layout, seed, heads_kv=Hk)
    td = torch_dtype(dtype)
    rng = np.random.default_rng(seed + 1)
    do = torch.from_numpy(rng.standard_normal(tuple(inp.q.shape)).astype(np.float32)).to(td)
    qf, kf, vf, dof = (f64(t) for t in (inp.q, inp.k, inp.v, do))
    scale = 1.0 / math.sqrt(D)
    q, k, v, dog = (t.cuda() for t in (inp.q, inp.k, inp.v, do))
    if use_gpu_forward:
        o, lse = attention(q, k, v, causal=causal, window_size=window, layout=layout)
    else:
        o_ref, lse_ref = oracle.attention(qf, kf, vf, scale, causal, window, layout)
        o = torch.from_numpy(o_ref).to(td).cuda()
        lse = torch.from_numpy(lse_ref).to(torch.float32).cuda()
    dq, dk, dv, delta = attention_backward(q, k, v, o, dog, lse, causal=causal, window_size=window, layout=layout)
    torch.cuda.synchronize()
    o16f = f64(o)
    dq_r, dk_r, dv_r, _ = oracle.attention_backward(qf, kf, vf, dof, scale, causal, window, layout)
    bq, bk, bv, bd = bounds(qf, kf, vf, dof, o16f, scale, causal, window, layout, dtype)
    if use_gpu_forward:
        # the forward's own O error enters D: |dD_i| <= sum_d |dO_id| |dO_i|, with
        # |dO| bounded by the forward's tolerance (2e-3 + one output ulp)
        o_exact, _ = oracle.attention(qf, kf, vf, scale, causal, window, layout)
        tol_o = 2e-3 + ulp16(o_exact, dtype)
        extra = np.sum(np.abs(dof) * tol_o, axis=-1)        # per query row, input layout [.., N, H] or [.., H, N]
        bq, bk = widen_for_forward_error(qf, kf, dof, scale, causal, window, layout, extra, bq, bk)
    res = {}
    for name, got, ref, bnd in (("dq", dq, dq_r, bq), ("dk", dk, dk_r, bk), ("dv", dv, dv_r, bv)):
        g = f64(got)
        assert np.isfinite(g).all(), f"{name} not finite"
        err = np.abs(g - ref)
        lim = bnd + ulp16(ref, dtype)
        worst = float((err - lim).max())
        res[name] = (float(err.max()), float((err / lim).max()))
        assert worst <= 0, f"{name}: error exceeds the bound by {worst:.3g} (max err {err.max():.3g}, ratio {res[name][1]:.3g})"
    d_exact = np.sum(dof * o16f, axis=-1)
    d_exact = d_exact if layout == "bhsd" else np.swapaxes(d_exact, 1, 2)
    derr = np.abs(f64(delta) - d_exact)
    assert (derr <= bd).all(), f"delta: max err {derr.max():.3g}"
    return res


def widen_for_forward_error(qf, kf, dof, scale, causal, window, layout, extra, bq, bk):
    """Add the effect of the forward's O error on D to the dq and dk bounds."""
    q, k = to_bhsd(qf, layout), to_bhsd(kf, layout)
    ex = extra if layout == "bhsd" else np.swapaxes(extra, 1, 2)       # [B, H, N]
    B, H, N, D = q.shape
    Hk = k.shape[1]
    bq = to_bhsd(bq, layout).copy()
    bk = to_bhsd(bk, layout).copy()
    for b in range(B):
        for h in range(H):
            g = oracle.kv_head_of(h, H, Hk)
            p = oracle.attention_probs_head(q[b, h], k[b, g], scale, causal, window[0], window[1])
            e = 2 * p * ex[b, h][:, None]
            bq[b, h] += scale * (e @ np.abs(k[b, g]))
            bk[b, g] += scale * (e.T @ np.abs(q[b, h]))
    back = (lambda x: x) if layout == "bhsd" else (lambda x: np.swapaxes(x, 1, 2))
    return back(bq), back(bk)


@pytest.mark.parametrize("mask", list(MASKS))
@pytest.mark.parametrize("n", [1, 63, 64, 65, 130, 333])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_bwd_small_sweep(dtype, d, n, mask):
    seed = 3000 + 10 * n + d + 7 * list(MASKS).index(mask) + (0 if dtype == "f16" else 100000)
    check_bwd(2, 3, 3, n, d, dtype, mask, "bshd", seed)


@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
@pytest.mark.parametrize("heads,heads_kv", [(4, 2), (4, 1), (6, 3)])
@pytest.mark.parametrize("mask", ["none", "causal", "w17_5"])
def test_bwd_shared_kv_and_layouts(heads, heads_kv, mask, layout):
    check_bwd(1, heads, heads_kv, 200, 128, "bf16", mask, layout, 4000 + heads * 10 + heads_kv)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64)])
@pytest.mark.parametrize("mask", ["causal", "none"])
def test_bwd_after_gpu_forward(dtype, d, mask):
    # the whole pipeline: our forward's O and LSE feed the backward
    check_bwd(2, 4, 2, 300, d, dtype, mask, "bshd", 4500 + d, use_gpu_forward=True)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_bwd_long_sequence(dtype):
    # one head pair at N=2048: several 128-key blocks and query tiles per workgroup
    check_bwd(1, 2, 1, 2048, 128, dtype, "causal", "bshd", 4600)


@pytest.mark.parametrize("batch,heads", [(1, 8), (2, 8), (4, 8), (5, 8)])
@pytest.mark.parametrize("mask", ["causal", "none"])
def test_bwd_head_groups_per_xcd(batch, heads, mask):
    # (batch, head) counts of 8, 16, 32 and 40: the kernels' work order puts
    # groups of 1, 2, 4 and 1 heads on each of the 8 XCDs; every workgroup's
    # unit and head must still be distinct
    check_bwd(batch, heads, heads, 300, 64, "f16", mask, "bshd", 4700 + batch)


@pytest.mark.parametrize("batch", [1, 2, 3])
def test_bwd_shared_kv_head_groups_per_xcd(batch):
    # (batch, K/V head) counts of 8, 16 and 24 with four query heads each: the
    # dQ kernel takes the query heads of one (8, 24) or two (16) K/V heads per
    # XCD at a time, the dK/dV kernel groups of K/V heads
    check_bwd(batch, 32, 8, 300, 64, "bf16", "causal", "bshd", 4800 + batch)


def test_bwd_deterministic():
    g = torch.Generator(device="cuda").manual_seed(5)
    q, k, v, do = (torch.randn((2, 1000, 8, 128), device="cuda", generator=g).to(torch.bfloat16) for _ in range(4))
    o, lse = attention(q, k, v, causal=True)
    r1 = attention_backward(q, k, v, o, do, lse, causal=True)
    for _ in range(3):
        r2 = attention_backward(q, k, v, o, do, lse, causal=True)
        torch.cuda.synchronize()
        for a, b in zip(r1, r2):
            assert torch.equal(a, b)


def test_bwd_empty_and_errors():
    x = torch.empty(0, 16, 2, 64, dtype=torch.float16, device="cuda")
    l = torch.empty(0, 2, 16, dtype=torch.float32, device="cuda")
    dq, dk, dv, delta = attention_backward(x, x, x, x, x, l)
    assert dq.shape == x.shape
    q = torch.zeros(1, 8, 2, 64, dtype=torch.float16, device="cuda")
    lse = torch.zeros(1, 2, 8, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        attention_backward(q.float(), q.float(), q.float(), q.float(), q.float(), lse)
    with pytest.raises(ValueError):   # k and v with different head counts
        attention_backward(q, q[:, :, :1].expand(1, 8, 3, 64), q, q, q, lse)
    # caller buffers must match what the kernels write (and lse must be fp32)
    f32 = dict(dtype=torch.float32, device="cuda")
    bad = [
        dict(dq=torch.empty(1, 8, 2, 32, dtype=torch.float16, device="cuda")),
        dict(dk=torch.empty(1, 8, 2, 64, dtype=torch.bfloat16, device="cuda")),
        dict(delta=torch.empty(1, 2, 8, dtype=torch.float16, device="cuda")),
        dict(delta=torch.empty(1, 8, 2, **f32).transpose(1, 2)),
    ]
    for kw in bad:
        with pytest.raises(ValueError):
            attention_backward(q, q, q, q, q, lse, **kw)
    with pytest.raises(ValueError):
        attention_backward(q, q, q, q, q, lse.to(torch.bfloat16))


@pytest.mark.parametrize("name", ["sdpa_b4h32n4096d128_bf16_causal", "gqa_b4h32kv8n4096d128_bf16_causal"])
def test_bwd_workload_full_size(name):
    # The timed backward pipeline at full size (the GPU forward's O and LSE,
    # then the backward, B=4 H=32 N=4096 d=128 bf16 causal, BSHD), compared
    # element by element on whole sampled heads: the first and last (batch,
    # K/V head) and two random ones; with shared K/V heads every query head
    # of those groups, whose dK and dV sum over the group.
    from exact_attention_04_amd.workloads import WORKLOADS, make_inputs
    w = WORKLOADS[name]
    inp = make_inputs(w)
    td = torch_dtype(w.dtype)
    rng = np.random.default_rng(w.seed + 7)
    do = torch.from_numpy(rng.standard_normal(tuple(inp.q.shape)).astype(np.float32)).to(td)
    scale, causal, window = w.softmax_scale, w.causal, (w.window_left, w.window_right)
    q, k, v, dog = (t.cuda() for t in (inp.q, inp.k, inp.v, do))
    o, lse = attention(q, k, v, causal=causal, window_size=window, softmax_scale=scale, layout=w.layout)
    dq, dk, dv, delta = attention_backward(q, k, v, o, dog, lse, causal=causal, window_size=window,
                                           softmax_scale=scale, layout=w.layout)
    torch.cuda.synchronize()
    assert all(bool(torch.isfinite(t.float()).all()) for t in (dq, dk, dv, delta))
    group = w.heads // w.kv_heads
    picks = [(0, 0), (w.batch - 1, w.kv_heads - 1)]
    picks += [(int(rng.integers(w.batch)), int(rng.integers(w.kv_heads))) for _ in range(2)]
    for b, g in picks:
        kf, vf = f64(inp.k[b, :, g]), f64(inp.v[b, :, g])
        dk_ref, dv_ref = np.zeros_like(kf), np.zeros_like(vf)
        bk, bv = np.zeros_like(kf), np.zeros_like(vf)
        for h in range(g * group, (g + 1) * group):
            qf, dof, o16 = f64(inp.q[b, :, h]), f64(do[b, :, h]), f64(o[b, :, h])
            dq_r, dk_r, dv_r, _ = oracle.attention_backward_head(qf, kf, vf, dof, scale, causal, *window)
            p = oracle.attention_probs_head(qf, kf, scale, causal, *window)
            hq, hk, hv, hd = head_bounds(qf, kf, vf, dof, o16, scale, causal, window, w.dtype, p=p)
            # the forward's own O error enters D (bounded by the forward's
            # tolerance, 2e-3 plus one output ulp), as in the pipeline tests
            o_exact, _ = oracle.attention_head(qf, kf, vf, scale, causal, *window)
            ex = np.sum(np.abs(dof) * (2e-3 + ulp16(o_exact, w.dtype)), axis=1)
            e = 2 * p * ex[:, None]
            hq = hq + scale * (e @ np.abs(kf)) + 1e-6
            hk = hk + scale * (e.T @ np.abs(qf))
            dk_ref += dk_r
            dv_ref += dv_r
            bk += hk
            bv += hv
            err = np.abs(f64(dq[b, :, h]) - dq_r)
            worst = float((err - hq - ulp16(dq_r, w.dtype)).max())
            assert worst <= 0, f"{name} dq (b={b}, h={h}) exceeds its bound by {worst:.3g}"
            d_exact = np.sum(dof * o16, axis=1)
            assert (np.abs(f64(delta[b, h]) - d_exact) <= hd).all(), f"{name} delta (b={b}, h={h})"
        for nm, got, ref, bnd in (("dk", dk[b, :, g], dk_ref, bk + 1e-6), ("dv", dv[b, :, g], dv_ref, bv + 1e-6)):
            err = np.abs(f64(got) - ref)
            worst = float((err - bnd - ulp16(ref, w.dtype)).max())
            assert worst <= 0, f"{name} {nm} (b={b}, K/V head {g}) exceeds its bound by {worst:.3g}"
        print(name, (b, g), "ok")
