"""Pins for the float64 backward oracle, against things other than itself.

  * torch autograd in float64 through torch's scaled_dot_product_attention
    (the routine of the "Flash Attention | Hermes Skill" Quick start), with
    boolean masks for every mask kind and enable_gqa for shared K/V heads;
  * central finite differences of the loss sum(dO * O), with O from the
    forward oracle, on tiny shapes;
  * invariants: dK sums to zero over the keys (each row's dS sums to zero
    over its visible keys), dV sums over the keys to the sum of dO over the
    query rows that see a key, delta_i = dO_i . O_i;
  * planted mistakes that must fail the autograd pin.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import sdpa_bwd_fp64
from oracle.sdpa_bwd_fp64 import attention_backward, attention_backward_head

MASKS = [
    (False, -1, -1),
    (True, -1, -1),
    (False, 3, 2),
    (True, 4, -1),
    (True, 0, 0),
    (False, 1, -1),
]


def torch_grads(q, k, v, do, scale, causal, wl, wr, gqa=False):
    """Gradients by autograd through torch SDPA (float64, CPU), BHSD arrays."""
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    nq, nk = q.shape[2], k.shape[2]
    mask = torch.from_numpy(oracle.visible(np.arange(nq)[:, None], np.arange(nk)[None, :], nk, causal, wl, wr))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale, enable_gqa=gqa)
    (o * torch.from_numpy(do)).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def rand(rng, *shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("causal,wl,wr", MASKS)
@pytest.mark.parametrize("n,d", [(1, 4), (7, 5), (33, 16)])
def test_matches_torch_autograd(n, d, causal, wl, wr):
    rng = np.random.default_rng(100 + n + d)
    q, k, v, do = (rand(rng, 2, 3, n, d) for _ in range(4))
    dq, dk, dv, _ = attention_backward(q, k, v, do, 0.45, causal, (wl, wr), "bhsd")
    tq, tk, tv = torch_grads(q, k, v, do, 0.45, causal, wl, wr)
    for a, b in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11)


@pytest.mark.parametrize("hk", [1, 2, 4])
@pytest.mark.parametrize("causal", [False, True])
def test_shared_kv_heads_match_torch_autograd(hk, causal):
    rng = np.random.default_rng(120 + hk)
    q, do = rand(rng, 2, 8, 29, 8), rand(rng, 2, 8, 29, 8)
    k, v = rand(rng, 2, hk, 29, 8), rand(rng, 2, hk, 29, 8)
    dq, dk, dv, _ = attention_backward(q, k, v, do, 0.3, causal, (-1, -1), "bhsd")
    tq, tk, tv = torch_grads(q, k, v, do, 0.3, causal, -1, -1, gqa=True)
    for a, b in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11)


@pytest.mark.parametrize("causal,wl,wr", [(False, -1, -1), (True, -1, -1), (False, 1, 1)])
def test_finite_differences(causal, wl, wr):
    # derivative of L = sum(dO * O) by central differences on the forward oracle
    rng = np.random.default_rng(7)
    n, d, scale = 5, 3, 0.7
    q, k, v, do = (rand(rng, n, d) for _ in range(4))

    def loss(q_, k_, v_):
        o, _ = oracle.attention_head(q_, k_, v_, scale, causal, wl, wr)
        return float(np.sum(o * do))

    dq, dk, dv, _ = attention_backward_head(q, k, v, do, scale, causal, wl, wr)
    h = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        num = np.zeros_like(grad)
        for idx in np.ndindex(*grad.shape):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=0, atol=2e-8)


@pytest.mark.parametrize("causal,wl,wr", MASKS)
def test_invariants(causal, wl, wr):
    rng = np.random.default_rng(31)
    n, d = 40, 8
    q, k, v, do = (rand(rng, n, d) for _ in range(4))
    dq, dk, dv, delta = attention_backward_head(q, k, v, do, 0.6, causal, wl, wr)
    # every row sees at least its diagonal key here
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-12)
    o, _ = oracle.attention_head(q, k, v, 0.6, causal, wl, wr)
    np.testing.assert_allclose(delta, np.sum(do * o, axis=1), atol=1e-12)


def test_layout_and_blocking(monkeypatch):
    rng = np.random.default_rng(9)
    q, k, v, do = (rand(rng, 2, 50, 3, 8) for _ in range(4))     # BSHD
    g1 = attention_backward(q, k, v, do, 0.5, True, (-1, -1), "bshd")
    g2 = attention_backward(*(np.swapaxes(x, 1, 2) for x in (q, k, v, do)), 0.5, True, (-1, -1), "bhsd")
    for a, b in zip(g1[:3], g2[:3]):
        np.testing.assert_allclose(a, np.swapaxes(b, 1, 2), rtol=0, atol=1e-13)
    # tiny row blocks give the same result as one block
    monkeypatch.setattr(oracle.sdpa_fp64, "_MAX_BLOCK_ELEMS", 64)
    g3 = attention_backward(q, k, v, do, 0.5, True, (-1, -1), "bshd")
    for a, b in zip(g1, g3):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Planted mistakes (in test doubles only): each must fail the autograd pin.
# ---------------------------------------------------------------------------

def _bwd_without_delta(q, k, v, do, scale, causal=False, wl=-1, wr=-1):
    nq, nk = len(q), len(k)
    s = (q @ k.T) * scale
    vis = oracle.visible(np.arange(nq)[:, None], np.arange(nk)[None, :], nk, causal, wl, wr)
    s = np.where(vis, s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    ds = p * (do @ v.T)                       # forgot the "- D_i" term
    return scale * ds @ k, scale * ds.T @ q, p.T @ do


def _bwd_untransposed_dv(q, k, v, do, scale, causal=False, wl=-1, wr=-1):
    dq, dk, dv, _ = attention_backward_head(q, k, v, do, scale, causal, wl, wr)
    nq, nk = len(q), len(k)
    s = np.where(oracle.visible(np.arange(nq)[:, None], np.arange(nk)[None, :], nk, causal, wl, wr),
                 (q @ k.T) * scale, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return dq, dk, p @ do                     # P dO instead of P^T dO


@pytest.mark.parametrize("mutation", ["no_delta", "untransposed_dv", "unscaled_dk"])
def test_planted_mistakes_are_caught(mutation):
    rng = np.random.default_rng(77)
    n, d, scale = 12, 4, 0.8
    q, k, v, do = (rand(rng, n, d) for _ in range(4))
    if mutation == "no_delta":
        g = _bwd_without_delta(q, k, v, do, scale, True)
    elif mutation == "untransposed_dv":
        g = _bwd_untransposed_dv(q, k, v, do, scale, True)
    else:
        dq, dk, dv, _ = attention_backward_head(q, k, v, do, scale, True)
        g = (dq, dk / scale, dv)
    t = torch_grads(q[None, None], k[None, None], v[None, None], do[None, None], scale, True, -1, -1)
    caught = any(not np.allclose(a, b[0, 0], rtol=0, atol=1e-9) for a, b in zip(g, t))
    assert caught, f"planted mistake {mutation} slipped past the autograd pin"
