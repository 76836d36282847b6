"""Float64 reference gradients of attention, from the materialised probabilities.

TEST INFRASTRUCTURE ONLY: imported by tests and the benchmark's CPU baseline,
never by the product path.

The pages reach the backward pass through recomputation ("Flash Attention |
Hermes Skill", Quick start: IO-aware tiling and recomputation; the FP8 section
notes that the 16-bit kernels run forward and backward, fp8 forward only).
What is differentiated is the same definition the forward oracle writes out
("standard attention", Workflow 1, Step 2).  For one head, with s_ij the
scaled, masked scores, P_ij = exp(s_ij - LSE_i) and O = P V, and dO the
gradient of a loss with respect to O, the chain rule gives

    dV = P^T dO                        (O_i = sum_j P_ij v_j)
    dP_ij = dO_i . v_j
    D_i = sum_j P_ij dP_ij = dO_i . O_i
    dS_ij = P_ij (dP_ij - D_i)         (softmax over each row's visible keys)
    dQ = scale * dS K,   dK = scale * dS^T Q

Masked pairs have P_ij = 0, so they carry no gradient.  With fewer K/V heads
than query heads (``kv_head_of`` in the forward oracle), a shared K/V head's
gradient is the sum over the query heads that read it.

Work layout: query rows are processed in blocks (probabilities materialised
for a block of rows over the keys they can see); dK and dV sum the blocks'
contributions.  No tiling over keys, no recomputation tricks.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np

from .sdpa_fp64 import _key_span, _row_blocks, _softmax_block, _to_bhsd, kv_head_of, visible

__all__ = ["attention_backward_head", "attention_backward", "attention_backward_parallel"]


def attention_backward_head(q, k, v, do, scale: float, causal: bool = False, window_left: int = -1,
                            window_right: int = -1):
    """One head: q, do [Nq, D], k, v [Nk, D] -> (dq, dk, dv, delta) in float64.

    ``delta`` is D_i = dO_i . O_i for every query row (0 for a row that sees no
    key).
    """
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    nq, nk = q.shape[0], k.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    delta = np.zeros(nq, dtype=np.float64)
    rows = np.arange(nq, dtype=np.int64)
    for blk in _row_blocks(rows, nk, causal, window_left, window_right):
        r0, r1 = int(blk[0]), int(blk[-1]) + 1
        lo, hi = _key_span(r0, r1, nk, causal, window_left, window_right)
        if hi <= lo:
            continue
        s = (q[blk] @ k[lo:hi].T) * np.float64(scale)
        vis = visible(blk[:, None], np.arange(lo, hi)[None, :], nk, causal, window_left, window_right)
        s = np.where(vis, s, -np.inf)
        p, _, _ = _softmax_block(s)                  # rows with no key: all zeros
        o = p @ v[lo:hi]
        dv[lo:hi] += p.T @ do[blk]
        dp = do[blk] @ v[lo:hi].T
        d = np.sum(do[blk] * o, axis=1)
        ds = p * (dp - d[:, None])
        dq[blk] = np.float64(scale) * (ds @ k[lo:hi])
        dk[lo:hi] += np.float64(scale) * (ds.T @ q[blk])
        delta[blk] = d
    return dq, dk, dv, delta


def attention_backward(q, k, v, do, scale: Optional[float] = None, causal: bool = False,
                       window: Tuple[int, int] = (-1, -1), layout: str = "bshd"):
    """Batched gradients over 4-D arrays in ``layout``; k and v may have fewer heads.

    Returns (dq, dk, dv) in the input layout (float64) and delta as [B, Hq, Nq].
    """
    qh, kh, vh, doh = (_to_bhsd(np.asarray(x), layout) for x in (q, k, v, do))
    B, H, Nq, D = qh.shape
    Hk, Nk = kh.shape[1], kh.shape[2]
    if vh.shape[1] != Hk or doh.shape != qh.shape:
        raise ValueError("shape mismatch")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    wl, wr = int(window[0]), int(window[1])
    dq = np.zeros((B, H, Nq, D), dtype=np.float64)
    dk = np.zeros((B, Hk, Nk, D), dtype=np.float64)
    dv = np.zeros((B, Hk, Nk, vh.shape[3]), dtype=np.float64)
    delta = np.zeros((B, H, Nq), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            g = kv_head_of(h, H, Hk)
            dq1, dk1, dv1, d1 = attention_backward_head(qh[b, h], kh[b, g], vh[b, g], doh[b, h], scale, causal,
                                                        wl, wr)
            dq[b, h] = dq1
            dk[b, g] += dk1
            dv[b, g] += dv1
            delta[b, h] = d1
    if layout == "bshd":
        dq, dk, dv = (np.swapaxes(x, 1, 2) for x in (dq, dk, dv))
    return dq, dk, dv, delta


def _pool_task(args):
    q, k, v, do, scale, causal, wl, wr = args
    return attention_backward_head(q, k, v, do, scale, causal, wl, wr)


def attention_backward_parallel(head_arrays, scale: float, causal: bool, window: Tuple[int, int], pool):
    """``attention_backward_head`` over a list of (q, k, v, dO) heads on a ready process pool."""
    tasks = [(q, k, v, do, scale, causal, int(window[0]), int(window[1])) for (q, k, v, do) in head_arrays]
    return list(pool.map(_pool_task, tasks))
