"""Float64 reference attention that materialises the score matrix.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the CPU
baseline of the benchmark, never by the product path.

What it computes (the plain definition the method must reproduce):

    O = softmax(Q K^T * scale + mask) V

This is the "standard attention" the pages replace with one fused call
("Flash Attention | Hermes Skill", Workflow 1, Step 2: softmax(q @ k^T /
sqrt(d_k)) @ v, and Step 4, the same with ``/ 8.0`` at d=64).  The fused
kernel computes "exactly the same attention" ("FlashAttention",
aiunderstanding.org, section "Djupdykning"), so the oracle is that definition
written out, not the tiled algorithm: for each query row i and key j

    s_ij = scale * sum_d q[i,d] k[j,d]            (float64, on stored values)
    s_ij = -inf        where key j is not visible from row i
    m_i = max_j s_ij,  e_ij = exp(s_ij - m_i),  l_i = sum_j e_ij
    O[i,:] = sum_j (e_ij / l_i) v[j,:],          LSE_i = m_i + ln(l_i)

Masks ("Flash Attention | Hermes Skill", Quick start: ``causal=True``;
Workflow 2, Steps 2-3: ``window_size=(left, right)``, -1 meaning no limit):
key j is visible from query i iff j < Nk, and j <= i when causal, and
i - left <= j when left >= 0, and j <= i + right when right >= 0.  Windows are
inclusive on both ends; with causal the right side is additionally capped at
i (so a (256, 256) window with causal sees keys [i-256, i]).

Heads: k and v may carry fewer heads than q (multi-query attention, K/V
shared across heads: "Flash Attention | Hermes Skill", Workflow 2, Step 3,
q as [batch, seq, num_q_heads, dim] with k, v as [batch, seq, num_kv_heads,
dim]).  The number of query heads must be a multiple of the number of K/V
heads; see ``kv_head_of`` for which K/V head each query head reads.

Readings where the pages say nothing (each listed in the design notes):
  * LSE is the natural-log logsumexp of the scaled, masked scores.
  * A row with no visible key gets O = 0 and LSE = -inf.  With Nq == Nk the
    diagonal key is always visible, so this does not arise for the GPU path.
  * Masks are aligned top-left (row i, key i on the diagonal).
  * fp8 inputs are dequantised as ``x_q * descale`` before anything else.
  * With Hk K/V heads and Hq = g * Hk query heads, query heads form
    contiguous groups of g: query head h reads K/V head h // g (one K/V head
    for all query heads when Hk = 1).

Work layout: rows are independent by definition, so they are processed in
blocks; per block only keys inside the union of the rows' visible ranges are
materialised.  Keys outside it have e_ij = 0 exactly, so leaving them out does
not change any sum.  The softmax is two-pass (max, then exp/sum) over whole
rows: no running rescale and no tiling over keys.
"""
from __future__ import annotations

import math
import os
from typing import Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "kv_head_of",
    "visible",
    "dequantize_e4m3",
    "attention_head",
    "attention_probs_head",
    "attention",
    "attention_parallel",
]

# Upper bound on the number of float64 score elements materialised at once.
_MAX_BLOCK_ELEMS = 1 << 24


def kv_head_of(h: int, hq: int, hk: int) -> int:
    """The K/V head that query head h reads when q has hq heads and k, v have hk.

    Query heads form contiguous groups of hq // hk (the reading taken where
    the pages only say that fewer K/V heads are shared across the heads).
    """
    if hk < 1 or hq % hk != 0:
        raise ValueError(f"{hq} query heads cannot share {hk} K/V heads")
    return h // (hq // hk)


def visible(i, j, nk: int, causal: bool, window_left: int, window_right: int):
    """Boolean visibility of key j from query i (broadcasts over arrays)."""
    i, j = np.broadcast_arrays(np.asarray(i), np.asarray(j))
    ok = j < nk
    if causal:
        ok = ok & (j <= i)
    if window_left >= 0:
        ok = ok & (j >= i - window_left)
    if window_right >= 0:
        ok = ok & (j <= i + window_right)
    return ok


def dequantize_e4m3(codes, descale: float) -> np.ndarray:
    """Decode OCP 8-bit float E4M3 ("fn": no infinities) codes and multiply by descale.

    Format (OCP 8-bit floating point specification): 1 sign bit, 4 exponent
    bits with bias 7, 3 mantissa bits.  Exponent field 0 is subnormal,
    value (-1)^s * 2^-6 * m/8.  Otherwise (-1)^s * 2^(e-7) * (1 + m/8).  The
    single code pattern S.1111.111 is NaN; there is no infinity, so the
    largest finite magnitude is 2^8 * 1.75 = 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = sign * np.ldexp(m.astype(np.float64) / 8.0, -6)
    nrm = sign * np.ldexp(1.0 + m.astype(np.float64) / 8.0, (e - 7).astype(np.int64))
    val = np.where(e == 0, sub, nrm)
    val = np.where((e == 0xF) & (m == 0x7), np.nan, val)
    return val * np.float64(descale)


def _key_span(r0: int, r1: int, nk: int, causal: bool, wl: int, wr: int) -> Tuple[int, int]:
    """Smallest [lo, hi) that holds every key visible from rows r0..r1-1."""
    lo = 0 if wl < 0 else max(0, r0 - wl)
    hi = nk
    if wr >= 0:
        hi = min(hi, (r1 - 1) + wr + 1)
    if causal:
        hi = min(hi, r1)
    return lo, max(lo, hi)


def _row_blocks(rows: np.ndarray, nk: int, causal: bool, wl: int, wr: int):
    """Split sorted query rows into contiguous-range blocks of bounded score size."""
    step = max(1, min(1024, _MAX_BLOCK_ELEMS // max(nk, 1)))
    start = 0
    n = len(rows)
    while start < n:
        end = min(n, start + step)
        yield rows[start:end]
        start = end


def _softmax_block(s: np.ndarray):
    """Two-pass softmax over the last axis of a masked score block (float64).

    Returns (p, m, l): probabilities, row max and row sum of exp(s - m).
    Rows that are entirely -inf give p = 0, m = -inf, l = 0.
    """
    m = np.max(s, axis=1)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe[:, None])          # exp(-inf) = 0 for masked keys
    l = np.sum(e, axis=1)
    denom = np.where(empty, 1.0, l)
    p = e / denom[:, None]
    return p, m, l


def attention_head(q, k, v, scale: float, causal: bool = False, window_left: int = -1,
                   window_right: int = -1, rows: Optional[Sequence[int]] = None):
    """One head: q [Nq, D], k [Nk, D], v [Nk, Dv] -> (O [R, Dv], LSE [R]) in float64.

    ``rows`` selects which query rows to compute (default: all, in order).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, nk = q.shape[0], k.shape[0]
    rows = np.arange(nq, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    order = np.argsort(rows, kind="stable")
    srows = rows[order]
    o_sorted = np.zeros((len(rows), v.shape[1]), dtype=np.float64)
    lse_sorted = np.full(len(rows), -np.inf, dtype=np.float64)
    pos = 0
    for blk in _row_blocks(srows, nk, causal, window_left, window_right):
        r0, r1 = int(blk[0]), int(blk[-1]) + 1
        lo, hi = _key_span(r0, r1, nk, causal, window_left, window_right)
        nb = len(blk)
        if hi > lo:
            s = (q[blk] @ k[lo:hi].T) * np.float64(scale)
            vis = visible(blk[:, None], np.arange(lo, hi)[None, :], nk, causal, window_left, window_right)
            s = np.where(vis, s, -np.inf)
            p, m, l = _softmax_block(s)
            o_sorted[pos:pos + nb] = p @ v[lo:hi]
            with np.errstate(divide="ignore"):
                lse_sorted[pos:pos + nb] = np.where(np.isfinite(m), m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
        pos += nb
    o = np.empty_like(o_sorted)
    lse = np.empty_like(lse_sorted)
    o[order] = o_sorted
    lse[order] = lse_sorted
    return o, lse


def attention_probs_head(q, k, scale: float, causal: bool = False, window_left: int = -1,
                         window_right: int = -1) -> np.ndarray:
    """The full probability matrix P [Nq, Nk] of one head (small shapes only)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    nq, nk = q.shape[0], k.shape[0]
    s = (q @ k.T) * np.float64(scale)
    vis = visible(np.arange(nq)[:, None], np.arange(nk)[None, :], nk, causal, window_left, window_right)
    s = np.where(vis, s, -np.inf)
    p, _, _ = _softmax_block(s)
    return p


def _to_bhsd(x: np.ndarray, layout: str) -> np.ndarray:
    if layout == "bhsd":
        return x
    if layout == "bshd":
        return np.swapaxes(x, 1, 2)
    raise ValueError(f"unknown layout {layout!r}")


def attention(q, k, v, scale: Optional[float] = None, causal: bool = False,
              window: Tuple[int, int] = (-1, -1), layout: str = "bshd",
              rows: Optional[Sequence[int]] = None,
              heads: Optional[Sequence[Tuple[int, int]]] = None):
    """Batched attention over 4-D arrays in ``layout`` ("bshd" or "bhsd").

    k and v may have fewer heads than q (``kv_head_of``).

    Returns (O, LSE).  With ``heads=None`` and ``rows=None``: O in the input
    layout (float64) and LSE as [B, H, Nq].  With ``heads`` (a list of
    (b, h) pairs) and/or ``rows``: O as [len(heads), R, D] and LSE as
    [len(heads), R], for the listed heads in order.
    ``scale=None`` means 1/sqrt(D) (the pages' "Auto-scale").
    """
    qh, kh, vh = (_to_bhsd(np.asarray(x), layout) for x in (q, k, v))
    B, H, Nq, D = qh.shape
    Hk = kh.shape[1]
    if vh.shape[1] != Hk:
        raise ValueError("k and v must have the same number of heads")
    kv = [kv_head_of(h, H, Hk) for h in range(H)]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    wl, wr = int(window[0]), int(window[1])
    if heads is None and rows is None:
        o = np.empty((B, H, Nq, vh.shape[3]), dtype=np.float64)
        lse = np.empty((B, H, Nq), dtype=np.float64)
        for b in range(B):
            for h in range(H):
                o[b, h], lse[b, h] = attention_head(qh[b, h], kh[b, kv[h]], vh[b, kv[h]], scale, causal, wl, wr)
        if layout == "bshd":
            o = np.swapaxes(o, 1, 2)
        return o, lse
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
    outs, lses = [], []
    for (b, h) in heads:
        o1, l1 = attention_head(qh[b, h], kh[b, kv[h]], vh[b, kv[h]], scale, causal, wl, wr, rows)
        outs.append(o1)
        lses.append(l1)
    return np.stack(outs), np.stack(lses)


def _pool_worker_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover - threadpoolctl is optional
        pass


def _pool_task(args):
    q, k, v, scale, causal, wl, wr = args
    return attention_head(q, k, v, scale, causal, wl, wr)


def attention_parallel(head_arrays, scale: float, causal: bool, window: Tuple[int, int],
                       processes: Optional[int] = None, pool=None):
    """Run ``attention_head`` over a list of (q, k, v) heads in a process pool.

    One process per core, one BLAS thread per process.  Returns the list of
    (O, LSE) per head.  ``pool`` may be a ready ``ProcessPoolExecutor`` (so a
    caller can time the work without the pool start-up).
    """
    import concurrent.futures as cf
    import multiprocessing as mp

    tasks = [(q, k, v, scale, causal, int(window[0]), int(window[1])) for (q, k, v) in head_arrays]
    own = pool is None
    if own:
        n = processes or len(os.sched_getaffinity(0))
        pool = cf.ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn"),
                                      initializer=_pool_worker_init)
    try:
        return list(pool.map(_pool_task, tasks))
    finally:
        if own:
            pool.shutdown()


def make_pool(processes: int):
    """A spawn-context process pool with one BLAS thread per worker."""
    import concurrent.futures as cf
    import multiprocessing as mp
    return cf.ProcessPoolExecutor(max_workers=processes, mp_context=mp.get_context("spawn"),
                                  initializer=_pool_worker_init)
