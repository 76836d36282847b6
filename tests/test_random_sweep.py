"""GPU parity on a seeded random sweep of launch shapes.

Forward: each case draws a batch, head counts (query heads a multiple of
the K/V heads), a sequence length, a head dim, an input type, a layout, a
mask (causal or not, window edges or none) and, for fp8, the format of P,
and compares the whole output and LSE with the float64 oracle, as the other
parity tests do.  The sizes span the planner's configurations (the plain
128-row one, key streams of 128, 64 and 32 rows, the key split for fp8) in
combinations the targeted tests do not enumerate.

Backward: the same kind of draw for fp16/bf16, checked element by element
against the float64 gradient oracle with the elementwise bounds of
test_bwd.py, from the oracle's O and LSE or from the GPU forward's.
"""
import numpy as np
import pytest
import torch

from exact_attention_04_amd import plan
from exact_attention_04_amd.workloads import small_case
from parity_helpers import full_check, upload
from test_bwd import check_bwd

pytestmark = pytest.mark.gpu


def _cases(count=40, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        dtype = str(rng.choice(["f16", "bf16", "fp8"], p=[0.4, 0.4, 0.2]))
        d = 128 if dtype == "fp8" else int(rng.choice([64, 128]))
        layout = str(rng.choice(["bshd", "bhsd"]))
        heads_kv = int(rng.choice([1, 2, 4, 8]))
        heads = heads_kv * int(rng.choice([1, 1, 2, 4]))
        batch = int(rng.integers(1, 5))
        n = int(rng.integers(1, 1600))
        # keep the float64 oracle's work per case small
        if batch * heads * n * n > 3e7:
            continue
        causal = bool(rng.random() < 0.5)
        wl = int(rng.choice([-1, -1, int(rng.integers(0, 400))]))
        wr = -1 if causal else int(rng.choice([-1, -1, int(rng.integers(0, 400))]))
        pv8 = dtype == "fp8" and bool(rng.random() < 0.5)
        out.append((batch, heads, heads_kv, n, d, dtype, layout, causal, (wl, wr), pv8, 9900 + len(out)))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "b{}h{}k{}n{}d{}_{}_{}_c{}_w{}_{}_{}".format(
    c[0], c[1], c[2], c[3], c[4], c[5], c[6], int(c[7]), c[8][0], c[8][1], "pv8" if c[9] else "pv16"))
def test_random_shapes(case):
    batch, heads, heads_kv, n, d, dtype, layout, causal, window, pv8, seed = case
    inp = small_case(batch, heads, n, d, dtype, layout, seed, heads_kv=heads_kv)
    q, k, v = upload(inp)
    pv = torch.float8_e4m3fn if pv8 else None
    o = torch.empty(q.shape, dtype=torch.bfloat16 if dtype == "fp8" else q.dtype, device=q.device)
    info = plan(q, k, v, o, causal=causal, window_size=window, layout=layout,
                descale=inp.descale if dtype == "fp8" else None, pv_dtype=pv)
    full_check(inp, dtype, causal=causal, window=window, layout=layout, pv_dtype=pv,
               what=f"{case} kernel {info.kernel.decode()} splits {info.splits}")


def _bwd_cases(count=30, seed=20261204):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        dtype = str(rng.choice(["f16", "bf16"]))
        d = int(rng.choice([64, 128]))
        layout = str(rng.choice(["bshd", "bhsd"]))
        heads_kv = int(rng.choice([1, 2, 4]))
        heads = heads_kv * int(rng.choice([1, 2, 3]))
        batch = int(rng.integers(1, 4))
        n = int(rng.integers(1, 700))
        if batch * heads * n * n > 6e6:
            continue
        causal = bool(rng.random() < 0.5)
        wl = int(rng.choice([-1, -1, int(rng.integers(0, 300))]))
        wr = -1 if causal else int(rng.choice([-1, -1, int(rng.integers(0, 300))]))
        gpu_fwd = bool(rng.random() < 0.3)
        out.append((batch, heads, heads_kv, n, d, dtype, layout, causal, (wl, wr), gpu_fwd, 7700 + len(out)))
    return out


@pytest.mark.parametrize("case", _bwd_cases(), ids=lambda c: "b{}h{}k{}n{}d{}_{}_{}_c{}_w{}_{}_{}".format(
    c[0], c[1], c[2], c[3], c[4], c[5], c[6], int(c[7]), c[8][0], c[8][1], "gpufwd" if c[9] else "oraclefwd"))
def test_random_shapes_backward(case):
    batch, heads, heads_kv, n, d, dtype, layout, causal, window, gpu_fwd, seed = case
    check_bwd(batch, heads, heads_kv, n, d, dtype, (causal, window), layout, seed, use_gpu_forward=gpu_fwd)
