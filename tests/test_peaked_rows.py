"""GPU parity on peaked rows: a few keys hold most of a query row's weight.

The fused kernel must give the same attention as the materialised definition
("FlashAttention", aiunderstanding.org, Översikt and Djupdykning) within the
tolerances of the other parity tests, including rows whose softmax is not
spread over many keys.  There the 16-bit rounding of P does not average out:
a dominant key that is not the row's reference maximum carries a relative
rounding error of up to 2^-8 (bf16) straight into O.  These inputs put such
keys in tiles without any mask element (a row's first visible tile, or one
further along), at several magnitudes of V, with the two dominant keys'
values of opposite sign so that O itself is small and its format's ulp gives
no slack.

Each case compares every element of O and LSE with the float64 oracle.
"""
import numpy as np
import pytest
import torch

from exact_attention_04_amd.workloads import Inputs, torch_dtype
from parity_helpers import full_check

pytestmark = pytest.mark.gpu


def _stored(q, k, v, dtype):
    td = torch_dtype(dtype)
    return Inputs(*(torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(td) for x in (q, k, v)),
                  (1.0, 1.0, 1.0))


def peaked_pairs(n, d, vmag, key_base, seed):
    """32 query rows near the end of the sequence, row j dominated by keys
    key_base + 2j and key_base + 2j + 1 along direction e_j: scores 16 and
    16 - (j + 1)/32 at scale 1/8, so the second key's p runs from 0.97 down
    to 0.37 of the first's and lands on many different rounding positions;
    V is +vmag on the first key and -vmag on the second in column j.  Every
    other score is about 0.01, some e^-16 below the dominant pair."""
    rng = np.random.default_rng(seed)
    q = 0.1 * rng.standard_normal((1, n, 1, d))
    k = 0.1 * rng.standard_normal((1, n, 1, d))
    v = rng.standard_normal((1, n, 1, d))
    for j in range(32):
        r, a, b = n - 64 + j, key_base + 2 * j, key_base + 2 * j + 1
        q[0, r, 0, j] = 64.0
        k[0, a, 0] = 0.0
        k[0, b, 0] = 0.0
        k[0, a, 0, j] = 2.0
        k[0, b, 0, j] = 2.0 - (j + 1) * 2.0 ** -8
        v[0, a, 0, j] = vmag
        v[0, b, 0, j] = -vmag
    return q, k, v


@pytest.mark.parametrize("key_base", [0, 128])
@pytest.mark.parametrize("vmag", [3.0, 8.0])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_dominant_key_pairs_in_unmasked_tiles(dtype, d, causal, vmag, key_base):
    # key_base 0: the pairs sit in every row's first key tile (which sets the
    # row's reference maximum); 128: in a later tile, past that reference
    # (with fp16 P this also exceeds P's range and takes the exact-maximum pass)
    q, k, v = peaked_pairs(384, d, vmag, key_base, 7 + d + key_base)
    full_check(_stored(q, k, v, dtype), dtype, causal=causal, scale=1.0 / 8.0,
               what=f"peaked pairs {dtype} d{d} causal={causal} |v|={vmag} keys@{key_base}")


@pytest.mark.parametrize("vmag", [3.0, 8.0])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_two_key_row_in_its_first_tile(dtype, causal, vmag):
    # One row (200) whose weight sits on keys 5 and 6, both in its first,
    # unmasked key tile; key 5 is the reference maximum (p = 1 exactly) and
    # key 6 has p = exp(-64 * 2^-7 / 8) = 0.939, which bf16 stores as
    # 0.9375; V of the two keys is +vmag and -vmag in column 1.
    n, d = 256, 64
    rng = np.random.default_rng(5)
    q = 0.1 * rng.standard_normal((1, n, 1, d))
    k = 0.1 * rng.standard_normal((1, n, 1, d))
    v = 0.1 * rng.standard_normal((1, n, 1, d))
    q[0, 200, 0] = 0.0
    q[0, 200, 0, 0] = 64.0
    k[0, 5, 0] = 0.0
    k[0, 6, 0] = 0.0
    k[0, 5, 0, 0] = 2.0
    k[0, 6, 0, 0] = 2.0 - 2.0 ** -7
    v[0, 5, 0, 1] = vmag
    v[0, 6, 0, 1] = -vmag
    full_check(_stored(q, k, v, dtype), dtype, causal=causal, scale=1.0 / 8.0,
               what=f"two-key row {dtype} causal={causal} |v|={vmag}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_sink_key_shared_by_every_row(dtype):
    # Every query row puts a large share of its weight on key 0 and a smaller
    # one on key 1 (a pair of "sink" keys along a direction all queries share),
    # over 1500 keys with a causal mask: the pair sits in each row's first
    # tile, unmasked for rows >= 64.
    n, d = 1500, 128
    rng = np.random.default_rng(11)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    q = rng.standard_normal((1, n, 2, d)) + 6.0 * u
    k = rng.standard_normal((1, n, 2, d))
    v = rng.standard_normal((1, n, 2, d))
    k[0, 0] = 12.0 * u
    k[0, 1] = 11.8 * u
    v[0, 0] = 4.0
    v[0, 1] = -4.0
    full_check(_stored(q, k, v, dtype), dtype, causal=True, what=f"sink keys {dtype}")


@pytest.mark.parametrize("pv8", [False, True])
@pytest.mark.parametrize("factor", [16.0, 64.0, 256.0])
@pytest.mark.parametrize("shape", [(2, 4, 4, 700, True, (-1, -1)), (1, 8, 2, 1000, False, (300, 40))])
def test_fp8_scores_with_large_scales(shape, factor, pv8):
    # fp8 inputs with the softmax scale 16-256 times 1/sqrt(d): very peaked
    # rows (at 256 the fixed reference overflows and the exact-maximum pass
    # runs), both formats of P; O within 3e-2, the LSE within the fp8 bound
    # that includes the 8-bit matrix instruction's truncated group sums
    # (parity_helpers)
    import math
    from exact_attention_04_amd.workloads import small_case
    batch, heads, heads_kv, n, causal, window = shape
    inp = small_case(batch, heads, n, 128, "fp8", "bshd", 6100 + int(factor) + (1 if pv8 else 0), heads_kv=heads_kv)
    full_check(inp, "fp8", causal=causal, window=window, scale=factor / math.sqrt(128),
               pv_dtype=torch.float8_e4m3fn if pv8 else None, what=f"fp8 x{factor} pv8={pv8} {shape}")
