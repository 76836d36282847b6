"""CPU check of the forward kernel's test for masked key tiles.

The kernel (csrc/fwd_kernel.hip, `tile_masked`) decides per 64-key tile
whether a wave's 32 query rows see every key of the tile.  Every visibility
condition (keys past the sequence end, causal, the left and right window
edges; the masks of "Flash Attention | Hermes Skill", Workflow 2) is
monotone in the tile index, so the fully visible tiles form one interval,
computed once per wave.  The interval formula is restated here and compared
with a brute-force scan of every (row, key) pair.
"""
import random

BN = 64


def visible(i, j, n, causal, wl, wr):
    if j >= n:
        return False
    if causal and j > i:
        return False
    if wl >= 0 and j < i - wl:
        return False
    if wr >= 0 and j > i + wr:
        return False
    return True


def masked_brute(kt, r0, r1, n, causal, wl, wr):
    return not all(visible(i, j, n, causal, wl, wr) for i in range(r0, r1) for j in range(kt * BN, kt * BN + BN))


def masked_interval(kt, r0, r1, n, causal, wl, wr):
    hi_key = n - BN
    if causal:
        hi_key = min(hi_key, r0 - (BN - 1))
    if wr >= 0:
        hi_key = min(hi_key, r0 + wr - (BN - 1))
    t_hi = 0 if hi_key < 0 else hi_key // BN + 1
    lo_key = (r1 - 1) - wl if wl >= 0 else 0
    t_lo = 0 if lo_key <= 0 else (lo_key + BN - 1) // BN
    span = max(t_hi - t_lo, 0)
    return ((kt - t_lo) & 0xFFFFFFFF) >= span


def test_interval_matches_brute_force():
    rng = random.Random(7)
    cases = 0
    for _ in range(400):
        n = rng.choice([1, 31, 64, 65, 127, 128, 200, 333, 700])
        r0 = 32 * rng.randrange(0, (n + 31) // 32)
        r1 = min(r0 + 32, n)
        causal = rng.random() < 0.5
        wl = rng.choice([-1, -1, 0, 1, 63, 64, 100, 4095])
        wr = rng.choice([-1, -1, 0, 1, 63, 64, 100])
        for kt in range(0, (n + BN - 1) // BN + 2):
            assert masked_interval(kt, r0, r1, n, causal, wl, wr) == masked_brute(kt, r0, r1, n, causal, wl, wr), \
                (kt, r0, r1, n, causal, wl, wr)
            cases += 1
    assert cases > 1000
