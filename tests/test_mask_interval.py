"""CPU checks of the kernels' tests for masked tiles.

The kernel (csrc/fwd_kernel.hip, `tile_masked`) decides per 64-key tile
whether a wave's 32 query rows see every key of the tile.  Every visibility
condition (keys past the sequence end, causal, the left and right window
edges; the masks of "Flash Attention | Hermes Skill", Workflow 2) is
monotone in the tile index, so the fully visible tiles form one interval,
computed once per wave.  The interval formula is restated here and compared
with a brute-force scan of every (row, key) pair.  The backward's dK/dV
kernel (csrc/bwd_kernel.hip) does the same along the query rows for a
wave's fixed 32 keys; its interval is compared with the block test.
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


def all_visible_block(r0, r1, k0, k1, n, causal, wl, wr):
    """Every (row, key) of rows [r0, r1) x keys [k0, k1) visible (the
    kernels' block test, restated)."""
    if k1 > n:
        return False
    if causal and k1 - 1 > r0:
        return False
    if wl >= 0 and k0 < (r1 - 1) - wl:
        return False
    if wr >= 0 and k1 - 1 > r0 + wr:
        return False
    return True


def row_interval(k0, k1, n, causal, wl, wr):
    """The backward dK/dV kernel's per-wave interval [lo, hi] of 32-row block
    starts r0 whose rows [r0, min(r0 + 32, n)) see all of keys [k0, k1)."""
    lo = 0
    if causal:
        lo = max(lo, k1 - 1)
    if wr >= 0:
        lo = max(lo, k1 - 1 - wr)
    hi = 1 << 30
    if wl >= 0 and n > k0 + wl + 1:
        hi = k0 + wl - 31
    if k1 > n:
        hi = -1
    return lo, hi


def test_row_interval_matches_the_block_test():
    rng = random.Random(11)
    for _ in range(3000):
        n = rng.choice([1, 31, 64, 100, 128, 300, 1000])
        k0 = 32 * rng.randrange(0, (n + 31) // 32)
        k1 = max(min(k0 + 32, n), k0 + 1)
        causal = rng.random() < 0.5
        wl = rng.choice([-1, -1, 0, 5, 31, 32, 64, 200])
        wr = rng.choice([-1, -1, 0, 5, 31, 32, 64, 200])
        lo, hi = row_interval(k0, k1, n, causal, wl, wr)
        for r0 in range(0, n, 32):
            r1 = min(r0 + 32, n)
            assert (lo <= r0 <= hi) == all_visible_block(r0, r1, k0, k1, n, causal, wl, wr), \
                (r0, k0, k1, n, causal, wl, wr, lo, hi)
