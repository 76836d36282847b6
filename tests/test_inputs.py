"""The seeded input generator's fp8 quantisation, checked against the
e4m3fn format's definition (sign, 4 exponent bits with bias 7, 3 mantissa
bits; largest finite value 448, smallest subnormal step 2^-9): per-tensor
scale s = amax |x| / 448, then x / s rounded to the nearest e4m3 value."""
import numpy as np
import torch

from exact_attention_04_amd.workloads import quantize_e4m3_per_tensor


def e4m3_spacing(y):
    """Distance between neighbouring e4m3 values around |y| (normal range
    2^-6 .. 448: 2^(e - 3); below 2^-6: the subnormal step 2^-9)."""
    a = np.abs(y)
    e = np.floor(np.log2(np.where(a >= 2.0 ** -6, a, 2.0 ** -6)))
    return 2.0 ** (e - 3)


def test_quantisation_uses_the_range_and_rounds_to_nearest():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((4, 257, 3, 64)).astype(np.float32) * 3.0
    xq, s = quantize_e4m3_per_tensor(x)
    assert xq.dtype == torch.float8_e4m3fn
    y = xq.to(torch.float64).numpy()
    assert np.isfinite(y).all() and np.abs(y).max() <= 448.0
    assert np.isclose(s, np.abs(x).max() / 448.0, rtol=1e-7)
    # the largest magnitude lands on the top of the range
    i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert abs(y[i]) == 448.0
    # every value within half a spacing of x / s (round to nearest)
    t = x.astype(np.float64) / s
    assert (np.abs(y - t) <= 0.5 * e4m3_spacing(t) * (1 + 1e-6)).all()


def test_quantisation_of_zero_and_exact_grid_values():
    xq, s = quantize_e4m3_per_tensor(np.zeros((2, 3), np.float32))
    assert s == 1.0 and (xq.to(torch.float32) == 0).all()
    # values already on the e4m3 grid (times a power-of-two scale) survive exactly
    grid = np.array([448.0, -448.0, 1.0, 1.125, -0.5, 2.0 ** -9, 3 * 2.0 ** -9, 240.0], np.float32)
    xq, s = quantize_e4m3_per_tensor(grid)
    assert s == 1.0
    assert np.array_equal(xq.to(torch.float32).numpy(), grid)
