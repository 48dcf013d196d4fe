"""CPU pins of the acceptance bound used by the INT8 parity tests.

half_ulp_bf16 must be exactly the largest error of rounding to bf16 (round to nearest
even) in each binade: torch's float -> bf16 conversion never errs by more, and errs by
exactly that much at the midpoints between neighbouring bf16 values.
"""

import numpy as np
import torch

from tolerance import half_ulp_bf16, int8_excess


def test_half_ulp_bounds_bf16_rounding():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(200_000) * np.exp2(rng.integers(-20, 20, 200_000))
    xr = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    x32 = x.astype(np.float32).astype(np.float64)
    assert np.all(np.abs(xr - x32) <= half_ulp_bf16(x32))


def test_half_ulp_is_reached_at_midpoints():
    e = np.arange(-10, 10)
    p = np.ldexp(1.0, e)
    mid = p + np.ldexp(1.0, e - 8)            # halfway between 2^e and its bf16 successor
    assert np.array_equal(half_ulp_bf16(p), np.ldexp(1.0, e - 8))
    assert np.array_equal(half_ulp_bf16(-mid), np.ldexp(1.0, e - 8))
    xr = torch.from_numpy(mid.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.abs(xr - mid), half_ulp_bf16(mid))
    # just below a power of two the bound is the lower binade's
    assert np.array_equal(half_ulp_bf16(np.nextafter(p, 0)), np.ldexp(1.0, e - 9))
    assert half_ulp_bf16(np.array([0.0]))[0] == 0.0


def test_int8_excess_is_the_half_ulp_bound():
    ref = np.array([[0.75, 1.0, -3.0, 0.0]])
    slack = 2e-3 + np.array([2.0 ** -9, 2.0 ** -8, 2.0 ** -7, 0.0])
    at = torch.from_numpy(ref + slack)
    assert int8_excess(at, ref) <= 1e-15
    over = torch.from_numpy(ref + slack * np.array([1, 1, 1.01, 1]))
    assert int8_excess(over, ref) > 0
