"""The chunk plan's device division, modelled on the host.

On the device, `div_small(a, b)` (csrc/da_internal.h) takes a / b for
0 <= a <= 2^22 from the float product a * rcp(b), truncated, then corrects it by
one either way from the remainder.  The hardware reciprocal is within one ulp, so
the model runs every dividend in range through the correctly rounded reciprocal
and through its neighbours one ulp below and above, rounds the product to float32
as the device does, and must reproduce Python's integer quotient every time.
"""
import numpy as np
import pytest

A_MAX = 1 << 22


def device_div_model(a: np.ndarray, b: int, ulps: int) -> np.ndarray:
    r = np.float32(1.0) / np.float32(b)
    for _ in range(abs(ulps)):
        r = np.nextafter(r, np.float32(np.inf if ulps > 0 else 0.0), dtype=np.float32)
    prod = a.astype(np.float32) * r                      # one float32 rounding
    q = prod.astype(np.int64)                            # truncation toward zero
    rem = a - q * b
    return q + (rem >= b) - (rem < 0)


@pytest.mark.parametrize("b", [1, 2, 3, 7, 31, 32, 33, 63, 64, 96, 1000, 1023, 1024, 1952, 2047, 2048,
                               4095, 4096, 8191, 8192, 65537, (1 << 20) - 1, 1 << 22])
def test_every_dividend_in_range(b):
    a = np.arange(A_MAX + 1, dtype=np.int64)
    want = a // b
    for ulps in (-1, 0, 1):
        got = device_div_model(a, b, ulps)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, f"b={b} ulps={ulps}: a={a[bad[:5]]} gives {got[bad[:5]]}, not {want[bad[:5]]}"


def test_random_divisors():
    rng = np.random.default_rng(7)
    a = np.concatenate([rng.integers(0, A_MAX + 1, 200_000), np.arange(0, 5000)]).astype(np.int64)
    for b in rng.integers(1, A_MAX + 1, 60):
        for ulps in (-1, 0, 1):
            assert np.array_equal(device_div_model(a, int(b), ulps), a // int(b)), int(b)


def test_one_correction_is_not_enough_past_the_range():
    """Past 2^22 the estimate can be two off: the bound the device code relies on is real."""
    a = np.arange(1 << 24, (1 << 24) + (1 << 20), dtype=np.int64)
    assert not np.array_equal(device_div_model(a, 1, -1), a)
