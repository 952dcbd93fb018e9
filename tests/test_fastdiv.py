"""The float-reciprocal division the kernels use for index arithmetic is exact.

The kernels compute q = trunc(float(a) * fl(1/d)) and repair q with one
remainder check. For 0 <= a < 2^22 and 1 <= d < 2^22 the float quotient is
within 0.5 of a/d, so one correction suffices. Emulated here in float32
(round-to-nearest multiply, truncating conversion), on boundary and random
numerators.
"""

import numpy as np


def fdiv(a: np.ndarray, d: int):
    inv = np.float32(1.0) / np.float32(d)
    q = (a.astype(np.float32) * inv).astype(np.int64)  # truncation toward zero
    r = a - q * d
    q = np.where(r < 0, q - 1, np.where(r >= d, q + 1, q))
    r = a - q * d
    return q, r


def test_fastdiv_exact_on_boundaries_and_random():
    rng = np.random.default_rng(0)
    divisors = list(range(1, 300)) + [1023, 1024, 1025, 4095, 4096, 16383, 65535, (1 << 21) + 3, (1 << 22) - 1]
    amax = 1 << 22
    for d in divisors:
        mult = np.arange(0, amax, d, dtype=np.int64)[-2000:]
        a = np.concatenate([mult, mult + 1, mult - 1, mult + d - 1,
                            rng.integers(0, amax, 5000), np.array([0, amax - 1])])
        a = a[(a >= 0) & (a < amax)]
        q, r = fdiv(a, d)
        assert np.array_equal(q, a // d), d
        assert np.array_equal(r, a % d), d


def test_halo_row_decode_by_float_reciprocal_is_exact():
    """Halo items of the local-context tiles are decoded as
    hy = trunc((pi + 0.5) * fl(1/pw)) in float32 with no fix-up; exact for
    every word count pw a tile can have and pi < 2^16 (far beyond any halo)."""
    pi = np.arange(1 << 16, dtype=np.int64)
    for pw in range(1, 40):
        inv = np.float32(1.0) / np.float32(pw)
        got = ((pi.astype(np.float32) + np.float32(0.5)) * inv).astype(np.int64)
        np.testing.assert_array_equal(got, pi // pw, err_msg=f"pw={pw}")
