"""Exhaustive host check of the multiply-shift division the kernels use to split
v-staging indices (n / d for n < 2**14, 1 <= d <= 256)."""
import numpy as np


def test_div_magic_exact():
    n = np.arange(1 << 14, dtype=np.uint64)
    for d in range(1, 257):
        m = np.uint64((1 << 24) // d + 1)
        q = (n * m) >> np.uint64(24)
        np.testing.assert_array_equal(q, n // np.uint64(d), err_msg=f"d={d}")
