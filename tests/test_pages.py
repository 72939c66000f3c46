"""LUT page order (host-side format helper), checked against its definition."""
import numpy as np
import pytest

from any_precision_bit_amd.pages import lut_page


@pytest.mark.parametrize("b", range(1, 9))
def test_lut_page_order(b):
    n = 1 << b
    R = 96
    lut = np.arange(R * n, dtype=np.float32).reshape(R, n).astype(np.float16) if R * n < 2048 else \
        np.random.default_rng(b).standard_normal((R, n)).astype(np.float16)
    page = lut_page(lut).reshape(-1)
    E = min(8, n)
    G = n // E
    for r in range(R):
        t, rr = divmod(r, 32)
        for i in range(n):
            g, j = divmod(i, E)
            assert page[((t * G + g) * 32 + rr) * E + j] == lut[r, i]
    assert lut_page(lut).shape == lut.shape and lut_page(lut).dtype == lut.dtype


def test_lut_page_rejects_bad_shapes():
    with pytest.raises(ValueError):
        lut_page(np.zeros((40, 8), np.float16))
    with pytest.raises(ValueError):
        lut_page(np.zeros((32, 6), np.float16))
