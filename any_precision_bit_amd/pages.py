"""Page formats of the library (host-side data preparation; no layer compute).

Bit-plane pages are row-major (row stride K/8 bytes, column c at bit c & 7 of
byte c >> 3). LUT pages are row-major per-row tables [R, 2^b] by default; a
layer created with PW_FLAG_LUT_TILED takes them in 32-row tiles instead, which
a work-group stages with contiguous loads: `lut_page` reorders a per-row table
(fp16, R a multiple of 32) into that order. The byte size is unchanged.
"""
from __future__ import annotations

import numpy as np


def lut_page(lut: np.ndarray) -> np.ndarray:
    """Tile t of the result holds, for entry groups g = 0 .. G-1 (E = min(8, 2^b)
    entries each, G = 2^b / E), the entries [g*E, g*E + E) of rows 32t .. 32t+31,
    row after row. Returns a contiguous array of the input's shape and dtype."""
    R, n = lut.shape
    if R % 32 or n & (n - 1):
        raise ValueError(f"LUT of shape {lut.shape}: rows must be a multiple of 32, entries a power of two")
    E = min(8, n)
    G = n // E
    return np.ascontiguousarray(lut.reshape(R // 32, 32, G, E).transpose(0, 2, 1, 3)).reshape(R, n)
