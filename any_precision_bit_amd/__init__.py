"""Fused mixed-precision MoE layer over Any-Precision bit-plane / LUT pages on
MI355X (gfx950). The compute lives in libpw.so (HIP kernels behind the C ABI in
include/pw.h); this package only marshals arguments to it."""
from . import binding  # noqa: F401  (raises ImportError when libpw.so is missing)
from .binding import PW_DOWN, PW_GATE, PW_UP, PwError  # noqa: F401
from .layer import PagedMoELayer, route_buffers  # noqa: F401
