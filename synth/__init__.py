"""Seeded synthetic inputs for the fused mixed-precision MoE layer.

This package produces input data only (tokens, router weights, 8-bit parent
indices stored as bit-planes, per-row LUTs and per-block bitwidth plans). It
holds none of the layer's arithmetic, so both the CPU oracle and the GPU path
can consume the same arrays.
"""
from .moe import *  # noqa: F401,F403
