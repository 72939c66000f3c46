"""Seeded synthetic serving trace for KV-cache pressure (input data only).

The PagedWeight pages motivate the planner with the KV cache competing with the
weights for GPU memory as contexts grow (arxivlens summary; legiblepapers
"Key Takeaways"). No trace is given, so this generator stands in for one:
requests arrive by a Poisson process whose rate rises and falls over the run
(one sine period), each with a prompt length and a number of decode tokens
drawn uniformly; at every decode step each active request's context grows by
one token, and a request leaves when its decode tokens are done. The output is
the number of cached tokens per step; KV bytes = tokens * bytes per token.
"""
from __future__ import annotations

import math

import numpy as np


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, elem_bytes: int = 2) -> int:
    """K and V of one token across `layers` attention layers."""
    return 2 * layers * kv_heads * head_dim * elem_bytes


def request_trace(steps: int, seed: int = 0, peak_rate: float = 2.0, prompt=(256, 2048), decode=(64, 512)):
    """Cached tokens (sum of active contexts) after each of `steps` decode steps."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([7, seed])))
    active = []   # [context tokens, decode tokens left]
    out = np.zeros(steps, dtype=np.int64)
    for s in range(steps):
        rate = peak_rate * 0.5 * (1.0 - math.cos(2.0 * math.pi * s / steps))
        for _ in range(int(g.poisson(rate))):
            active.append([int(g.integers(prompt[0], prompt[1] + 1)), int(g.integers(decode[0], decode[1] + 1))])
        for r in active:
            r[0] += 1
            r[1] -= 1
        active = [r for r in active if r[1] > 0]
        out[s] = sum(r[0] for r in active)
    return out
