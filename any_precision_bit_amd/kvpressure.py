"""Byte targets for the planner from KV-cache pressure.

The PagedWeight planner frees weight bytes when the KV cache needs memory and
may spend them again when it shrinks (arxivlens summary: precision balanced
against KV-cache size; legiblepapers "Key Takeaways": bitwidths adjusted to KV
cache pressure). Reading: with a memory budget M for one layer's weights plus
its share of the KV cache, the bytes to free are

    target = resident weight bytes + KV bytes - M

a positive target is passed to pw_plan_greedy as bytes to free; when the target
is below -hysteresis the layer may spend -(target + hysteresis) bytes on
upgrades (never above max_bits, the quality plan). Host logic only: the plan is
applied through a PageManager or pw_moe_plan_set.
"""
from __future__ import annotations

from typing import Callable, Optional

import numpy as np

from . import binding as B


class KVPressurePlanner:
    def __init__(self, layer, budget_bytes: float, sensitivity, hysteresis_bytes: float,
                 resident_bytes: Callable[[], float], min_bits=None, max_bits=None):
        self.layer = layer
        self.budget = float(budget_bytes)
        self.sens = np.ascontiguousarray(sensitivity, dtype=np.float32)
        self.hyst = float(hysteresis_bytes)
        self.resident = resident_bytes
        self.min_bits, self.max_bits = min_bits, max_bits

    def target(self, kv_bytes: float) -> float:
        return self.resident() + float(kv_bytes) - self.budget

    def decide(self, kv_bytes: float, expert_count, n_tokens: int) -> Optional[tuple]:
        """(new bits, bytes moved, damage, actions) when the plan should change, else None."""
        t = self.target(kv_bytes)
        if t > 0:
            goal = t
        elif t < -self.hyst:
            goal = t + self.hyst          # negative: a budget to spend on upgrades
        else:
            return None
        new, moved, dmg, n = B.pw_plan_greedy(self.layer.handle, self.sens, expert_count, n_tokens, goal,
                                              min_bits=self.min_bits, max_bits=self.max_bits)
        return (new, moved, dmg, n) if n > 0 else None
