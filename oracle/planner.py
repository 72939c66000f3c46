"""Plain planner oracle -- TEST INFRASTRUCTURE (only tests/, the smoke check and
bench.py's cpu_baseline leg may import it).

The quality-aware runtime planner of the PagedWeight pages (legiblepapers
"Summary & Methodology Analysis" and FAQ Q8: identify the bytes to free, then
greedily select the cheapest quantisation actions by damage per released byte,
the damage drawing on offline sensitivity, online routing mass and prompt
residuals). The pages give no formula; this oracle takes the plainest reading,
stated step by step:

  * an action changes one block (expert, linear) by one bit;
  * a block [R x K] at bitwidth b occupies R*K*b/8 bytes of bit-planes
    (planes 0..b-1) plus R*2^b*2 bytes of LUT (LUT_b), so b -> b-1 releases
    the difference;
  * the damage of b -> b-1 is (sensitivity + residual) * mass * (4^-(b-1) - 4^-b):
    a b-bit quantiser's noise power scales as 4^-b;
  * mass: a routed expert's routed assignments / T (how often it is used); the
    shared expert's mass is 1 (every token uses it).

Downgrades (bytes_to_free > 0): while fewer than bytes_to_free bytes are
released, scan every block's next downgrade (b > min) and take the one with the
smallest damage per released byte, ties to the lower block index.
Upgrades (bytes_to_free < 0: a budget of -bytes_to_free bytes): scan every
block's next upgrade (b < max) among blocks still eligible, take the one with
the largest damage reduction per added byte (ties to the lower block index) if
it fits in what is left of the budget, else drop that block from eligibility;
stop when no block is eligible.

It rescans every block at every step: quadratic, and obviously the definition.
"""
from __future__ import annotations

import numpy as np


def block_bytes(R: int, K: int, b: int) -> float:
    """Resident bytes of an [R x K] block at bitwidth b: planes 0..b-1 and LUT_b."""
    return R * K * b / 8.0 + R * float(1 << b) * 2.0


def noise(b: int) -> float:
    """Relative quantisation noise power of a b-bit quantiser, 4^-b."""
    return 2.0 ** (-2 * b)


def block_shapes(d: int, E: int, F: int, Fs: int, rows_per_block: int = 0):
    """(R, K) of every block in (expert, linear, row-block) order: gate and up [F x d], down
    [d x F], the shared expert (id E, when Fs > 0) with Fs; with rows_per_block = rb > 0 each
    linear is cut into blocks of rb rows."""
    shapes = []
    for e in range(E + (1 if Fs > 0 else 0)):
        f = Fs if e == E else F
        for R, K in ((f, d), (f, d), (d, f)):
            rows = rows_per_block or R
            shapes += [(rows, K)] * (R // rows)
    return shapes


def masses(E: int, has_shared: bool, expert_count, T: int, blocks_per_expert=None):
    """Routing mass per block: count_e / T for routed experts, 1 for the shared expert;
    blocks_per_expert[e] blocks per expert (3 when linears are whole)."""
    m = []
    for e in range(E + (1 if has_shared else 0)):
        me = 1.0 if e == E else float(expert_count[e]) / float(T)
        m += [me] * (3 if blocks_per_expert is None else blocks_per_expert[e])
    return m


def plan(shapes, bits, sensitivity, mass, bytes_to_free, residual=None, min_bits=None, max_bits=None):
    """Returns (new bits u8, bytes released (>0) or added (<0), damage added, actions)."""
    n = len(shapes)
    bits = [int(b) for b in np.asarray(bits).reshape(-1)]
    sens = [float(np.float32(s)) for s in np.asarray(sensitivity, dtype=np.float32).reshape(-1)]
    res = [0.0] * n if residual is None else [float(np.float32(r)) for r in np.asarray(residual, dtype=np.float32).reshape(-1)]
    lo = [3] * n if min_bits is None else [int(v) for v in np.asarray(min_bits).reshape(-1)]
    hi = [8] * n if max_bits is None else [int(v) for v in np.asarray(max_bits).reshape(-1)]
    weight = [(sens[i] + res[i]) * mass[i] for i in range(n)]
    done, damage, actions = 0.0, 0.0, 0
    if bytes_to_free > 0:
        while done < bytes_to_free:
            best, best_i = None, -1
            for i, (R, K) in enumerate(shapes):
                b = bits[i]
                if b <= lo[i]:
                    continue
                dB = block_bytes(R, K, b) - block_bytes(R, K, b - 1)
                ratio = weight[i] * (noise(b - 1) - noise(b)) / dB
                if best is None or ratio < best:
                    best, best_i = ratio, i
            if best_i < 0:
                break
            R, K = shapes[best_i]
            b = bits[best_i]
            done += block_bytes(R, K, b) - block_bytes(R, K, b - 1)
            damage += weight[best_i] * (noise(b - 1) - noise(b))
            bits[best_i] = b - 1
            actions += 1
        return np.array(bits, dtype=np.uint8), done, damage, actions
    budget = -bytes_to_free
    eligible = [True] * n
    while True:
        best, best_i = None, -1
        for i, (R, K) in enumerate(shapes):
            b = bits[i]
            if not eligible[i] or b >= hi[i]:
                continue
            dB = block_bytes(R, K, b + 1) - block_bytes(R, K, b)
            ratio = weight[i] * (noise(b) - noise(b + 1)) / dB
            if best is None or ratio > best:
                best, best_i = ratio, i
        if best_i < 0:
            break
        R, K = shapes[best_i]
        b = bits[best_i]
        add = block_bytes(R, K, b + 1) - block_bytes(R, K, b)
        if done + add > budget:
            eligible[best_i] = False
            continue
        done += add
        damage -= weight[best_i] * (noise(b) - noise(b + 1))
        bits[best_i] = b + 1
        actions += 1
    return np.array(bits, dtype=np.uint8), -done, damage, actions
