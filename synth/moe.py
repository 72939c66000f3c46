"""Workload shapes and seeded generators for the Any-Precision MoE layer.

Format of the generated weights (the PagedWeight pages: "PagedWeight: Efficient
MoE LLM Serving with Dynamic Quality-Aware Weight Quantization", arxivlens
summary and legiblepapers "Summary & Methodology Analysis" -- Any-Precision
bit-plane and LUT buffers held as GPU-resident pages):

* Every linear of every expert is an [R x K] matrix (R output rows, K inputs).
  gate and up are [F x d]; down is [d x F].
* Each weight has an 8-bit parent index q in 0..255. Bit-plane p (p = 0 is the
  most significant bit of q) is an [R x K/8] byte array, row-major, column c
  of a row stored in byte c >> 3 at bit c & 7 (least significant bit first).
* The bitwidth-b view of a weight uses planes 0..b-1, i.e. the index q >> (8-b),
  and looks it up in that row's LUT_b, a table of 2^b fp16 values.
* LUT_b values are independent N(0, 0.02) draws rounded to fp16 and sorted
  ascending within the row, separately for every b.

Every tensor draws from its own PCG64 stream keyed by
(config, run seed, layer, expert, linear, kind, b, step), so any tensor can be
regenerated alone and in any order.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

GATE, UP, DOWN = 0, 1, 2
LINEARS = (GATE, UP, DOWN)

KIND_PARENT = 1
KIND_LUT = 2
KIND_X = 3
KIND_ROUTER = 4
KIND_BITS = 5
KIND_REWRITE = 6


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    cid: int
    d: int            # hidden size
    E: int            # routed experts
    F: int            # routed expert ffn size
    k: int            # top-k
    T: int            # tokens per call
    Fs: int = 0       # shared expert ffn size (0: none); the shared expert has id E
    bits_rule: str = "uniform"
    bits_values: tuple = (3, 4)
    bits_probs: Optional[tuple] = None
    zipf: float = 0.0  # router bias skew (0: no bias)
    layers: int = 1
    steps: int = 1
    rewrite_every: int = 0
    rewrite_frac: float = 0.0
    rewrite_drop: int = 0

    @property
    def has_shared(self) -> bool:
        return self.Fs > 0

    @property
    def n_experts_total(self) -> int:
        return self.E + (1 if self.has_shared else 0)

    @property
    def n_blocks(self) -> int:
        return 3 * self.n_experts_total

    def ffn(self, e: int) -> int:
        return self.Fs if e == self.E else self.F

    def block_shape(self, e: int, lin: int):
        """(R, K) of linear `lin` of expert `e`."""
        f = self.ffn(e)
        return (f, self.d) if lin in (GATE, UP) else (self.d, f)

    def with_tokens(self, T: int) -> "MoEConfig":
        return dataclasses.replace(self, T=T)


# The five workloads: shapes follow the pages' evaluation models
# (legiblepapers FAQ Q6: Qwen1.5-MoE-A2.7B, Mixtral-8x7B-v0.1) at synthetic values.
CONFIGS = {
    "tiny_d256": MoEConfig("tiny_d256", 0, d=256, E=8, F=512, k=2, T=4,
                    bits_rule="uniform", bits_values=(3, 4)),
    "qwen_d2048_t16": MoEConfig("qwen_d2048_t16", 1, d=2048, E=60, F=1408, k=4, T=16, Fs=5632,
                    bits_rule="uniform", bits_values=(3, 4, 5, 6, 8)),
    "mixtral_d4096": MoEConfig("mixtral_d4096", 2, d=4096, E=8, F=14336, k=2, T=1,
                    bits_rule="choice", bits_values=(3, 4, 6, 8),
                    bits_probs=(0.3, 0.3, 0.2, 0.2), zipf=1.2),
    "fine_e128_t128": MoEConfig("fine_e128_t128", 3, d=2048, E=128, F=768, k=8, T=128,
                    bits_rule="frequency", bits_values=(8, 4, 3), zipf=1.1),
    "qwen_stack24_t256": MoEConfig("qwen_stack24_t256", 4, d=2048, E=60, F=1408, k=4, T=256, Fs=5632,
                    bits_rule="uniform", bits_values=(3, 4, 5, 6, 8),
                    layers=24, steps=64, rewrite_every=16, rewrite_frac=0.25,
                    rewrite_drop=2),
    # the decode layer's shape at prefill scale, with linear-blocks of 128 rows
    "qwen_rows128_t1024": MoEConfig("qwen_rows128_t1024", 5, d=2048, E=60, F=1408, k=4, T=1024, Fs=5632,
                    bits_rule="uniform", bits_values=(3, 4, 5, 6, 8)),
}

# rows per linear-block of the workloads cut into row-blocks (the rest: whole linears)
ROWS_PER_BLOCK = {"qwen_rows128_t1024": 128}

WORKLOAD_TEXT = {
    "tiny_d256": "d256 E8 F512 top2 T4, bits U{3,4}",
    "qwen_d2048_t16": "Qwen1.5-MoE-A2.7B-shaped decode layer: d2048 E60 F1408 top4 T16 + shared F5632, bits U{3,4,5,6,8}",
    "mixtral_d4096": "Mixtral-8x7B-shaped layer: d4096 E8 F14336 top2, bits {3,4,6,8} p=(.3,.3,.2,.2), Zipf(1.2) routing",
    "fine_e128_t128": "fine-grained layer: d2048 E128 F768 top8 T128, Zipf(1.1) routing, bits by routed frequency 8/4/3",
    "qwen_stack24_t256": "24-layer stack of the d2048 E60 F1408 top4 (+shared F5632) layer, T256, 64 steps, plan rewrite every 16",
    "qwen_rows128_t1024": "prefill of the d2048 E60 F1408 top4 (+shared F5632) layer, T1024, linear-blocks of 128 rows, bits U{3,4,5,6,8} per block",
}


def rng_for(cfg: MoEConfig, run_seed: int, *, layer: int = 0, expert: int = 0,
            linear: int = 0, kind: int = 0, b: int = 0, step: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence([cfg.cid, run_seed, layer, expert, linear, kind, b, step])
    return np.random.Generator(np.random.PCG64(ss))


# ----------------------------------------------------------------------------- weights
def parent_indices(cfg: MoEConfig, e: int, lin: int, *, layer: int = 0, run_seed: int = 0) -> np.ndarray:
    """8-bit parent indices q, uniform on 0..255, u8 [R, K]."""
    R, K = cfg.block_shape(e, lin)
    g = rng_for(cfg, run_seed, layer=layer, expert=e, linear=lin, kind=KIND_PARENT)
    return g.integers(0, 256, size=(R, K), dtype=np.uint8)


def pack_planes(q: np.ndarray, n_planes: int = 8) -> np.ndarray:
    """Bit-planes 0..n_planes-1 of q (plane 0 = MSB), u8 [n_planes, R, K/8],
    row-major, LSB-first within each byte."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    R, K = q.shape
    assert K % 8 == 0
    out = np.empty((n_planes, R, K // 8), dtype=np.uint8)
    for p in range(n_planes):
        out[p] = np.packbits((q >> (7 - p)) & 1, axis=1, bitorder="little")
    return out


def lut(cfg: MoEConfig, e: int, lin: int, b: int, *, layer: int = 0, run_seed: int = 0) -> np.ndarray:
    """Per-row LUT for bitwidth b: fp16 [R, 2^b], N(0, 0.02) draws rounded to
    fp16 (round-to-nearest-even), sorted ascending within each row."""
    R, _ = cfg.block_shape(e, lin)
    g = rng_for(cfg, run_seed, layer=layer, expert=e, linear=lin, kind=KIND_LUT, b=b)
    v = (g.standard_normal((R, 1 << b)) * 0.02).astype(np.float16)
    return np.sort(v, axis=1)


# ----------------------------------------------------------------------------- activations / router
def tokens(cfg: MoEConfig, T: Optional[int] = None, *, run_seed: int = 0, layer: int = 0,
           step: int = 0) -> np.ndarray:
    """x ~ N(0, 1) rounded to fp16, [T, d]."""
    T = cfg.T if T is None else T
    g = rng_for(cfg, run_seed, layer=layer, kind=KIND_X, step=step, b=T)
    return g.standard_normal((T, cfg.d)).astype(np.float16)


def router(cfg: MoEConfig, *, layer: int = 0, run_seed: int = 0):
    """Router weight fp16 [E, d] ~ N(0, 0.02), and an optional fp16 logit bias [E].

    The skewed workloads add a fixed bias beta_e = fp16(s_g * ln p_e) with
    p_e proportional to (e+1)^-zipf (expert 0 most popular) and s_g the Gumbel
    scale matching the logit spread (logit std 0.02*sqrt(d) times sqrt(6)/pi),
    so that top-1 usage approximately follows the Zipf law."""
    g = rng_for(cfg, run_seed, layer=layer, kind=KIND_ROUTER)
    w = (g.standard_normal((cfg.E, cfg.d)) * 0.02).astype(np.float16)
    if cfg.zipf <= 0.0:
        return w, None
    ranks = np.arange(1, cfg.E + 1, dtype=np.float64)
    p = ranks ** (-cfg.zipf)
    p /= p.sum()
    scale = 0.02 * math.sqrt(cfg.d) * math.sqrt(6.0) / math.pi
    beta = (scale * np.log(p)).astype(np.float16)
    return w, beta


# ----------------------------------------------------------------------------- plans
def initial_bits(cfg: MoEConfig, *, layer: int = 0, run_seed: int = 0,
                 counts: Optional[np.ndarray] = None) -> np.ndarray:
    """Per-(expert, linear) bitwidths, u8 [E + has_shared, 3].

    uniform / choice rules draw per block. The frequency rule needs the routed
    counts per expert of the measured batch (`counts`, length E) and gives the
    32 most-routed experts 8 bits, the next 32 4 bits and the rest 3 bits
    (ties go to the lower expert index)."""
    n = cfg.n_experts_total
    if cfg.bits_rule == "frequency":
        if counts is None:
            raise ValueError("frequency rule needs the routed counts per expert")
        return plan_by_frequency(np.asarray(counts), n, cfg.bits_values)
    g = rng_for(cfg, run_seed, layer=layer, kind=KIND_BITS)
    vals = np.asarray(cfg.bits_values, dtype=np.uint8)
    if cfg.bits_rule == "uniform":
        return g.choice(vals, size=(n, 3)).astype(np.uint8)
    if cfg.bits_rule == "choice":
        return g.choice(vals, size=(n, 3), p=np.asarray(cfg.bits_probs)).astype(np.uint8)
    raise ValueError(cfg.bits_rule)


def n_row_blocks(cfg: MoEConfig, rows_per_block: int) -> int:
    """Blocks of a layer when every linear is split into blocks of rows_per_block rows
    (0: whole linears): per expert 2 * ffn / rb + d / rb."""
    if rows_per_block <= 0:
        return cfg.n_blocks
    n = 0
    for e in range(cfg.n_experts_total):
        n += 2 * cfg.ffn(e) // rows_per_block + cfg.d // rows_per_block
    return n


def rowblock_bits(cfg: MoEConfig, rows_per_block: int, *, layer: int = 0, run_seed: int = 0) -> np.ndarray:
    """Flat per-block bitwidths for row-blocks of rows_per_block rows (order: expert, linear,
    row-block), drawn per block like the config's uniform / choice rule."""
    n = n_row_blocks(cfg, rows_per_block)
    g = rng_for(cfg, run_seed, layer=layer, kind=KIND_BITS, b=rows_per_block)
    vals = np.asarray(cfg.bits_values, dtype=np.uint8)
    p = None if cfg.bits_rule == "uniform" else np.asarray(cfg.bits_probs)
    return g.choice(vals, size=n, p=p).astype(np.uint8)


def plan_by_frequency(counts: np.ndarray, n_experts_total: int, tiers=(8, 4, 3),
                      tier_size: int = 32) -> np.ndarray:
    counts = np.asarray(counts, dtype=np.int64)
    E = counts.shape[0]
    order = sorted(range(E), key=lambda e: (-int(counts[e]), e))
    bits = np.full((n_experts_total, 3), tiers[-1], dtype=np.uint8)
    for rank, e in enumerate(order):
        tier = min(rank // tier_size, len(tiers) - 1)
        bits[e, :] = tiers[tier]
    return bits


def rewrite_plan(cfg: MoEConfig, bits: np.ndarray, *, layer: int, epoch: int,
                 run_seed: int = 0):
    """One plan rewrite: a seeded floor(frac * n_blocks) of the blocks drop
    `rewrite_drop` bits (floor 3). Returns (new_bits, list of changed flat block ids)."""
    n_blocks = bits.size
    n_pick = int(math.floor(cfg.rewrite_frac * n_blocks))
    g = rng_for(cfg, run_seed, layer=layer, kind=KIND_REWRITE, step=epoch)
    pick = g.permutation(n_blocks)[:n_pick]
    new = bits.copy().reshape(-1)
    changed = []
    for blk in sorted(int(i) for i in pick):
        nb = max(3, int(new[blk]) - cfg.rewrite_drop)
        if nb != new[blk]:
            changed.append(blk)
        new[blk] = nb
    return new.reshape(bits.shape), changed


# ----------------------------------------------------------------------------- bundles
@dataclasses.dataclass
class Block:
    e: int
    lin: int
    R: int
    K: int
    planes: np.ndarray      # u8 [n_planes, R, K/8]
    luts: dict              # b -> fp16 [R, 2^b]
    q: Optional[np.ndarray] = None


def make_block(cfg: MoEConfig, e: int, lin: int, *, layer: int = 0, run_seed: int = 0,
               n_planes: int = 8, lut_bits=(3, 4, 5, 6, 8), keep_parent: bool = False) -> Block:
    q = parent_indices(cfg, e, lin, layer=layer, run_seed=run_seed)
    R, K = q.shape
    planes = pack_planes(q, n_planes)
    luts = {b: lut(cfg, e, lin, b, layer=layer, run_seed=run_seed) for b in lut_bits}
    return Block(e, lin, R, K, planes, luts, q if keep_parent else None)


def make_layer_blocks(cfg: MoEConfig, bits: np.ndarray, *, layer: int = 0, run_seed: int = 0,
                      all_luts: bool = False, keep_parent: bool = False, workers: int = 8):
    """Blocks for every (expert, linear) of one layer. Only planes 0..b-1 and
    the LUT for b are generated unless all_luts is set (then planes 0..7 and
    LUTs for 3..8, enough for any later plan that lowers bits)."""
    from concurrent.futures import ThreadPoolExecutor

    jobs = [(e, lin) for e in range(cfg.n_experts_total) for lin in LINEARS]

    def one(job):
        e, lin = job
        b = int(bits[e, lin])
        if all_luts:
            lb = tuple(sorted(set((3, 4, 5, 6, 8)) | {b}))
            return make_block(cfg, e, lin, layer=layer, run_seed=run_seed, n_planes=8,
                              lut_bits=lb, keep_parent=keep_parent)
        return make_block(cfg, e, lin, layer=layer, run_seed=run_seed, n_planes=b,
                          lut_bits=(b,), keep_parent=keep_parent)

    with ThreadPoolExecutor(max_workers=max(1, workers)) as ex:
        blocks = list(ex.map(one, jobs))
    return {(blk.e, blk.lin): blk for blk in blocks}
