"""The quality-aware planner (legiblepapers "Summary & Methodology Analysis", FAQ Q8):
the oracle (oracle/planner.py) pinned to brute force and to the data it
describes, then the library's pw_plan_greedy against the oracle."""
import itertools

import numpy as np
import pytest

import synth
from oracle import planner as P


# ----------------------------------------------------------------------------- oracle pins
def test_block_bytes_match_generated_pages():
    """The resident size of a block at b is the byte size of its planes 0..b-1 plus its LUT_b,
    measured on generated pages of several shapes."""
    cfg = synth.CONFIGS["tiny_d256"]
    for e, lin in [(0, 0), (3, 2)]:
        blk = synth.make_block(cfg, e, lin, n_planes=8, lut_bits=(1, 2, 3, 4, 5, 6, 7, 8))
        R, K = blk.R, blk.K
        for b in range(1, 9):
            measured = blk.planes[:b].nbytes + blk.luts[b].nbytes
            assert P.block_bytes(R, K, b) == measured, (b, R, K)


def test_noise_ratio_of_a_uniform_quantiser():
    """One bit less multiplies a quantiser's mean squared error by 4: measured by rounding uniform
    samples to b-bit grids."""
    x = np.random.default_rng(0).random(2_000_000)
    mse = {}
    for b in range(3, 9):
        step = 2.0 ** -b
        q = (np.floor(x / step) + 0.5) * step
        mse[b] = float(np.mean((x - q) ** 2))
    for b in range(4, 9):
        assert abs(mse[b - 1] / mse[b] - P.noise(b - 1) / P.noise(b)) < 0.02


def _equal_step_instance(n, b, seed):
    """n blocks of one shape at bitwidth b that may each drop exactly one bit: every action
    releases the same bytes, so the cheapest set of j actions is the j smallest damages."""
    g = np.random.default_rng(seed)
    shapes = [(64, 256)] * n
    sens = g.random(n).astype(np.float32)
    mass = list(g.random(n))
    bits = np.full(n, b, np.uint8)
    return shapes, bits, sens, mass


@pytest.mark.parametrize("seed", range(4))
def test_downgrades_match_brute_force_when_steps_are_equal(seed):
    n, b = 7, 5
    shapes, bits, sens, mass = _equal_step_instance(n, b, seed)
    step = P.block_bytes(64, 256, b) - P.block_bytes(64, 256, b - 1)
    dmg = [(float(sens[i])) * mass[i] * (P.noise(b - 1) - P.noise(b)) for i in range(n)]
    for j in range(1, n + 1):
        new, moved, damage, actions = P.plan(shapes, bits, sens, mass, j * step - 1.0,
                                             min_bits=np.full(n, b - 1, np.uint8))
        best = min(sum(dmg[i] for i in c) for c in itertools.combinations(range(n), j))
        assert actions == j and moved == j * step
        assert abs(damage - best) <= 1e-15 * max(1.0, best)
        chosen = [i for i in range(n) if new[i] == b - 1]
        assert abs(sum(dmg[i] for i in chosen) - best) <= 1e-15 * max(1.0, best)


@pytest.mark.parametrize("seed", range(4))
def test_upgrades_match_brute_force_when_steps_are_equal(seed):
    n, b = 6, 4
    shapes, bits, sens, mass = _equal_step_instance(n, b, seed)
    step = P.block_bytes(64, 256, b + 1) - P.block_bytes(64, 256, b)
    gain = [float(sens[i]) * mass[i] * (P.noise(b) - P.noise(b + 1)) for i in range(n)]
    for j in range(0, n + 1):
        new, moved, damage, actions = P.plan(shapes, bits, sens, mass, -(j * step + 1.0),
                                             max_bits=np.full(n, b + 1, np.uint8))
        best = max(sum(gain[i] for i in c) for c in itertools.combinations(range(n), j))
        assert actions == j and moved == -j * step
        assert abs(-damage - best) <= 1e-15 * max(1.0, best)


def test_greedy_definition_step_by_step():
    """On a mixed-shape instance every chosen action is, at its step, the cheapest damage per
    released byte among all available ones (brute-force rescan from the definition)."""
    g = np.random.default_rng(5)
    shapes = P.block_shapes(256, 5, 384, 512)
    n = len(shapes)
    bits = g.choice([3, 4, 5, 6, 8], size=n).astype(np.uint8)
    sens = g.random(n).astype(np.float32)
    mass = P.masses(5, True, g.integers(0, 9, size=5), 8)
    target = 0.4 * sum(P.block_bytes(R, K, int(b)) for (R, K), b in zip(shapes, bits))
    cur = bits.copy()
    released = 0.0
    while released < target:
        opts = []
        for i, (R, K) in enumerate(shapes):
            if cur[i] > 3:
                dB = P.block_bytes(R, K, int(cur[i])) - P.block_bytes(R, K, int(cur[i]) - 1)
                opts.append(((float(sens[i]) * mass[i]) * (P.noise(int(cur[i]) - 1) - P.noise(int(cur[i]))) / dB, i, dB))
        if not opts:
            break
        r, i, dB = min(opts)
        cur[i] -= 1
        released += dB
    new, moved, _, _ = P.plan(shapes, bits, sens, mass, target)
    assert np.array_equal(new, cur) and moved == released


def test_mass_residual_and_stopping():
    shapes = [(32, 128)] * 3
    bits = np.array([6, 6, 6], np.uint8)
    step = P.block_bytes(32, 128, 6) - P.block_bytes(32, 128, 5)
    sens = np.array([1.0, 1.0, 1.0], np.float32)
    # an expert with no routed tokens (mass 0) is the free first choice
    new, moved, dmg, n = P.plan(shapes, bits, sens, [0.5, 0.0, 0.5], step)
    assert new.tolist() == [6, 5, 6] and dmg == 0.0 and n == 1 and moved == step
    # a prompt residual on block 0 makes block 2 cheaper than block 0
    new, *_ = P.plan(shapes, bits, sens, [0.5, 1.0, 0.5], step, residual=np.array([1.0, 0, 0], np.float32))
    assert new.tolist() == [6, 6, 5]
    # a single block downgraded as far as the floor allows
    one = [(64, 512)]
    new, moved, _, n = P.plan(one, np.array([8], np.uint8), np.ones(1, np.float32), [1.0], 1e12)
    assert new.tolist() == [3] and n == 5 and moved == P.block_bytes(64, 512, 8) - P.block_bytes(64, 512, 3)
    # a budget below the cheapest upgrade changes nothing
    new, moved, _, n = P.plan(one, np.array([3], np.uint8), np.ones(1, np.float32), [1.0], -100.0)
    assert new.tolist() == [3] and moved == 0.0 and n == 0


# ----------------------------------------------------------------------------- library vs oracle
@pytest.fixture(scope="module")
def B():
    from any_precision_bit_amd import binding
    return binding


@pytest.mark.parametrize("seed", range(6))
def test_library_planner_matches_oracle(B, seed):
    g = np.random.default_rng(100 + seed)
    cfg = synth.CONFIGS["qwen_d2048_t16"]
    h = B.pw_layer_create(cfg.d, cfg.E, cfg.F, cfg.k, cfg.Fs, cfg.T)
    try:
        n = cfg.n_blocks
        bits = g.choice([3, 4, 5, 6, 8], size=n).astype(np.uint8)
        B.pw_moe_plan_set(h, bits)
        sens = (g.random(n) * 2).astype(np.float32)
        resid = (g.random(n) * 0.3).astype(np.float32) if seed % 2 else None
        counts = g.multinomial(cfg.T * cfg.k, np.ones(cfg.E) / cfg.E).astype(np.int32)
        lo = np.minimum(bits, g.choice([1, 2, 3], size=n)).astype(np.uint8) if seed % 3 == 0 else None
        hi = np.maximum(bits, 8).astype(np.uint8)
        total = sum(P.block_bytes(R, K, int(b)) for (R, K), b in zip(P.block_shapes(cfg.d, cfg.E, cfg.F, cfg.Fs), bits))
        shapes = P.block_shapes(cfg.d, cfg.E, cfg.F, cfg.Fs)
        mass = P.masses(cfg.E, True, counts, cfg.T)
        for frac in (0.05, 0.3, -0.1, -0.5):
            tgt = frac * total
            got = B.pw_plan_greedy(h, sens, counts, cfg.T, tgt, residual=resid, min_bits=lo, max_bits=hi)
            ref = P.plan(shapes, bits, sens, mass, tgt, residual=resid, min_bits=lo, max_bits=hi)
            assert np.array_equal(got[0], ref[0]), frac
            assert got[1] == ref[1] and got[3] == ref[3]
            assert abs(got[2] - ref[2]) <= 1e-12 * max(1e-30, abs(ref[2]))
    finally:
        B.pw_layer_destroy(h)


def test_library_planner_validation(B):
    h = B.pw_layer_create(256, 4, 512, 2, 0, 8)
    try:
        sens = np.ones(12, np.float32)
        cnt = np.array([2, 2, 2, 2], np.int32)
        with pytest.raises(B.PwError) as ei:
            B.pw_plan_greedy(h, sens, cnt, 8, 1e5)
        assert ei.value.status == 7                        # no plan yet
        B.pw_moe_plan_set(h, [3, 4, 5] * 4)
        with pytest.raises(B.PwError) as ei:
            B.pw_plan_greedy(h, np.full(12, -1.0, np.float32), cnt, 8, 1e5)
        assert ei.value.status == 1
        with pytest.raises(B.PwError) as ei:
            B.pw_plan_greedy(h, sens, cnt, 0, 1e5)
        assert ei.value.status == 1
        with pytest.raises(B.PwError) as ei:
            B.pw_plan_greedy(h, sens, cnt, 8, 1e5, min_bits=np.full(12, 4, np.uint8))
        assert ei.value.status == 3                        # current plan below the floor
        out, moved, dmg, n = B.pw_plan_greedy(h, sens, cnt, 8, 0.0)
        assert out.tolist() == [3, 4, 5] * 4 and n >= 0
    finally:
        B.pw_layer_destroy(h)


def test_library_planner_row_blocks_matches_oracle(B):
    """Linear-blocks of 128 rows: the planner works on every row-block."""
    g = np.random.default_rng(7)
    cfg = synth.CONFIGS["qwen_d2048_t16"]
    rb = 128
    h = B.pw_layer_create(cfg.d, cfg.E, cfg.F, cfg.k, cfg.Fs, cfg.T, rows_per_block=rb)
    try:
        bits = synth.rowblock_bits(cfg, rb)
        n = bits.shape[0]
        B.pw_moe_plan_set(h, bits)
        shapes = P.block_shapes(cfg.d, cfg.E, cfg.F, cfg.Fs, rb)
        assert len(shapes) == n == synth.n_row_blocks(cfg, rb)
        per = [2 * cfg.ffn(e) // rb + cfg.d // rb for e in range(cfg.n_experts_total)]
        sens = g.random(n).astype(np.float32)
        counts = g.multinomial(cfg.T * cfg.k, np.ones(cfg.E) / cfg.E).astype(np.int32)
        mass = P.masses(cfg.E, True, counts, cfg.T, per)
        total = sum(P.block_bytes(R, K, int(b)) for (R, K), b in zip(shapes, bits))
        for frac in (0.1, -0.2):
            got = B.pw_plan_greedy(h, sens, counts, cfg.T, frac * total)
            ref = P.plan(shapes, bits, sens, mass, frac * total)
            assert np.array_equal(got[0], ref[0]) and got[1] == ref[1] and got[3] == ref[3]
    finally:
        B.pw_layer_destroy(h)
