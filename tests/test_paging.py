"""Page bookkeeping of asynchronous page movement (host logic, no GPU)."""
import itertools

import numpy as np

import synth
from any_precision_bit_amd.paging import page_delta, pages_of
from oracle import planner as OP


def test_page_delta_transforms_residency_exactly():
    for a, b in itertools.product(range(1, 9), repeat=2):
        load, drop = page_delta([a], [b])
        have = pages_of(a)
        ld, dr = load.get(0, set()), drop.get(0, set())
        assert not (ld & have) and dr <= have
        assert (have - dr) | ld == pages_of(b)
        if a == b:
            assert not ld and not dr


def test_page_delta_bytes_match_plan_bytes():
    """The bytes a plan change loads minus the bytes it drops equal the change of the plan's resident
    bytes, with page sizes taken from generated pages."""
    cfg = synth.CONFIGS["tiny_d256"]
    blk = synth.make_block(cfg, 0, 2, n_planes=8, lut_bits=tuple(range(1, 9)))
    size = lambda pg: blk.planes[pg[1]].nbytes if pg[0] == "plane" else blk.luts[pg[1]].nbytes
    g = np.random.default_rng(3)
    old = g.integers(1, 9, size=12)
    new = g.integers(1, 9, size=12)
    load, drop = page_delta(old, new)
    moved = sum(size(p) for s in load.values() for p in s) - sum(size(p) for s in drop.values() for p in s)
    expect = sum(OP.block_bytes(blk.R, blk.K, int(b)) for b in new) - sum(OP.block_bytes(blk.R, blk.K, int(b)) for b in old)
    assert moved == expect
