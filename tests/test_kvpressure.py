"""KV-pressure byte targets (host logic) and the synthetic request trace."""
import numpy as np
import pytest

import synth
from oracle import planner as OP
from synth.kvtrace import kv_bytes_per_token, request_trace


def test_kv_bytes_per_token_of_a_known_shape():
    # Qwen1.5-MoE-A2.7B attention: 24 layers, 16 KV heads of 128, fp16: 2 * 24 * 16 * 128 * 2 bytes
    assert kv_bytes_per_token(24, 16, 128) == 196608
    assert kv_bytes_per_token(1, 16, 128) == 8192


def test_trace_is_seeded_and_follows_its_definition():
    a = request_trace(400, seed=1)
    assert np.array_equal(a, request_trace(400, seed=1)) and not np.array_equal(a, request_trace(400, seed=2))
    assert a[0] >= 0 and a.max() > 5 * max(1, a[0])       # the load rises from an empty start
    assert a[-1] < a.max()                                   # and falls again


@pytest.fixture(scope="module")
def B():
    from any_precision_bit_amd import binding
    return binding


class _Lay:
    def __init__(self, h):
        self.handle = h


def test_targets_drive_the_planner_like_the_oracle(B):
    from any_precision_bit_amd.kvpressure import KVPressurePlanner

    cfg = synth.CONFIGS["qwen_d2048_t16"]
    h = B.pw_layer_create(cfg.d, cfg.E, cfg.F, cfg.k, cfg.Fs, cfg.T)
    try:
        bits = synth.initial_bits(cfg)
        B.pw_moe_plan_set(h, bits)
        shapes = OP.block_shapes(cfg.d, cfg.E, cfg.F, cfg.Fs)
        plan_bytes = lambda bb: sum(OP.block_bytes(R, K, int(b)) for (R, K), b in zip(shapes, np.asarray(bb).reshape(-1)))
        state = {"bits": bits.reshape(-1).copy()}
        sens = np.random.default_rng(2).random(cfg.n_blocks).astype(np.float32)
        counts = np.random.default_rng(3).multinomial(cfg.T * cfg.k, np.ones(cfg.E) / cfg.E)
        w0 = plan_bytes(bits)
        ctl = KVPressurePlanner(_Lay(h), budget_bytes=w0 + 50e6, sensitivity=sens, hysteresis_bytes=5e6,
                                resident_bytes=lambda: plan_bytes(state["bits"]), max_bits=bits.reshape(-1))
        mass = OP.masses(cfg.E, True, counts, cfg.T)
        for kv in (10e6, 48e6, 90e6, 130e6, 60e6, 20e6):
            tgt = plan_bytes(state["bits"]) + kv - (w0 + 50e6)
            d = ctl.decide(kv, counts, cfg.T)
            if -5e6 <= tgt <= 0:
                assert d is None
                continue
            goal = tgt if tgt > 0 else tgt + 5e6
            ref = OP.plan(shapes, state["bits"], sens, mass, goal, max_bits=bits.reshape(-1))
            if ref[3] == 0:
                assert d is None
                continue
            assert np.array_equal(d[0], ref[0])
            if tgt > 0:
                assert plan_bytes(d[0]) + kv <= w0 + 50e6 + 1e-6 or (d[0] == 3).all()
            state["bits"] = d[0].copy()
            B.pw_moe_plan_set(h, d[0])
    finally:
        B.pw_layer_destroy(h)
