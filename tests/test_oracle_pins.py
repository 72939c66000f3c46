"""Pins of the CPU oracle to things other than itself (no GPU needed).

Each test fixes one part of the oracle against a definition, a brute force,
a closed form, a library routine, or a value worked by hand under
tests/golden/ -- chosen so that a dropped term, a wrong sign, a wrong bit or
plane order, or a transposed operand fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth
from synth import GATE, UP, DOWN

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def hand_pack(q, n_planes=8):
    """Bit-planes written out from the format definition, one bit at a time."""
    R, K = q.shape
    planes = np.zeros((n_planes, R, K // 8), dtype=np.uint8)
    for p in range(n_planes):
        for r in range(R):
            for c in range(K):
                bit = (int(q[r, c]) >> (7 - p)) & 1
                planes[p, r, c >> 3] |= bit << (c & 7)
    return planes


# ----------------------------------------------------------------------------- O5 format
def test_golden_format_fixture():
    g = json.load(open(os.path.join(GOLDEN, "ap_format_tiny.json")))
    q = np.array([g["q"]], dtype=np.uint8)
    planes = np.array(g["planes"], dtype=np.uint8).reshape(8, 1, 1)
    # the generator's packing equals the hand-worked planes
    assert np.array_equal(synth.pack_planes(q), planes)
    assert np.array_equal(hand_pack(q), planes)
    # the oracle's bit-by-bit assembly reads them as the hand-worked indices
    assert oracle.unpack_indices(planes, 3).tolist() == [g["idx_b3"]]
    assert oracle.unpack_indices(planes, 5).tolist() == [g["idx_b5"]]


def test_index_truncation_bruteforce():
    rng = np.random.default_rng(7)
    q_all = np.arange(256, dtype=np.uint8).reshape(1, 256)       # every parent value
    q_rand = rng.integers(0, 256, size=(5, 128), dtype=np.uint8)
    for q in (q_all, q_rand):
        planes = hand_pack(q)
        assert np.array_equal(planes, synth.pack_planes(q))
        for b in range(1, 9):
            idx = oracle.unpack_indices(planes, b)
            assert np.array_equal(idx, q >> (8 - b)), b


def test_index_uses_only_top_planes():
    # Corrupting planes b..7 must not change the bitwidth-b view.
    rng = np.random.default_rng(3)
    q = rng.integers(0, 256, size=(3, 64), dtype=np.uint8)
    planes = synth.pack_planes(q)
    for b in range(1, 8):
        bad = planes.copy()
        bad[b:] ^= 0xFF
        assert np.array_equal(oracle.unpack_indices(bad, b), q >> (8 - b))


def test_b8_reproduces_parent_dequant():
    cfg = synth.CONFIGS["tiny_d256"]
    for lin in (GATE, DOWN):
        q = synth.parent_indices(cfg, 2, lin)
        planes = synth.pack_planes(q)
        lut8 = synth.lut(cfg, 2, lin, 8)
        W = oracle.dequant(planes, 8, lut8)
        ref = lut8[np.arange(q.shape[0])[:, None], q].astype(np.float32)
        assert np.array_equal(W.view(np.uint32), ref.view(np.uint32))


def test_dequant_bitwidth_b_matches_truncated_parent():
    cfg = synth.CONFIGS["tiny_d256"]
    q = synth.parent_indices(cfg, 1, UP)
    planes = synth.pack_planes(q)
    for b in (3, 4, 5, 6, 8):
        lut_b = synth.lut(cfg, 1, UP, b)
        W = oracle.dequant(planes, b, lut_b)
        ref = lut_b[np.arange(q.shape[0])[:, None], q >> (8 - b)].astype(np.float32)
        assert np.array_equal(W, ref)


def test_identity_lut_closed_form():
    # LUT_b[r][i] = i (exact in fp16) and a one-hot input e_c: g[r] = q[r][c] >> (8-b).
    rng = np.random.default_rng(11)
    R, K = 24, 256
    q = rng.integers(0, 256, size=(R, K), dtype=np.uint8)
    planes = synth.pack_planes(q)
    for b in (1, 3, 4, 6, 8):
        lut_id = np.tile(np.arange(1 << b, dtype=np.float16), (R, 1))
        for c in (0, 7, 8, 131, 255):
            x = np.zeros(K, dtype=np.float16)
            x[c] = 1.0
            g = oracle.linear(planes, b, lut_id, x)
            assert np.array_equal(g, (q[:, c] >> (8 - b)).astype(np.float32)), (b, c)


# ----------------------------------------------------------------------------- O1..O4 routing
def exact_logits_py(x, wr, bias=None):
    """Python-integer logits in units of 2^-48 (each fp16 value times 2^24 is an integer)."""
    X = [[int(float(v) * 2 ** 24) for v in row] for row in np.asarray(x, np.float16)]
    W = [[int(float(v) * 2 ** 24) for v in row] for row in np.asarray(wr, np.float16)]
    out = []
    for xr in X:
        row = []
        for e, wrow in enumerate(W):
            s = sum(a * b for a, b in zip(xr, wrow))
            if bias is not None:
                s += int(float(np.float16(bias[e])) * 2 ** 48)
            row.append(s)
        out.append(row)
    return out


def test_golden_router_fixture():
    g = json.load(open(os.path.join(GOLDEN, "router_tiny.json")))
    x = np.array(g["x"], dtype=np.float16)
    wr = np.array(g["router_w"], dtype=np.float16)
    L, st = oracle.router_logits(x, wr)
    assert st == oracle.ORC_OK
    assert L.tolist() == g["logits_2m48"]
    ids, w = oracle.topk_softmax(L, g["k"])
    assert ids.tolist() == g["ids"]
    assert np.allclose(w, np.array(g["w"]), rtol=0, atol=1e-7)
    counts, offsets, srt = oracle.bucket_sort(ids, wr.shape[0])
    assert counts.tolist() == g["counts"]
    assert offsets.tolist() == g["offsets"]
    assert srt.tolist() == g["sorted"]


@pytest.mark.parametrize("cname", ["tiny_d256", "mixtral_d4096"])
def test_router_exact_vs_python_int(cname):
    cfg = synth.CONFIGS[cname]
    if cname == "mixtral_d4096":
        # a slice of the Zipf-biased Mixtral-shaped router, exercising the bias term
        wr, bias = synth.router(cfg)
        wr = wr[:, :512]
        x = synth.tokens(cfg, 3)[:, :512]
    else:
        wr, bias = synth.router(cfg)
        x = synth.tokens(cfg)
    L, st = oracle.router_logits(x, wr, bias)
    assert st == oracle.ORC_OK
    assert L.tolist() == exact_logits_py(x, wr, bias)


def test_router_range_flag():
    x = np.full((1, 128), 60000.0, dtype=np.float16)
    wr = np.full((2, 128), 60000.0, dtype=np.float16)
    _, st = oracle.router_logits(x, wr)
    assert st == oracle.ORC_E_RANGE


def test_topk_and_bucket_sort_bruteforce():
    rng = np.random.default_rng(5)
    T, E, k = 37, 12, 3
    # few distinct values -> many exact ties
    L = rng.integers(-3, 4, size=(T, E)).astype(np.int64) * (1 << 40)
    ids, w = oracle.topk_softmax(L, k)
    ref = np.argsort(-L, axis=1, kind="stable")[:, :k]   # stable: ties keep the lower index
    assert np.array_equal(ids, ref)
    counts, offsets, srt = oracle.bucket_sort(ids, E)
    assert np.array_equal(counts, np.bincount(ids.reshape(-1), minlength=E))
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    flat = ids.reshape(-1)
    assert np.array_equal(srt, np.argsort(flat, kind="stable"))


def test_topk_all_experts_and_identical_rows():
    cfg = synth.CONFIGS["tiny_d256"]
    x = synth.tokens(cfg)
    wr, _ = synth.router(cfg)
    wr = wr.copy()
    wr[5] = wr[2]                       # identical rows -> identical logits
    L, _ = oracle.router_logits(x, wr)
    assert np.array_equal(L[:, 5], L[:, 2])
    ids, w = oracle.topk_softmax(L, cfg.E)
    for t in range(x.shape[0]):
        assert sorted(ids[t].tolist()) == list(range(cfg.E))
        pos = ids[t].tolist()
        assert pos.index(2) == pos.index(5) - 1   # tie: lower index first, adjacent


def test_softmax_weights():
    rng = np.random.default_rng(9)
    T, E = 50, 16
    L = rng.integers(-(1 << 50), 1 << 50, size=(T, E)).astype(np.int64)
    for k in (1, 2, 4, 8):
        ids, w = oracle.topk_softmax(L, k)
        assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= k * 2.0 ** -23)
        if k == 1:
            assert np.all(w == 1.0)
        assert np.all(np.diff(w, axis=1) <= 0)          # descending logits -> descending w
    # two experts at logit gap delta: w0 = 1 / (1 + exp(-delta))
    for delta in (0.0, 0.25, 1.0, 3.5, -0.0):
        L2 = np.array([[int(delta * 2 ** 48), 0]], dtype=np.int64)
        ids, w = oracle.topk_softmax(L2, 2)
        assert abs(w[0, 0] - 1.0 / (1.0 + math.exp(-abs(delta)))) <= 1e-6


# ----------------------------------------------------------------------------- O5..O7 whole layer
SMALL = synth.MoEConfig("small", 90, d=128, E=6, F=256, k=3, T=5, Fs=384,
                        bits_rule="uniform", bits_values=(3, 4, 5, 6, 8))


def dense_reference(cfg, bits, blocks, x, wr, bias):
    """Independent fp64 layer: routing from Python-integer logits, weights
    materialised from the parent indices (not the planes), dense products."""
    L = exact_logits_py(x, wr, bias)
    T = x.shape[0]
    xf = x.astype(np.float64)
    y = np.zeros((T, cfg.d))
    W = {}
    for (e, lin), blk in blocks.items():
        b = int(bits[e, lin])
        W[(e, lin)] = blk.luts[b][np.arange(blk.R)[:, None], blk.q >> (8 - b)].astype(np.float64)

    def expert(e, v):
        g = W[(e, GATE)] @ v
        u = W[(e, UP)] @ v
        a = g / (1.0 + np.exp(-g)) * u
        return W[(e, DOWN)] @ a

    ids_all = []
    for t in range(T):
        order = sorted(range(cfg.E), key=lambda e: (-L[t][e], e))[:cfg.k]
        ids_all.append(order)
        lg = np.array([L[t][e] for e in order], dtype=np.float64) * 2.0 ** -48
        ww = np.exp(lg - lg[0])
        ww /= ww.sum()
        for j, e in enumerate(order):
            y[t] += ww[j] * expert(e, xf[t])
        if cfg.has_shared:
            y[t] += expert(cfg.E, xf[t])
    return y, np.array(ids_all)


def rel_err_per_token(y, ref):
    num = np.abs(y - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    return num / np.maximum(den, 1e-30)


@pytest.mark.parametrize("cfg", [synth.CONFIGS["tiny_d256"], SMALL], ids=["tiny_d256", "small_shared"])
def test_whole_layer_vs_dense_fp64(cfg):
    bits = synth.initial_bits(cfg)
    blocks = synth.make_layer_blocks(cfg, bits, keep_parent=True)
    x = synth.tokens(cfg)
    wr, bias = synth.router(cfg)
    lay = oracle.OracleLayer.from_config(cfg, bits, blocks)
    out = lay.forward(x, wr, bias)
    ref, ref_ids = dense_reference(cfg, bits, blocks, x, wr, bias)
    assert np.array_equal(out["ids"], ref_ids)
    assert rel_err_per_token(out["y"].astype(np.float64), ref).max() <= 1e-5


def test_single_expert_is_textbook_swiglu_mlp():
    import torch
    import torch.nn.functional as Fn

    cfg = synth.MoEConfig("one", 91, d=128, E=1, F=384, k=1, T=6, bits_values=(3, 5, 8))
    bits = synth.initial_bits(cfg)
    blocks = synth.make_layer_blocks(cfg, bits, keep_parent=True)
    x = synth.tokens(cfg)
    wr, _ = synth.router(cfg)
    out = oracle.OracleLayer.from_config(cfg, bits, blocks).forward(x, wr)
    assert np.all(out["w"] == 1.0)
    Wt = {}
    for lin in (GATE, UP, DOWN):
        blk, b = blocks[(0, lin)], int(bits[0, lin])
        Wt[lin] = torch.tensor(blk.luts[b][np.arange(blk.R)[:, None], blk.q >> (8 - b)],
                               dtype=torch.float64)
    xt = torch.tensor(x, dtype=torch.float64)
    ref = (Fn.silu(xt @ Wt[GATE].T) * (xt @ Wt[UP].T)) @ Wt[DOWN].T
    assert rel_err_per_token(out["y"].astype(np.float64), ref.numpy()).max() <= 1e-6


def _layer(cfg, seed=0):
    bits = synth.initial_bits(cfg, run_seed=seed)
    blocks = synth.make_layer_blocks(cfg, bits, run_seed=seed)
    wr, bias = synth.router(cfg, run_seed=seed)
    return bits, blocks, wr, bias


def test_invariances():
    cfg = SMALL
    bits, blocks, wr, bias = _layer(cfg)
    lay = oracle.OracleLayer.from_config(cfg, bits, blocks)
    x = synth.tokens(cfg, 9)
    base = lay.forward(x, wr, bias)
    # token permutation permutes y (bitwise)
    perm = np.random.default_rng(1).permutation(x.shape[0])
    out = lay.forward(x[perm], wr, bias)
    assert np.array_equal(out["y"], base["y"][perm])
    # batch invariance: a token alone equals its row in the batch (bitwise)
    for t in (0, 4, 8):
        alone = lay.forward(x[t:t + 1], wr, bias)
        assert np.array_equal(alone["y"][0], base["y"][t])
    # expert relabeling: permute routed experts' blocks and router rows
    rel = np.random.default_rng(2).permutation(cfg.E)     # new id n holds old expert rel[n]
    blocks2 = dict(blocks)
    bits2 = bits.copy()
    for n in range(cfg.E):
        for lin in range(3):
            blocks2[(n, lin)] = blocks[(int(rel[n]), lin)]
        bits2[n] = bits[int(rel[n])]
    lay2 = oracle.OracleLayer.from_config(cfg, bits2, blocks2)
    out2 = lay2.forward(x, wr[rel], None if bias is None else bias[rel])
    assert np.array_equal(out2["y"], base["y"])
    assert np.array_equal(rel[out2["ids"]], base["ids"])
    # subset evaluation equals the full evaluation on those rows
    sub = lay.forward(x, wr, bias, subset=[7, 2])
    assert np.array_equal(sub["y"][[7, 2]], base["y"][[7, 2]])
    assert np.isnan(sub["y"][0]).all()


def test_zero_input():
    cfg = SMALL
    bits, blocks, wr, _ = _layer(cfg)
    x = np.zeros((3, cfg.d), dtype=np.float16)
    out = oracle.OracleLayer.from_config(cfg, bits, blocks).forward(x, wr, None)
    assert np.all(out["logits"] == 0)
    assert np.array_equal(out["ids"], np.tile(np.arange(cfg.k), (3, 1)))
    assert np.allclose(out["w"], 1.0 / cfg.k, rtol=0, atol=2 ** -24)
    assert np.all(out["y"] == 0.0)


# ----------------------------------------------------------------------------- O8 / O9
def test_plan_change_is_stateless():
    cfg = SMALL
    bits = synth.initial_bits(cfg)
    rng = np.random.default_rng(4)
    blocks = synth.make_layer_blocks(cfg, bits, all_luts=True)
    wr, bias = synth.router(cfg)
    x = synth.tokens(cfg)
    lay = oracle.OracleLayer.from_config(cfg, bits, blocks)
    lay.forward(x, wr, bias)
    new = bits.copy()
    flip = rng.random(new.shape) < 0.5
    new[flip] = np.maximum(3, new[flip].astype(int) - 2).astype(np.uint8)
    lay.set_bits(new)
    fresh = oracle.OracleLayer.from_config(cfg, new, blocks)
    assert np.array_equal(lay.forward(x, wr, bias)["y"], fresh.forward(x, wr, bias)["y"])


def test_rewrite_plan_rule():
    cfg = synth.CONFIGS["qwen_stack24_t256"]
    bits = synth.initial_bits(cfg, layer=3)
    assert bits.shape == (61, 3)
    new, changed = synth.rewrite_plan(cfg, bits, layer=3, epoch=1)
    diff = np.flatnonzero(new.reshape(-1) != bits.reshape(-1))
    assert sorted(changed) == diff.tolist()
    b0, b1 = bits.reshape(-1), new.reshape(-1)
    n_picked = 0
    g = synth.rng_for(cfg, 0, layer=3, kind=synth.KIND_REWRITE, step=1)
    pick = set(int(i) for i in g.permutation(bits.size)[:45])
    for i in range(bits.size):
        if i in pick:
            n_picked += 1
            assert b1[i] == max(3, int(b0[i]) - 2)
        else:
            assert b1[i] == b0[i]
    assert n_picked == math.floor(0.25 * 183) == 45


def test_residual_rounding_matches_numpy():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal(20000) * 4).astype(np.float16)
    y = rng.standard_normal(20000).astype(np.float32) * np.float32(3)
    y[:50] = np.float32(2.0 ** -20) * rng.standard_normal(50).astype(np.float32)
    x[:50] = np.float16(0)
    y[50:60] = np.float32(70000.0)
    out = oracle.residual(x, y)
    with np.errstate(over="ignore"):
        ref = (x.astype(np.float32) + y).astype(np.float16)   # numpy rounds to nearest even
    assert np.array_equal(out.view(np.uint16), ref.view(np.uint16))


def test_frequency_plan():
    counts = np.array([5, 9, 9, 0, 7] + [1] * 70)
    bits = synth.plan_by_frequency(counts, 75, (8, 4, 3), tier_size=2)
    assert bits[1].tolist() == [8, 8, 8] and bits[2].tolist() == [8, 8, 8]
    assert bits[4].tolist() == [4, 4, 4] and bits[0].tolist() == [4, 4, 4]
    assert bits[3].tolist() == [3, 3, 3]


# ----------------------------------------------------------------------------- linear-blocks of row-blocks
def test_rowblocks_with_one_bitwidth_per_linear_equal_whole_linears():
    """Row-blocks that all carry their linear's bitwidth reproduce the whole-linear layer bitwise."""
    cfg = SMALL
    bits = synth.initial_bits(cfg)
    blocks = synth.make_layer_blocks(cfg, bits)
    x = synth.tokens(cfg)
    wr, bias = synth.router(cfg)
    whole = oracle.OracleLayer.from_config(cfg, bits, blocks).forward(x, wr, bias)
    rb = 64
    flat = []
    for e in range(cfg.n_experts_total):
        for lin in range(3):
            R = cfg.d if lin == DOWN else cfg.ffn(e)
            flat += [bits[e, lin]] * (R // rb)
    rows = oracle.OracleLayer.from_config(cfg, np.array(flat, np.uint8), blocks, rows_per_block=rb).forward(x, wr, bias)
    assert np.array_equal(whole["y"].view(np.uint32), rows["y"].view(np.uint32))


@pytest.mark.parametrize("rb", [64, 128])
def test_rowblocks_vs_dense_fp64(rb):
    """Per-row-block bitwidths against a dense fp64 layer whose weights are materialised row by row
    from the parent indices at the row's block bitwidth."""
    cfg = SMALL
    flat = synth.rowblock_bits(cfg, rb)
    assert len(set(flat.tolist())) > 2
    blocks = {(e, lin): synth.make_block(cfg, e, lin, n_planes=8, lut_bits=(3, 4, 5, 6, 8), keep_parent=True)
              for e in range(cfg.n_experts_total) for lin in range(3)}
    x = synth.tokens(cfg)
    wr, bias = synth.router(cfg)
    out = oracle.OracleLayer.from_config(cfg, flat, blocks, rows_per_block=rb).forward(x, wr, bias)
    # materialise every linear row by row at its block's bitwidth
    W, i = {}, 0
    for e in range(cfg.n_experts_total):
        for lin in range(3):
            blk = blocks[(e, lin)]
            Wm = np.zeros((blk.R, blk.K))
            for j in range(blk.R // rb):
                b = int(flat[i])
                i += 1
                rr = np.arange(j * rb, (j + 1) * rb)
                Wm[rr] = blk.luts[b][rr[:, None], blk.q[rr] >> (8 - b)]
            W[(e, lin)] = Wm
    L = exact_logits_py(x, wr, bias)
    y = np.zeros((cfg.T, cfg.d))
    xf = x.astype(np.float64)
    expert = lambda e, v: W[(e, DOWN)] @ ((lambda g, u: g / (1.0 + np.exp(-g)) * u)(W[(e, GATE)] @ v, W[(e, UP)] @ v))
    for t in range(cfg.T):
        order = sorted(range(cfg.E), key=lambda e: (-L[t][e], e))[:cfg.k]
        lg = np.array([L[t][e] for e in order], dtype=np.float64) * 2.0 ** -48
        ww = np.exp(lg - lg[0])
        ww /= ww.sum()
        for j, e in enumerate(order):
            y[t] += ww[j] * expert(e, xf[t])
        y[t] += expert(cfg.E, xf[t])
    assert rel_err_per_token(out["y"].astype(np.float64), y).max() <= 1e-5
