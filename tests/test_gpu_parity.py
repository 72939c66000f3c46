"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs. Routing and indices bit-exact; outputs per token within
max |y - y_ref| / max |y_ref| <= 2e-3; routing weights within 1e-6 relative."""
import numpy as np
import pytest

import oracle
import synth
from helpers import (REL_TOL, bind_all, device_pages, f16_host, gpu_layer, layer_inputs,
                     rel_err_per_token, sample_tokens, to_dev_f16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch, torch.device("cuda:0")


def _say(*a):
    print(*a, flush=True)


# ----------------------------------------------------------------------------- debug hooks
@pytest.mark.parametrize("R,K", [(64, 384), (32, 2048)])
def test_unpack_and_dequant_bit_exact(torch_dev, R, K):
    torch, dev = torch_dev
    from any_precision_bit_amd import binding as B
    from any_precision_bit_amd.pages import lut_page

    rng = np.random.default_rng(R + K)
    q = rng.integers(0, 256, size=(R, K), dtype=np.uint8)
    planes_h = synth.pack_planes(q)
    planes = torch.from_numpy(planes_h).to(dev)
    for b in range(1, 9):
        _say(f"unpack/dequant R={R} K={K} b={b}")
        idx = torch.zeros((R, K), dtype=torch.uint8, device=dev)
        B.pw_debug_unpack([planes[p].data_ptr() for p in range(b)], b, R, K, idx.data_ptr())
        torch.cuda.synchronize()
        ref_idx = oracle.unpack_indices(planes_h, b)
        assert np.array_equal(idx.cpu().numpy(), ref_idx), b
        lut_h = (rng.standard_normal((R, 1 << b)) * 0.02).astype(np.float16)
        lut = to_dev_f16(lut_page(lut_h), dev)
        w = torch.zeros((R, K), dtype=torch.float16, device=dev)
        B.pw_debug_dequant([planes[p].data_ptr() for p in range(b)], b, lut.data_ptr(), R, K, w.data_ptr())
        torch.cuda.synchronize()
        ref_w = oracle.dequant(planes_h, b, lut_h).astype(np.float16)
        assert np.array_equal(f16_host(w).view(np.uint16), ref_w.view(np.uint16)), b


# ----------------------------------------------------------------------------- layer parity
def check_routing(route, ref, T, E, k):
    ids = route["topk_ids"].cpu().numpy()
    assert np.array_equal(ids, ref["ids"]), "top-k ids differ"
    assert np.array_equal(route["expert_count"].cpu().numpy(), ref["counts"])
    assert np.array_equal(route["expert_offset"].cpu().numpy(), ref["offsets"])
    assert np.array_equal(route["sorted_assign"].cpu().numpy(), ref["sorted"])
    w = route["topk_w"].cpu().numpy()
    assert np.all(np.abs(w - ref["w"]) <= 1e-6 * np.abs(ref["w"]) + 1e-7)
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= k * 2.0 ** -23 + 1e-6)


def run_parity(torch_dev, cfg, bits, blocks, x, wr, bias, subset, layer=None, pages=None):
    torch, dev = torch_dev
    from any_precision_bit_amd import route_buffers

    T = x.shape[0]
    pages = pages or device_pages(blocks, bits, dev)
    lay = layer or gpu_layer(cfg, bits, pages, max_tokens=T)
    xd, wd = to_dev_f16(x, dev), to_dev_f16(wr, dev)
    bd = None if bias is None else to_dev_f16(bias, dev)
    route = route_buffers(T, cfg.E, cfg.k, dev)
    y = lay.forward(xd, wd, bd, route=route)
    torch.cuda.synchronize()
    assert lay.status() == 0
    ref = oracle.OracleLayer.from_config(cfg, bits, blocks).forward(x, wr, bias, subset=subset)
    check_routing(route, ref, T, cfg.E, cfg.k)
    yh = y.cpu().numpy()
    err = rel_err_per_token(yh[subset], ref["y"][subset])
    _say(f"{cfg.name} T={T}: max rel err {err.max():.3e} over {len(subset)} tokens")
    assert err.max() <= REL_TOL
    return lay, y, ref


def _blocks(cfg, bits, **kw):
    return synth.make_layer_blocks(cfg, bits, **kw)


def test_tiny_full(torch_dev):
    cfg = synth.CONFIGS["tiny_d256"]
    _say("tiny_d256")
    bits = synth.initial_bits(cfg)
    blocks = _blocks(cfg, bits)
    x, wr, bias = layer_inputs(cfg)
    run_parity(torch_dev, cfg, bits, blocks, x, wr, bias, np.arange(cfg.T, dtype=np.int32))


def test_qwen_decode_full(torch_dev):
    cfg = synth.CONFIGS["qwen_d2048_t16"]
    _say("qwen_d2048_t16")
    bits = synth.initial_bits(cfg)
    blocks = _blocks(cfg, bits)
    x, wr, bias = layer_inputs(cfg)
    run_parity(torch_dev, cfg, bits, blocks, x, wr, bias, np.arange(cfg.T, dtype=np.int32))


@pytest.fixture(scope="module")
def c2_data():
    cfg = synth.CONFIGS["mixtral_d4096"]
    bits = synth.initial_bits(cfg)
    return cfg, bits, _blocks(cfg, bits)


@pytest.mark.parametrize("T,n_check", [(1, 1), (64, 8)])
def test_mixtral(torch_dev, c2_data, T, n_check):
    cfg, bits, blocks = c2_data
    _say(f"mixtral_d4096 T={T}")
    cfgT = cfg.with_tokens(T)
    x, wr, bias = layer_inputs(cfgT)
    run_parity(torch_dev, cfgT, bits, blocks, x, wr, bias, sample_tokens(T, n_check, seed=T))


def test_fine_e128(torch_dev):
    cfg = synth.CONFIGS["fine_e128_t128"]
    _say("fine_e128_t128")
    x, wr, bias = layer_inputs(cfg)
    L, _ = oracle.router_logits(x, wr, bias)
    ids, _ = oracle.topk_softmax(L, cfg.k)
    counts = np.bincount(ids.reshape(-1), minlength=cfg.E)
    bits = synth.initial_bits(cfg, counts=counts)
    blocks = _blocks(cfg, bits)
    _, _, ref = run_parity(torch_dev, cfg, bits, blocks, x, wr, bias, sample_tokens(cfg.T, 24, seed=3))
    assert ref["counts"].max() > 32          # exercises the multi-tile (large) kernels


def test_qwen_stack_teacher_forced(torch_dev):
    """A 3-layer slice of the 24-layer stack, 64 decode steps at T=256 with the
    plan rewritten (and pages rebound) before steps 16, 32 and 48. Every step
    runs on the GPU; routing is checked in full and outputs on 4 sampled tokens
    at the steps around each rewrite, each layer on the GPU's own input."""
    torch, dev = torch_dev
    from any_precision_bit_amd import route_buffers

    cfg = synth.CONFIGS["qwen_stack24_t256"]
    n_layers, T = 3, cfg.T
    layers = []
    for l in range(n_layers):
        bits = synth.initial_bits(cfg, layer=l)
        blocks = _blocks(cfg, bits, layer=l, all_luts=True)
        pages = device_pages(blocks, bits, dev, all_luts=True)
        lay = gpu_layer(cfg, bits, pages, max_tokens=T)
        wr, bias = synth.router(cfg, layer=l)
        layers.append(dict(bits=bits, blocks=blocks, pages=pages, lay=lay, wr=wr,
                           wd=to_dev_f16(wr, dev), orc=oracle.OracleLayer.from_config(cfg, bits, blocks)))
    check_steps = {0, 15, 16, 31, 32, 47, 48, 63}
    route = route_buffers(T, cfg.E, cfg.k, dev)
    y = torch.empty((T, cfg.d), dtype=torch.float32, device=dev)
    for s in range(cfg.steps):
        if s > 0 and s % cfg.rewrite_every == 0:
            for l, L in enumerate(layers):
                new, changed = synth.rewrite_plan(cfg, L["bits"], layer=l, epoch=s // cfg.rewrite_every)
                L["bits"] = new
                L["lay"].plan_set(new)
                for blk in changed:
                    e, lin = divmod(blk, 3)
                    planes, luts = L["pages"][(e, lin)]
                    b = int(new[e, lin])
                    L["lay"].bind(e, lin, [planes[p] for p in range(b)], luts[b], b)
                L["orc"].set_bits(new)
        x = to_dev_f16(synth.tokens(cfg, T, step=s), dev)
        for l, L in enumerate(layers):
            x_next = torch.empty_like(x)
            L["lay"].forward(x, L["wd"], None, y=y, x_next=x_next, route=route)
            if s in check_steps:
                torch.cuda.synchronize()
                xh = f16_host(x)
                sub = sample_tokens(T, 4, seed=100 * s + l)
                ref = L["orc"].forward(xh, L["wr"], None, subset=sub)
                check_routing(route, ref, T, cfg.E, cfg.k)
                err = rel_err_per_token(y.cpu().numpy()[sub], ref["y"][sub])
                _say(f"qwen_stack24_t256 step {s} layer {l}: max rel err {err.max():.3e}")
                assert err.max() <= REL_TOL
                xn_ref = oracle.residual(xh, y.cpu().numpy())   # O9 on the GPU's own y
                assert np.array_equal(f16_host(x_next).view(np.uint16), xn_ref.view(np.uint16))
            x = x_next
    torch.cuda.synchronize()
    for L in layers:
        assert L["lay"].status() == 0



def test_dependency_wait_limit_flags_and_recovers(torch_dev):
    """With the down items' dependency wait limited to zero polls, a down item that finds its
    gate_up rows unfinished gives up: the forward still completes, and the status word reports
    PW_STATUS_DEP_TIMEOUT (every item of this small layer starts in the first round, so the down
    items poll before their gate_up items can have finished). Back at the default limit the
    same layer and pages are exact again."""
    torch, dev = torch_dev
    from any_precision_bit_amd import binding as B

    cfg = synth.CONFIGS["tiny_d256"]
    bits = synth.initial_bits(cfg)
    blocks = _blocks(cfg, bits)
    x, wr, bias = layer_inputs(cfg)
    pages = device_pages(blocks, bits, dev)
    lay = gpu_layer(cfg, bits, pages, max_tokens=cfg.T)
    _say("dependency wait limit 0")
    lay.set_wait_limit(0)
    lay.forward(to_dev_f16(x, dev), to_dev_f16(wr, dev))
    torch.cuda.synchronize()
    flags = lay.status()
    assert flags & B.PW_STATUS_DEP_TIMEOUT, flags
    assert lay.status() == 0                      # read and cleared
    lay.set_wait_limit(1 << 20)
    run_parity(torch_dev, cfg, bits, blocks, x, wr, bias, np.arange(cfg.T, dtype=np.int32),
               layer=lay, pages=pages)



def test_qwen_stack_all_layers_independent_inputs(torch_dev):
    """All 24 layers of the stack at T=256, with the plan rewritten (and pages rebound) before steps
    16, 32 and 48, in the configuration `bench.py --stack` times: each layer takes its own seeded
    input per step. The steps on both sides of each rewrite run: routing is checked on every token
    of every layer, and outputs on one sampled token of a quarter of the layers (rotating) at the
    first step of each plan epoch. A forward leaves no state behind but the plan and the pages, so
    the steps in between, which only repeat the same kernels, are skipped."""
    torch, dev = torch_dev
    from any_precision_bit_amd import route_buffers

    from concurrent.futures import ThreadPoolExecutor

    cfg = synth.CONFIGS["qwen_stack24_t256"]
    T = cfg.T

    def reachable(b):   # bitwidths a block at b passes through under the rewrites
        out = {b}
        for _ in range(cfg.steps // cfg.rewrite_every):
            b = max(3, b - 2)
            out.add(b)
        return tuple(sorted(out))

    def stack_blocks(bits, l):   # planes 0..b-1 and the LUTs of every reachable bitwidth
        jobs = [(e, lin) for e in range(cfg.n_experts_total) for lin in synth.LINEARS]
        with ThreadPoolExecutor(max_workers=16) as ex:
            made = list(ex.map(lambda j: synth.make_block(cfg, j[0], j[1], layer=l, n_planes=int(bits[j]),
                                                          lut_bits=reachable(int(bits[j]))), jobs))
        return {(blk.e, blk.lin): blk for blk in made}

    layers = []
    for l in range(cfg.layers):
        bits = synth.initial_bits(cfg, layer=l)
        blocks = stack_blocks(bits, l)
        pages = device_pages(blocks, bits, dev, all_luts=True)
        lay = gpu_layer(cfg, bits, pages, max_tokens=T)
        wr, _ = synth.router(cfg, layer=l)
        layers.append(dict(bits=bits, pages=pages, lay=lay, wr=wr, wd=to_dev_f16(wr, dev),
                           orc=oracle.OracleLayer.from_config(cfg, bits, blocks)))
    _say(f"stack: {cfg.layers} layers ready")
    check_steps = {0, 15, 16, 31, 32, 47, 48, 63}
    route = route_buffers(T, cfg.E, cfg.k, dev)
    y = torch.empty((T, cfg.d), dtype=torch.float32, device=dev)
    x_next = torch.empty((T, cfg.d), dtype=torch.float16, device=dev)
    worst = 0.0
    for s in range(cfg.steps):
        if s > 0 and s % cfg.rewrite_every == 0:
            for l, L in enumerate(layers):
                new, changed = synth.rewrite_plan(cfg, L["bits"], layer=l, epoch=s // cfg.rewrite_every)
                L["bits"] = new
                L["lay"].plan_set(new)
                for blk in changed:
                    e, lin = divmod(int(blk), 3)
                    planes, luts = L["pages"][(e, lin)]
                    b = int(new[e, lin])
                    L["lay"].bind(e, lin, [planes[p] for p in range(b)], luts[b], b)
                L["orc"].set_bits(new)
        if s not in check_steps:
            continue
        epoch = s // cfg.rewrite_every
        for l, L in enumerate(layers):
            x = synth.tokens(cfg, T, step=s, layer=l)
            L["lay"].forward(to_dev_f16(x, dev), L["wd"], None, y=y, x_next=x_next, route=route)
            torch.cuda.synchronize()
            outputs = s % cfg.rewrite_every == 0 and l % 4 == epoch % 4
            sub = sample_tokens(T, 1, seed=1000 * s + l) if outputs else np.zeros(0, dtype=np.int32)
            ref = L["orc"].forward(x, L["wr"], None, subset=sub)
            check_routing(route, ref, T, cfg.E, cfg.k)
            if outputs:
                err = rel_err_per_token(y.cpu().numpy()[sub], ref["y"][sub])
                worst = max(worst, float(err.max()))
                assert err.max() <= REL_TOL, (s, l, err.max())
        _say(f"stack step {s}: routing exact on all {cfg.layers} layers, worst rel err so far {worst:.3e}")
    torch.cuda.synchronize()
    for L in layers:
        assert L["lay"].status() == 0


# ----------------------------------------------------------------------------- edge cases
SMALL = synth.MoEConfig("gsmall", 92, d=256, E=6, F=384, k=3, T=40, Fs=512,
                        bits_rule="uniform", bits_values=(1, 2, 3, 4, 5, 6, 7, 8))


def test_all_bitwidths_shared_and_ragged(torch_dev):
    """b = 1..8 mixed per block, a shared expert, F % 256 == 128 (ragged chunk)
    and T = 40 > 32 (both kernel variants)."""
    cfg = SMALL
    bits = synth.initial_bits(cfg)
    for b in range(1, 9):
        assert (bits == b).any() or True
    blocks = synth.make_layer_blocks(cfg, bits, all_luts=False)
    x, wr, bias = layer_inputs(cfg)
    run_parity(torch_dev, cfg, bits, blocks, x, wr, bias, np.arange(cfg.T, dtype=np.int32))


TWO_GROUPS = synth.MoEConfig("gtwo", 93, d=256, E=4, F=384, k=2, T=32, Fs=512,
                             bits_rule="uniform", bits_values=(3, 4, 5, 6, 8))


def test_two_token_groups_one_kernel(torch_dev):
    """T = 32: experts with 17..32 tokens (and the 32-token shared expert) run as two
    16-token groups in the one-tile kernel; no 64-token launch."""
    cfg = TWO_GROUPS
    bits = synth.initial_bits(cfg)
    blocks = synth.make_layer_blocks(cfg, bits)
    x, wr, bias = layer_inputs(cfg)
    _, _, ref = run_parity(torch_dev, cfg, bits, blocks, x, wr, bias, np.arange(cfg.T, dtype=np.int32))
    assert ((ref["counts"] > 16) & (ref["counts"] <= 32)).any(), ref["counts"]


def test_t0_noop_and_max_tokens(torch_dev):
    torch, dev = torch_dev
    cfg = synth.CONFIGS["tiny_d256"]
    bits = synth.initial_bits(cfg)
    blocks = _blocks(cfg, bits)
    pages = device_pages(blocks, bits, dev)
    lay = gpu_layer(cfg, bits, pages, max_tokens=64)
    x, wr, bias = layer_inputs(cfg, 64)
    y = torch.full((64, cfg.d), 7.0, device=dev)
    lay.forward(to_dev_f16(x, dev)[:0], to_dev_f16(wr, dev), None, y=y[:0])
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
    run_parity(torch_dev, cfg.with_tokens(64), bits, blocks, x, wr, bias,
               np.arange(64, dtype=np.int32), layer=lay, pages=pages)


def test_ties_zero_input_and_determinism(torch_dev):
    torch, dev = torch_dev
    from any_precision_bit_amd import route_buffers

    cfg = synth.CONFIGS["tiny_d256"].with_tokens(16)
    bits = synth.initial_bits(cfg)
    blocks = _blocks(cfg, bits)
    x, wr, _ = layer_inputs(cfg)
    wr = wr.copy()
    wr[6] = wr[1]
    wr[7] = wr[1]                  # three identical experts -> exact logit ties
    x[3] = 0.0                     # all-zero token: every logit 0, ids 0..k-1, y = 0
    lay, y, ref = run_parity(torch_dev, cfg, bits, blocks, x, wr, None, np.arange(16, dtype=np.int32))
    assert ref["ids"][3].tolist() == [0, 1]
    assert float(y[3].abs().max()) == 0.0
    route2 = route_buffers(16, cfg.E, cfg.k, dev)
    y2 = lay.forward(to_dev_f16(x, dev), to_dev_f16(wr, dev), None, route=route2)
    torch.cuda.synchronize()
    assert np.array_equal(route2["topk_ids"].cpu().numpy(), ref["ids"])
    assert np.array_equal(route2["sorted_assign"].cpu().numpy(), ref["sorted"])
    assert rel_err_per_token(y2.cpu().numpy(), y.cpu().numpy()).max() <= 1e-5


def test_plan_rewrite_and_rebind(torch_dev):
    torch, dev = torch_dev
    cfg = synth.CONFIGS["qwen_d2048_t16"].with_tokens(8)
    bits = synth.initial_bits(cfg)
    blocks = _blocks(cfg, bits, all_luts=True)
    pages = device_pages(blocks, bits, dev, all_luts=True)
    x, wr, bias = layer_inputs(cfg)
    lay, _, _ = run_parity(torch_dev, cfg, bits, blocks, x, wr, bias, np.arange(8, dtype=np.int32),
                           pages=pages)
    new = bits.copy()
    new[::2, :] = np.maximum(3, new[::2, :].astype(int) - 2).astype(np.uint8)
    new[1::3, 2] = 8
    lay.plan_set(new)
    bind_all(lay, new, pages)
    run_parity(torch_dev, cfg, new, blocks, x, wr, bias, np.arange(8, dtype=np.int32), layer=lay,
               pages=pages)


def test_router_range_flag(torch_dev):
    torch, dev = torch_dev
    cfg = synth.CONFIGS["tiny_d256"]
    bits = synth.initial_bits(cfg)
    blocks = _blocks(cfg, bits)
    lay = gpu_layer(cfg, bits, device_pages(blocks, bits, dev))
    x, wr, _ = layer_inputs(cfg)
    x = x.copy()
    x[1, 5] = 300.0                # outside the exact-router range
    lay.forward(to_dev_f16(x, dev), to_dev_f16(wr, dev), None)
    torch.cuda.synchronize()
    assert lay.status() == 1
    assert lay.status() == 0       # cleared by the read
