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
        ref_w = oracle.dequant(planes_h, b, lut_h).astype(np.float16)
        for tiled in (False, True):
            lut = to_dev_f16(lut_page(lut_h) if tiled else lut_h, dev)
            w = torch.zeros((R, K), dtype=torch.float16, device=dev)
            B.pw_debug_dequant([planes[p].data_ptr() for p in range(b)], b, lut.data_ptr(), R, K, w.data_ptr(),
                               lut_flags=B.PW_FLAG_LUT_TILED if tiled else 0)
            torch.cuda.synchronize()
            assert np.array_equal(f16_host(w).view(np.uint16), ref_w.view(np.uint16)), (b, tiled)


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


def run_parity(torch_dev, cfg, bits, blocks, x, wr, bias, subset, layer=None, pages=None, lut_tiled=False,
               max_tokens=None, path=None, ref=None):
    torch, dev = torch_dev
    from any_precision_bit_amd import route_buffers

    T = x.shape[0]
    pages = pages or device_pages(blocks, bits, dev, lut_tiled=lut_tiled)
    lay = layer or gpu_layer(cfg, bits, pages, max_tokens=max_tokens or T, lut_tiled=lut_tiled)
    if path is not None:
        lay.set_path(path)
    xd, wd = to_dev_f16(x, dev), to_dev_f16(wr, dev)
    bd = None if bias is None else to_dev_f16(bias, dev)
    route = route_buffers(T, cfg.E, cfg.k, dev)
    y = lay.forward(xd, wd, bd, route=route)
    torch.cuda.synchronize()
    assert lay.status() == 0
    if ref is None:
        ref = oracle.OracleLayer.from_config(cfg, bits, blocks, rows_per_block=lay.rows_per_block).forward(
            x, wr, bias, subset=subset)
    check_routing(route, ref, T, cfg.E, cfg.k)
    yh = y.cpu().numpy()
    err = rel_err_per_token(yh[subset], ref["y"][subset])
    _say(f"{cfg.name} T={T}{'' if path is None else ' path=' + str(path)}: max rel err {err.max():.3e} "
         f"over {len(subset)} tokens")
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


@pytest.mark.parametrize("lut_tiled", [False, True])
def test_qwen_decode_full(torch_dev, lut_tiled):
    cfg = synth.CONFIGS["qwen_d2048_t16"]
    _say(f"qwen_d2048_t16 lut_tiled={lut_tiled}")
    bits = synth.initial_bits(cfg)
    blocks = _blocks(cfg, bits)
    x, wr, bias = layer_inputs(cfg)
    run_parity(torch_dev, cfg, bits, blocks, x, wr, bias, np.arange(cfg.T, dtype=np.int32), lut_tiled=lut_tiled)


@pytest.fixture(scope="module")
def c2_data():
    cfg = synth.CONFIGS["mixtral_d4096"]
    bits = synth.initial_bits(cfg)
    return cfg, bits, _blocks(cfg, bits)


@pytest.mark.parametrize("T", [1, 64])
def test_mixtral(torch_dev, c2_data, T):
    cfg, bits, blocks = c2_data
    _say(f"mixtral_d4096 T={T}")
    cfgT = cfg.with_tokens(T)
    x, wr, bias = layer_inputs(cfgT)
    run_parity(torch_dev, cfgT, bits, blocks, x, wr, bias, np.arange(T, dtype=np.int32))


def test_fine_e128(torch_dev):
    cfg = synth.CONFIGS["fine_e128_t128"]
    _say("fine_e128_t128")
    x, wr, bias = layer_inputs(cfg)
    L, _ = oracle.router_logits(x, wr, bias)
    ids, _ = oracle.topk_softmax(L, cfg.k)
    counts = np.bincount(ids.reshape(-1), minlength=cfg.E)
    bits = synth.initial_bits(cfg, counts=counts)
    blocks = _blocks(cfg, bits)
    _, _, ref = run_parity(torch_dev, cfg, bits, blocks, x, wr, bias, np.arange(cfg.T, dtype=np.int32))
    assert ref["counts"].max() > 32          # exercises the multi-tile (large) kernels


@pytest.mark.parametrize("name,T", [("tiny_d256", 200), ("fine_e128_t128", 128), ("qwen_d2048_t16", 300)])
def test_expert_paths(torch_dev, name, T):
    """Every A/B path of the expert kernels on the same layer and batch: the one-tile kernel alone,
    the two-tile kernel alone (32-token groups, ragged last groups), the four-tile kernel for
    experts above 32 tokens, the dequantise-once kernel for them (the default) and for every
    expert. T = 300 puts the qwen shared expert in three 128-token passes (a ragged 44-token third
    pass); tiny_d256 and fine_e128_t128 have routed experts above 32 tokens."""
    cfg = synth.CONFIGS[name].with_tokens(T)
    _say(f"{name} T={T}: expert paths")
    x, wr, bias = layer_inputs(cfg)
    L, _ = oracle.router_logits(x, wr, bias)
    ids, _ = oracle.topk_softmax(L, cfg.k)
    counts = np.bincount(ids.reshape(-1), minlength=cfg.E)
    bits = synth.initial_bits(cfg, counts=counts) if name == "fine_e128_t128" else synth.initial_bits(cfg)
    blocks = _blocks(cfg, bits)
    if T <= 200:
        subset = np.arange(T, dtype=np.int32)
    else:   # tokens of the largest routed experts, and both shared-expert passes
        big = np.argsort(-counts, kind="stable")[:3]
        toks = np.unique(np.nonzero(np.isin(ids, big))[0])
        subset = np.unique(np.concatenate([toks[:12], np.arange(0, T, 23), [T - 1]])).astype(np.int32)
    assert counts.max() > 32 or (cfg.Fs > 0 and T > 256)
    lay, ref = None, None
    for path in ["auto", "small", "two", "four", "big"]:
        lay, _, ref = run_parity(torch_dev, cfg, bits, blocks, x, wr, bias, subset, layer=lay, path=path, ref=ref)


@pytest.mark.parametrize("name,T", [("qwen_d2048_t16", 300), ("mixtral_d4096", 64)])
def test_deterministic_accumulation(torch_dev, name, T):
    """PW_FLAG_DETERMINISTIC: two forwards of the same batch give bit-identical y on every expert
    path, and each matches the oracle. qwen T = 300 runs the two-tile kernel (routed experts, T k
    above 16 per expert) and the dequantise-once kernel (the shared expert in three passes, three
    K-pieces); mixtral T = 64 runs the one- and four-tile kernels with seven K-pieces per routed
    down projection; the two path runs both layers in the two-tile kernel."""
    torch, dev = torch_dev
    cfg = synth.CONFIGS[name].with_tokens(T)
    _say(f"{name} T={T}: deterministic accumulation")
    x, wr, bias = layer_inputs(cfg)
    bits = synth.initial_bits(cfg)
    blocks = _blocks(cfg, bits)
    pages = device_pages(blocks, bits, dev)
    lay = gpu_layer(cfg, bits, pages, max_tokens=T, deterministic=True)
    subset = sample_tokens(T, 12, seed=5)
    ref = None
    for path in ["auto", "small", "two", "four", "big"]:
        lay, y, ref = run_parity(torch_dev, cfg, bits, blocks, x, wr, bias, subset, layer=lay, path=path, ref=ref)
        y2 = lay.forward(to_dev_f16(x, dev), to_dev_f16(wr, dev), None if bias is None else to_dev_f16(bias, dev))
        torch.cuda.synchronize()
        assert torch.equal(y, y2), path
    lay.close()


def _rewrite_all(cfg, layers, s):
    """The plan rewrite before step s (a multiple of the rewrite period): each layer's seeded blocks
    lose bits; the GPU layer is re-planned and the changed blocks rebound; the oracle follows."""
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


def test_qwen_stack_teacher_forced(torch_dev):
    """A 3-layer slice of the 24-layer stack, 64 decode steps at T=256 with the plan rewritten (and
    pages rebound) before steps 16, 32 and 48, each layer fed by the previous layer's residual output.
    Every step of every layer is checked on the GPU's own input (teacher forcing): routing on all 256
    tokens (ids, weights, counts, offsets, sorted order), the residual bit-exactly, and outputs on 2
    seeded tokens (8 at the steps on both sides of a rewrite)."""
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
    around = {0, 15, 16, 31, 32, 47, 48, 63}
    route = route_buffers(T, cfg.E, cfg.k, dev)
    y = torch.empty((T, cfg.d), dtype=torch.float32, device=dev)
    worst = 0.0
    for s in range(cfg.steps):
        if s > 0 and s % cfg.rewrite_every == 0:
            _rewrite_all(cfg, layers, s)
        x = to_dev_f16(synth.tokens(cfg, T, step=s), dev)
        for l, L in enumerate(layers):
            x_next = torch.empty_like(x)
            L["lay"].forward(x, L["wd"], None, y=y, x_next=x_next, route=route)
            torch.cuda.synchronize()
            xh = f16_host(x)
            sub = sample_tokens(T, 8 if s in around else 2, seed=100 * s + l)
            ref = L["orc"].forward(xh, L["wr"], None, subset=sub)
            check_routing(route, ref, T, cfg.E, cfg.k)
            yh = y.cpu().numpy()
            err = rel_err_per_token(yh[sub], ref["y"][sub])
            worst = max(worst, float(err.max()))
            assert err.max() <= REL_TOL, (s, l, err.max())
            xn_ref = oracle.residual(xh, yh)   # O9 on the GPU's own y
            assert np.array_equal(f16_host(x_next).view(np.uint16), xn_ref.view(np.uint16)), (s, l)
            x = x_next
        if s % 8 == 7:
            _say(f"qwen_stack24_t256 3-layer slice: steps 0..{s} checked, worst rel err {worst:.3e}")
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
    """All 24 layers of the stack at T=256 over all 64 decode steps, with the plan rewritten (and pages
    rebound) before steps 16, 32 and 48, in the configuration `bench.py` times: each layer takes its own
    seeded input per step and writes its residual. Every (layer, step) runs on the GPU and its routing
    is checked on every token (ids, weights, counts, offsets, sorted order). Outputs are checked on one
    seeded token in three layers per step, rotating so that each layer is output-checked twice in every
    plan epoch, and the residual of those layers bit-exactly."""
    torch, dev = torch_dev
    from any_precision_bit_amd import route_buffers

    from concurrent.futures import ThreadPoolExecutor

    cfg = synth.CONFIGS["qwen_stack24_t256"]
    T, n_layers = cfg.T, cfg.layers

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
    for l in range(n_layers):
        bits = synth.initial_bits(cfg, layer=l)
        blocks = stack_blocks(bits, l)
        pages = device_pages(blocks, bits, dev, all_luts=True)
        lay = gpu_layer(cfg, bits, pages, max_tokens=T)
        wr, _ = synth.router(cfg, layer=l)
        layers.append(dict(bits=bits, pages=pages, lay=lay, wr=wr, wd=to_dev_f16(wr, dev),
                           orc=oracle.OracleLayer.from_config(cfg, bits, blocks)))
    _say(f"stack: {n_layers} layers ready")
    route = route_buffers(T, cfg.E, cfg.k, dev)
    y = torch.empty((T, cfg.d), dtype=torch.float32, device=dev)
    x_next = torch.empty((T, cfg.d), dtype=torch.float16, device=dev)
    per_step = 3
    seen = set()
    worst = 0.0
    for s in range(cfg.steps):
        if s > 0 and s % cfg.rewrite_every == 0:
            _rewrite_all(cfg, layers, s)
        # layers (3s .. 3s + 2) mod 24: every layer twice per 16-step plan epoch
        out_layers = {(per_step * s + i) % n_layers for i in range(per_step)}
        for l, L in enumerate(layers):
            x = synth.tokens(cfg, T, step=s, layer=l)
            xd = to_dev_f16(x, dev)
            L["lay"].forward(xd, L["wd"], None, y=y, x_next=x_next, route=route)
            torch.cuda.synchronize()
            outputs = l in out_layers
            sub = sample_tokens(T, 1, seed=1000 * s + l) if outputs else np.zeros(0, dtype=np.int32)
            ref = L["orc"].forward(x, L["wr"], None, subset=sub)
            check_routing(route, ref, T, cfg.E, cfg.k)
            if outputs:
                yh = y.cpu().numpy()
                err = rel_err_per_token(yh[sub], ref["y"][sub])
                worst = max(worst, float(err.max()))
                assert err.max() <= REL_TOL, (s, l, err.max())
                xn_ref = oracle.residual(x, yh)   # O9 on the GPU's own y
                assert np.array_equal(f16_host(x_next).view(np.uint16), xn_ref.view(np.uint16)), (s, l)
                seen.add((s // cfg.rewrite_every, l))
        if s % 4 == 3:
            _say(f"stack steps 0..{s}: routing exact on all {n_layers} layers, worst rel err {worst:.3e}")
    n_epochs = (cfg.steps + cfg.rewrite_every - 1) // cfg.rewrite_every
    assert seen == {(ep, l) for ep in range(n_epochs) for l in range(n_layers)}
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
    assert sorted(set(int(v) for v in bits.reshape(-1))) == list(range(1, 9)), bits
    blocks = synth.make_layer_blocks(cfg, bits, all_luts=False)
    x, wr, bias = layer_inputs(cfg)
    run_parity(torch_dev, cfg, bits, blocks, x, wr, bias, np.arange(cfg.T, dtype=np.int32))


TWO_GROUPS = synth.MoEConfig("gtwo", 93, d=256, E=4, F=384, k=2, T=32, Fs=512,
                             bits_rule="uniform", bits_values=(3, 4, 5, 6, 8))


def test_two_token_groups_one_kernel(torch_dev):
    """T = 32: experts with 17..32 tokens (and the 32-token shared expert) run as two 16-token
    groups in the one-tile kernel (the default at this T k / E) and as one 32-token group in the
    two-tile kernel (the two path); no 64-token launch."""
    cfg = TWO_GROUPS
    bits = synth.initial_bits(cfg)
    blocks = synth.make_layer_blocks(cfg, bits)
    x, wr, bias = layer_inputs(cfg)
    lay, ref = None, None
    for path in ["auto", "two"]:
        lay, _, ref = run_parity(torch_dev, cfg, bits, blocks, x, wr, bias, np.arange(cfg.T, dtype=np.int32),
                                 layer=lay, path=path, ref=ref)
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


@pytest.mark.parametrize("T", [16, 48])
def test_router_near_ties(torch_dev, T):
    """Experts whose logits differ by one fp16 ulp of a single weight (times that column's x), and
    an exact tie, at the top of every token; the oracle decides. At T = 16 the router computes
    every logit exactly; at T = 48 its fp32 pass cannot order these experts, so the selection rests
    on the exact logits of its candidates."""
    cfg = synth.CONFIGS["tiny_d256"].with_tokens(T)
    bits = synth.initial_bits(cfg)
    blocks = _blocks(cfg, bits)
    x, wr, _ = layer_inputs(cfg)
    x = np.abs(x).astype(np.float16)
    wr = wr.copy()
    wr[1] = np.float16(0.02)
    wr[2] = wr[1]
    wr[2, 17] = np.nextafter(wr[1, 17], np.float16(1))      # one ulp up: expert 2 just ahead of 1
    wr[3] = wr[1]
    wr[3, 200] = np.nextafter(wr[1, 200], np.float16(0))    # one ulp down: expert 3 just behind 1
    wr[4] = wr[1]                                           # exact tie with 1: the lower index wins
    lay, y, ref = run_parity(torch_dev, cfg, bits, blocks, x, wr, None, np.arange(T, dtype=np.int32))
    assert (ref["ids"] == np.array([2, 1])).all()           # (the construction: checked on the oracle)


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


@pytest.mark.parametrize("T", [4, 48])
def test_router_range_flag(torch_dev, T):
    """Outside the exact router's range (sum |x w| >= 2^15) or with a non-finite input the device
    status word raises PW_STATUS_ROUTER_RANGE; reading it clears it (T = 4: every logit exact in
    the first pass; T = 48: fp32 bounds first)."""
    torch, dev = torch_dev
    cfg = synth.CONFIGS["tiny_d256"].with_tokens(T)
    bits = synth.initial_bits(cfg)
    blocks = _blocks(cfg, bits)
    lay = gpu_layer(cfg, bits, device_pages(blocks, bits, dev))
    x, wr, _ = layer_inputs(cfg)
    for bad in ("huge", "inf"):
        xb = x.copy()
        if bad == "huge":
            xb[1, :] = 60000.0     # sum |x w| ~ 60000 * 256 * 0.016 >> 2^15
        else:
            xb[2, 7] = np.inf
        _say(f"router range flag: {bad}")
        lay.forward(to_dev_f16(xb, dev), to_dev_f16(wr, dev), None)
        torch.cuda.synchronize()
        assert lay.status() == 1, bad
        assert lay.status() == 0       # cleared by the read


@pytest.mark.parametrize("T", [16, 48])
def test_router_full_fp16_range(torch_dev, T):
    """Exact routing for large but in-range inputs. Tokens 0..7 carry 16 columns with |x| in
    [128, 4096], the other tokens two columns with |x| in [128, 512]; router weights |w| in
    [128, 512] on 4 other columns of every third expert; sum |x w| stays far below 2^15. Routing
    (ids, weights, counts, offsets, sorted order) must match the oracle's __int128 logits on every
    token with no range flag (T = 16: every logit exact in the first pass; T = 48: fp32 bounds,
    then exact candidates). Outputs are compared on tokens 8 on: on tokens 0..7 the SwiGLU output
    exceeds fp16's range, and the layer rounds it to fp16 as the down projection's MFMA operand."""
    torch, dev = torch_dev
    from any_precision_bit_amd import route_buffers

    cfg = synth.CONFIGS["tiny_d256"].with_tokens(T)
    bits = synth.initial_bits(cfg)
    blocks = _blocks(cfg, bits)
    x, wr, _ = layer_inputs(cfg)
    g = np.random.default_rng(77)
    x = x.copy()
    wr = wr.copy()
    sign = lambda shape: g.choice([-1.0, 1.0], size=shape)
    x[:8, :16] = (sign((8, 16)) * g.uniform(128, 4096, size=(8, 16))).astype(np.float16)
    x[8:, 20:22] = (sign((T - 8, 2)) * g.uniform(128, 512, size=(T - 8, 2))).astype(np.float16)
    wr[::3, 16:20] = (sign(wr[::3, 16:20].shape) * g.uniform(128, 512, size=wr[::3, 16:20].shape)).astype(np.float16)
    assert float((np.abs(x.astype(np.float64)) @ np.abs(wr.astype(np.float64)).T).max()) < 2 ** 15
    assert np.abs(x[:8].astype(np.float64)).max() > 2048
    _say("router full fp16 range")
    pages = device_pages(blocks, bits, dev)
    lay = gpu_layer(cfg, bits, pages, max_tokens=T)
    route = route_buffers(T, cfg.E, cfg.k, dev)
    y = lay.forward(to_dev_f16(x, dev), to_dev_f16(wr, dev), None, route=route)
    torch.cuda.synchronize()
    assert lay.status() == 0
    sub = np.arange(8, T, dtype=np.int32)
    ref = oracle.OracleLayer.from_config(cfg, bits, blocks).forward(x, wr, None, subset=sub)
    assert ref["status"] == 0
    check_routing(route, ref, T, cfg.E, cfg.k)
    err = rel_err_per_token(y.cpu().numpy()[sub], ref["y"][sub])
    _say(f"router full fp16 range: routing exact on {T} tokens, max rel err {err.max():.3e} on tokens 8..")
    assert err.max() <= REL_TOL


LIMITS = synth.MoEConfig("limits", 94, d=8192, E=256, F=128, k=16, T=40, Fs=256,
                         bits_rule="uniform", bits_values=(3, 4, 5, 6, 8))


def test_abi_limits(torch_dev):
    """The header's limits in one layer: d_model 8192, 256 routed experts, top-16, max_tokens 65536
    (the workspace at its largest T), plus a shared expert: the router's single-pass offsets scan at
    E = 256, gate/up items over 8 K-chunks, and the four-tile kernel for the shared expert
    (T = 40 > 32). All 40 tokens checked."""
    cfg = LIMITS
    bits = synth.initial_bits(cfg)
    _say("ABI limits: generating pages")
    blocks = _blocks(cfg, bits, workers=16)
    x, wr, bias = layer_inputs(cfg)
    _say("ABI limits: d8192 E256 k16 max_tokens 65536")
    run_parity(torch_dev, cfg, bits, blocks, x, wr, bias, np.arange(cfg.T, dtype=np.int32), max_tokens=65536)


def test_planner_plan_forward(torch_dev):
    """The planner's plan on the GPU: a qwen_d2048_t16 forward's routed counts feed pw_plan_greedy
    (seeded synthetic sensitivities) with a target of 25 % of the resident bytes; the emitted plan
    is set, its pages bound, and the next forward checked against the oracle on every token. Then
    an upgrade with half of the freed bytes as budget, checked the same way."""
    torch, dev = torch_dev
    from any_precision_bit_amd import binding as B
    from any_precision_bit_amd import route_buffers
    from oracle import planner as OP

    cfg = synth.CONFIGS["qwen_d2048_t16"]
    bits = synth.initial_bits(cfg)
    jobs = [(e, lin) for e in range(cfg.n_experts_total) for lin in synth.LINEARS]
    blocks = {(e, lin): synth.make_block(cfg, e, lin, n_planes=8, lut_bits=tuple(range(3, 9))) for e, lin in jobs}
    pages = device_pages(blocks, bits, dev, all_luts=True)
    lay = gpu_layer(cfg, bits, pages, max_tokens=cfg.T)
    x, wr, bias = layer_inputs(cfg)
    route = route_buffers(cfg.T, cfg.E, cfg.k, dev)
    lay.forward(to_dev_f16(x, dev), to_dev_f16(wr, dev), None, route=route)
    torch.cuda.synchronize()
    counts = route["expert_count"].cpu().numpy()
    sens = np.random.default_rng(11).random(cfg.n_blocks).astype(np.float32)
    shapes = OP.block_shapes(cfg.d, cfg.E, cfg.F, cfg.Fs)
    resident = sum(OP.block_bytes(R, K, int(b)) for (R, K), b in zip(shapes, bits.reshape(-1)))
    cur = bits
    for step, tgt in (("downgrade", 0.25 * resident), ("upgrade", None)):
        if tgt is None:
            tgt = -0.5 * freed
        new, moved, dmg, n = B.pw_plan_greedy(lay.handle, sens, counts, cfg.T, tgt)
        ref = OP.plan(shapes, cur.reshape(-1), sens, OP.masses(cfg.E, True, counts, cfg.T), tgt)
        assert np.array_equal(new, ref[0]) and n > 0
        if step == "downgrade":
            freed = moved
            assert moved >= tgt
        new = new.reshape(cur.shape)
        lay.plan_set(new)
        bind_all(lay, new, pages)
        _say(f"planner {step}: {n} actions, {moved / 1e6:.1f} MB, mean bits {cur.mean():.2f} -> {new.mean():.2f}")
        run_parity(torch_dev, cfg, new, blocks, x, wr, bias, np.arange(cfg.T, dtype=np.int32), layer=lay,
                   pages=pages)
        cur = new


def test_async_page_movement(torch_dev):
    """Asynchronous page movement on qwen_d2048_t16: pages of a planner downgrade (25 % of the
    resident bytes) and then of an upgrade back are copied on a side stream while forwards keep
    running on the compute stream with the old plan; after each commit the device holds exactly the
    pages the plan reads, and the next forward matches the oracle on every token."""
    torch, dev = torch_dev
    from any_precision_bit_amd import PagedMoELayer, route_buffers
    from any_precision_bit_amd import binding as B
    from any_precision_bit_amd.paging import PageManager
    from oracle import planner as OP

    cfg = synth.CONFIGS["qwen_d2048_t16"]
    bits = synth.initial_bits(cfg)
    jobs = [(e, lin) for e in range(cfg.n_experts_total) for lin in synth.LINEARS]
    blocks = {(e, lin): synth.make_block(cfg, e, lin, n_planes=8, lut_bits=tuple(range(3, 9))) for e, lin in jobs}
    lay = PagedMoELayer(cfg.d, cfg.E, cfg.F, cfg.k, cfg.Fs, cfg.T)
    pm = PageManager(lay, {k: (b.planes, b.luts) for k, b in blocks.items()}, bits, dev)
    shapes = OP.block_shapes(cfg.d, cfg.E, cfg.F, cfg.Fs)
    plan_bytes = lambda bb: sum(OP.block_bytes(R, K, int(b)) for (R, K), b in zip(shapes, np.asarray(bb).reshape(-1)))
    assert pm.resident_bytes() == plan_bytes(bits)
    x, wr, bias = layer_inputs(cfg)
    xd, wd = to_dev_f16(x, dev), to_dev_f16(wr, dev)
    route = route_buffers(cfg.T, cfg.E, cfg.k, dev)
    lay.forward(xd, wd, None, route=route)
    torch.cuda.synchronize()
    counts = route["expert_count"].cpu().numpy()
    sens = np.random.default_rng(11).random(cfg.n_blocks).astype(np.float32)
    cur = bits
    for step in ("downgrade", "upgrade"):
        tgt = 0.25 * plan_bytes(cur) if step == "downgrade" else -0.25 * plan_bytes(bits)
        new, moved, _, n = B.pw_plan_greedy(lay.handle, sens, counts, cfg.T, tgt, max_bits=np.full(cfg.n_blocks, 8, np.uint8))
        staged = pm.stage(new)
        y = torch.empty((cfg.T, cfg.d), dtype=torch.float32, device=dev)
        for _ in range(8):                      # forwards with the old plan while the copies run
            lay.forward(xd, wd, None, y=y)
        pm.commit(staged)
        _say(f"paging {step}: {n} actions, {staged.nbytes / 1e6:.1f} MB copied in {staged.copy_ms():.2f} ms")
        torch.cuda.synchronize()
        cur = new.reshape(cur.shape)
        assert pm.resident_bytes() == plan_bytes(cur)
        run_parity(torch_dev, cfg, cur, blocks, x, wr, bias, np.arange(cfg.T, dtype=np.int32), layer=lay,
                   pages=pm.dev)


def test_kv_pressure_plans(torch_dev):
    """KV-cache pressure driving the planner through the page manager on qwen_d2048_t16: KV bytes
    rising past the budget force downgrades (weights + KV back within the budget), falling KV allows
    upgrades back toward the starting plan; after every committed change the layer matches the
    oracle on every token."""
    torch, dev = torch_dev
    from any_precision_bit_amd import PagedMoELayer, route_buffers
    from any_precision_bit_amd.kvpressure import KVPressurePlanner
    from any_precision_bit_amd.paging import PageManager

    cfg = synth.CONFIGS["qwen_d2048_t16"]
    bits = synth.initial_bits(cfg)
    jobs = [(e, lin) for e in range(cfg.n_experts_total) for lin in synth.LINEARS]
    blocks = {(e, lin): synth.make_block(cfg, e, lin, n_planes=8, lut_bits=tuple(range(3, 9))) for e, lin in jobs}
    lay = PagedMoELayer(cfg.d, cfg.E, cfg.F, cfg.k, cfg.Fs, cfg.T)
    pm = PageManager(lay, {k: (b.planes, b.luts) for k, b in blocks.items()}, bits, dev)
    x, wr, bias = layer_inputs(cfg)
    route = route_buffers(cfg.T, cfg.E, cfg.k, dev)
    lay.forward(to_dev_f16(x, dev), to_dev_f16(wr, dev), None, route=route)
    torch.cuda.synchronize()
    counts = route["expert_count"].cpu().numpy()
    w0 = float(pm.resident_bytes())
    budget = w0 + 100e6
    ctl = KVPressurePlanner(lay, budget, np.random.default_rng(4).random(cfg.n_blocks).astype(np.float32),
                            hysteresis_bytes=5e6, resident_bytes=pm.resident_bytes, max_bits=bits.reshape(-1))
    seen = set()
    for kv in (50e6, 160e6, 220e6, 120e6, 20e6):
        d = ctl.decide(kv, counts, cfg.T)
        if d is None:
            continue
        staged = pm.stage(d[0].reshape(bits.shape))
        pm.commit(staged)
        torch.cuda.synchronize()
        seen.add("down" if d[1] > 0 else "up")
        if d[1] > 0:
            assert pm.resident_bytes() + kv <= budget
        _say(f"kv {kv / 1e6:.0f} MB: {d[3]} actions, weights {pm.resident_bytes() / 1e6:.1f} MB")
        run_parity(torch_dev, cfg, pm.bits, blocks, x, wr, bias, np.arange(cfg.T, dtype=np.int32), layer=lay,
                   pages=pm.dev)
    assert seen == {"down", "up"}


def _row_block_layer(torch_dev, cfg, rb, bits, lut_tiled=False, max_tokens=None):
    """A layer of rb-row linear-blocks bound block by block to its rows of whole-linear pages."""
    torch, dev = torch_dev
    from any_precision_bit_amd import PagedMoELayer

    jobs = [(e, lin) for e in range(cfg.n_experts_total) for lin in synth.LINEARS]
    blocks = {(e, lin): synth.make_block(cfg, e, lin, n_planes=8, lut_bits=(3, 4, 5, 6, 8)) for e, lin in jobs}
    pages = device_pages(blocks, np.full((cfg.n_experts_total, 3), 8), dev, all_luts=True, lut_tiled=lut_tiled)
    lay = PagedMoELayer(cfg.d, cfg.E, cfg.F, cfg.k, cfg.Fs, max_tokens or cfg.T, lut_tiled=lut_tiled,
                        rows_per_block=rb)
    lay.plan_set(bits)
    i = 0
    for e, lin in jobs:
        planes, luts = pages[(e, lin)]
        R = planes.shape[1]
        for j in range(R // rb):
            b = int(bits[i])
            i += 1
            rows = slice(j * rb, (j + 1) * rb)
            lay.bind_rows(e, lin, j, [planes[p][rows] for p in range(b)], luts[b][rows], b)
    assert i == bits.shape[0]
    return lay, blocks, pages


@pytest.mark.parametrize("lut_tiled", [False, True])
def test_row_blocks_decode(torch_dev, lut_tiled):
    """qwen_d2048_t16 with linear-blocks of 128 rows, each at its own bitwidth (per-block pages bound
    one by one), against the oracle on every token."""
    cfg = synth.CONFIGS["qwen_d2048_t16"]
    bits = synth.rowblock_bits(cfg, 128)
    _say(f"row-blocks of 128 rows, lut_tiled={lut_tiled}: {bits.shape[0]} blocks")
    lay, blocks, pages = _row_block_layer(torch_dev, cfg, 128, bits, lut_tiled)
    x, wr, bias = layer_inputs(cfg)
    run_parity(torch_dev, cfg, bits, blocks, x, wr, bias, np.arange(cfg.T, dtype=np.int32), layer=lay,
               pages=pages)


def test_prefill_t1024_row_blocks(torch_dev):
    """The T = 1024 prefill workload (qwen_rows128_t1024): routing on all 1024 tokens, outputs on 48
    seeded tokens, linear-blocks of 128 rows."""
    cfg = synth.CONFIGS["qwen_rows128_t1024"]
    rb = synth.ROWS_PER_BLOCK[cfg.name]
    bits = synth.rowblock_bits(cfg, rb)
    lay, blocks, pages = _row_block_layer(torch_dev, cfg, rb, bits)
    x, wr, bias = layer_inputs(cfg)
    _say("qwen_rows128_t1024")
    run_parity(torch_dev, cfg, bits, blocks, x, wr, bias, sample_tokens(cfg.T, 48, seed=9), layer=lay, pages=pages)
