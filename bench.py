"""Benchmark of the fused mixed-precision MoE layer on one MI355X.

Workload: the Qwen1.5-MoE-A2.7B-shaped decode layer (d 2048, 60 routed experts
of ffn 1408, top-4, a shared expert of ffn 5632, T = 16 tokens, bitwidths drawn
uniformly from {3,4,5,6,8} per (expert, linear)), synthetic seeded data.
A step is one full forward (routing, gate/up + SwiGLU, down + weighted
accumulation) of one layer over the batch. Steps rotate over byte-identical
clones of the pages at distinct addresses so that the working set exceeds the
on-chip caches and the weights stream from HBM.

Prints one JSON line on stdout; diagnostics go to stderr. With --sweep it
instead times one layer forward of every workload shape (tiny_d256, qwen_d2048_t16,
mixtral_d4096 at T=1 and T=64, fine_e128_t128, one layer of qwen_stack24_t256) and
prints a markdown table; with --stack it times the whole 24-layer qwen_stack24_t256
workload over its 64 steps and plan rewrites.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0   # dense fp16 MFMA, MI355X


def log(*a):
    print(*a, file=sys.stderr, flush=True)


KERNEL_SRC = os.path.join(ROOT, "any_precision_bit_amd", "csrc", "pw_kernels.hip")
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "expert_kernel_qwen_d2048_t16_traffic.md")
SQ_PROFILE = os.path.join(ROOT, "profiles", "expert_kernel_qwen_d2048_t16_sq_counters.md")


def kernel_code_digest():
    """sha256 of the kernel source with // comments and blank lines removed."""
    import hashlib
    code = [ln.split("//", 1)[0].rstrip() for ln in open(KERNEL_SRC)]
    return hashlib.sha256("\n".join(c for c in code if c).encode()).hexdigest()


def profile_values(path, keys):
    """The "key: value" lines of a committed rocprofv3 counter summary, as floats, or None when
    the file is missing or the kernel code has changed since those counters were taken."""
    try:
        text = open(path).read()
    except OSError:
        return None
    fields = dict(line.split(":", 1) for line in text.splitlines() if line.startswith(tuple(k + ":" for k in keys)))
    if fields.get("kernel_code_sha256", "").strip() != kernel_code_digest():
        return None
    return {k: float(fields[k]) for k in keys if k != "kernel_code_sha256" and k in fields}


def measured_traffic():
    """HBM bytes per expert-kernel launch from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE runs, scaled by a 1 GiB copy's readings), or None
    when the kernel code has changed since those counters were taken."""
    v = profile_values(TRAFFIC_PROFILE, ["kernel_code_sha256", "traffic_bytes_per_launch"])
    return None if not v else v["traffic_bytes_per_launch"]


def measured_alu():
    """The expert kernel's VALU and LDS lane-instructions per dequantised weight and its
    VALU-issue time from the committed SQ counter summary (None if the kernel changed)."""
    return profile_values(SQ_PROFILE, ["kernel_code_sha256", "valu_lane_instr_per_weight",
                                       "lds_lane_instr_per_weight", "valu_bound_us"])


# (label, workload, tokens or None for the workload's own, rotation clones); tiny_d256 is cache-resident
SWEEP = [("tiny_d256", "tiny_d256", None, 1), ("qwen_d2048_t16", "qwen_d2048_t16", None, 8),
         ("mixtral_d4096 T=1", "mixtral_d4096", 1, 8), ("mixtral_d4096 T=64", "mixtral_d4096", 64, 4),
         ("fine_e128_t128", "fine_e128_t128", None, 4),
         ("qwen_stack24_t256 layer 0, first plan", "qwen_stack24_t256", None, 4)]


def sweep(args, torch, synth, PagedMoELayer, lut_page, dev):
    """Per-call times of one layer forward (routing + experts) for every workload shape (or the one
    labelled --only): warm-up calls, then timed calls each bracketed by HIP events on the launch
    stream, rotating over byte-identical page clones. Useful MFMA work is the dense-equivalent
    2 * tokens * rows * K of every (expert, linear) over the tokens routed to it (and all T for the
    shared expert), from the routed counts of one more forward."""
    from any_precision_bit_amd import route_buffers
    def f16(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.float16).view(np.int16).copy()).to(dev).view(
            torch.float16)

    rows = []
    stream = torch.cuda.current_stream(dev)
    for label, key, T, M in SWEEP:
        if args.only and label != args.only:
            continue
        cfg = synth.CONFIGS[key]
        if T is not None:
            cfg = cfg.with_tokens(T)
        t0 = time.time()
        x = f16(synth.tokens(cfg))
        wr_h, bias_h = synth.router(cfg)
        wr = f16(wr_h)
        bias = f16(bias_h) if bias_h is not None else None
        counts = None
        if cfg.bits_rule == "frequency":
            # the plan follows the batch's routing counts; ranked here in fp64 (input set-up only)
            lg = x.double() @ wr.double().T + (bias.double() if bias is not None else 0.0)
            ids = torch.topk(lg, cfg.k, dim=1).indices
            counts = torch.bincount(ids.reshape(-1), minlength=cfg.E).cpu().numpy()
        bits = synth.initial_bits(cfg, counts=counts)
        blocks = synth.make_layer_blocks(cfg, bits)
        base = {}
        for (e, lin), blk in blocks.items():
            b = int(bits[e, lin])
            base[(e, lin)] = (torch.from_numpy(np.ascontiguousarray(blk.planes[:b])).to(dev),
                              f16(lut_page(blk.luts[b]) if args.lut_tiled else blk.luts[b]), b)
        del blocks
        lays = []
        for c in range(M):
            pages = base if c == 0 else {kk: (p.clone(), l.clone(), b) for kk, (p, l, b) in base.items()}
            lay = PagedMoELayer(cfg.d, cfg.E, cfg.F, cfg.k, cfg.Fs, cfg.T, lut_tiled=args.lut_tiled)
            lay.plan_set(bits)
            for (e, lin), (p, l, b) in pages.items():
                lay.bind(e, lin, [p[i] for i in range(b)], l, b)
            lays.append((lay, pages, torch.empty((cfg.T, cfg.d), device=dev)))
        torch.cuda.synchronize()
        log(f"{label}: pages ready in {time.time() - t0:.1f}s")
        for i in range(args.warmup):
            lay, _, y = lays[i % M]
            lay.forward(x, wr, bias, y=y, stream=stream)
        n = max(args.steps // 4, 50)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i in range(n):
            lay, _, y = lays[i % M]
            evs[i][0].record(stream)
            lay.forward(x, wr, bias, y=y, stream=stream)
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
        nb = lays[0][0].last_bytes(stream)
        layer_bytes = nb[0] + nb[1] + nb[2]
        route = route_buffers(cfg.T, cfg.E, cfg.k, dev)
        lays[0][0].forward(x, wr, bias, y=lays[0][2], route=route, stream=stream)
        torch.cuda.synchronize()
        check_status([lay for lay, _, _ in lays], label)
        counts = route["expert_count"].cpu().numpy().astype(np.float64)
        flops = 2.0 * 3 * cfg.F * cfg.d * counts.sum() + (2.0 * 3 * cfg.Fs * cfg.d * cfg.T if cfg.Fs else 0.0)
        med = float(np.median(us))
        rows.append((label, cfg.T, M, layer_bytes / 1e6, med, float(np.percentile(us, 10)),
                     float(np.percentile(us, 90)), layer_bytes / (med * 1e-6) / 1e9, cfg.T / (med * 1e-6),
                     flops / (med * 1e-6) / 1e12))
        log(f"{label}: median {med:.1f} us")
        for lay, _, _ in lays:
            lay.close()
        del lays, base
        torch.cuda.empty_cache()
    print("| workload | T | clones | algorithmic MB | median us | p10 us | p90 us | GB/s | HBM % | tokens/s | "
          "useful MFMA TFLOP/s | % of fp16 MFMA peak |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|")
    for label, T, M, mb, med, p10, p90, gbs, tps, tf in rows:
        print(f"| {label} | {T} | {M} | {mb:.1f} | {med:.1f} | {p10:.1f} | {p90:.1f} | {gbs:.0f} | "
              f"{100 * gbs / HBM_PEAK_GBS:.1f} | {tps:,.0f} | {tf:.1f} | {100 * tf / MFMA_F16_PEAK_TFLOPS:.2f} |",
              flush=True)


def layer_stack(args, torch, synth, PagedMoELayer, lut_page, dev, print_table=True):
    """The whole qwen_stack24_t256 workload: 24 layers, each with its own seeded weights, router and pages, over 64
    decode steps of 256 tokens. Before steps 16, 32 and 48 every layer's plan is rewritten (45 seeded
    blocks lose two bits, not below 3) and the changed blocks are rebound to their lower planes and
    LUTs. Every layer also writes its residual x + y. With these synthetic weights a free-running
    residual chain grows past the exact router's input range within five layers, so each layer takes
    its own seeded N(0, 1) input per step (independent inputs per step and layer). One HIP event pair
    on the launch stream brackets each step, rewrite calls included. Algorithmic bytes per layer are
    read back after the last step of each plan epoch."""
    from concurrent.futures import ThreadPoolExecutor

    cfg = synth.CONFIGS["qwen_stack24_t256"]
    T, L, every = cfg.T, cfg.layers, cfg.rewrite_every
    stream = torch.cuda.current_stream(dev)

    def f16(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.float16).view(np.int16).copy()).to(dev).view(
            torch.float16)

    def reachable(b):   # bitwidths a block at b can reach under the rewrites
        out = {b}
        for _ in range(cfg.steps // every):
            b = max(3, b - 2)
            out.add(b)
        return tuple(sorted(out))

    t0 = time.time()
    layers = []
    for l in range(L):
        bits = synth.initial_bits(cfg, layer=l)
        jobs = [(e, lin) for e in range(cfg.n_experts_total) for lin in synth.LINEARS]

        def one(job, l=l, bits=bits):
            e, lin = job
            b = int(bits[e, lin])
            return synth.make_block(cfg, e, lin, layer=l, n_planes=b, lut_bits=reachable(b))

        with ThreadPoolExecutor(max_workers=16) as ex:
            blocks = list(ex.map(one, jobs))
        pages = {}
        for blk in blocks:
            pages[(blk.e, blk.lin)] = (torch.from_numpy(np.ascontiguousarray(blk.planes)).to(dev),
                                       {b: f16(lut_page(v) if args.lut_tiled else v) for b, v in blk.luts.items()})
        del blocks
        lay = PagedMoELayer(cfg.d, cfg.E, cfg.F, cfg.k, cfg.Fs, T, lut_tiled=args.lut_tiled)
        lay.plan_set(bits)
        for (e, lin), (p, luts) in pages.items():
            b = int(bits[e, lin])
            lay.bind(e, lin, [p[i] for i in range(b)], luts[b], b)
        wr_h, _ = synth.router(cfg, layer=l)
        layers.append(dict(bits=bits, pages=pages, lay=lay, wr=f16(wr_h)))
        log(f"stack layer {l}: pages ready ({time.time() - t0:.0f}s)")
    xs = [[f16(synth.tokens(cfg, T, step=s, layer=l)) for l in range(L)] for s in range(cfg.steps)]
    log(f"stack inputs ready ({time.time() - t0:.0f}s)")
    y = torch.empty((T, cfg.d), dtype=torch.float32, device=dev)
    x_next = torch.empty((T, cfg.d), dtype=torch.float16, device=dev)

    def step(s):
        if s > 0 and s % every == 0:
            for l, Ly in enumerate(layers):
                new, changed = synth.rewrite_plan(cfg, Ly["bits"], layer=l, epoch=s // every)
                Ly["bits"] = new
                Ly["lay"].plan_set(new)
                for blk in changed:
                    e, lin = divmod(int(blk), 3)
                    p, luts = Ly["pages"][(e, lin)]
                    b = int(new[e, lin])
                    Ly["lay"].bind(e, lin, [p[i] for i in range(b)], luts[b], b)
        for l, Ly in enumerate(layers):
            Ly["lay"].forward(xs[s][l], Ly["wr"], None, y=y, x_next=x_next, stream=stream)

    # warm-up: the first steps of the first epoch, on their own copy of the plan state
    for s in range(min(args.warmup, 2)):
        step(s)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(cfg.steps)]
    epoch_bytes = []
    for s in range(cfg.steps):
        evs[s][0].record(stream)
        step(s)
        evs[s][1].record(stream)
        if (s + 1) % every == 0 or s + 1 == cfg.steps:
            nb = [Ly["lay"].last_bytes(stream) for Ly in layers]
            epoch_bytes.append((float(np.mean([sum(b[:3]) for b in nb])),
                                float(np.mean([Ly["bits"].mean() for Ly in layers]))))
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    check_status([Ly["lay"] for Ly in layers], "qwen_stack24_t256")
    n_ep = (cfg.steps + every - 1) // every
    epochs = []
    for ep in range(n_ep):
        sl = ms[ep * every:(ep + 1) * every]
        mb, bits_mean = epoch_bytes[ep]
        per_layer_us = float(np.median(sl)) * 1e3 / L
        gbs = mb / (per_layer_us * 1e-6) / 1e9
        epochs.append({"steps": f"{ep * every}..{min(cfg.steps, (ep + 1) * every) - 1}", "mean_bits": round(bits_mean, 3),
                       "layer_bytes": mb, "step_ms_median": round(float(np.median(sl)), 4),
                       "step_ms_p10": round(float(np.percentile(sl, 10)), 4),
                       "step_ms_p90": round(float(np.percentile(sl, 90)), 4),
                       "layer_us_median": round(per_layer_us, 2), "layer_GBps": round(gbs, 1),
                       "layer_hbm_frac": round(gbs / HBM_PEAK_GBS, 4)})
    summary = {"workload": synth.WORKLOAD_TEXT["qwen_stack24_t256"], "tokens_per_step": T, "layers": L,
               "steps": cfg.steps, "value": round(T * cfg.steps / (ms.sum() * 1e-3), 1), "unit": "tokens/s",
               "step_ms_median": round(float(np.median(ms)), 4), "step_ms_p10": round(float(np.percentile(ms, 10)), 4),
               "step_ms_p90": round(float(np.percentile(ms, 90)), 4), "epochs": epochs,
               "status_checked": True}
    if print_table:
        print("| plan epoch | steps | mean bits | algorithmic MB per layer | median step ms | p10 | p90 | per-layer us | "
              "GB/s | HBM % | stack tokens/s |")
        print("|---|---|---|---|---|---|---|---|---|---|---|")
        for ep, e in enumerate(epochs):
            print(f"| {ep} | {e['steps']} | {e['mean_bits']:.2f} | {e['layer_bytes'] / 1e6:.1f} | {e['step_ms_median']:.2f} | "
                  f"{e['step_ms_p10']:.2f} | {e['step_ms_p90']:.2f} | {e['layer_us_median']:.1f} | {e['layer_GBps']:.0f} | "
                  f"{100 * e['layer_hbm_frac']:.1f} | {T / (e['step_ms_median'] * 1e-3):,.0f} |")
        print(f"| all | 0..{cfg.steps - 1} | | | {summary['step_ms_median']:.2f} | {summary['step_ms_p10']:.2f} | "
              f"{summary['step_ms_p90']:.2f} | {summary['step_ms_median'] * 1e3 / L:.1f} | | | {summary['value']:,.0f} |",
              flush=True)
    for Ly in layers:
        Ly["lay"].close()
    del layers, xs
    torch.cuda.empty_cache()
    return summary


def paging_run(args, torch, synth, PagedMoELayer, dev, print_table=True):
    """Asynchronous page movement on the qwen_d2048_t16 layer: forwards run back to back on the compute
    stream, each bracketed by HIP events, first with no page movement, then while plan changes chosen
    by the planner (a downgrade freeing 25 % of the resident bytes, then an upgrade back, repeated)
    copy their pages host-to-device on a side stream; each change is committed as soon as its copies
    have landed. Also times the planner itself on the host."""
    from any_precision_bit_amd import binding as B
    from any_precision_bit_amd import route_buffers
    from any_precision_bit_amd.paging import PageManager

    def f16(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.float16).view(np.int16).copy()).to(dev).view(
            torch.float16)

    cfg = synth.CONFIGS["qwen_d2048_t16"]
    t0 = time.time()
    bits = synth.initial_bits(cfg)
    jobs = [(e, lin) for e in range(cfg.n_experts_total) for lin in synth.LINEARS]
    blocks = {(e, lin): synth.make_block(cfg, e, lin, n_planes=8, lut_bits=tuple(range(3, 9))) for e, lin in jobs}
    lay = PagedMoELayer(cfg.d, cfg.E, cfg.F, cfg.k, cfg.Fs, cfg.T)
    pm = PageManager(lay, {k: (b.planes, b.luts) for k, b in blocks.items()}, bits, dev)
    del blocks
    x, wr = f16(synth.tokens(cfg)), f16(synth.router(cfg)[0])
    y = torch.empty((cfg.T, cfg.d), device=dev)
    stream = pm.compute
    route = route_buffers(cfg.T, cfg.E, cfg.k, dev)
    lay.forward(x, wr, None, y=y, route=route, stream=stream)
    torch.cuda.synchronize()
    counts = route["expert_count"].cpu().numpy()
    sens = np.random.default_rng(11).random(cfg.n_blocks).astype(np.float32)
    log(f"paging: layer ready ({time.time() - t0:.1f}s), {pm.resident_bytes() / 1e6:.1f} MB resident")

    # the planner on the host: one downgrade of 25 % of the resident bytes
    resident = pm.resident_bytes()
    reps = 200
    tt = time.perf_counter()
    for _ in range(reps):
        down, moved, dmg, n_act = B.pw_plan_greedy(lay.handle, sens, counts, cfg.T, 0.25 * resident)
    plan_us = (time.perf_counter() - tt) / reps * 1e6
    # for comparison: the same bytes freed one random bit at a time (the seeded rewrite's style),
    # scored with the planner's damage measure
    g = np.random.default_rng(5)
    cur = bits.reshape(-1).astype(int).copy()
    shape = lambda i: ((cfg.Fs if i // 3 == cfg.E else cfg.F, cfg.d) if i % 3 < 2 else
                       (cfg.d, cfg.Fs if i // 3 == cfg.E else cfg.F))
    nbytes = lambda R, K, b: R * K * b / 8.0 + R * float(1 << b) * 2.0
    mass = lambda i: 1.0 if i // 3 == cfg.E else counts[i // 3] / cfg.T
    freed_r, dmg_r = 0.0, 0.0
    while freed_r < 0.25 * resident:
        i = int(g.integers(0, len(cur)))
        if cur[i] <= 3:
            continue
        R, K = shape(i)
        freed_r += nbytes(R, K, cur[i]) - nbytes(R, K, cur[i] - 1)
        dmg_r += float(sens[i]) * mass(i) * (4.0 ** -(cur[i] - 1) - 4.0 ** -cur[i])
        cur[i] -= 1

    def run(n, changes):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        copied, copy_ms, overlapped, staged, plans, n_changes = 0, [], [], None, list(changes), 0
        since = 0
        for i in range(n):
            if staged is None and plans:
                staged = pm.stage(plans.pop(0))
                since = 0
            evs[i][0].record(stream)
            lay.forward(x, wr, None, y=y, stream=stream)
            evs[i][1].record(stream)
            since += 1
            if staged is not None and staged.ready():
                pm.commit(staged)
                copied += staged.nbytes
                copy_ms.append(staged.copy_ms())
                overlapped.append(since)
                n_changes += 1
                staged = None
        if staged is not None:
            pm.commit(staged)
        torch.cuda.synchronize()
        us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
        return us, copied, copy_ms, overlapped, n_changes

    n = max(args.steps, 200)
    for _ in range(args.warmup):
        lay.forward(x, wr, None, y=y, stream=stream)
    quiet, *_ = run(n, [])
    cycle = [down.reshape(bits.shape), bits] * 8
    moving, copied, copy_ms, overlapped, n_changes = run(n, cycle)
    check_status([lay], "paging")
    stat = lambda a: {"p50": round(float(np.percentile(a, 50)), 2), "p90": round(float(np.percentile(a, 90)), 2),
                      "p99": round(float(np.percentile(a, 99)), 2), "max": round(float(a.max()), 2)}
    out = {"workload": synth.WORKLOAD_TEXT["qwen_d2048_t16"], "forwards": n,
           "forward_us_quiet": stat(quiet), "forward_us_while_moving": stat(moving),
           "plan_changes_committed": n_changes, "copied_MB": round(copied / 1e6, 1),
           "copy_ms_mean": round(float(np.mean(copy_ms)), 3) if copy_ms else None,
           "copy_GBps": round(copied / 1e9 / (np.sum(copy_ms) * 1e-3), 1) if copy_ms else None,
           "forwards_overlapped_per_change": round(float(np.mean(overlapped)), 1) if overlapped else None,
           "planner": {"host_us": round(plan_us, 1), "blocks": cfg.n_blocks, "target_MB": round(0.25 * resident / 1e6, 1),
                       "freed_MB": round(moved / 1e6, 1), "actions": n_act, "damage": dmg,
                       "damage_random_same_bytes": dmg_r, "freed_random_MB": round(freed_r / 1e6, 1)},
           "status_checked": True}
    if print_table:
        print(json.dumps(out, indent=1))
    lay.close()
    del pm
    torch.cuda.empty_cache()
    return out


def kv_pressure_run(args, torch, synth, PagedMoELayer, dev, print_table=True):
    """KV-cache pressure driving the planner on the qwen_d2048_t16 layer: one forward per decode step of
    a seeded request trace (the forward's batch stays the workload's 16 tokens; the trace sets the
    layer's share of KV bytes, 16 KV heads x 128 x fp16 per token). The memory budget is the starting
    plan's page bytes plus the trace's median KV bytes; every 8 steps the byte target (resident pages
    + KV - budget) is passed to the planner, the plan's pages move on a side stream and are committed
    when they have landed. Reports weight bytes, plan changes, damage, the worst overshoot of the
    budget, and forward latency."""
    from any_precision_bit_amd import route_buffers
    from any_precision_bit_amd.kvpressure import KVPressurePlanner
    from any_precision_bit_amd.paging import PageManager
    from synth.kvtrace import kv_bytes_per_token, request_trace

    def f16(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.float16).view(np.int16).copy()).to(dev).view(
            torch.float16)

    cfg = synth.CONFIGS["qwen_d2048_t16"]
    bits = synth.initial_bits(cfg)
    jobs = [(e, lin) for e in range(cfg.n_experts_total) for lin in synth.LINEARS]
    blocks = {(e, lin): synth.make_block(cfg, e, lin, n_planes=8, lut_bits=tuple(range(3, 9))) for e, lin in jobs}
    lay = PagedMoELayer(cfg.d, cfg.E, cfg.F, cfg.k, cfg.Fs, cfg.T)
    pm = PageManager(lay, {k: (b.planes, b.luts) for k, b in blocks.items()}, bits, dev)
    del blocks
    x, wr = f16(synth.tokens(cfg)), f16(synth.router(cfg)[0])
    y = torch.empty((cfg.T, cfg.d), device=dev)
    stream = pm.compute
    route = route_buffers(cfg.T, cfg.E, cfg.k, dev)
    lay.forward(x, wr, None, y=y, route=route, stream=stream)
    torch.cuda.synchronize()
    counts = route["expert_count"].cpu().numpy()
    steps = 800
    # a request rate whose KV swing (about 0.3 GB) is what one layer's plan can absorb
    kv = request_trace(steps, seed=3, peak_rate=0.12).astype(np.float64) * kv_bytes_per_token(1, 16, 128)
    w0 = float(pm.resident_bytes())
    budget = w0 + float(np.median(kv))
    sens = np.random.default_rng(11).random(cfg.n_blocks).astype(np.float32)
    ctl = KVPressurePlanner(lay, budget, sens, hysteresis_bytes=0.02 * w0, resident_bytes=pm.resident_bytes,
                            max_bits=bits.reshape(-1))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    staged, n_down, n_up, moved_total, damage, over, wmin, wmax = None, 0, 0, 0.0, 0.0, 0.0, w0, w0
    for s_ in range(steps):
        if staged is None and s_ % 8 == 0:
            d = ctl.decide(kv[s_], counts, cfg.T)
            if d is not None:
                staged = pm.stage(d[0].reshape(bits.shape))
                moved_total += abs(d[1])
                damage += max(d[2], 0.0)
                n_down += d[1] > 0
                n_up += d[1] < 0
        evs[s_][0].record(stream)
        lay.forward(x, wr, None, y=y, stream=stream)
        evs[s_][1].record(stream)
        if staged is not None and staged.ready():
            pm.commit(staged)
            staged = None
        w = float(pm.resident_bytes())
        wmin, wmax = min(wmin, w), max(wmax, w)
        over = max(over, w + kv[s_] - budget)
    if staged is not None:
        pm.commit(staged)
    torch.cuda.synchronize()
    check_status([lay], "kv pressure")
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    out = {"workload": synth.WORKLOAD_TEXT["qwen_d2048_t16"], "steps": steps,
           "kv_MB": {"min": round(kv.min() / 1e6, 1), "median": round(float(np.median(kv)) / 1e6, 1),
                     "max": round(kv.max() / 1e6, 1)},
           "budget_MB": round(budget / 1e6, 1), "weights_MB": {"start": round(w0 / 1e6, 1), "min": round(wmin / 1e6, 1),
                                                               "max": round(wmax / 1e6, 1)},
           "plan_changes": {"down": int(n_down), "up": int(n_up)}, "moved_MB": round(moved_total / 1e6, 1),
           "downgrade_damage_sum": damage, "final_bits_equal_start": bool((pm.bits == bits).all()),
           "worst_overshoot_MB": round(over / 1e6, 1),
           "forward_us": {"p50": round(float(np.percentile(us, 50)), 2), "p99": round(float(np.percentile(us, 99)), 2),
                          "max": round(float(us.max()), 2)},
           "tokens_per_s": round(cfg.T * steps / (us.sum() * 1e-6), 1), "status_checked": True}
    if print_table:
        print(json.dumps(out, indent=1))
    lay.close()
    del pm
    torch.cuda.empty_cache()
    return out


def prefill_run(args, torch, synth, PagedMoELayer, dev, print_table=True):
    """The T = 1024 prefill workload with linear-blocks of 128 rows (qwen_rows128_t1024): every
    block at its own bitwidth, bound block by block; per-call times of whole forwards over two
    byte-identical page clones, HIP events on the launch stream. Useful MFMA work counts
    2 * tokens * rows * K of every block over the tokens routed to its expert."""
    from any_precision_bit_amd import route_buffers

    def f16(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.float16).view(np.int16).copy()).to(dev).view(
            torch.float16)

    cfg = synth.CONFIGS["qwen_rows128_t1024"]
    rb = synth.ROWS_PER_BLOCK[cfg.name]
    bits = synth.rowblock_bits(cfg, rb)
    t0 = time.time()
    jobs = [(e, lin) for e in range(cfg.n_experts_total) for lin in synth.LINEARS]
    base = {}
    for e, lin in jobs:
        blk = synth.make_block(cfg, e, lin, n_planes=8, lut_bits=(3, 4, 5, 6, 8))
        base[(e, lin)] = (torch.from_numpy(np.ascontiguousarray(blk.planes)).to(dev),
                          {b: f16(v) for b, v in blk.luts.items()})
    lays = []
    for c in range(2):
        pages = base if c == 0 else {k: (p.clone(), {b: l.clone() for b, l in ls.items()}) for k, (p, ls) in base.items()}
        lay = PagedMoELayer(cfg.d, cfg.E, cfg.F, cfg.k, cfg.Fs, cfg.T, rows_per_block=rb)
        lay.plan_set(bits)
        i = 0
        for e, lin in jobs:
            planes, luts = pages[(e, lin)]
            for j in range(planes.shape[1] // rb):
                b = int(bits[i])
                i += 1
                rows = slice(j * rb, (j + 1) * rb)
                lay.bind_rows(e, lin, j, [planes[p][rows] for p in range(b)], luts[b][rows], b)
        lays.append(dict(lay=lay, pages=pages, x=f16(synth.tokens(cfg)), wr=f16(synth.router(cfg)[0]), bias=None,
                         y=torch.empty((cfg.T, cfg.d), device=dev)))
    torch.cuda.synchronize()
    log(f"qwen_rows128_t1024: pages ready ({time.time() - t0:.1f}s)")
    stream = torch.cuda.current_stream(dev)
    us = time_per_call(torch, lays, stream, 40, 4)
    check_status([c["lay"] for c in lays], "qwen_rows128_t1024")
    nb = lays[0]["lay"].last_bytes(stream)
    layer_bytes = nb[0] + nb[1] + nb[2]
    route = route_buffers(cfg.T, cfg.E, cfg.k, dev)
    c0 = lays[0]
    c0["lay"].forward(c0["x"], c0["wr"], None, y=c0["y"], route=route, stream=stream)
    torch.cuda.synchronize()
    counts = route["expert_count"].cpu().numpy().astype(np.float64)
    flops = 2.0 * 3 * cfg.F * cfg.d * counts.sum() + 2.0 * 3 * cfg.Fs * cfg.d * cfg.T
    med = float(np.median(us))
    out = {"workload": synth.WORKLOAD_TEXT[cfg.name], "tokens": cfg.T, "rows_per_block": rb,
           "blocks": int(bits.shape[0]), "mean_bits": round(float(bits.mean()), 3), "value": round(cfg.T / (med * 1e-6), 1),
           "unit": "tokens/s", "us_median": round(med, 1), "us_p10": round(float(np.percentile(us, 10)), 1),
           "us_p90": round(float(np.percentile(us, 90)), 1), "layer_bytes": layer_bytes,
           "layer_hbm_frac": round(layer_bytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
           "useful_mfma_TFLOPs": round(flops / (med * 1e-6) / 1e12, 1),
           "mfma_frac_of_fp16_peak": round(flops / (med * 1e-6) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
           "rotation_clones": 2, "status_checked": True}
    if print_table:
        print(json.dumps(out, indent=1))
    for c in lays:
        c["lay"].close()
    del lays, base
    torch.cuda.empty_cache()
    return out


def check_status(lays, what):
    """Reads (and clears) the device status word of every layer; a set flag means a forward's output
    was not valid (router range, or a dependency wait that gave up), so no figure is published."""
    for lay in lays:
        flags = lay.status()
        if flags:
            log(f"{what}: layer status flags 0x{flags:x} after the timed forwards; no result is reported")
            sys.exit(3)


def make_clones(torch, synth, PagedMoELayer, dev, cfg, n_clones, lut_tiled=False, bits=None, blocks=None):
    """Pages of one seeded layer, then byte-identical clones at distinct addresses, each bound to its own
    layer handle. Returns (clones, x_host, wr_host, bias_host, bits, blocks, page_bytes)."""
    from any_precision_bit_amd.pages import lut_page

    def f16(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.float16).view(np.int16).copy()).to(dev).view(
            torch.float16)

    if bits is None:
        bits = synth.initial_bits(cfg)
    if blocks is None:
        blocks = synth.make_layer_blocks(cfg, bits)
    x_h = synth.tokens(cfg)
    wr_h, bias_h = synth.router(cfg)
    order = lut_page if lut_tiled else np.ascontiguousarray
    base_pages = {}
    for (e, lin), blk in blocks.items():
        b = int(bits[e, lin])
        base_pages[(e, lin)] = (torch.from_numpy(np.ascontiguousarray(blk.planes[:b])).to(dev),
                                f16(order(blk.luts[b])), b)
    clones = []
    for c in range(n_clones):
        pages = base_pages if c == 0 else {key: (p.clone(), l.clone(), b) for key, (p, l, b) in base_pages.items()}
        lay = PagedMoELayer(cfg.d, cfg.E, cfg.F, cfg.k, cfg.Fs, cfg.T, lut_tiled=lut_tiled)
        lay.plan_set(bits)
        for (e, lin), (p, l, b) in pages.items():
            lay.bind(e, lin, [p[i] for i in range(b)], l, b)
        clones.append(dict(lay=lay, pages=pages, x=f16(x_h), wr=f16(wr_h),
                           bias=None if bias_h is None else f16(bias_h),
                           y=torch.empty((cfg.T, cfg.d), device=dev)))
    torch.cuda.synchronize()
    page_bytes = sum(p.numel() + l.numel() * 2 for (p, l, _) in base_pages.values())
    return clones, x_h, wr_h, bias_h, bits, blocks, page_bytes


def fwd(c, stream):
    c["lay"].forward(c["x"], c["wr"], c["bias"], y=c["y"], stream=stream)


def time_per_call(torch, clones, stream, n, warmup):
    """Per-call durations (us) of n forwards rotating over the clones, each bracketed by HIP events on
    the launch stream, after `warmup` untimed forwards."""
    for i in range(warmup):
        fwd(clones[i % len(clones)], stream)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):
        evs[i][0].record(stream)
        fwd(clones[i % len(clones)], stream)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) * 1e3 for a, b in evs])


def oracle_rate(oracle, cfg, bits, blocks, x_h, wr_h, bias_h, threads, seconds, subset=None, max_reps=32):
    """Oracle tokens/s (untuned) over repeated forwards of the batch (or of `subset` of its tokens: the
    routing of every token plus the expert outputs of those) until `seconds` of oracle time."""
    lay_o = oracle.OracleLayer.from_config(cfg, bits, blocks)
    n_tok, t_cpu, reps = 0, 0.0, 0
    while (t_cpu < seconds or reps == 0) and reps < max_reps:
        tt = time.perf_counter()
        lay_o.forward(x_h, wr_h, bias_h, subset=subset, threads=threads)
        t_cpu += time.perf_counter() - tt
        n_tok += cfg.T if subset is None else len(subset)
        reps += 1
    return n_tok / t_cpu, reps, n_tok, t_cpu


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--clones", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sub-results", action="store_true",
                    help="headline only: skip the mixtral_d4096 T=1 and qwen_stack24_t256 sub-results")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--lut-tiled", action="store_true", help="LUT pages in the 32-row tiled order")
    ap.add_argument("--sweep", action="store_true",
                    help="time every workload shape (per-call median, p10, p90) and print a table")
    ap.add_argument("--only", default="", metavar="LABEL",
                    help="with --sweep: time only the workload of this label (e.g. 'mixtral_d4096 T=64')")
    ap.add_argument("--stack", action="store_true",
                    help="time the 24-layer qwen_stack24_t256 workload over 64 steps with plan rewrites")
    ap.add_argument("--paging", action="store_true",
                    help="forward latency with and without asynchronous page movement, and the planner's host time")
    ap.add_argument("--prefill", action="store_true",
                    help="the T = 1024 prefill workload with 128-row linear-blocks")
    ap.add_argument("--kv-pressure", action="store_true",
                    help="a seeded KV-cache trace driving the planner and page movement on the decode layer")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run torch copies of MIB MiB (HBM counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    from any_precision_bit_amd import PagedMoELayer
    from any_precision_bit_amd.pages import lut_page

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = args.copy_calibration << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"copied {args.copy_calibration} MiB x 5 (reads and writes {n} bytes per copy)")
        return
    if args.sweep:
        sweep(args, torch, synth, PagedMoELayer, lut_page, dev)
        return
    if args.stack:
        layer_stack(args, torch, synth, PagedMoELayer, lut_page, dev)
        return
    if args.paging:
        paging_run(args, torch, synth, PagedMoELayer, dev)
        return
    if args.kv_pressure:
        kv_pressure_run(args, torch, synth, PagedMoELayer, dev)
        return
    if args.prefill:
        prefill_run(args, torch, synth, PagedMoELayer, dev)
        return
    cfg = synth.CONFIGS["qwen_d2048_t16"]
    T = cfg.T
    t0 = time.time()
    clones, x_h, wr_h, _, bits, blocks, page_bytes = make_clones(torch, synth, PagedMoELayer, dev, cfg,
                                                                 args.clones, lut_tiled=args.lut_tiled)
    log(f"qwen_d2048_t16: {args.clones} clones x {page_bytes / 1e6:.1f} MB of pages resident "
        f"({time.time() - t0:.1f}s)")

    stream = torch.cuda.current_stream(dev)
    for i in range(args.warmup):
        fwd(clones[i % len(clones)], stream)
    torch.cuda.synchronize()

    # headline: whole forwards back to back, events only around the timed region
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        fwd(clones[i % len(clones)], stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = ev0.elapsed_time(ev1)
    ms_per_step = ms_total / args.steps

    # per-phase durations: each phase of the last forward of every clone replayed
    # back to back over the same rotation, HIP events on the launch stream around it
    ran = min(len(clones), max(args.warmup, args.steps))   # clones that have run a forward
    n_rep = max(args.steps // 2, ran)
    avg_ms = []
    for phase in range(2):   # 0 routing, 1 experts
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n_rep):
            clones[i % ran]["lay"].replay(phase, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        avg_ms.append(e0.elapsed_time(e1) / n_rep)
    check_status([c["lay"] for c in clones], "qwen_d2048_t16")
    nb = clones[0]["lay"].last_bytes(stream)   # route, gate_up, down, residual
    phase_bytes = [nb[0], nb[1] + nb[2]]
    names = ["routing", "experts"]
    for i in range(2):
        gbs = phase_bytes[i] / (avg_ms[i] * 1e-3) / 1e9 if avg_ms[i] > 0 else 0.0
        log(f"  {names[i]:8s} {avg_ms[i] * 1e3:8.2f} us  {phase_bytes[i] / 1e6:8.2f} MB  {gbs:8.1f} GB/s")
    layer_bytes = nb[0] + nb[1] + nb[2]
    layer_gbs = layer_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"step {ms_per_step * 1e3:.2f} us (phases sum {sum(avg_ms) * 1e3:.2f} us), layer bytes "
        f"{layer_bytes / 1e6:.1f} MB -> {layer_gbs:.0f} GB/s ({layer_gbs / HBM_PEAK_GBS:.1%} of HBM peak); "
        f"wall {wall:.3f}s")

    # dominant kernel: the expert kernel (gate_up + SwiGLU + down, >99 % of the layer's bytes)
    ex_gbs = phase_bytes[1] / (avg_ms[1] * 1e-3) / 1e9
    roofline = {"bound": "hbm", "kernel": "expert_kernel<1> (gate_up + SwiGLU + down + accumulation)",
                "achieved": round(ex_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ex_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                "bytes_per_launch": phase_bytes[1], "avg_launch_us": round(avg_ms[1] * 1e3, 3),
                "alu": measured_alu()}
    for c in clones:
        c["lay"].close()
    del clones
    torch.cuda.empty_cache()

    # sub-results: the other decode-shaped workloads, same run
    subs = None
    if not args.no_sub_results:
        subs = {}
        c2 = synth.CONFIGS["mixtral_d4096"].with_tokens(1)
        t0 = time.time()
        cl2, *_ = make_clones(torch, synth, PagedMoELayer, dev, c2, args.clones, lut_tiled=args.lut_tiled)
        log(f"mixtral_d4096 T=1: pages ready ({time.time() - t0:.1f}s)")
        us = time_per_call(torch, cl2, stream, max(args.steps, 50), args.warmup)
        check_status([c["lay"] for c in cl2], "mixtral_d4096 T=1")
        nb2 = cl2[0]["lay"].last_bytes(stream)
        b2 = nb2[0] + nb2[1] + nb2[2]
        med = float(np.median(us))
        subs["mixtral_d4096_t1"] = {
            "workload": synth.WORKLOAD_TEXT["mixtral_d4096"] + ", T1", "value": round(1 / (med * 1e-6), 1),
            "unit": "tokens/s", "us_median": round(med, 2), "us_p10": round(float(np.percentile(us, 10)), 2),
            "us_p90": round(float(np.percentile(us, 90)), 2), "layer_bytes": b2,
            "layer_GBps": round(b2 / (med * 1e-6) / 1e9, 1), "layer_hbm_frac": round(b2 / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "rotation_clones": args.clones, "calls": int(len(us)), "status_checked": True}
        for c in cl2:
            c["lay"].close()
        del cl2
        torch.cuda.empty_cache()
        log(f"mixtral_d4096 T=1: median {med:.1f} us")
        # the headline layer with its LUT pages in the other accepted order (the 32-row tiled
        # order is the kernel's preferred one; row-major is the per-row table of the pages)
        other = "row-major" if args.lut_tiled else "tiled"
        clt, *_ = make_clones(torch, synth, PagedMoELayer, dev, cfg, args.clones, lut_tiled=not args.lut_tiled)
        ust = time_per_call(torch, clt, stream, max(args.steps, 50), args.warmup)
        check_status([c["lay"] for c in clt], f"qwen_d2048_t16 ({other} LUT pages)")
        medt = float(np.median(ust))
        subs["qwen_d2048_t16_lut_" + other.replace("-", "_")] = {
            "workload": synth.WORKLOAD_TEXT["qwen_d2048_t16"] + f", LUT pages {other}", "lut_pages": other,
            "value": round(T / (medt * 1e-6), 1), "unit": "tokens/s", "us_median": round(medt, 2),
            "us_p10": round(float(np.percentile(ust, 10)), 2), "us_p90": round(float(np.percentile(ust, 90)), 2),
            "rotation_clones": args.clones, "calls": int(len(ust)), "status_checked": True}
        for c in clt:
            c["lay"].close()
        del clt
        torch.cuda.empty_cache()
        log(f"qwen_d2048_t16 with {other} LUT pages: median {medt:.1f} us per forward")
        subs["qwen_stack24_t256"] = layer_stack(args, torch, synth, PagedMoELayer, lut_page, dev, print_table=False)
        log(f"qwen_stack24_t256: {subs['qwen_stack24_t256']['value']:,.0f} tokens/s")
        subs["page_movement"] = paging_run(args, torch, synth, PagedMoELayer, dev, print_table=False)
        pg = subs["page_movement"]
        log(f"page movement: forward p50 {pg['forward_us_quiet']['p50']} -> {pg['forward_us_while_moving']['p50']} us, "
            f"p99 {pg['forward_us_quiet']['p99']} -> {pg['forward_us_while_moving']['p99']} us, "
            f"{pg['copied_MB']} MB at {pg['copy_GBps']} GB/s; planner {pg['planner']['host_us']} us")
        subs["prefill_t1024"] = prefill_run(args, torch, synth, PagedMoELayer, dev, print_table=False)
        log(f"prefill T=1024: {subs['prefill_t1024']['value']:,.0f} tokens/s, "
            f"{subs['prefill_t1024']['useful_mfma_TFLOPs']} useful MFMA TFLOP/s")
        subs["kv_pressure"] = kv_pressure_run(args, torch, synth, PagedMoELayer, dev, print_table=False)
        kp = subs["kv_pressure"]
        log(f"kv pressure: {kp['plan_changes']} plan changes, weights {kp['weights_MB']} MB, "
            f"worst overshoot {kp['worst_overshoot_MB']} MB")

    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        cores = len(os.sched_getaffinity(0))
        threads = min(cores, 16)
        rate, reps, n_tok, t_cpu = oracle_rate(oracle, cfg, bits, blocks, x_h, wr_h, None, threads, args.cpu_seconds)
        cpu = {"value": round(rate, 3), "unit": "tokens/s", "cores": cores, "threads": threads, "kind": "oracle",
               "sample": f"{reps} full forward(s) of the same 16-token qwen_d2048_t16 batch ({n_tok} tokens), "
                         f"{t_cpu:.1f}s on {threads} threads"}
        log(f"oracle: {cpu['value']} tokens/s on {threads} threads ({cores} cores in the affinity set)")
        # one host thread, bounded samples: tiny_d256 (whole batches) and qwen_d2048_t16 (2 of its 16 tokens)
        one = {}
        r1, reps1, n1, t1 = oracle_rate(oracle, cfg, bits, blocks, x_h, wr_h, None, 1, 1.0,
                                        subset=np.array([0, 1], dtype=np.int32), max_reps=1)
        one["qwen_d2048_t16"] = {"value": round(r1, 3), "unit": "tokens/s",
                                 "sample": f"routing of all 16 tokens + expert outputs of 2 tokens, {t1:.1f}s"}
        c0 = synth.CONFIGS["tiny_d256"]
        bits0 = synth.initial_bits(c0)
        blocks0 = synth.make_layer_blocks(c0, bits0)
        wr0, _ = synth.router(c0)
        r0, reps0, n0, t0c = oracle_rate(oracle, c0, bits0, blocks0, synth.tokens(c0), wr0, None, 1, 1.0)
        one["tiny_d256"] = {"value": round(r0, 1), "unit": "tokens/s",
                            "sample": f"{reps0} forward(s) of the 4-token batch, {t0c:.2f}s"}
        cpu["one_thread"] = one
        log(f"oracle, one thread: qwen_d2048_t16 {r1:.3f} tokens/s, tiny_d256 {r0:.1f} tokens/s")

    out = {
        "metric": "MoE-layer decode tokens/sec on 1 MI355X; achieved HBM GB/s vs peak",
        "value": round(T * args.steps / (ms_total * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": "Qwen1.5-MoE-A2.7B-shaped decode layer: d2048, 60 routed experts ffn1408 "
                               "top-4 + shared expert ffn5632, T16, bits U{3,4,5,6,8} per (expert, linear)",
                   "tokens": T, "rotation_clones": args.clones,
                   "lut_pages": "32-row tiled" if args.lut_tiled else "row-major",
                   "layer_bytes": layer_bytes, "layer_GBps": round(layer_gbs, 1),
                   "layer_hbm_frac": round(layer_gbs / HBM_PEAK_GBS, 4), "status_checked": True},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "sub_results": subs,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
