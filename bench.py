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


def kernel_code_digest():
    """sha256 of the kernel source with // comments and blank lines removed."""
    import hashlib
    code = [ln.split("//", 1)[0].rstrip() for ln in open(KERNEL_SRC)]
    return hashlib.sha256("\n".join(c for c in code if c).encode()).hexdigest()


def measured_traffic():
    """HBM bytes per expert-kernel launch from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE runs, scaled by a 1 GiB copy's readings), or None
    when the kernel code has changed since those counters were taken."""
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    fields = dict(line.split(":", 1) for line in text.splitlines() if line.startswith(("kernel_code_sha256:", "traffic_bytes_per_launch:")))
    if fields.get("kernel_code_sha256", "").strip() != kernel_code_digest():
        return None
    return float(fields["traffic_bytes_per_launch"])


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
                              f16(lut_page(blk.luts[b])), b)
        del blocks
        lays = []
        for c in range(M):
            pages = base if c == 0 else {kk: (p.clone(), l.clone(), b) for kk, (p, l, b) in base.items()}
            lay = PagedMoELayer(cfg.d, cfg.E, cfg.F, cfg.k, cfg.Fs, cfg.T)
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


def layer_stack(args, torch, synth, PagedMoELayer, lut_page, dev):
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
                                       {b: f16(lut_page(v)) for b, v in blk.luts.items()})
        del blocks
        lay = PagedMoELayer(cfg.d, cfg.E, cfg.F, cfg.k, cfg.Fs, T)
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
    print("| plan epoch | steps | mean bits | algorithmic MB per layer | mean step ms | per-layer us | "
          "GB/s | HBM % | stack tokens/s |")
    print("|---|---|---|---|---|---|---|---|---|")
    n_ep = (cfg.steps + every - 1) // every
    for ep in range(n_ep):
        sl = ms[ep * every:(ep + 1) * every]
        mb, bits_mean = epoch_bytes[ep]
        per_layer_us = sl.mean() * 1e3 / L
        print(f"| {ep} | {ep * every}..{min(cfg.steps, (ep + 1) * every) - 1} | {bits_mean:.2f} | {mb / 1e6:.1f} | "
              f"{sl.mean():.2f} | {per_layer_us:.1f} | {mb / (per_layer_us * 1e-6) / 1e9:.0f} | "
              f"{100 * mb / (per_layer_us * 1e-6) / 1e9 / HBM_PEAK_GBS:.1f} | {T / (sl.mean() * 1e-3):,.0f} |")
    print(f"| all | 0..{cfg.steps - 1} | | | {ms.mean():.2f} | {ms.mean() * 1e3 / L:.1f} | | | "
          f"{T * cfg.steps / (ms.sum() * 1e-3):,.0f} |", flush=True)
    for Ly in layers:
        assert Ly["lay"].status() == 0, "layer status flag set"
        Ly["lay"].close()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--clones", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--sweep", action="store_true",
                    help="time every workload shape (per-call median, p10, p90) and print a table")
    ap.add_argument("--only", default="", metavar="LABEL",
                    help="with --sweep: time only the workload of this label (e.g. 'mixtral_d4096 T=64')")
    ap.add_argument("--stack", action="store_true",
                    help="time the 24-layer qwen_stack24_t256 workload over 64 steps with plan rewrites")
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
    cfg = synth.CONFIGS["qwen_d2048_t16"]
    T = cfg.T
    t0 = time.time()
    bits = synth.initial_bits(cfg)
    blocks = synth.make_layer_blocks(cfg, bits)
    x_h = synth.tokens(cfg)
    wr_h, _ = synth.router(cfg)
    log(f"generated qwen_d2048_t16 pages in {time.time() - t0:.1f}s")

    def f16(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.float16).view(np.int16).copy()).to(dev).view(
            torch.float16)

    # one set of pages, then byte-identical clones at distinct addresses
    base_pages = {}
    for (e, lin), blk in blocks.items():
        b = int(bits[e, lin])
        base_pages[(e, lin)] = (torch.from_numpy(np.ascontiguousarray(blk.planes[:b])).to(dev),
                                f16(lut_page(blk.luts[b])), b)
    x = f16(x_h)
    clones = []
    for c in range(args.clones):
        pages = base_pages if c == 0 else {key: (p.clone(), l.clone(), b) for key, (p, l, b) in
                                           base_pages.items()}
        lay = PagedMoELayer(cfg.d, cfg.E, cfg.F, cfg.k, cfg.Fs, T)
        lay.plan_set(bits)
        for (e, lin), (p, l, b) in pages.items():
            lay.bind(e, lin, [p[i] for i in range(b)], l, b)
        clones.append(dict(lay=lay, pages=pages, wr=f16(wr_h), y=torch.empty((T, cfg.d), device=dev)))
    torch.cuda.synchronize()
    page_bytes = sum(p.numel() + l.numel() * 2 for (p, l, _) in base_pages.values())
    log(f"{args.clones} clones x {page_bytes / 1e6:.1f} MB of pages resident")

    stream = torch.cuda.current_stream(dev)
    for i in range(args.warmup):
        c = clones[i % len(clones)]
        c["lay"].forward(x, c["wr"], None, y=c["y"], stream=stream)
    torch.cuda.synchronize()

    # headline: whole forwards back to back, events only around the timed region
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        c = clones[i % len(clones)]
        c["lay"].forward(x, c["wr"], None, y=c["y"], stream=stream)
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
                "bytes_per_launch": phase_bytes[1], "avg_launch_us": round(avg_ms[1] * 1e3, 3)}

    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        lay_o = oracle.OracleLayer.from_config(cfg, bits, blocks)
        cores = len(os.sched_getaffinity(0))
        threads = min(cores, 16)
        n_tok, t_cpu, reps = 0, 0.0, 0
        while t_cpu < args.cpu_seconds and reps < 32:
            tt = time.perf_counter()
            lay_o.forward(x_h, wr_h, None, threads=threads)
            t_cpu += time.perf_counter() - tt
            n_tok += T
            reps += 1
        cpu = {"value": round(n_tok / t_cpu, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"{reps} full forward(s) of the same 16-token qwen_d2048_t16 batch ({n_tok} tokens), "
                         f"{t_cpu:.1f}s on {threads} threads"}
        log(f"oracle: {cpu['value']} tokens/s on {threads} threads")

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
                   "layer_bytes": layer_bytes, "layer_GBps": round(layer_gbs, 1),
                   "layer_hbm_frac": round(layer_gbs / HBM_PEAK_GBS, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    for c in clones:
        c["lay"].close()


if __name__ == "__main__":
    main()
