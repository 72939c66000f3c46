"""Shared test utilities: device placement of generated pages, a GPU layer
built through the C ABI, and the parity metrics. No layer arithmetic here."""
from __future__ import annotations

import numpy as np

import synth

# Parity bar on floating-point outputs: per token, max |y - y_ref| / max |y_ref| <= 2e-3.
REL_TOL = 2e-3


def rel_err_per_token(y, ref):
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.abs(y - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    return num / np.maximum(den, 1e-30)


def device_pages(blocks, bits, device, all_luts=False, lut_tiled=False):
    """Copies each block's planes 0..b-1 (all generated planes when all_luts)
    and its LUT(s), row-major (or in the 32-row tiled page order), to the device.
    Returns {(e, lin): (planes u8 [n,R,K/8], {b: lut fp16})}."""
    import torch
    from any_precision_bit_amd.pages import lut_page

    order = lut_page if lut_tiled else np.ascontiguousarray
    out = {}
    for (e, lin), blk in blocks.items():
        b = int(bits[e, lin])
        n = blk.planes.shape[0] if all_luts else b
        planes = torch.from_numpy(np.ascontiguousarray(blk.planes[:n])).to(device)
        lb = blk.luts.keys() if all_luts else [b]
        luts = {int(bb): torch.from_numpy(order(blk.luts[bb]).view(np.int16).copy()).to(device)
                .view(torch.float16) for bb in lb}
        out[(e, lin)] = (planes, luts)
    return out


def bind_all(layer, bits, pages):
    for (e, lin), (planes, luts) in pages.items():
        b = int(bits[e, lin])
        layer.bind(e, lin, [planes[p] for p in range(b)], luts[b], b)


def gpu_layer(cfg, bits, pages, max_tokens=None, lut_tiled=False, deterministic=False):
    from any_precision_bit_amd import PagedMoELayer

    lay = PagedMoELayer(cfg.d, cfg.E, cfg.F, cfg.k, cfg.Fs, max_tokens or max(cfg.T, 1), lut_tiled=lut_tiled,
                        deterministic=deterministic)
    lay.plan_set(bits)
    bind_all(lay, bits, pages)
    return lay


def to_dev_f16(a, device):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16).view(np.int16).copy()).to(
        device).view(torch.float16)


def f16_host(t):
    import torch

    return t.detach().view(torch.int16).cpu().numpy().view(np.float16)


def sample_tokens(T, n, seed=0):
    if n >= T:
        return np.arange(T, dtype=np.int32)
    g = np.random.default_rng(seed)
    return np.sort(g.choice(T, size=n, replace=False)).astype(np.int32)


def layer_inputs(cfg, T=None, *, layer=0, run_seed=0, step=0):
    x = synth.tokens(cfg, T, layer=layer, run_seed=run_seed, step=step)
    wr, bias = synth.router(cfg, layer=layer, run_seed=run_seed)
    return x, wr, bias
