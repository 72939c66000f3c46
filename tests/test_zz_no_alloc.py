"""pw_moe_forward_noalloc (the forward for callers that cannot allocate) against
pw_moe_forward on the same layer and inputs, two calls in a row with the second
smaller: routing bit-exact, outputs within the parity bar, and each call's
residual bit-exact for its own y (fp32 atomics may add in another order)."""
import ctypes

import numpy as np
import pytest

import synth
from helpers import REL_TOL, device_pages, f16_host, gpu_layer, layer_inputs, rel_err_per_token, to_dev_f16

pytestmark = pytest.mark.gpu


def _route_struct(B, r):
    return B.pw_route_out(*[int(r[k].data_ptr()) for k in
                            ("topk_ids", "topk_w", "expert_count", "expert_offset", "sorted_assign")])


@pytest.mark.parametrize("name,T_first,T_second", [("qwen_d2048_t16", 16, 5), ("qwen_stack24_t256", 256, 40)])
def test_noalloc_matches_forward(name, T_first, T_second):
    import torch
    from any_precision_bit_amd import binding as B
    from any_precision_bit_amd import route_buffers

    assert torch.cuda.is_available()
    dev = torch.device("cuda:0")
    cfg = synth.CONFIGS[name]
    bits = synth.initial_bits(cfg)
    blocks = synth.make_layer_blocks(cfg, bits)
    pages = device_pages(blocks, bits, dev)
    lay = gpu_layer(cfg, bits, pages, max_tokens=T_first)
    wr, bias = synth.router(cfg)
    wd = to_dev_f16(wr, dev)
    bd = None if bias is None else to_dev_f16(bias, dev)
    stream = torch.cuda.current_stream(dev)
    for call, T in enumerate((T_first, T_second)):
        print(f"no-alloc vs forward: {name} call {call} T={T}", flush=True)
        x, _, _ = layer_inputs(cfg, T, step=call)
        xd = to_dev_f16(x, dev)
        ra, rb = route_buffers(T, cfg.E, cfg.k, dev), route_buffers(T, cfg.E, cfg.k, dev)
        ya = torch.full((T, cfg.d), np.nan, device=dev)
        yb = torch.full((T, cfg.d), np.nan, device=dev)
        xa = torch.empty_like(xd)
        xb = torch.empty_like(xd)
        lay.forward(xd, wd, bd, y=ya, x_next=xa, route=ra)
        B.pw_moe_forward_noalloc(lay.handle, int(xd.data_ptr()), T, int(wd.data_ptr()),
                                 0 if bd is None else int(bd.data_ptr()), int(yb.data_ptr()), int(xb.data_ptr()),
                                 _route_struct(B, rb), int(stream.cuda_stream))
        torch.cuda.synchronize()
        assert lay.status() == 0
        for key in ("topk_ids", "expert_count", "expert_offset", "sorted_assign", "topk_w"):
            assert torch.equal(ra[key], rb[key]), key
        err = rel_err_per_token(yb.cpu().numpy(), ya.cpu().numpy())
        assert np.isfinite(err).all() and err.max() <= REL_TOL, err.max()
        # the residual is exact for each call's own y: x_next = fp16_rne(fp32(x) + y). (The two
        # calls' y may differ in the last fp32 bit, since fp32 atomics add in another order; where
        # x + y cancels that bit can move x_next by more than one fp16 ulp.)
        xh = np.asarray(x, np.float16).astype(np.float32)
        for xn, yv in ((xa, ya), (xb, yb)):
            want = (xh + yv.cpu().numpy()).astype(np.float16)
            assert np.array_equal(f16_host(xn).view(np.uint16), want.view(np.uint16))
        print(f"  routing identical, max rel err {err.max():.2e}", flush=True)
    lay.close()
