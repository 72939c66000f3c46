"""Torch-facing wrapper of the C ABI: passes tensor addresses and the current
stream to libpw.so. No computation happens here."""
from __future__ import annotations

from typing import Optional, Sequence

import torch

from . import binding as B


def _ptr(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else int(t.data_ptr())


class PagedMoELayer:
    """One fused mixed-precision MoE layer (handle of pw_layer_create).

    The caller owns every device tensor; the wrapper keeps references to the
    bound pages so they outlive the forwards that read them."""

    def __init__(self, d_model: int, n_experts: int, d_ffn: int, top_k: int,
                 d_ffn_shared: int = 0, max_tokens: int = 256, lut_tiled: bool = False,
                 rows_per_block: int = 0, deterministic: bool = False):
        self.d_model, self.n_experts, self.d_ffn = d_model, n_experts, d_ffn
        self.top_k, self.d_ffn_shared, self.max_tokens = top_k, d_ffn_shared, max_tokens
        self.n_total = n_experts + (1 if d_ffn_shared > 0 else 0)
        self.lut_tiled = lut_tiled
        self.rows_per_block = rows_per_block
        self.deterministic = deterministic
        flags = (B.PW_FLAG_LUT_TILED if lut_tiled else 0) | (B.PW_FLAG_DETERMINISTIC if deterministic else 0)
        self.handle = B.pw_layer_create(d_model, n_experts, d_ffn, top_k, d_ffn_shared, max_tokens,
                                        flags=flags, rows_per_block=rows_per_block)
        self._pages = {}

    def close(self):
        if self.handle:
            B.pw_layer_destroy(self.handle)
            self.handle = 0
            self._pages.clear()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def plan_set(self, bits) -> None:
        B.pw_moe_plan_set(self.handle, bits)

    def bind(self, expert: int, linear: int, planes: Sequence[torch.Tensor] | torch.Tensor,
             lut: torch.Tensor, lut_bits: int) -> None:
        """planes: a tensor [n, R, K/8] (u8) or a list of per-plane tensors."""
        if isinstance(planes, torch.Tensor):
            addrs = [int(planes[p].data_ptr()) for p in range(planes.shape[0])]
        else:
            addrs = [int(p.data_ptr()) for p in planes]
        B.pw_page_table_bind(self.handle, expert, linear, addrs, int(lut.data_ptr()), lut_bits)
        self._pages[(expert, linear)] = (planes, lut)

    def bind_rows(self, expert: int, linear: int, row_block: int, planes: Sequence[torch.Tensor],
                  lut: torch.Tensor, lut_bits: int) -> None:
        """Pages of one row-block: per-plane tensors of its rows and its rows of the LUT."""
        B.pw_page_table_bind_rows(self.handle, expert, linear, row_block, [int(p.data_ptr()) for p in planes],
                                  int(lut.data_ptr()), lut_bits)
        self._pages[(expert, linear, row_block)] = (planes, lut)

    def forward(self, x: torch.Tensor, router_w: torch.Tensor, router_b: Optional[torch.Tensor] = None,
                y: Optional[torch.Tensor] = None, x_next: Optional[torch.Tensor] = None,
                route: Optional[dict] = None, stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
        T = x.shape[0]
        if y is None:
            y = torch.empty((T, self.d_model), dtype=torch.float32, device=x.device)
        r = None
        if route is not None:
            r = B.pw_route_out(*[_ptr(route.get(k)) or None for k in
                                 ("topk_ids", "topk_w", "expert_count", "expert_offset", "sorted_assign")])
        s = stream if stream is not None else torch.cuda.current_stream(x.device)
        B.pw_moe_forward(self.handle, _ptr(x), T, _ptr(router_w), _ptr(router_b), _ptr(y), _ptr(x_next),
                         r, int(s.cuda_stream))
        return y

    def status(self, stream: Optional[torch.cuda.Stream] = None) -> int:
        s = stream if stream is not None else torch.cuda.current_stream()
        return B.pw_layer_status(self.handle, int(s.cuda_stream))

    def replay(self, phase: int, stream: Optional[torch.cuda.Stream] = None) -> None:
        s = stream if stream is not None else torch.cuda.current_stream()
        B.pw_moe_replay(self.handle, phase, int(s.cuda_stream))

    def set_wait_limit(self, polls: int) -> None:
        """Test hook: polls of a down item's dependency counter before it gives up."""
        B.pw_debug_set_wait_limit(self.handle, polls)

    def set_path(self, path) -> None:
        """A/B switch of the expert kernels: 'auto', 'small', 'four' or 'big'."""
        B.pw_debug_set_path(self.handle, path)

    def last_bytes(self, stream: Optional[torch.cuda.Stream] = None):
        s = stream if stream is not None else torch.cuda.current_stream()
        return B.pw_layer_last_bytes(self.handle, int(s.cuda_stream))


def route_buffers(T: int, E: int, k: int, device) -> dict:
    """Device buffers for the optional routing outputs of a forward."""
    return dict(topk_ids=torch.empty((T, k), dtype=torch.int32, device=device),
                topk_w=torch.empty((T, k), dtype=torch.float32, device=device),
                expert_count=torch.empty((E,), dtype=torch.int32, device=device),
                expert_offset=torch.empty((E + 1,), dtype=torch.int32, device=device),
                sorted_assign=torch.empty((T * k,), dtype=torch.int32, device=device))
