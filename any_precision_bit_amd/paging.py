"""Asynchronous page movement for one layer's Any-Precision pages.

The PagedWeight pages treat the bit-plane and LUT buffers as GPU-resident pages
that are reloaded or offloaded asynchronously, overlapped with serving
(arxivlens summary; legiblepapers "Summary & Methodology Analysis"); the
limitations note rare latency spikes from it. This module is that mechanism on
one GPU, as plumbing around the library: PyTorch supplies pinned host memory,
device memory, streams and events; the layer's pw_moe_plan_set and
pw_page_table_bind take the result. No layer arithmetic happens here.

Host tier: every block's planes 0..n-1 and its LUT for every bitwidth a plan
may use, in pinned host memory (the pages are read-only weights, so the host
copy is always current and offloading never writes back). Device tier: for
every block, exactly the pages its current bitwidth b reads, planes 0..b-1 and
LUT_b. A plan change is staged on a copy stream: the pages the new plan reads
and the device lacks are copied host-to-device there while forwards keep
running on the compute stream with the old plan. commit() makes the compute
stream wait for those copies, sets the plan, binds the pages, and drops the
device pages the new plan no longer reads; the caching allocator reuses their
memory only after the compute stream has passed every forward that read them.
"""
from __future__ import annotations

from typing import Dict, Optional, Tuple

import numpy as np
import torch


def pages_of(b: int):
    """The device pages a block at bitwidth b reads: planes 0..b-1 and LUT_b."""
    return {("plane", p) for p in range(b)} | {("lut", b)}


def page_delta(old_bits, new_bits):
    """Pages to load and to drop, per block index, when the plan goes from old_bits to new_bits:
    (load, drop), each a dict block -> set of ("plane", p) / ("lut", b)."""
    old = np.asarray(old_bits).reshape(-1)
    new = np.asarray(new_bits).reshape(-1)
    load, drop = {}, {}
    for i, (a, b) in enumerate(zip(old.tolist(), new.tolist())):
        have, need = pages_of(int(a)), pages_of(int(b))
        if need - have:
            load[i] = need - have
        if have - need:
            drop[i] = have - need
    return load, drop


class Staged:
    """A plan change whose copies have been issued on the copy stream."""

    def __init__(self, bits, new_pages, drop, event, nbytes, t0, t1):
        self.bits, self.new_pages, self.drop = bits, new_pages, drop
        self.event, self.nbytes = event, nbytes
        self.t0, self.t1 = t0, t1           # timing events around the copies

    def ready(self) -> bool:
        return self.event.query()

    def copy_ms(self) -> float:
        """Duration of the copies on the copy stream (synchronises with them)."""
        self.t1.synchronize()
        return self.t0.elapsed_time(self.t1)


class PageManager:
    """Device residency of one layer's pages.

    layer: a PagedMoELayer; host: {(e, lin): (planes u8 [n, R, K/8] numpy or torch, {b: LUT fp16 [R, 2^b]})}
    (the LUT page order must match the layer's); bits: the initial plan u8 [E + has_shared, 3]."""

    def __init__(self, layer, host: Dict[Tuple[int, int], tuple], bits, device,
                 compute_stream: Optional[torch.cuda.Stream] = None,
                 copy_stream: Optional[torch.cuda.Stream] = None):
        self.layer = layer
        self.device = device
        self.compute = compute_stream or torch.cuda.current_stream(device)
        self.copy = copy_stream or torch.cuda.Stream(device)   # default priority
        self.keys = [(e, lin) for e in range(layer.n_total) for lin in range(3)]
        self.host = {}
        for key in self.keys:
            planes, luts = host[key]
            hp = torch.as_tensor(np.ascontiguousarray(planes) if isinstance(planes, np.ndarray) else planes)
            self.host[key] = (hp.pin_memory(),
                              {int(b): torch.as_tensor(np.ascontiguousarray(v).view(np.int16)).pin_memory()
                               .view(torch.float16) for b, v in luts.items()})
        self.bits = np.asarray(bits, dtype=np.uint8).reshape(layer.n_total, 3).copy()
        self.dev: Dict[Tuple[int, int], dict] = {k: {} for k in self.keys}
        # initial residency, synchronously
        for i, key in enumerate(self.keys):
            for page in pages_of(int(self.bits.reshape(-1)[i])):
                self.dev[key][page] = self._host_page(key, page).to(device)
        torch.cuda.synchronize(device)
        layer.plan_set(self.bits)
        for key in self.keys:
            self._bind(key, int(self.bits[key]))

    def _host_page(self, key, page):
        planes, luts = self.host[key]
        kind, v = page
        if kind == "plane":
            if v >= planes.shape[0]:
                raise ValueError(f"block {key}: plane {v} is not in the host tier")
            return planes[v]
        if v not in luts:
            raise ValueError(f"block {key}: LUT for b={v} is not in the host tier")
        return luts[v]

    def _bind(self, key, b):
        pages = self.dev[key]
        self.layer.bind(key[0], key[1], [pages[("plane", p)] for p in range(b)], pages[("lut", b)], b)

    def resident_bytes(self) -> int:
        return sum(t.numel() * t.element_size() for pg in self.dev.values() for t in pg.values())

    def stage(self, new_bits) -> Staged:
        """Issues, on the copy stream, the host-to-device copies of every page new_bits reads that
        the device lacks. Returns at once; forwards may keep running with the current plan."""
        new_bits = np.asarray(new_bits, dtype=np.uint8).reshape(self.bits.shape)
        load, drop = page_delta(self.bits, new_bits)
        new_pages = {}
        nbytes = 0
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(self.copy):
            t0.record(self.copy)
            for i, pages in load.items():
                key = self.keys[i]
                for page in sorted(pages):
                    src = self._host_page(key, page)
                    dst = torch.empty_like(src, device=self.device)
                    dst.copy_(src, non_blocking=True)
                    new_pages[(key, page)] = dst
                    nbytes += src.numel() * src.element_size()
            t1.record(self.copy)
            ev = torch.cuda.Event()
            ev.record(self.copy)
        return Staged(new_bits, new_pages, {self.keys[i]: pg for i, pg in drop.items()}, ev, nbytes, t0, t1)

    def commit(self, staged: Staged) -> None:
        """Makes the compute stream wait for the staged copies, then sets the new plan and binds
        its pages; the next forward on the compute stream reads them. Pages the new plan no longer
        reads are dropped (their memory is reused only after the compute stream passes this point)."""
        self.compute.wait_event(staged.event)
        for (key, page), t in staged.new_pages.items():
            t.record_stream(self.compute)   # allocated on the copy stream, read on the compute stream
            self.dev[key][page] = t
        for key, pages in staged.drop.items():
            for page in pages:
                self.dev[key].pop(page).record_stream(self.compute)
        self.bits = staged.bits.copy()
        self.layer.plan_set(self.bits)
        for i, key in enumerate(self.keys):
            self._bind(key, int(self.bits[key]))
