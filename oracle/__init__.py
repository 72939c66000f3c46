"""CPU oracle for the fused mixed-precision MoE layer -- TEST INFRASTRUCTURE.

Only `tests/`, `__graft_entry__.smoke()` and the `cpu_baseline` leg of
`bench.py` may import this package. It is a plain, slow, obviously correct
implementation of the layer (see oracle.c for the step list and the reading
of the PagedWeight pages it follows). It shares no code with the GPU library:
it takes the generator's arrays (`synth`) directly, never the page table.

Pins (checked by the `-m "not gpu"` tests): brute-force index truncation, the
b = 8 parent dequant, an identity-LUT closed form, dense fp64 equality with an
independently materialised weight matrix and an exact Python-integer router,
a textbook SwiGLU MLP when E = k = 1, routing weights summing to 1, and
permutation / relabeling / batch invariances.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# ORACLE_LIBRARY names another build of oracle.c (a sanitizer build for the pins)
_LOAD_PATH = os.environ.get("ORACLE_LIBRARY") or _LIB_PATH
_lib = None

ORC_OK, ORC_E_RANGE, ORC_E_ARG = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (plain C, OpenMP, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def build_sanitized(out_dir: str) -> str:
    """oracle.c with AddressSanitizer and UBSan (gcc) in out_dir; load it with
    gcc's libasan preloaded and ORACLE_LIBRARY pointing at it."""
    os.makedirs(out_dir, exist_ok=True)
    out = os.path.join(out_dir, "liboracle_san.so")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-fPIC", "-shared", "-o", out, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def lib():
    global _lib
    if _lib is None:
        if _LOAD_PATH == _LIB_PATH and not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LOAD_PATH)
        P = ctypes.c_void_p
        i32 = ctypes.c_int
        L.orc_router_logits.argtypes = [P, i32, i32, P, i32, P, P]
        L.orc_router_logits.restype = i32
        L.orc_topk_softmax.argtypes = [P, i32, i32, i32, P, P]
        L.orc_topk_softmax.restype = None
        L.orc_bucket_sort.argtypes = [P, i32, i32, i32, P, P, P]
        L.orc_bucket_sort.restype = None
        L.orc_unpack_indices.argtypes = [P, i32, i32, i32, P]
        L.orc_unpack_indices.restype = None
        L.orc_dequant.argtypes = [P, i32, P, i32, i32, P]
        L.orc_dequant.restype = None
        L.orc_linear.argtypes = [P, i32, P, i32, i32, P, P]
        L.orc_linear.restype = None
        L.orc_moe_forward.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, P, i32, P, P, P, i32, P,
                                      P, P, P, P, P, P, i32]
        L.orc_moe_forward.restype = i32
        L.orc_residual.argtypes = [P, P, ctypes.c_size_t, P]
        L.orc_residual.restype = None
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _h(a) -> np.ndarray:
    """fp16 array -> contiguous uint16 view (bit patterns)."""
    a = np.ascontiguousarray(a, dtype=np.float16)
    return a.view(np.uint16)


def _plane_ptrs(planes: np.ndarray, b: int):
    planes = np.ascontiguousarray(planes, dtype=np.uint8)
    assert planes.shape[0] >= b
    arr = (ctypes.c_void_p * 8)()
    for p in range(b):
        arr[p] = planes[p].ctypes.data
    return arr, planes


# ----------------------------------------------------------------------------- steps
def router_logits(x, wr, bias=None):
    """O1: exact logits as int64 in units of 2^-48, [T, E]. Returns (L, status)."""
    xh, wh = _h(x), _h(wr)
    T, d = xh.shape
    E = wh.shape[0]
    bh = None if bias is None else _h(bias)
    L = np.zeros((T, E), dtype=np.int64)
    st = lib().orc_router_logits(_p(xh), T, d, _p(wh), E, _p(bh), _p(L))
    return L, st


def topk_softmax(L, k):
    """O2 + O3: ids int32 [T, k], w fp32 [T, k]."""
    L = np.ascontiguousarray(L, dtype=np.int64)
    T, E = L.shape
    ids = np.zeros((T, k), dtype=np.int32)
    w = np.zeros((T, k), dtype=np.float32)
    lib().orc_topk_softmax(_p(L), T, E, k, _p(ids), _p(w))
    return ids, w


def bucket_sort(ids, E):
    """O4: counts [E], offsets [E+1], sorted [T*k]."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    counts = np.zeros(E, dtype=np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    srt = np.zeros(T * k, dtype=np.int32)
    lib().orc_bucket_sort(_p(ids), T, E, k, _p(counts), _p(offsets), _p(srt))
    return counts, offsets, srt


def unpack_indices(planes, b):
    """O5: indices u8 [R, K] at bitwidth b, read bit by bit from planes [>=b, R, K/8]."""
    ptrs, keep = _plane_ptrs(planes, b)
    R, K8 = keep.shape[1], keep.shape[2]
    out = np.zeros((R, K8 * 8), dtype=np.uint8)
    lib().orc_unpack_indices(ptrs, b, R, K8 * 8, _p(out))
    return out


def dequant(planes, b, lut):
    """O5: weights fp32 [R, K] = LUT_b[r][idx]."""
    ptrs, keep = _plane_ptrs(planes, b)
    R, K8 = keep.shape[1], keep.shape[2]
    lh = _h(lut)
    assert lh.shape == (R, 1 << b)
    out = np.zeros((R, K8 * 8), dtype=np.float32)
    lib().orc_dequant(ptrs, b, _p(lh), R, K8 * 8, _p(out))
    return out


def linear(planes, b, lut, x):
    """One linear out[r] = sum_c W[r][c] x[c] (fp32, c ascending)."""
    ptrs, keep = _plane_ptrs(planes, b)
    R, K8 = keep.shape[1], keep.shape[2]
    lh = _h(lut)
    xh = _h(x).reshape(-1)
    assert xh.shape[0] == K8 * 8
    out = np.zeros(R, dtype=np.float32)
    lib().orc_linear(ptrs, b, _p(lh), R, K8 * 8, _p(xh), _p(out))
    return out


def residual(x, y):
    """O9: fp16_rne(float(x) + y) as float16."""
    xh = _h(x)
    y = np.ascontiguousarray(y, dtype=np.float32)
    assert y.shape == xh.shape
    out = np.zeros(xh.shape, dtype=np.uint16)
    lib().orc_residual(_p(xh), _p(y), xh.size, _p(out))
    return out.view(np.float16)


# ----------------------------------------------------------------------------- layer
class OracleLayer:
    """The oracle's own copy of one layer: bitwidth plan plus the generator's
    planes and LUTs per (expert, linear). A plan change is a new `bits` array;
    the layer keeps no other state (O8).

    rows_per_block = 0: one linear-block per linear, bits [E + has_shared, 3].
    rows_per_block = rb > 0: each linear is split into blocks of rb rows, bits is
    flat, one entry per block in the order expert (routed, then shared), linear
    (gate, up, down), row-block; block j of a linear reads rows j*rb .. j*rb+rb-1
    of that linear's planes and of its LUT at the block's own bitwidth."""

    def __init__(self, d, E, F, k, Fs, bits, blocks, rows_per_block=0):
        self.d, self.E, self.F, self.k, self.Fs = int(d), int(E), int(F), int(k), int(Fs)
        self.rb = int(rows_per_block)
        self.n_total = self.E + (1 if self.Fs > 0 else 0)
        self.blocks = blocks            # (e, lin) -> object with .planes and .luts
        self.set_bits(bits)

    @classmethod
    def from_config(cls, cfg, bits, blocks, rows_per_block=0):
        return cls(cfg.d, cfg.E, cfg.F, cfg.k, cfg.Fs, bits, blocks, rows_per_block)

    def block_list(self):
        """(e, lin, first row, rows) of every block in order."""
        out = []
        for e in range(self.n_total):
            f = self.Fs if e == self.E else self.F
            for lin in range(3):
                R = self.d if lin == 2 else f
                rows = self.rb or R
                for j in range(R // rows):
                    out.append((e, lin, j * rows, rows))
        return out

    def set_bits(self, bits):
        blist = self.block_list()
        bits = np.ascontiguousarray(np.asarray(bits, dtype=np.uint8).reshape(-1))
        if bits.shape[0] != len(blist):
            raise ValueError(f"{bits.shape[0]} bitwidths for {len(blist)} blocks")
        self._bits = bits
        self._plane_arr = (ctypes.c_void_p * (len(blist) * 8))()
        self._lut_arr = (ctypes.c_void_p * len(blist))()
        self._keep = []
        for i, (e, lin, r0, rows) in enumerate(blist):
            b = int(bits[i])
            blk = self.blocks[(e, lin)]
            planes = np.ascontiguousarray(blk.planes, dtype=np.uint8)
            if planes.shape[0] < b:
                raise ValueError(f"block {(e, lin)} has {planes.shape[0]} planes < b={b}")
            lut_b = _h(blk.luts[b])
            self._keep += [planes, lut_b]
            for p in range(b):
                self._plane_arr[i * 8 + p] = planes[p, r0:r0 + rows].ctypes.data
            self._lut_arr[i] = lut_b[r0:r0 + rows].ctypes.data

    @property
    def bits(self):
        return self._bits.reshape(self.n_total, 3).copy() if not self.rb else self._bits.copy()

    def forward(self, x, router_w, router_b=None, subset=None, threads: int = 0):
        """Returns dict(y, logits, ids, w, counts, offsets, sorted, status).
        y rows outside `subset` are NaN."""
        xh = _h(x)
        T, d = xh.shape
        assert d == self.d
        wh = _h(router_w)
        bh = None if router_b is None else _h(router_b)
        sub = None if subset is None else np.ascontiguousarray(subset, dtype=np.int32)
        y = np.full((T, d), np.nan, dtype=np.float32)
        L = np.zeros((T, self.E), dtype=np.int64)
        ids = np.zeros((T, self.k), dtype=np.int32)
        w = np.zeros((T, self.k), dtype=np.float32)
        counts = np.zeros(self.E, dtype=np.int32)
        offsets = np.zeros(self.E + 1, dtype=np.int32)
        srt = np.zeros(T * self.k, dtype=np.int32)
        st = lib().orc_moe_forward(
            self.d, self.E, self.F, self.Fs, self.k, self.rb, _p(self._bits), self._plane_arr, self._lut_arr,
            _p(xh), T, _p(wh), _p(bh), _p(sub), 0 if sub is None else len(sub), _p(y), _p(L),
            _p(ids), _p(w), _p(counts), _p(offsets), _p(srt), int(threads))
        return dict(y=y, logits=L, ids=ids, w=w, counts=counts, offsets=offsets, sorted=srt,
                    status=st)
