"""ctypes binding of libpw.so (include/pw.h), argument marshalling only.

Every compute step runs in the library's HIP kernels. Functions keep the C
names; pointers are plain integers (e.g. `tensor.data_ptr()`), streams are
`hipStream_t` handles as integers (`torch.cuda.current_stream().cuda_stream`).
Raises PwError on any non-OK status. Import fails loudly when the library has
not been built.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# PW_LIBRARY names another build of the same ABI (a sanitizer build for host-side tests)
LIB_PATH = os.environ.get("PW_LIBRARY") or os.path.join(_HERE, "libpw.so")

PW_ABI_VERSION = 2
PW_FLAG_LUT_TILED = 1
PW_FLAG_DETERMINISTIC = 2
PW_GATE, PW_UP, PW_DOWN = 0, 1, 2
PW_STATUS_ROUTER_RANGE = 1
PW_STATUS_DEP_TIMEOUT = 2
STATUS_NAMES = {0: "PW_OK", 1: "PW_E_ARG", 2: "PW_E_SHAPE", 3: "PW_E_BITS", 4: "PW_E_UNBOUND",
                5: "PW_E_ALIGN", 6: "PW_E_RANGE", 7: "PW_E_STATE", 8: "PW_E_NOMEM", 9: "PW_E_HIP"}
EXPORTED = ["pw_layer_create", "pw_layer_destroy", "pw_last_error", "pw_moe_plan_set",
            "pw_page_table_bind", "pw_moe_forward", "pw_layer_status", "pw_moe_replay",
            "pw_layer_last_bytes", "pw_debug_unpack", "pw_debug_dequant", "pw_debug_set_wait_limit", "pw_debug_set_path",
            "pw_moe_forward_noalloc", "pw_plan_greedy", "pw_page_table_bind_rows"]


class PwError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class pw_moe_desc(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("d_ffn", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("d_ffn_shared", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("rows_per_block", ctypes.c_int32)]


class pw_route_out(ctypes.Structure):
    _fields_ = [("topk_ids", ctypes.c_void_p), ("topk_w", ctypes.c_void_p),
                ("expert_count", ctypes.c_void_p), ("expert_offset", ctypes.c_void_p),
                ("sorted_assign", ctypes.c_void_p)]


def _load():
    # PyTorch supplies device memory and streams; its HIP runtime must be the one
    # libpw.so binds to, so it is loaded first (one HIP runtime per process).
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "or python any_precision_bit_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, u32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32
    st = ctypes.c_int
    sig = {
        "pw_layer_create": ([ctypes.POINTER(pw_moe_desc), ctypes.POINTER(P)], st),
        "pw_layer_destroy": ([P], st),
        "pw_last_error": ([], ctypes.c_char_p),
        "pw_moe_plan_set": ([P, P, i32], st),
        "pw_page_table_bind": ([P, i32, i32, P, i32, P, i32], st),
        "pw_page_table_bind_rows": ([P, i32, i32, i32, P, i32, P, i32], st),
        "pw_moe_forward": ([P, P, i32, P, P, P, P, ctypes.POINTER(pw_route_out), P], st),
        "pw_moe_forward_noalloc": ([P, P, i32, P, P, P, P, ctypes.POINTER(pw_route_out), P], st),
        "pw_layer_status": ([P, P, ctypes.POINTER(u32)], st),
        "pw_plan_greedy": ([P, P, P, P, i32, P, P, ctypes.c_double, P, P], st),
        "pw_moe_replay": ([P, i32, P], st),
        "pw_layer_last_bytes": ([P, P, ctypes.POINTER(ctypes.c_double)], st),
        "pw_debug_unpack": ([P, i32, i32, i32, P, P], st),
        "pw_debug_dequant": ([P, i32, P, u32, i32, i32, P, P], st),
        "pw_debug_set_wait_limit": ([P, u32], st),
        "pw_debug_set_path": ([P, i32], st),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    return L


lib = _load()


def pw_last_error() -> str:
    return (lib.pw_last_error() or b"").decode()


def _check(status: int):
    if status != 0:
        raise PwError(status, pw_last_error())


def pw_layer_create(d_model, n_experts, d_ffn, top_k, d_ffn_shared, max_tokens, flags=0,
                    abi_version=PW_ABI_VERSION, rows_per_block=0) -> int:
    desc = pw_moe_desc(abi_version, d_model, n_experts, d_ffn, top_k, d_ffn_shared, max_tokens, flags,
                       rows_per_block)
    out = ctypes.c_void_p()
    _check(lib.pw_layer_create(ctypes.byref(desc), ctypes.byref(out)))
    return out.value


def pw_layer_destroy(layer: int):
    _check(lib.pw_layer_destroy(layer))


def pw_moe_plan_set(layer: int, bits) -> None:
    """bits: any sequence of ints, flattened in (expert, linear) order."""
    flat = [int(b) for b in (bits.reshape(-1).tolist() if hasattr(bits, "reshape") else bits)]
    arr = (ctypes.c_uint8 * len(flat))(*flat)
    _check(lib.pw_moe_plan_set(layer, arr, len(flat)))


def pw_page_table_bind(layer: int, expert: int, linear: int, planes, lut: int, lut_bits: int) -> None:
    """planes: sequence of device addresses (ints) of planes 0..n-1."""
    arr = (ctypes.c_void_p * max(1, len(planes)))(*[int(p) for p in planes])
    _check(lib.pw_page_table_bind(layer, expert, linear, arr, len(planes), lut, lut_bits))


def pw_page_table_bind_rows(layer: int, expert: int, linear: int, row_block: int, planes, lut: int,
                            lut_bits: int) -> None:
    """planes: sequence of device addresses (ints) of the block's rows of planes 0..n-1."""
    arr = (ctypes.c_void_p * max(1, len(planes)))(*[int(p) for p in planes])
    _check(lib.pw_page_table_bind_rows(layer, expert, linear, row_block, arr, len(planes), lut, lut_bits))


def pw_moe_forward(layer: int, x: int, T: int, router_w: int, router_b, y: int, x_next=None,
                   route: pw_route_out | None = None, stream: int = 0) -> None:
    _check(lib.pw_moe_forward(layer, x, T, router_w, router_b or None, y, x_next or None,
                              ctypes.byref(route) if route is not None else None, stream or None))


def pw_moe_forward_noalloc(layer: int, x: int, T: int, router_w: int, router_b, y: int, x_next=None,
                           route: pw_route_out | None = None, stream: int = 0) -> None:
    _check(lib.pw_moe_forward_noalloc(layer, x, T, router_w, router_b or None, y, x_next or None,
                                      ctypes.byref(route) if route is not None else None, stream or None))


def pw_plan_greedy(layer: int, sensitivity, expert_count, n_tokens: int, bytes_to_free: float,
                   residual=None, min_bits=None, max_bits=None):
    """Host arrays in, (new bits u8 [n_blocks], bytes moved, damage, actions) out."""
    import numpy as np

    sens = np.ascontiguousarray(sensitivity, dtype=np.float32).reshape(-1)
    cnt = np.ascontiguousarray(expert_count, dtype=np.int32).reshape(-1)
    res = None if residual is None else np.ascontiguousarray(residual, dtype=np.float32).reshape(-1)
    lo = None if min_bits is None else np.ascontiguousarray(min_bits, dtype=np.uint8).reshape(-1)
    hi = None if max_bits is None else np.ascontiguousarray(max_bits, dtype=np.uint8).reshape(-1)
    out = np.zeros(sens.shape[0], dtype=np.uint8)
    r = (ctypes.c_double * 3)()
    p = lambda a: None if a is None else a.ctypes.data_as(ctypes.c_void_p)
    _check(lib.pw_plan_greedy(layer, p(sens), p(res), p(cnt), n_tokens, p(lo), p(hi), float(bytes_to_free),
                              p(out), r))
    return out, r[0], r[1], int(r[2])


def pw_layer_status(layer: int, stream: int = 0) -> int:
    flags = ctypes.c_uint32(0)
    st = lib.pw_layer_status(layer, stream or None, ctypes.byref(flags))
    if st not in (0, 7):
        _check(st)
    return flags.value


def pw_moe_replay(layer: int, phase: int, stream: int = 0) -> None:
    _check(lib.pw_moe_replay(layer, phase, stream or None))


def pw_layer_last_bytes(layer: int, stream: int = 0):
    b = (ctypes.c_double * 4)()
    _check(lib.pw_layer_last_bytes(layer, stream or None, b))
    return list(b)


def pw_debug_unpack(planes, b: int, R: int, K: int, idx_out: int, stream: int = 0) -> None:
    arr = (ctypes.c_void_p * 8)(*([int(p) for p in planes] + [None] * (8 - len(planes))))
    _check(lib.pw_debug_unpack(arr, b, R, K, idx_out, stream or None))


def pw_debug_dequant(planes, b: int, lut: int, R: int, K: int, w_out: int, stream: int = 0,
                     lut_flags: int = 0) -> None:
    arr = (ctypes.c_void_p * 8)(*([int(p) for p in planes] + [None] * (8 - len(planes))))
    _check(lib.pw_debug_dequant(arr, b, lut, lut_flags, R, K, w_out, stream or None))


def pw_debug_set_wait_limit(layer: int, polls: int) -> None:
    _check(lib.pw_debug_set_wait_limit(layer, polls))


PATHS = {"auto": 0, "small": 1, "four": 2, "big": 3, "two": 4}


def pw_debug_set_path(layer: int, path) -> None:
    """Which expert kernel takes which experts: 'auto', 'small', 'four', 'big' (or 0..3)."""
    _check(lib.pw_debug_set_path(layer, PATHS[path] if isinstance(path, str) else int(path)))
