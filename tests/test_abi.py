"""C-ABI library checks that need no GPU: the library loads, exports every
function include/pw.h declares, and validates arguments before touching the
device (every error path returns before any HIP call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "pw.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(pw_[a-z_0-9]+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def B():
    from any_precision_bit_amd import binding
    return binding


def test_exports_every_declared_symbol(B):
    names = declared_functions()
    assert len(names) >= 11
    lib = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(B.EXPORTED) == names


def test_create_validation(B):
    ok = dict(d_model=256, n_experts=8, d_ffn=512, top_k=2, d_ffn_shared=0, max_tokens=16)
    h = B.pw_layer_create(**ok)
    B.pw_layer_destroy(h)
    bad = [dict(d_model=200), dict(d_model=0), dict(d_model=8320), dict(n_experts=0), dict(n_experts=257),
           dict(d_ffn=100), dict(top_k=0), dict(top_k=9), dict(d_ffn_shared=-128),
           dict(d_ffn_shared=100), dict(max_tokens=0), dict(max_tokens=70000)]
    for b in bad:
        with pytest.raises(B.PwError) as ei:
            B.pw_layer_create(**{**ok, **b})
        assert ei.value.status == 2, b
    with pytest.raises(B.PwError) as ei:
        B.pw_layer_create(**ok, abi_version=99)
    assert ei.value.status == 1
    for good in (B.PW_FLAG_LUT_TILED, B.PW_FLAG_DETERMINISTIC, B.PW_FLAG_LUT_TILED | B.PW_FLAG_DETERMINISTIC):
        B.pw_layer_destroy(B.pw_layer_create(**ok, flags=good))   # the defined flags
    for bad_flags in (4, 0x80000000):
        with pytest.raises(B.PwError) as ei:
            B.pw_layer_create(**ok, flags=bad_flags)
        assert ei.value.status == 1
    B.pw_layer_destroy(None)   # no-op


def test_plan_bind_forward_validation(B):
    h = B.pw_layer_create(256, 4, 512, 2, 384, 8)
    try:
        nb = 3 * 5
        with pytest.raises(B.PwError) as ei:
            B.pw_moe_plan_set(h, [3] * (nb - 1))
        assert ei.value.status == 1
        for bad in (0, 9):
            with pytest.raises(B.PwError) as ei:
                B.pw_moe_plan_set(h, [3] * (nb - 1) + [bad])
            assert ei.value.status == 3
        # forward before any plan: state error
        with pytest.raises(B.PwError) as ei:
            B.pw_moe_forward(h, 4096, 1, 4096, 0, 4096)
        assert ei.value.status == 7
        B.pw_moe_plan_set(h, [3, 4, 5] * 5)
        # fake, aligned device addresses: bind only records them
        base = 1 << 40
        planes = [base + 4096 * p for p in range(8)]
        lut = base + (1 << 20)
        with pytest.raises(B.PwError) as ei:
            B.pw_page_table_bind(h, 5, 0, planes, lut, 3)       # expert out of range
        assert ei.value.status == 1
        with pytest.raises(B.PwError) as ei:
            B.pw_page_table_bind(h, 0, 3, planes, lut, 3)       # linear out of range
        assert ei.value.status == 1
        with pytest.raises(B.PwError) as ei:
            B.pw_page_table_bind(h, 0, 0, [planes[0] + 8] + planes[1:], lut, 3)
        assert ei.value.status == 5
        with pytest.raises(B.PwError) as ei:
            B.pw_page_table_bind(h, 0, 0, planes, lut + 2, 3)
        assert ei.value.status == 5
        with pytest.raises(B.PwError) as ei:
            B.pw_page_table_bind(h, 0, 0, planes, lut, 0)
        assert ei.value.status == 3
        with pytest.raises(B.PwError) as ei:
            B.pw_page_table_bind(h, 0, 0, [planes[0], 0], lut, 3)
        assert ei.value.status == 1
        # bind everything at the planned bits except one block with too few planes
        for e in range(5):
            for lin, b in zip(range(3), (3, 4, 5)):
                B.pw_page_table_bind(h, e, lin, planes[:b], lut, b)
        B.pw_page_table_bind(h, 2, 2, planes[:4], lut, 5)
        with pytest.raises(B.PwError) as ei:
            B.pw_moe_forward(h, 4096, 1, 4096, 0, 4096)
        assert ei.value.status == 4 and "expert 2, linear 2" in B.pw_last_error()
        B.pw_page_table_bind(h, 2, 2, planes[:5], lut, 4)       # LUT bits mismatch
        with pytest.raises(B.PwError) as ei:
            B.pw_moe_forward(h, 4096, 1, 4096, 0, 4096)
        assert ei.value.status == 4
        B.pw_page_table_bind(h, 2, 2, planes[:8], lut, 5)       # extra planes are fine
        # T range, T == 0 no-op, null / misaligned activations
        with pytest.raises(B.PwError) as ei:
            B.pw_moe_forward(h, 4096, 9, 4096, 0, 4096)
        assert ei.value.status == 6
        with pytest.raises(B.PwError) as ei:
            B.pw_moe_forward(h, 4096, -1, 4096, 0, 4096)
        assert ei.value.status == 6
        B.pw_moe_forward(h, 0, 0, 0, 0, 0)
        with pytest.raises(B.PwError) as ei:
            B.pw_moe_forward(h, 0, 1, 4096, 0, 4096)
        assert ei.value.status == 1
        with pytest.raises(B.PwError) as ei:
            B.pw_moe_forward(h, 4104, 1, 4096, 0, 4096)
        assert ei.value.status == 5
        with pytest.raises(B.PwError) as ei:
            B.pw_moe_forward(h, 4096, 1, 4096, 4097, 4096)
        assert ei.value.status == 5
        # a plan that raises a bit above the bound planes is caught at the next forward
        B.pw_moe_plan_set(h, [3, 4, 6] * 5)
        with pytest.raises(B.PwError) as ei:
            B.pw_moe_forward(h, 4096, 1, 4096, 0, 4096)
        assert ei.value.status == 4
    finally:
        B.pw_layer_destroy(h)


def test_debug_hook_validation(B):
    p = [1 << 40] * 8
    with pytest.raises(B.PwError) as ei:
        B.pw_debug_unpack(p, 9, 32, 128, 1 << 41)
    assert ei.value.status == 3
    with pytest.raises(B.PwError) as ei:
        B.pw_debug_unpack(p, 3, 33, 128, 1 << 41)
    assert ei.value.status == 2
    with pytest.raises(B.PwError) as ei:
        B.pw_debug_dequant(p, 3, (1 << 40) + 2, 32, 128, 1 << 41)
    assert ei.value.status == 5
    with pytest.raises(B.PwError) as ei:
        B.pw_debug_dequant(p, 3, 1 << 40, 32, 128, 1 << 41, lut_flags=2)
    assert ei.value.status == 1


def test_status_and_replay_without_device_state(B):
    h = B.pw_layer_create(256, 8, 512, 2, 0, 16)
    try:
        assert B.pw_layer_status(h) == 0            # nothing allocated yet: flags 0
        with pytest.raises(B.PwError) as ei:
            B.pw_moe_replay(h, 1)
        assert ei.value.status == 7
        with pytest.raises(B.PwError) as ei:
            B.pw_layer_last_bytes(h)
        assert ei.value.status == 7
    finally:
        B.pw_layer_destroy(h)


def test_wait_limit_hook(B):
    with pytest.raises(B.PwError) as ei:
        B.pw_debug_set_wait_limit(0, 0)               # null layer
    assert ei.value.status == 1
    h = B.pw_layer_create(256, 8, 512, 2, 0, 16)
    try:
        B.pw_debug_set_wait_limit(h, 0)
        B.pw_debug_set_wait_limit(h, 1 << 20)
    finally:
        B.pw_layer_destroy(h)



def test_noalloc_validation(B):
    """pw_moe_forward_noalloc checks its arguments and the static scratch size before any HIP call."""
    with pytest.raises(B.PwError) as ei:
        B.pw_moe_forward_noalloc(0, 4096, 1, 4096, 0, 4096)
    assert ei.value.status == 1
    # the 24-layer qwen shape at T = 1024 needs ~58 MB of workspace: beyond the 32 MiB scratch
    h = B.pw_layer_create(2048, 60, 1408, 4, 5632, 1024)
    try:
        with pytest.raises(B.PwError) as ei:
            B.pw_moe_forward_noalloc(h, 4096, 1, 4096, 0, 4096)
        assert ei.value.status == 7                     # no plan yet
        B.pw_moe_plan_set(h, [3] * (3 * 61))
        base = 1 << 40
        for e in range(61):
            for lin in range(3):
                B.pw_page_table_bind(h, e, lin, [base + 4096 * p for p in range(3)], base + (1 << 20), 3)
        with pytest.raises(B.PwError) as ei:
            B.pw_moe_forward_noalloc(h, 4096, 1025, 4096, 0, 4096)
        assert ei.value.status == 6                     # T above max_tokens
        with pytest.raises(B.PwError) as ei:
            B.pw_moe_forward_noalloc(h, 4097, 16, 4096, 0, 4096)
        assert ei.value.status == 5                     # misaligned x
        with pytest.raises(B.PwError) as ei:
            B.pw_moe_forward_noalloc(h, 4096, 1024, 4096, 0, 4096)
        assert ei.value.status == 6 and "scratch" in str(ei.value)
        B.pw_moe_forward_noalloc(h, 4096, 0, 4096, 0, 4096)   # T = 0: a no-op
    finally:
        B.pw_layer_destroy(h)


def test_row_block_validation(B):
    ok = dict(d_model=256, n_experts=4, d_ffn=384, top_k=2, d_ffn_shared=512, max_tokens=8)
    for rb in (32, 96, 100, -64, 256):   # not a multiple of 64, not dividing every size, negative
        with pytest.raises(B.PwError) as ei:
            B.pw_layer_create(**ok, rows_per_block=rb)
        assert ei.value.status == 2, rb
    h = B.pw_layer_create(**ok, rows_per_block=128)
    try:
        # blocks: per routed expert 2*384/128 + 256/128 = 8, the shared 2*512/128 + 2 = 10
        with pytest.raises(B.PwError) as ei:
            B.pw_moe_plan_set(h, [3] * 3 * 5)
        assert ei.value.status == 1
        B.pw_moe_plan_set(h, [3] * (4 * 8 + 10))
        base = 1 << 40
        planes = [base + 4096 * p for p in range(3)]
        with pytest.raises(B.PwError) as ei:
            B.pw_page_table_bind_rows(h, 0, 0, 3, planes, base + (1 << 20), 3)   # gate has 3 row-blocks
        assert ei.value.status == 1
        B.pw_page_table_bind_rows(h, 4, 2, 1, planes, base + (1 << 20), 3)       # shared down, row-block 1
        with pytest.raises(B.PwError) as ei:
            B.pw_moe_forward(h, 4096, 1, 4096, 0, 4096)
        assert ei.value.status == 4                                                # others unbound
    finally:
        B.pw_layer_destroy(h)


def test_path_hook(B):
    """pw_debug_set_path takes the five declared paths by name or number and rejects the rest."""
    with pytest.raises(B.PwError) as ei:
        B.pw_debug_set_path(0, "auto")                # null layer
    assert ei.value.status == 1
    h = B.pw_layer_create(256, 8, 512, 2, 0, 16)
    try:
        for name, num in B.PATHS.items():
            B.pw_debug_set_path(h, name)
            B.pw_debug_set_path(h, num)
        assert sorted(B.PATHS.values()) == [0, 1, 2, 3, 4]
        for bad in (-1, 5):
            with pytest.raises(B.PwError) as ei:
                B.pw_debug_set_path(h, bad)
            assert ei.value.status == 1
    finally:
        B.pw_layer_destroy(h)
