"""The C-ABI library loads, exports every entry point include/moe.h declares,
and its host-side checks (no GPU needed) behave as documented."""
import ctypes
import os
import re

import pytest

from moe_expert_ffn_plan_amd import binding as B
from oracle.routing import capacity_rows

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe.h")


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"MOE_API\s+[\w\s\*]*?\b(moe_\w+)\s*\(", text)))


def test_header_declares_entry_points():
    syms = declared_symbols()
    assert {"moe_plan", "moe_forward", "moe_plan_workspace_bytes", "moe_forward_workspace_bytes"} <= set(syms)


def test_library_exports_declared_symbols():
    lib = B.lib()
    for s in declared_symbols():
        assert hasattr(lib, s), s
    assert sorted(B.EXPORTS) == declared_symbols()


def test_status_strings():
    assert B.status_str(0) == "ok"
    assert B.status_str(-5) == "device is not gfx950"
    assert B.status_str(123) == "unknown status"


@pytest.mark.parametrize("T,H,I,E,k,bm", [(64, 256, 128, 8, 2, 128), (2048, 4096, 768, 64, 8, 128),
                                          (128, 7168, 2048, 32, 8, 16), (4096, 7168, 2048, 32, 8, 32),
                                          (16384, 7168, 2048, 32, 8, 128), (1, 256, 128, 1, 1, 16)])
def test_capacity_matches_oracle(T, H, I, E, k, bm):
    s = B.make_shape(T, H, I, E, k, bm)
    assert B.capacity_rows(s) == capacity_rows(T, k, E, bm)
    assert B.plan_workspace_bytes(s) > 0
    assert B.forward_workspace_bytes(s) > B.capacity_rows(s) * (H * 2 + I)


@pytest.mark.parametrize("bad,status", [
    (dict(block_m=48), -2), (dict(block_m=8), -2), (dict(num_experts=0), -2), (dict(num_experts=513), -2),
    (dict(topk=0), -2), (dict(topk=65), -2), (dict(num_tokens=-1), -2), (dict(hidden=384), -3),
    (dict(intermediate=192), -3), (dict(hidden=0), -2)])
def test_shape_validation(bad, status):
    kw = dict(num_tokens=64, hidden=256, intermediate=128, num_experts=8, topk=2, block_m=128)
    kw.update(bad)
    s = B.make_shape(**kw)
    v = ctypes.c_size_t()
    assert B.lib().moe_forward_workspace_bytes(ctypes.byref(s), ctypes.byref(v)) == status


def test_null_and_empty_inputs_return_before_gpu_work():
    lib = B.lib()
    s = B.make_shape(64, 256, 128, 8, 2, 128)
    assert lib.moe_plan(None, None, None, 0, None) == -1
    assert lib.moe_plan(ctypes.byref(s), None, None, 0, None) == -1
    assert lib.moe_forward(ctypes.byref(s), *([None] * 11), 0, None) == -1
    empty = B.make_shape(0, 256, 128, 8, 2, 128)
    assert lib.moe_plan(ctypes.byref(empty), None, None, 0, None) == 0
    assert lib.moe_forward(ctypes.byref(empty), *([None] * 11), 0, None) == 0


def test_misaligned_and_small_workspace():
    lib = B.lib()
    s = B.make_shape(64, 256, 128, 8, 2, 128)
    need = B.plan_workspace_bytes(s)
    assert lib.moe_plan(ctypes.byref(s), ctypes.c_void_p(0x1004), ctypes.c_void_p(0x10000), need, None) == -3
    assert lib.moe_plan(ctypes.byref(s), ctypes.c_void_p(0x1000), ctypes.c_void_p(0x10000), need - 1, None) == -4
