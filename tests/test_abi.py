"""The C ABI: the library loads and exports every symbol include/moe.h declares.

CPU-only checks (no kernel is launched): symbol table against the header,
status strings, and a clean error from moe_create when no GPU is visible.
"""
import ctypes
import os
import re

import pytest

from sparse_moe_expert_sigmoid_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(moe_[a-z_]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for f in ("moe_route", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_create",
              "moe_destroy", "moe_last_error", "moe_workspace_size", "moe_status_string"):
        assert f in names
    assert set(names) == set(binding.EXPORTS)


def test_library_exports_every_declared_symbol():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libmoe_mi355x.so is not built (python -m sparse_moe_expert_sigmoid_amd.build)")
    lib = ctypes.CDLL(binding.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    lib = binding.load_library()
    for st, name in enumerate(["MOE_OK", "MOE_E_INVALID", "MOE_E_UNSUPPORTED", "MOE_E_DEVICE",
                               "MOE_E_WORKSPACE"]):
        assert lib.moe_status_string(st).decode() == name


def test_null_context_is_rejected_without_touching_a_device():
    lib = binding.load_library()
    n = ctypes.c_size_t()
    assert lib.moe_workspace_size(None, 8, 8, 256, 2304, 2048, 1, ctypes.byref(n)) == \
        binding.MOE_E_INVALID
    assert lib.moe_route(None, 0, None, None, None, 8, 2304, 256, 8, 2.446, None, None, None, 0,
                         None) == binding.MOE_E_INVALID
    assert lib.moe_combine(None, None, None, None, None, None, 1, 8, 64, None, None) == \
        binding.MOE_E_INVALID


def test_create_reports_missing_device_cleanly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible; covered by the GPU tests")
    lib = binding.load_library()
    h = ctypes.c_void_p()
    st = lib.moe_create(0, ctypes.byref(h))
    assert st in (binding.MOE_E_DEVICE, binding.MOE_E_UNSUPPORTED)
    assert h.value is None
    assert len(lib.moe_last_error(None).decode()) > 0
