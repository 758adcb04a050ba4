"""Host-side checks of the C ABI: the library loads, exports what include/moe.h declares, and
rejects bad arguments with status codes (no GPU needed: nothing here launches a kernel)."""
import ctypes
import os
import re

import pytest

from fp4_routed_expert_moe_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from fp4_routed_expert_moe_amd import build
        build.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_abi():
    names = declared_functions()
    for must in ("moe_layer_create", "moe_route", "moe_forward", "moe_layer_destroy", "moe_workspace_bytes"):
        assert must in names
    assert set(names) == set(_lib.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.moe_abi_version() == _lib.MOE_ABI_VERSION


def test_status_strings(lib):
    for code in range(6):
        assert lib.moe_status_string(code)
    assert lib.moe_status_string(_lib.MOE_OK) == b"ok"
    assert lib.moe_status_string(99) == b"unknown status"


def _desc(**kw):
    base = dict(abi_version=_lib.MOE_ABI_VERSION, hidden=256, n_experts=8, top_k=2, n_shared=1, inter=128,
                path=0, device=0, w_router=0x10000, router_bias=None, gate_codes=0x20000, gate_scales=0x30000,
                up_codes=0x40000, up_scales=0x50000, down_codes=0x60000, down_scales=0x70000)
    base.update(kw)
    return _lib.LayerDesc(**base)


@pytest.mark.parametrize("bad,status", [
    (dict(hidden=100), _lib.MOE_ERR_INVALID),
    (dict(hidden=16), _lib.MOE_ERR_INVALID),
    (dict(hidden=16384), _lib.MOE_ERR_INVALID),
    (dict(inter=48), _lib.MOE_ERR_INVALID),
    (dict(n_experts=0), _lib.MOE_ERR_INVALID),
    (dict(n_experts=2000), _lib.MOE_ERR_INVALID),
    (dict(top_k=0), _lib.MOE_ERR_INVALID),
    (dict(top_k=9), _lib.MOE_ERR_INVALID),
    (dict(n_shared=2), _lib.MOE_ERR_INVALID),
    (dict(path=7), _lib.MOE_ERR_INVALID),
    (dict(gate_codes=None), _lib.MOE_ERR_INVALID),
    (dict(down_codes=0x60004), _lib.MOE_ERR_INVALID),
    (dict(abi_version=99), _lib.MOE_ERR_UNSUPPORTED),
])
def test_create_rejects_bad_descriptors(lib, bad, status):
    out = ctypes.c_void_p(1234)
    desc = _desc(**bad)
    assert lib.moe_layer_create(ctypes.byref(desc), ctypes.byref(out)) == status
    assert out.value is None
    assert lib.moe_last_error()


def test_create_null_arguments(lib):
    out = ctypes.c_void_p()
    assert lib.moe_layer_create(None, ctypes.byref(out)) == _lib.MOE_ERR_INVALID
    desc = _desc()
    assert lib.moe_layer_create(ctypes.byref(desc), None) == _lib.MOE_ERR_INVALID


def test_calls_on_null_layer(lib):
    assert lib.moe_workspace_bytes(None, 8) == 0
    assert lib.moe_forward(None, None, 0, None, None, None, 0, None) == _lib.MOE_ERR_INVALID
    assert lib.moe_route(None, None, 4, None, None, 0, None) == _lib.MOE_ERR_INVALID
    assert b"NULL layer" in lib.moe_last_error()
    lib.moe_layer_destroy(None)


def test_no_device_is_unsupported_here(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; covered by the GPU tests")
    buf = ctypes.create_string_buffer(64)
    assert lib.moe_device_supported(0, buf, 64) == 0
    out = ctypes.c_void_p()
    desc = _desc()
    assert lib.moe_layer_create(ctypes.byref(desc), ctypes.byref(out)) == _lib.MOE_ERR_UNSUPPORTED
    assert out.value is None


def test_timing_api_without_launches(lib):
    lib.moe_timing_reset()
    lib.moe_timing_enable(1)
    assert lib.moe_timing_read(None, None, None, 0) == 0
    lib.moe_timing_enable(0)
