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
                path=0, device=0, block=32, flags=0, routed_scale=1.0, reserved=0, w_router=0x10000, router_bias=None, gate_codes=0x20000, gate_scales=0x30000,
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
    (dict(abi_version=1), _lib.MOE_ERR_UNSUPPORTED),
    (dict(block=16), _lib.MOE_ERR_INVALID),
    (dict(reserved=1), _lib.MOE_ERR_INVALID),
    (dict(routed_scale=0.0), _lib.MOE_ERR_INVALID),
    (dict(routed_scale=float("nan")), _lib.MOE_ERR_INVALID),
    (dict(routed_scale=float("inf")), _lib.MOE_ERR_INVALID),
    (dict(flags=2), _lib.MOE_ERR_INVALID),
    (dict(flags=1), _lib.MOE_ERR_INVALID),                               # FP8 pointers missing
    (dict(flags=1, n_shared=0, shared_gate_fp8=0x80000, shared_gate_fp8_scales=0x90000, shared_up_fp8=0xa0000,
          shared_up_fp8_scales=0xb0000, shared_down_fp8=0xc0000, shared_down_fp8_scales=0xd0000),
     _lib.MOE_ERR_INVALID),                                              # FP8 shared with S = 0
    (dict(flags=1, inter=96, shared_gate_fp8=0x80000, shared_gate_fp8_scales=0x90000, shared_up_fp8=0xa0000,
          shared_up_fp8_scales=0xb0000, shared_down_fp8=0xc0000, shared_down_fp8_scales=0xd0000),
     _lib.MOE_ERR_INVALID),                                              # I not a multiple of 128
    (dict(shared_up_fp8=0xa0000), _lib.MOE_ERR_INVALID),                 # FP8 pointer without the flag
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
    assert lib.moe_forward_noalloc(None, None, 4, None, None, None) == _lib.MOE_ERR_INVALID
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


# ---- test hooks and the sanitized host build ---------------------------------------------


def _fake_desc(**kw):
    return _desc(hidden=4096, n_experts=256, top_k=6, n_shared=1, inter=2048, **kw)


def test_fake_arch_hook_creates_layers_without_a_gpu(lib, monkeypatch):
    monkeypatch.setenv("MOE_FAKE_ARCH", "gfx950")
    buf = ctypes.create_string_buffer(64)
    assert lib.moe_device_supported(0, buf, 64) == 1 and buf.value == b"gfx950"
    out = ctypes.c_void_p()
    desc = _fake_desc()
    assert lib.moe_layer_create(ctypes.byref(desc), ctypes.byref(out)) == _lib.MOE_OK
    try:
        ws = [lib.moe_workspace_bytes(out, t) for t in (1, 8, 512, 4096)]
        assert all(w % 256 == 0 for w in ws) and ws == sorted(ws)
        # the no-allocation entry point's limit at these dims, and its rejection (no launch)
        assert lib.moe_workspace_bytes(out, 340) <= _lib.MOE_NOALLOC_SCRATCH_BYTES
        assert lib.moe_workspace_bytes(out, 341) > _lib.MOE_NOALLOC_SCRATCH_BYTES
        assert lib.moe_forward_noalloc(out, 0x100000, 341, 0x200000, None, None) == _lib.MOE_ERR_WORKSPACE
        assert b"scratch" in lib.moe_last_error()
    finally:
        lib.moe_layer_destroy(out)
    monkeypatch.setenv("MOE_FAKE_ARCH", "gfx942")
    assert lib.moe_layer_create(ctypes.byref(desc), ctypes.byref(out)) == _lib.MOE_ERR_UNSUPPORTED
    assert b"gfx942" in lib.moe_last_error()


def test_fail_alloc_hook(lib, monkeypatch):
    monkeypatch.setenv("MOE_FAKE_ARCH", "gfx950")
    monkeypatch.setenv("MOE_FAIL_ALLOC", "1")
    out = ctypes.c_void_p(1234)
    desc = _fake_desc()
    assert lib.moe_layer_create(ctypes.byref(desc), ctypes.byref(out)) == _lib.MOE_ERR_ALLOC
    assert out.value is None


def test_host_abi_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    """The library's host code (api.hip) built with ASan + UBSan on its host pass only, linked
    with a C++ driver (abi_host_check.cpp) that walks the ABI's host paths on the CPU; leaks are
    checked at exit."""
    import shutil
    import subprocess
    from fp4_routed_expert_moe_amd import build
    llvm = "/opt/rocm/llvm/bin/clang++"
    if not os.path.exists(llvm):
        pytest.skip("ROCm clang++ not found")
    objs = [os.path.join(build.BUILD_DIR, s.replace(".hip", ".o")) for s in build.SOURCES if s != "api.hip"]
    if not all(os.path.exists(o) for o in objs):
        build.build()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    api_o, drv_o, exe = tmp_path / "api.o", tmp_path / "drv.o", tmp_path / "abi_host_check"
    flags = [f for f in build.HIP_FLAGS if f != "-O3"] + ["-O1", "-g"]
    build._run([build.hipcc(), *flags, *san, "-c", os.path.join(build.CSRC, "api.hip"), "-o", str(api_o)])
    host_san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
    build._run([llvm, "-O1", "-g", *host_san, "-I", build.INCLUDE, "-c",
                os.path.join(ROOT, "tests", "abi_host_check.cpp"), "-o", str(drv_o)])
    rocm_lib = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(build.hipcc()))), "lib")
    build._run([llvm, *host_san, str(drv_o), str(api_o), *objs, "-L", rocm_lib, "-lamdhip64",
                f"-Wl,-rpath,{rocm_lib}", "-o", str(exe)])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("MOE_FAKE_ARCH", None)
    env.pop("MOE_FAIL_ALLOC", None)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi host checks: ok" in r.stdout
    shutil.rmtree(tmp_path, ignore_errors=True)
