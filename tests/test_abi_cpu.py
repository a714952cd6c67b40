"""The C-ABI library loads, exports every symbol include/gqa.h declares, and
returns each validation error before touching a device (CPU only)."""

import ctypes
import os
import subprocess

import pytest

from gqa_attention_forward_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_loads_and_exports_header_symbols():
    lib = _lib.load()
    names = _lib.header_functions()
    assert set(names) == set(_lib.SIGNATURES), names
    for name in names:
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, f"{name} has no ctypes signature"
    assert lib.gqa_abi_version() == _lib.ABI_VERSION == 2


def test_workspace_size_matches_layout():
    ws = ctypes.c_size_t()
    lib = _lib.load()
    assert lib.gqa_attention_workspace_size(16, 32, 1, 8192, 128, 1024, ctypes.byref(ws)) == 0
    assert ws.value == 16 * 32 * 1 * 8 * (128 + 2) * 4
    assert lib.gqa_attention_workspace_size(2, 3, 5, 100, 64, 64, ctypes.byref(ws)) == 0
    assert ws.value == -(-(2 * 3 * 5 * 2 * 66 * 4) // 256) * 256
    assert lib.gqa_attention_workspace_size(1, 1, 1, 1, 64, 0, ctypes.byref(ws)) == 0
    assert ws.value == 0


def test_pure_c_validation_paths(tmp_path):
    exe = tmp_path / "abi_check"
    lib_dir = os.path.dirname(_lib.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-O1", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_check.c"), "-L", lib_dir, "-lgqa",
           f"-Wl,-rpath,{lib_dir}", "-lm", "-o", str(exe)]
    subprocess.run(cmd, check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "ALL OK" in res.stdout


def test_python_errors_map_to_exceptions():
    lib = _lib.load()
    s = _lib.strides3([4096, 1024, 64])
    st = lib.gqa_attention_prefill(None, s, None, s, None, s, None, s, 1, 4, 1, 16, 128, 64,
                                   None, 0.125, None, 0, 0, None, 0, None)
    assert st == _lib.GQA_ERR_INVALID_ARGUMENT
    with pytest.raises(ValueError):
        _lib.check(st)
    p = ctypes.c_void_p(0x10000)
    st = lib.gqa_attention_prefill(p, s, p, s, p, s, p, s, 1, 4, 1, 16, 128, 96,
                                   None, 0.125, None, 0, 0, None, 0, None)
    with pytest.raises(NotImplementedError):
        _lib.check(st)
    assert "head dim" in lib.gqa_last_error().decode()


def test_decode_tile_rule():
    """About one (b, kv head, split) unit per compute unit (256 on MI355X; the
    same fallback where no device answers), powers of two from 128 to 8192."""
    import gqa_attention_forward_amd as gqa
    assert gqa.decode_tile(1, 8, 1024) == 128
    assert gqa.decode_tile(1, 8, 4096) == 128
    assert gqa.decode_tile(1, 8, 16384) == 512
    assert gqa.decode_tile(1, 8, 32768) == 1024
    assert gqa.decode_tile(4, 8, 4096) == 512
    assert gqa.decode_tile(4, 8, 32768) == 4096
    assert gqa.decode_tile(1, 8, 0) == 128
    assert gqa.decode_tile(64, 8, 1 << 20) == 8192
    with pytest.raises(ValueError):
        gqa.decode_tile(0, 8, 1024)
