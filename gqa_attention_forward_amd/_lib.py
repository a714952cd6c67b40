"""ctypes loader for libgqa.so (built in-tree next to this file).

Argument marshalling only: the library does every step of the computation.
A missing or unloadable library is an error, never a fallback.
"""

from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgqa.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "gqa.h")

GQA_OK = 0
GQA_ERR_INVALID_ARGUMENT = 1
GQA_ERR_UNSUPPORTED = 2
GQA_ERR_WORKSPACE = 3
GQA_ERR_HIP = 4
NOALLOC_SCRATCH_BYTES = 8 << 20  # GQA_NOALLOC_SCRATCH_BYTES


class GQAError(RuntimeError):
    """A libgqa call returned a status other than GQA_OK."""

    def __init__(self, status: int, message: str):
        super().__init__(f"libgqa status {status}: {message}")
        self.status = status


class GQAInvalidArgument(GQAError, ValueError):
    pass


class GQAUnsupported(GQAError, NotImplementedError):
    pass


class GQAWorkspaceError(GQAError, ValueError):
    pass


_EXC = {
    GQA_ERR_INVALID_ARGUMENT: GQAInvalidArgument,
    GQA_ERR_UNSUPPORTED: GQAUnsupported,
    GQA_ERR_WORKSPACE: GQAWorkspaceError,
}

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F = ctypes.c_float
_STR3 = ctypes.POINTER(ctypes.c_int64)

# name -> argtypes (order as in include/gqa.h)
SIGNATURES = {
    "gqa_abi_version": [],
    "gqa_last_error": [],
    "gqa_attention_workspace_size": [_I64, _I64, _I64, _I64, _I64, _I32,
                                     ctypes.POINTER(ctypes.c_size_t)],
    "gqa_attention_prefill": [_P, _STR3, _P, _STR3, _P, _STR3, _P, _STR3,
                              _I32, _I32, _I32, _I32, _I32, _I32, _P, _F, _P, _I32, _I32,
                              _P, ctypes.c_size_t, _P],
    "gqa_attention_decode_splitkv": [_P, _STR3, _P, _STR3, _P, _STR3, _P, _STR3,
                                     _I32, _I32, _I32, _I32, _I32, _P, _F, _P, _I32,
                                     _P, ctypes.c_size_t, _P],
    "gqa_attention_decode_tile": [_I32, _I32, _I32, ctypes.POINTER(ctypes.c_int32)],
    "gqa_attention_decode_splitkv_fused": [_P, _STR3, _P, _STR3, _P, _STR3, _P, _STR3,
                                           _I32, _I32, _I32, _I32, _I32, _P, _F, _P, _I32,
                                           _P, ctypes.c_size_t, _P, _I64, _P],
    "gqa_attention_decode_splitkv_noalloc": [_P, _STR3, _P, _STR3, _P, _STR3, _P, _STR3,
                                             _I32, _I32, _I32, _I32, _I32, _P, _F, _P, _I32, _P],
    "gqa_attention_splitkv_partial": [_P, _STR3, _P, _STR3, _P, _STR3,
                                      _I32, _I32, _I32, _I32, _I32, _I32, _P, _F, _I32, _I32,
                                      _P, ctypes.c_size_t, _P],
    "gqa_attention_splitkv_merge": [_P, ctypes.c_size_t, _P, _STR3, _I32, _I32, _I32, _I32,
                                    _I32, _P, _P],
    "gqa_attention_paged": [_P, _I64, _I64, _P, _P, _P, _I64, _I64, _I64, _P, _I32, _P,
                            _P, _I64, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _F, _P,
                            _I32, _I32, _P, ctypes.c_size_t, _P],
    "gqa_attention_paged_append": [_P, _I64, _I64, _P, _P, _P, _I64, _I64, _I64, _P, _I32, _P,
                                   _P, _P, _I64, _I64,
                                   _P, _I64, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                   _F, _P, _I32, _I32, _P, ctypes.c_size_t, _P],
}

ABI_VERSION = 2

_lib = None


def header_functions(path: str = HEADER_PATH) -> list[str]:
    """Names of the functions include/gqa.h declares."""
    text = open(path).read()
    return sorted(set(re.findall(r"\b(gqa_[a-z0-9_]+)\s*\(", text)))


def load() -> ctypes.CDLL:
    """Load libgqa.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with "
            "`python -c 'import __graft_entry__ as g; g.build()'` from the repository root")
    lib = ctypes.CDLL(LIB_PATH)
    for name, argtypes in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = ctypes.c_int32
    lib.gqa_last_error.restype = ctypes.c_char_p
    if lib.gqa_abi_version() != ABI_VERSION:
        raise RuntimeError(f"libgqa ABI version {lib.gqa_abi_version()} != {ABI_VERSION}")
    _lib = lib
    return lib


def check(status: int) -> None:
    if status == GQA_OK:
        return
    msg = load().gqa_last_error().decode(errors="replace")
    raise _EXC.get(status, GQAError)(status, msg)


_I64x3 = ctypes.c_int64 * 3


def strides3(values) -> ctypes.Array:
    return _I64x3(int(values[0]), int(values[1]), int(values[2]))
