"""ctypes loader for libcpattn.so (the C ABI declared in include/cpattn.h).

Loading fails loudly if the library has not been built: there is no
fallback implementation of any entry point.
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libcpattn.so")

# enum values of include/cpattn.h
OK, E_NULL, E_SHAPE, E_DTYPE, E_HEADDIM, E_ALIGN, E_ALIAS, E_HIP, E_SCALE, E_FLAGS = range(10)
BF16, F32, F16, E4M3 = 0, 1, 2, 3
SEQ_TO_HEAD, HEAD_TO_SEQ = 0, 1
ABI_VERSION = 4
STATIC_SCRATCH_BYTES = 32 << 20     # CPATTN_STATIC_SCRATCH_BYTES
SCHED_BYTES = 2048                  # CPATTN_WORKSPACE_COUNTER_BYTES
FLAG_ACCUMULATE = 1
FLAG_SEQ_MAJOR = 2
FLAG_K_SEQ_LAST = 4

STATUS_NAMES = {OK: "OK", E_NULL: "E_NULL", E_SHAPE: "E_SHAPE", E_DTYPE: "E_DTYPE", E_HEADDIM: "E_HEADDIM",
                E_ALIGN: "E_ALIGN", E_ALIAS: "E_ALIAS", E_HIP: "E_HIP", E_SCALE: "E_SCALE",
                E_FLAGS: "E_FLAGS"}

# (name, restype, argtypes) of every exported function
_P, _I64, _F, _E = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
_U32, _U64 = ctypes.c_uint32, ctypes.c_uint64
_PI64, _PU64 = ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_uint64)
_PP = ctypes.POINTER(ctypes.c_void_p)
SIGNATURES = [
    ("cpattn_attn_fwd", _E, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _F, _E, _E, _P]),
    ("cpattn_attn_fwd_ex", _E, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _F, _E, _E, _U32, _P, _U64, _P]),
    ("cpattn_attn_fwd_ex_static", _E, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _F, _E, _E, _U32, _U64, _P]),
    ("cpattn_attn_fwd_fp8", _E, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _F, _F, _F, _F, _E, _U32, _P, _U64,
                                 _P]),
    ("cpattn_attn_fwd_workspace_size", _E, [_I64, _I64, _I64, _I64, _I64, _E, _E, _PU64]),
    ("cpattn_attn_fwd_split_plan", _E, [_I64, _I64, _I64, _I64, _I64, _I64, _U64, _PI64, _PI64, _PU64]),
    ("cpattn_attn_merge", _E, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _E, _P]),
    ("cpattn_ring_attn_fwd", _E, [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _F, _P]),
    ("cpattn_qk_rmsnorm", _E, [_P, _P, _P, _I64, _I64, _F, _F, _E, _P]),
    ("cpattn_ulysses_pack", _E, [_P, _P, _I64, _I64, _I64, _I64, _I64, _E, _E, _P]),
    ("cpattn_ulysses_unpack", _E, [_P, _P, _I64, _I64, _I64, _I64, _I64, _E, _E, _P]),
    ("cpattn_ulysses_pack_n", _E, [_PP, _PP, _I64, _I64, _I64, _I64, _I64, _I64, _E, _E, _P]),
    ("cpattn_ulysses_unpack_n", _E, [_PP, _PP, _I64, _I64, _I64, _I64, _I64, _I64, _E, _E, _P]),
    ("cpattn_status_string", ctypes.c_char_p, [_E]),
    ("cpattn_abi_version", ctypes.c_int, []),
]

_lib = None


class CpattnError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed: {STATUS_NAMES.get(status, status)} ({message})")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library with argument types set (loaded once per process)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m long_sequence_bidirectional_amd.build` "
                "(there is no fallback implementation)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            f = getattr(handle, name)
            f.restype = res
            f.argtypes = args
        if handle.cpattn_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH}: ABI version {handle.cpattn_abi_version()} != {ABI_VERSION}")
        _lib = handle
    return _lib


def check(fn: str, status: int) -> None:
    if status != OK:
        raise CpattnError(fn, status, lib().cpattn_status_string(status).decode())
