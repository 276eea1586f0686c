"""ctypes view of libfp8q.so (the C ABI declared in include/fp8q.h).

torch is imported first on purpose: the library links libamdhip64.so.7, and
loading it after torch makes the dynamic loader reuse the HIP runtime torch
already loaded, so device pointers and streams from torch are valid in it.
There is no fallback: if the library is not built, loading raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch  # noqa: F401  (load order, see above)

PKG = os.path.dirname(os.path.abspath(__file__))
# FP8Q_LIBRARY names another build of the library to load (the test suite's
# sanitizer build of the host code uses it); the default is the in-tree build.
LIB_PATH = os.environ.get("FP8Q_LIBRARY") or os.path.join(PKG, "libfp8q.so")

FP8Q_OK = 0
FP8Q_ERR_INVALID_ARG = 1
FP8Q_ERR_UNSUPPORTED = 2
FP8Q_ERR_HIP = 3
FP8Q_ERR_WORKSPACE = 4

FP8Q_W8A16 = 0
FP8Q_W8A8 = 1
FP8Q_W8A16_F16 = 2

_lock = threading.Lock()
_lib = None

P = ctypes.c_void_p
I64 = ctypes.c_int64
SZ = ctypes.c_size_t
ST = ctypes.c_int

# name -> (restype, argtypes); mirrors include/fp8q.h
SIGNATURES = {
    "fp8q_abi_version": (ctypes.c_int, []),
    "fp8q_status_string": (ctypes.c_char_p, [ST]),
    "fp8q_last_error": (ctypes.c_char_p, []),
    "fp8q_quantize_weight": (ST, [P, I64, I64, I64, P, I64, P, P, P]),
    "fp8q_quantize_act_workspace_size": (SZ, [I64, I64]),
    "fp8q_quantize_act": (ST, [P, I64, I64, I64, P, I64, P, P, SZ, P, P]),
    "fp8q_quantize_act_static": (ST, [P, I64, I64, I64, P, P, I64, P, P]),
    "fp8q_quantize_act_ema": (ST, [P, I64, I64, I64, P, I64, P, P, ctypes.c_float,
                                   ctypes.c_float, ctypes.c_int, P, SZ, P, P]),
    "fp8q_quantize_weight_grouped": (ST, [P, I64, I64, I64, I64, P, I64, P, P, P]),
    "fp8q_linear_grouped_workspace_size": (SZ, [ST, I64, I64, I64, I64]),
    "fp8q_linear_grouped": (ST, [ST, P, I64, I64, I64, P, P, I64, I64, P, I64, P, I64, P, SZ, P]),
    "fp8q_kv_cache_workspace_size": (SZ, [I64, I64, I64]),
    "fp8q_kv_cache_write": (ST, [P, P, I64, I64, I64, I64, P, P, P, I64, P, P, ctypes.c_int, P,
                                 SZ, P, P]),
    "fp8q_linear_workspace_size": (SZ, [ST, I64, I64, I64]),
    "fp8q_linear": (ST, [ST, P, I64, I64, I64, P, P, I64, I64, P, P, I64, P, SZ, P]),
    "fp8q_cast_f32_to_e4m3": (ST, [P, I64, P, P]),
    "fp8q_linear_noalloc": (ST, [ST, P, I64, I64, I64, P, P, I64, I64, P, P, I64, P]),
    "fp8q_linear_w8a8_dynamic_workspace_size": (SZ, [I64, I64, I64]),
    "fp8q_linear_w8a8_dynamic": (ST, [P, I64, I64, I64, P, I64, I64, P, P, I64, P, P, SZ, P, P]),
    "fp8q_linear_describe": (ST, [ST, I64, I64, I64, ctypes.c_char_p, SZ]),
    "fp8q_linear_w8a8_dynamic_describe": (ST, [I64, I64, I64, ctypes.c_char_p, SZ]),
    "fp8q_linear_grouped_describe": (ST, [ST, I64, I64, I64, I64, ctypes.c_char_p, SZ]),
}


class Fp8qError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.detail = detail
        super().__init__(f"{status_string(status)}: {detail}")


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(
                        f"{LIB_PATH} is not built; run `python -m fp8_weight_quantized_amd.build`")
                handle = ctypes.CDLL(LIB_PATH)
                for name, (res, args) in SIGNATURES.items():
                    fn = getattr(handle, name)
                    fn.restype = res
                    fn.argtypes = args
                _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().fp8q_status_string(status).decode()


def last_error() -> str:
    return lib().fp8q_last_error().decode()


def check(status: int) -> None:
    if status != FP8Q_OK:
        raise Fp8qError(status, last_error())
