"""CPU oracle for the FP8 weight-quantized linear path -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product (the HIP library under
``fp8_weight_quantized_amd/`` and its binding) never imports it, and the two
share no code: the only thing both sides consume is the seeded synthetic
input from ``workloads.py``.

The arithmetic lives in ``fp8q_oracle.c`` (plain C, fp64 GEMM, IEEE fp32
division, table-search E4M3 cast); this module only marshals numpy arrays.
Each function names the passage of the pages it follows in the C source.

Functions whose result has no independent pin would be listed here as
"parity unpinned"; every function below is pinned by tests/test_oracle_*.py.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8q_oracle.c")

# -fno-fast-math / -ffp-contract=off keep every fp32 division IEEE and every
# multiply-add unfused, which the bit-exact codes depend on.
CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
          "-fPIC", "-shared", "-Wall", "-Wextra"]
# ORACLE_SANITIZE=1 (the test suite's sanitizer run, with libasan preloaded)
# builds and loads a copy with AddressSanitizer + UndefinedBehaviorSanitizer.
SANITIZE = os.environ.get("ORACLE_SANITIZE") == "1"
if SANITIZE:
    CFLAGS = CFLAGS + ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                       "-fno-omit-frame-pointer", "-g"]
_LIB = os.path.join(_HERE, "liboracle_sanitize.so" if SANITIZE else "liboracle.so")

_lock = threading.Lock()
_lib = None

MODE_W8A16 = 0
MODE_W8A8 = 1
MODE_W8A16_F16 = 2


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (the checker, not the product)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            I64 = ctypes.c_int64
            lib.oracle_abi_version.restype = ctypes.c_int
            lib.oracle_e4m3_value.restype = ctypes.c_double
            lib.oracle_e4m3_value.argtypes = [ctypes.c_uint]
            lib.oracle_f16_value.restype = ctypes.c_double
            lib.oracle_f16_value.argtypes = [ctypes.c_uint]
            lib.oracle_e4m3_table.argtypes = [P]
            lib.oracle_cast_e4m3.restype = ctypes.c_uint
            lib.oracle_cast_e4m3.argtypes = [ctypes.c_float]
            lib.oracle_cast_e4m3_scan.restype = ctypes.c_uint
            lib.oracle_cast_e4m3_scan.argtypes = [ctypes.c_float]
            lib.oracle_cast_e4m3_array.argtypes = [P, I64, P]
            lib.oracle_cast_e4m3_bits.argtypes = [ctypes.c_uint32, I64, P]
            lib.oracle_scale_from_amax.restype = ctypes.c_float
            lib.oracle_scale_from_amax.argtypes = [ctypes.c_float]
            lib.oracle_quantize_weight.restype = ctypes.c_int
            lib.oracle_quantize_weight.argtypes = [P, I64, I64, I64, P, I64, P]
            lib.oracle_quantize_act.restype = ctypes.c_int
            lib.oracle_quantize_act.argtypes = [P, I64, I64, I64, P, I64, P]
            lib.oracle_quantize_act_static.restype = ctypes.c_int
            lib.oracle_quantize_act_static.argtypes = [P, I64, I64, I64, ctypes.c_float, P, I64]
            lib.oracle_ema_scale.restype = ctypes.c_float
            lib.oracle_ema_scale.argtypes = [ctypes.c_float] * 4
            lib.oracle_quantize_act_ema.restype = ctypes.c_int
            lib.oracle_quantize_act_ema.argtypes = [P, I64, I64, I64, P, I64, P, ctypes.c_float,
                                                    ctypes.c_float, ctypes.c_int, P]
            lib.oracle_kv_cache_write.restype = ctypes.c_int
            lib.oracle_kv_cache_write.argtypes = [P, P, I64, I64, I64, I64, P, P, P, I64, P, P,
                                                  ctypes.c_int]
            lib.oracle_quantize_weight_grouped.restype = ctypes.c_int
            lib.oracle_quantize_weight_grouped.argtypes = [P, I64, I64, I64, I64, P, I64, P]
            lib.oracle_linear_grouped.restype = None
            lib.oracle_linear_grouped.argtypes = [ctypes.c_int, P, I64, I64, I64, ctypes.c_float,
                                                  P, I64, I64, P, I64, P, I64, P]
            lib.oracle_linear.restype = None
            lib.oracle_linear.argtypes = [ctypes.c_int, P, I64, I64, I64, ctypes.c_float,
                                          P, I64, I64, P, P, I64, P]
            _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _need(a: np.ndarray, dtype, name: str) -> np.ndarray:
    if a.dtype != dtype:
        raise TypeError(f"{name}: expected {np.dtype(dtype)}, got {a.dtype}")
    if a.ndim == 2 and a.size and a.strides[1] != a.itemsize:
        raise ValueError(f"{name}: last dimension must be contiguous")
    return a


def _ld(a: np.ndarray) -> int:
    return a.strides[0] // a.itemsize if a.shape[0] > 1 else a.shape[1]


# ---------------------------------------------------------------- format ----
def e4m3_table() -> np.ndarray:
    """Decoded value of each of the 256 E4M3 codes (NaN for 0x7F, 0xFF)."""
    out = np.empty(256, np.float64)
    _load().oracle_e4m3_table(_ptr(out))
    return out


def e4m3_value(code: int) -> float:
    return _load().oracle_e4m3_value(int(code))


def cast_e4m3(t: float) -> int:
    """RNE, saturating fp32 -> E4M3 code by table search."""
    return _load().oracle_cast_e4m3(float(np.float32(t)))


def cast_e4m3_scan(t: float) -> int:
    """The same cast by linear arg-min scan (independent route)."""
    return _load().oracle_cast_e4m3_scan(float(np.float32(t)))


def cast_e4m3_array(t: np.ndarray) -> np.ndarray:
    t = np.ascontiguousarray(t, dtype=np.float32)
    out = np.empty(t.shape, np.uint8)
    _load().oracle_cast_e4m3_array(_ptr(t), t.size, _ptr(out))
    return out


def cast_e4m3_bits(first: int, count: int) -> np.ndarray:
    """Codes for the fp32 bit patterns first .. first+count-1."""
    out = np.empty(count, np.uint8)
    _load().oracle_cast_e4m3_bits(ctypes.c_uint32(first), count, _ptr(out))
    return out


def scale_from_amax(amax: float) -> np.float32:
    return np.float32(_load().oracle_scale_from_amax(float(np.float32(amax))))


# ---------------------------------------------------------- quantization ----
def quantize_weight(w_bf16: np.ndarray):
    """bf16 bits uint16 [N, K] -> (codes uint8 [N, K], scale float32 [N], nonfinite)."""
    _need(w_bf16, np.uint16, "w_bf16")
    n, k = w_bf16.shape
    q = np.empty((n, k), np.uint8)
    s = np.empty(n, np.float32)
    nf = _load().oracle_quantize_weight(_ptr(w_bf16), n, k, _ld(w_bf16), _ptr(q), k, _ptr(s))
    return q, s, bool(nf)


def quantize_weight_grouped(w_bf16: np.ndarray, group: int):
    """bf16 bits [N, K] -> (codes uint8 [N, K], scale float32 [N, ceil(K/group)], nonfinite)."""
    _need(w_bf16, np.uint16, "w_bf16")
    if group < 1:
        raise ValueError("group must be >= 1")
    n, k = w_bf16.shape
    q = np.empty((n, k), np.uint8)
    s = np.empty((n, -(-k // group)), np.float32)
    nf = _load().oracle_quantize_weight_grouped(_ptr(w_bf16), n, k, _ld(w_bf16), group, _ptr(q),
                                                k, _ptr(s))
    return q, s, bool(nf)


def quantize_act(x_bf16: np.ndarray):
    """bf16 bits uint16 [M, K] -> (codes uint8 [M, K], scale float32, nonfinite)."""
    _need(x_bf16, np.uint16, "x_bf16")
    m, k = x_bf16.shape
    q = np.empty((m, k), np.uint8)
    s = np.empty(1, np.float32)
    nf = _load().oracle_quantize_act(_ptr(x_bf16), m, k, _ld(x_bf16), _ptr(q), k, _ptr(s))
    return q, np.float32(s[0]), bool(nf)


def quantize_act_static(x_bf16: np.ndarray, scale: float):
    """bf16 bits [M, K] and a given fp32 scale -> (codes uint8 [M, K], nonfinite)."""
    _need(x_bf16, np.uint16, "x_bf16")
    m, k = x_bf16.shape
    q = np.empty((m, k), np.uint8)
    nf = _load().oracle_quantize_act_static(_ptr(x_bf16), m, k, _ld(x_bf16),
                                            float(np.float32(scale)), _ptr(q), k)
    return q, bool(nf)


def ema_scale(s_old: float, s_new: float, decay: float, temperature: float = 0.0) -> np.float32:
    """One EMA step of the activation scale, in fp32."""
    f = lambda v: float(np.float32(v))
    return np.float32(_load().oracle_ema_scale(f(s_old), f(s_new), f(decay), f(temperature)))


def quantize_act_ema(x_bf16: np.ndarray, state: float, decay: float, temperature: float = 0.0,
                     seed: bool = False):
    """One EMA-scaled quantization call.

    Returns (codes uint8 [M, K], scale_used float32, new_state float32, nonfinite).
    With seed=True the call is the dynamic quantization and `state` is ignored.
    """
    _need(x_bf16, np.uint16, "x_bf16")
    m, k = x_bf16.shape
    q = np.empty((m, k), np.uint8)
    st = np.array([state], np.float32)
    used = np.empty(1, np.float32)
    nf = _load().oracle_quantize_act_ema(_ptr(x_bf16), m, k, _ld(x_bf16), _ptr(q), k, _ptr(st),
                                         float(np.float32(decay)), float(np.float32(temperature)),
                                         1 if seed else 0, _ptr(used))
    return q, np.float32(used[0]), np.float32(st[0]), bool(nf)


def kv_cache_write(k_bf16: np.ndarray, v_bf16: np.ndarray, heads: int, slot: np.ndarray,
                   k_cache: np.ndarray, v_cache: np.ndarray, running, calibrate: bool):
    """Write new K/V tokens ([T, heads*head_dim] bf16 bits) into the E4M3 caches
    ([heads, S, head_dim] uint8, updated in place) at rows `slot` (int64 [T]).

    Returns (running float32 [2], scales float32 [2], flags int)."""
    _need(k_bf16, np.uint16, "k")
    _need(v_bf16, np.uint16, "v")
    t, width = k_bf16.shape
    if v_bf16.shape != (t, width) or width % heads:
        raise ValueError("shape mismatch")
    hd = width // heads
    for c in (k_cache, v_cache):
        if c.dtype != np.uint8 or c.ndim != 3 or c.shape[0] != heads or c.shape[2] != hd \
                or not c.flags.c_contiguous:
            raise ValueError("caches must be contiguous uint8 [heads, S, head_dim]")
    if _ld(k_bf16) != _ld(v_bf16):
        raise ValueError("k and v must share a row stride")
    slot = np.ascontiguousarray(slot, dtype=np.int64)
    run = np.array(running, np.float32).reshape(2).copy()
    sc = np.empty(2, np.float32)
    fl = _load().oracle_kv_cache_write(_ptr(k_bf16), _ptr(v_bf16), t, heads, hd, _ld(k_bf16),
                                       _ptr(slot), _ptr(k_cache), _ptr(v_cache), k_cache.shape[1],
                                       _ptr(run), _ptr(sc), 1 if calibrate else 0)
    return run, sc, int(fl)


# ---------------------------------------------------------------- linear ----
def linear_grouped(mode: int, x: np.ndarray, wq: np.ndarray, w_scale: np.ndarray, group: int,
                   x_scale: float | None = None, rows: np.ndarray | None = None) -> np.ndarray:
    """fp64 Y = X . dequant(Wq)^T with per-group weight scales [N, ceil(K/group)]."""
    if mode in (MODE_W8A16, MODE_W8A16_F16):
        _need(x, np.uint16, "x")
        if x_scale is not None:
            raise ValueError("the 16-bit activation modes take no activation scale")
        xs = 0.0
    elif mode == MODE_W8A8:
        _need(x, np.uint8, "x")
        if x_scale is None:
            raise ValueError("fp8_w_fp8_a needs the activation scale")
        xs = float(np.float32(x_scale))
    else:
        raise ValueError("unknown mode")
    _need(wq, np.uint8, "wq")
    m, k = x.shape
    n, k2 = wq.shape
    w_scale = np.ascontiguousarray(w_scale, dtype=np.float32)
    if k2 != k or group < 1 or w_scale.shape != (n, -(-k // group)):
        raise ValueError("shape mismatch")
    if rows is None:
        nrows, rp = m, None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        if rows.size and (rows.min() < 0 or rows.max() >= m):
            raise IndexError("row index out of range")
        nrows, rp = rows.size, _ptr(rows)
    y = np.empty((nrows, n), np.float64)
    if nrows and n:
        _load().oracle_linear_grouped(mode, _ptr(x), m, k, _ld(x), xs, _ptr(wq), n, _ld(wq),
                                      _ptr(w_scale), group, rp, nrows, _ptr(y))
    return y


def f16_value(bits: int) -> float:
    """IEEE binary16 value of a 16-bit pattern, decoded from its bit fields."""
    return _load().oracle_f16_value(int(bits) & 0xFFFF)


def linear(mode: int, x: np.ndarray, wq: np.ndarray, w_scale: np.ndarray,
           x_scale: float | None = None, rows: np.ndarray | None = None) -> np.ndarray:
    """fp64 Y = X . dequant(Wq)^T for the selected rows of X.

    mode 0 (fp8_w_bf16_a): x is bf16 bits uint16 [M, K], x_scale must be None.
    mode 1 (fp8_w_fp8_a):  x is E4M3 codes uint8 [M, K], x_scale is the fp32 scale.
    mode 2 (fp8_w_fp16_a): x is fp16 bits uint16 [M, K], x_scale must be None.
    """
    if mode in (MODE_W8A16, MODE_W8A16_F16):
        _need(x, np.uint16, "x")
        if x_scale is not None:
            raise ValueError("the 16-bit activation modes take no activation scale")
        xs = 0.0
    elif mode == MODE_W8A8:
        _need(x, np.uint8, "x")
        if x_scale is None:
            raise ValueError("fp8_w_fp8_a needs the activation scale")
        xs = float(np.float32(x_scale))
    else:
        raise ValueError("unknown mode")
    _need(wq, np.uint8, "wq")
    w_scale = np.ascontiguousarray(w_scale, dtype=np.float32)
    m, k = x.shape
    n, k2 = wq.shape
    if k2 != k or w_scale.shape != (n,):
        raise ValueError("shape mismatch")
    if rows is None:
        nrows, rp = m, None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        if rows.size and (rows.min() < 0 or rows.max() >= m):
            raise IndexError("row index out of range")
        nrows, rp = rows.size, _ptr(rows)
    y = np.empty((nrows, n), np.float64)
    if nrows and n:
        _load().oracle_linear(mode, _ptr(x), m, k, _ld(x), xs, _ptr(wq), n, _ld(wq),
                              _ptr(w_scale), rp, nrows, _ptr(y))
    return y
