"""fp8q: FP8 (E4M3) weight-quantized linear layers on AMD MI355X (gfx950).

A thin binding over the C ABI of libfp8q.so (include/fp8q.h): it checks
tensor metadata, allocates outputs and scratch with torch (device memory
only) and passes raw pointers and the current HIP stream.  Every step of the
computation runs in the library's HIP kernels; there is no CPU path.

    wq, w_scale = quantize_weight(w_bf16)             # per output channel
    wq, w_scale = quantize_weight_grouped(w_bf16, 128)  # per group of 128 inputs
    xq, x_scale = quantize_act(x_bf16)                # per tensor, dynamic
    xq = quantize_act_static(x_bf16, held_scale)      # per tensor, held scale
    ema = EmaActScale(dev); xq, x_scale = ema(x_bf16) # per tensor, EMA scale
    kv_scale = kv_cache_write(k, v, slot, k_cache, v_cache, running, calibrate)
    y = linear(x_bf16, wq, w_scale)                   # fp8_w_bf16_a (decode)
    y = linear(xq, wq, w_scale, x_scale=x_scale)      # fp8_w_fp8_a  (prefill)
    y, x_scale = linear_w8a8_dynamic(x_bf16, wq, w_scale)  # fp8_w_fp8_a, X quantized inside

Codes are returned as uint8 tensors holding raw e4m3fn bit patterns (view
them with .view(torch.float8_e4m3fn)).  Code matrices are allocated with a
row stride rounded up to 16 bytes, as the GEMM requires.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import FP8Q_W8A8, FP8Q_W8A16, FP8Q_W8A16_F16, Fp8qError, check

__all__ = [
    "quantize_weight", "quantize_weight_grouped", "quantize_act", "quantize_act_static", "quantize_act_ema",
    "EmaActScale", "kv_cache_write", "linear", "linear_w8a8_dynamic", "cast_f32_to_e4m3",
    "describe_linear",
    "FP8Q_W8A16", "FP8Q_W8A8", "Fp8qError", "library_path",
]


def library_path() -> str:
    _lib.lib()
    return _lib.LIB_PATH


def _round_up(v: int, a: int) -> int:
    return (v + a - 1) // a * a


def _stream(dev: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr() if t is not None and t.numel() > 0 else None)


def _matrix(t: torch.Tensor, name: str, dtypes) -> tuple[int, int, int]:
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must be one of {dtypes}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    rows, cols = t.shape
    if t.numel() == 0:
        return rows, cols, cols        # nothing is read: the strides of an empty tensor are moot
    if cols > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have a contiguous last dimension")
    ld = t.stride(0) if rows > 1 else max(cols, t.stride(0))
    return rows, cols, ld


def _codes(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t


def _new_codes(rows: int, cols: int, dev: torch.device) -> torch.Tensor:
    ld = _round_up(max(cols, 1), 16)
    return torch.empty((rows, ld), dtype=torch.uint8, device=dev)[:, :cols]


def quantize_weight(w: torch.Tensor, nonfinite_flag: torch.Tensor | None = None):
    """Per-output-channel E4M3 quantization of a bf16 [N, K] weight.

    Returns (codes uint8 [N, K], scale float32 [N]).  `nonfinite_flag`, an
    int32 GPU tensor, is set to 1 if any weight is NaN or infinite.
    """
    n, k, ld = _matrix(w, "w", (torch.bfloat16,))
    dev = w.device
    q = _new_codes(n, k, dev)
    scale = torch.empty(n, dtype=torch.float32, device=dev)
    check(_lib.lib().fp8q_quantize_weight(
        _ptr(w), n, k, ld, _ptr(q), q.stride(0) if n else _round_up(k, 16), _ptr(scale),
        _ptr(nonfinite_flag), _stream(dev)))
    return q, scale


def quantize_act(x: torch.Tensor, nonfinite_flag: torch.Tensor | None = None):
    """Dynamic per-tensor E4M3 quantization of bf16 activations [M, K].

    Returns (codes uint8 [M, K], scale float32 [1]) -- the scale stays on the GPU.
    """
    m, k, ld = _matrix(x, "x", (torch.bfloat16,))
    dev = x.device
    q = _new_codes(m, k, dev)
    scale = torch.empty(1, dtype=torch.float32, device=dev)
    L = _lib.lib()
    nws = L.fp8q_quantize_act_workspace_size(m, k)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    check(L.fp8q_quantize_act(
        _ptr(x), m, k, ld, _ptr(q), q.stride(0) if m else _round_up(k, 16), _ptr(scale),
        _ptr(ws), nws, _ptr(nonfinite_flag), _stream(dev)))
    return q, scale


def _scalar_f32(t: torch.Tensor, name: str, dev: torch.device) -> None:
    if t.dtype != torch.float32 or t.numel() != 1 or t.device != dev:
        raise ValueError(f"{name} must be one float32 on {dev}")


def quantize_act_static(x: torch.Tensor, scale: torch.Tensor,
                        nonfinite_flag: torch.Tensor | None = None) -> torch.Tensor:
    """Per-tensor E4M3 quantization of bf16 activations with a held scale.

    `scale` is a float32 [1] GPU tensor (positive, finite); values beyond
    448 * scale saturate.  Returns the codes, uint8 [M, K].
    """
    m, k, ld = _matrix(x, "x", (torch.bfloat16,))
    dev = x.device
    _scalar_f32(scale, "scale", dev)
    q = _new_codes(m, k, dev)
    check(_lib.lib().fp8q_quantize_act_static(
        _ptr(x), m, k, ld, _ptr(scale), _ptr(q), q.stride(0) if m else _round_up(k, 16),
        _ptr(nonfinite_flag), _stream(dev)))
    return q


def quantize_act_ema(x: torch.Tensor, state: torch.Tensor, decay: float = 0.9999,
                     temperature: float = 0.0, seed: bool = False,
                     nonfinite_flag: torch.Tensor | None = None):
    """Per-tensor E4M3 quantization with an EMA scale carried in `state`.

    `state` is a float32 [1] GPU tensor.  seed=True quantizes dynamically and
    sets the state to that scale; otherwise the codes use the state as it was,
    and the state then takes one EMA step towards this tensor's dynamic scale.
    Returns (codes uint8 [M, K], scale float32 [1] the codes were made with).
    """
    m, k, ld = _matrix(x, "x", (torch.bfloat16,))
    dev = x.device
    _scalar_f32(state, "state", dev)
    q = _new_codes(m, k, dev)
    scale = torch.empty(1, dtype=torch.float32, device=dev)
    L = _lib.lib()
    nws = L.fp8q_quantize_act_workspace_size(m, k)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    check(L.fp8q_quantize_act_ema(
        _ptr(x), m, k, ld, _ptr(q), q.stride(0) if m else _round_up(k, 16), _ptr(scale),
        _ptr(state), float(decay), float(temperature), 1 if seed else 0, _ptr(ws), nws,
        _ptr(nonfinite_flag), _stream(dev)))
    return q, scale


class EmaActScale:
    """The EMA activation scale of one linear layer's input: a device state
    and whether it has been seeded.  Calling it quantizes a bf16 [M, K]
    activation and returns (codes, scale) for fp8_w_fp8_a."""

    def __init__(self, device, decay: float = 0.9999, temperature: float = 0.0):
        self.state = torch.zeros(1, dtype=torch.float32, device=device)
        self.decay = float(decay)
        self.temperature = float(temperature)
        self.seeded = False

    def __call__(self, x: torch.Tensor, nonfinite_flag: torch.Tensor | None = None):
        out = quantize_act_ema(x, self.state, self.decay, self.temperature,
                               seed=not self.seeded, nonfinite_flag=nonfinite_flag)
        self.seeded = True
        return out


def kv_cache_write(k: torch.Tensor, v: torch.Tensor, slot: torch.Tensor,
                   k_cache: torch.Tensor, v_cache: torch.Tensor, running_max: torch.Tensor,
                   calibrate: bool, flags: torch.Tensor | None = None) -> torch.Tensor:
    """Write new K/V tokens of one layer into its E4M3 caches.

    k, v: bf16 [T, heads * head_dim] (token-major); slot: int64 [T] cache rows;
    k_cache, v_cache: uint8 [heads, S, head_dim], contiguous; running_max:
    float32 [2] (max |K|, max |V|), raised when `calibrate` (prefill), read as
    it stands otherwise (decode).  Returns the float32 [2] K/V scales used.
    """
    t, width, ld = _matrix(k, "k", (torch.bfloat16,))
    t2, width2, ld2 = _matrix(v, "v", (torch.bfloat16,))
    if (t2, width2) != (t, width) or (t and ld2 != ld):
        raise ValueError("k and v must have the same shape and row stride")
    dev = k.device
    for c, name in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        if c.dtype != torch.uint8 or c.dim() != 3 or not c.is_contiguous() or c.device != dev:
            raise ValueError(f"{name} must be a contiguous uint8 [heads, S, head_dim] on {dev}")
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache differ in shape")
    heads, slots, head_dim = k_cache.shape
    if heads * head_dim != width:
        raise ValueError(f"k has {width} values per token, the cache holds {heads} x {head_dim}")
    if slot.dtype != torch.int64 or slot.shape != (t,) or slot.device != dev or \
            (t and slot.stride(0) != 1):
        raise ValueError(f"slot must be a contiguous int64 [{t}] on {dev}")
    if running_max.dtype != torch.float32 or running_max.numel() != 2 or \
            running_max.device != dev or not running_max.is_contiguous():
        raise ValueError("running_max must be a contiguous float32 [2] on the same device")
    scale = torch.empty(2, dtype=torch.float32, device=dev)
    L = _lib.lib()
    nws = L.fp8q_kv_cache_workspace_size(t, heads, head_dim)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    check(L.fp8q_kv_cache_write(
        _ptr(k), _ptr(v), t, heads, head_dim, ld if t else width, _ptr(slot), _ptr(k_cache),
        _ptr(v_cache), slots, _ptr(running_max), _ptr(scale), 1 if calibrate else 0, _ptr(ws),
        nws, _ptr(flags), _stream(dev)))
    return scale


def quantize_weight_grouped(w: torch.Tensor, group: int = 128,
                            nonfinite_flag: torch.Tensor | None = None):
    """Per-group E4M3 quantization of a bf16 [N, K] weight: groups of `group`
    (64, 128, 256 or 512) consecutive input values per output row.

    Returns (codes uint8 [N, K], scale float32 [N, ceil(K / group)]).
    """
    n, k, ld = _matrix(w, "w", (torch.bfloat16,))
    dev = w.device
    q = _new_codes(n, k, dev)
    scale = torch.empty((n, -(-k // group)), dtype=torch.float32, device=dev)
    check(_lib.lib().fp8q_quantize_weight_grouped(
        _ptr(w), n, k, ld, group, _ptr(q), q.stride(0) if n else _round_up(k, 16), _ptr(scale),
        _ptr(nonfinite_flag), _stream(dev)))
    return q, scale


def linear(x: torch.Tensor, wq: torch.Tensor, w_scale: torch.Tensor,
           x_scale: torch.Tensor | None = None, out: torch.Tensor | None = None,
           group: int | None = None) -> torch.Tensor:
    """Y = X . dequant(Wq)^T.

    x bf16 [M, K] with x_scale None  -> fp8_w_bf16_a (W8A16), bf16 Y.
    x fp16 [M, K] with x_scale None  -> fp8_w_fp16_a (W8A16, fp16), fp16 Y.
    x E4M3 codes [M, K] with x_scale -> fp8_w_fp8_a  (W8A8), bf16 Y.
    group None: w_scale [N] (per channel); else w_scale [N, ceil(K / group)].
    """
    wq = _codes(wq)
    x = _codes(x)
    if x.dtype in (torch.bfloat16, torch.float16):
        mode = FP8Q_W8A16 if x.dtype == torch.bfloat16 else FP8Q_W8A16_F16
        if x_scale is not None:
            raise ValueError("a 16-bit activation takes no x_scale (fp8_w_bf16_a / fp8_w_fp16_a)")
    elif x.dtype == torch.uint8:
        mode = FP8Q_W8A8
        if x_scale is None:
            raise ValueError("E4M3 activations need x_scale (fp8_w_fp8_a)")
    else:
        raise TypeError(f"x must be bf16, fp16 or E4M3 codes, got {x.dtype}")
    m, k, ldx = _matrix(x, "x", (torch.bfloat16, torch.float16, torch.uint8))
    n, k2, ldw = _matrix(wq, "wq", (torch.uint8,))
    if k2 != k:
        raise ValueError(f"inner dimensions differ: x has K={k}, wq has K={k2}")
    n_scales = n if group is None else n * -(-k // group)
    if w_scale.dtype != torch.float32 or w_scale.numel() != n_scales or not w_scale.is_cuda:
        raise ValueError(f"w_scale must be a float32 GPU tensor with {n_scales} elements")
    if not w_scale.is_contiguous():
        raise ValueError("w_scale must be contiguous")
    w_scale = w_scale.reshape(-1)
    if x_scale is not None and (x_scale.dtype != torch.float32 or x_scale.numel() != 1 or not x_scale.is_cuda):
        raise ValueError("x_scale must be a float32 GPU tensor with one element")
    dev = x.device
    ydt = torch.float16 if mode == FP8Q_W8A16_F16 else torch.bfloat16
    if out is None:
        out = torch.empty((m, _round_up(max(n, 1), 8)), dtype=ydt, device=dev)[:, :n]
    om, on, ldy = _matrix(out, "out", (ydt,))
    if (om, on) != (m, n):
        raise ValueError(f"out must be [{m}, {n}]")
    L = _lib.lib()
    if group is None:
        nws = L.fp8q_linear_workspace_size(mode, m, n, k)
        ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
        check(L.fp8q_linear(mode, _ptr(x), m, k, ldx, _ptr(x_scale), _ptr(wq), n, ldw,
                            _ptr(w_scale), _ptr(out), ldy, _ptr(ws), nws, _stream(dev)))
    else:
        nws = L.fp8q_linear_grouped_workspace_size(mode, m, n, k, group)
        ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
        check(L.fp8q_linear_grouped(mode, _ptr(x), m, k, ldx, _ptr(x_scale), _ptr(wq), n, ldw,
                                    _ptr(w_scale), group, _ptr(out), ldy, _ptr(ws), nws,
                                    _stream(dev)))
    return out


def linear_w8a8_dynamic(x: torch.Tensor, wq: torch.Tensor, w_scale: torch.Tensor,
                        out: torch.Tensor | None = None,
                        nonfinite_flag: torch.Tensor | None = None):
    """fp8_w_fp8_a on bf16 activations quantized per tensor inside the call.

    Equals quantize_act(x) followed by linear(xq, wq, w_scale, x_scale=...):
    same codes and scale, same sums.  Returns (Y bf16 [M, N], x_scale float32 [1]).
    """
    wq = _codes(wq)
    m, k, ldx = _matrix(x, "x", (torch.bfloat16,))
    n, k2, ldw = _matrix(wq, "wq", (torch.uint8,))
    if k2 != k:
        raise ValueError(f"inner dimensions differ: x has K={k}, wq has K={k2}")
    if w_scale.dtype != torch.float32 or w_scale.numel() != n or not w_scale.is_cuda \
            or not w_scale.is_contiguous():
        raise ValueError(f"w_scale must be a contiguous float32 GPU tensor with {n} elements")
    dev = x.device
    if out is None:
        out = torch.empty((m, _round_up(max(n, 1), 8)), dtype=torch.bfloat16, device=dev)[:, :n]
    om, on, ldy = _matrix(out, "out", (torch.bfloat16,))
    if (om, on) != (m, n):
        raise ValueError(f"out must be [{m}, {n}]")
    scale = torch.empty(1, dtype=torch.float32, device=dev)
    L = _lib.lib()
    nws = L.fp8q_linear_w8a8_dynamic_workspace_size(m, n, k)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    check(L.fp8q_linear_w8a8_dynamic(_ptr(x), m, k, ldx, _ptr(wq), n, ldw, _ptr(w_scale),
                                     _ptr(out), ldy, _ptr(scale), _ptr(ws), nws,
                                     _ptr(nonfinite_flag), _stream(dev)))
    return out, scale


def cast_f32_to_e4m3(x: torch.Tensor) -> torch.Tensor:
    """RNE, saturating fp32 -> E4M3 codes, elementwise (any shape, contiguous)."""
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 GPU tensor")
    out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    check(_lib.lib().fp8q_cast_f32_to_e4m3(_ptr(x), x.numel(), _ptr(out), _stream(x.device)))
    return out


def describe_linear(mode: int, m: int, n: int, k: int, group: int | None = None,
                    dynamic: bool = False) -> str:
    """The kernels a linear call of these sizes launches (dynamic=True: the
    fp8_w_fp8_a entry point that quantizes bf16 activations itself)."""
    buf = ctypes.create_string_buffer(256)
    if dynamic:
        check(_lib.lib().fp8q_linear_w8a8_dynamic_describe(m, n, k, buf, 256))
    elif group is None:
        check(_lib.lib().fp8q_linear_describe(mode, m, n, k, buf, 256))
    else:
        check(_lib.lib().fp8q_linear_grouped_describe(mode, m, n, k, group, buf, 256))
    return buf.value.decode()
