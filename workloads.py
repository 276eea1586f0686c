"""Seeded synthetic inputs for the FP8 weight-quantized linear path.

This module is the only code that both the CPU oracle side (tests, benchmark
baseline) and the HIP side consume.  It holds no arithmetic of the method
itself: it draws numbers with numpy's PCG64 generator and rounds them to
bf16 bit patterns, nothing more.

Workloads are Llama-3-shaped linear layers.  The weight statistics follow the
pages' description of Llama 3 linear weights ("Llama 3 精读" FP8 + 128K
write-up, §2.1: standard deviation around 0.08-0.15 and a few percent of
entries with |w| > 2), modelled as N(0, 0.1) with 3% of entries replaced by
+-U(2, 4).  No real checkpoint is used.

All arrays are returned as uint16 bf16 bit patterns, row-major, last
dimension contiguous.  Weights are [N=out, K=in]; activations are [M, K].
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np


# ---------------------------------------------------------------------------
# fp32 -> bf16 bit patterns, round to nearest even (input preparation only).
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    u = np.array(a, dtype=np.float32, copy=True, order="C").view(np.uint32)
    nan = np.isnan(u.view(np.float32))
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u += np.uint32(0x7FFF)          # wraps only for NaN patterns, fixed below
    u += lsb
    u >>= np.uint32(16)
    out = u.astype(np.uint16)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------
# Generators.  A matrix is drawn in row blocks of about 2^22 elements; block b
# comes from PCG64(seed) jumped b times (numpy's jumped(b) advances the state
# by b * 2^128 draws), and within a block the draws happen in a fixed order.
# The result is therefore a pure function of (shape, seed), whatever number of
# threads fills the blocks.
# ---------------------------------------------------------------------------
_BLOCK_ELEMS = 1 << 22


def _threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return max(1, min(16, os.cpu_count() or 1))


def _blocked(rows: int, cols: int, seed: int, fill) -> np.ndarray:
    """Fill a [rows, cols] bf16-bit matrix block by block; fill(rng, r, c) -> fp32 [r, c]."""
    out = np.empty((rows, cols), np.uint16)
    if rows == 0 or cols == 0:
        return out
    rb = max(1, _BLOCK_ELEMS // cols)
    starts = list(range(0, rows, rb))
    base = np.random.PCG64(seed)

    def one(b: int) -> None:
        r0 = starts[b]
        r1 = min(rows, r0 + rb)
        rng = np.random.Generator(base.jumped(b))
        out[r0:r1] = f32_to_bf16_bits(fill(rng, r1 - r0, cols))

    if len(starts) == 1:
        one(0)
    else:
        with ThreadPoolExecutor(max_workers=_threads()) as ex:
            list(ex.map(one, range(len(starts))))
    return out


def _heavy_tail_fill(rng: np.random.Generator, r: int, c: int) -> np.ndarray:
    w = rng.standard_normal((r, c), dtype=np.float32)
    w *= np.float32(0.1)
    mask = rng.random((r, c), dtype=np.float32) < np.float32(0.03)
    nnz = int(np.count_nonzero(mask))
    sign = np.where(rng.random(nnz, dtype=np.float32) < np.float32(0.5),
                    np.float32(-1.0), np.float32(1.0))
    mag = rng.uniform(2.0, 4.0, nnz).astype(np.float32)
    w[mask] = sign * mag
    return w


def _normal_fill(rng: np.random.Generator, r: int, c: int) -> np.ndarray:
    return rng.standard_normal((r, c), dtype=np.float32)


def _outlier_fill(rng: np.random.Generator, r: int, c: int) -> np.ndarray:
    x = rng.standard_normal((r, c), dtype=np.float32)
    mask = rng.random((r, c), dtype=np.float32) < np.float32(0.001)
    x[mask] *= np.float32(20.0)
    return x


def _swiglu_fill(rng: np.random.Generator, r: int, c: int) -> np.ndarray:
    a = rng.standard_normal((r, c), dtype=np.float32)
    b = rng.standard_normal((r, c), dtype=np.float32)
    return a / (np.float32(1.0) + np.exp(-a)) * b


def heavy_tail_weight(n: int, k: int, seed: int) -> np.ndarray:
    """W [n, k]: N(0, 0.1), then 3% of entries replaced by +-U(2, 4)."""
    return _blocked(n, k, seed, _heavy_tail_fill)


def normal_act(m: int, k: int, seed: int) -> np.ndarray:
    """X [m, k] ~ N(0, 1)."""
    return _blocked(m, k, seed, _normal_fill)


def outlier_act(m: int, k: int, seed: int) -> np.ndarray:
    """X [m, k] ~ N(0, 1) with 0.1% of entries multiplied by 20."""
    return _blocked(m, k, seed, _outlier_fill)


def swiglu_act(m: int, k: int, seed: int) -> np.ndarray:
    """X [m, k] = SiLU(a) * b with a, b ~ N(0, 1): the input of a down projection."""
    return _blocked(m, k, seed, _swiglu_fill)


# ---------------------------------------------------------------------------
# Workload registry (shapes of Llama 3 8B / 70B linear layers).
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class Linear:
    name: str
    n: int          # out features (rows of W)
    k: int          # in features
    seed: int       # weight seed


@dataclass(frozen=True)
class Workload:
    key: str
    title: str
    mode: str                     # "w8a16" (fp8_w_bf16_a) or "w8a8" (fp8_w_fp8_a)
    linears: tuple
    ms: tuple                     # activation rows (tokens) per call
    act: str = "normal"           # normal | outlier | swiglu
    notes: str = field(default="")

    def act_seed(self, m: int) -> int:
        """Activation seed: 1000 + M (the weight seeds are the matrix index)."""
        return 1000 + m


WORKLOADS = {
    "tiny": Workload(
        "tiny", "Tiny W[256,512], X[16,512], seed 0", "w8a16",
        (Linear("w", 256, 512, 0),), (16,), notes="weight seed 0; activation seed 1000 + M like every workload"),
    "q_proj_decode": Workload(
        "q_proj_decode", "Llama-3-8B q_proj decode, W[4096,4096], M in {1,8,32,64}", "w8a16",
        (Linear("q_proj", 4096, 4096, 0),), (1, 8, 32, 64)),
    "mlp_prefill": Workload(
        "mlp_prefill", "Llama-3-8B fused gate+up prefill, W[28672,4096], X[8192,4096]", "w8a8",
        (Linear("gate_up", 28672, 4096, 0),), (8192,), act="outlier"),
    "down_prefill_70b": Workload(
        "down_prefill_70b", "Llama-3-70B down_proj prefill, W[8192,28672], X[4096,28672]", "w8a8",
        (Linear("down_proj", 8192, 28672, 0),), (4096,), act="swiglu"),
    "layer_decode_70b": Workload(
        "layer_decode_70b", "Llama-3-70B decoder-layer linears at decode M=12", "w8a16",
        (Linear("q_proj", 8192, 8192, 0), Linear("k_proj", 1024, 8192, 1),
         Linear("v_proj", 1024, 8192, 2), Linear("o_proj", 8192, 8192, 3),
         Linear("gate_proj", 28672, 8192, 4), Linear("up_proj", 28672, 8192, 5),
         Linear("down_proj", 8192, 28672, 6)), (12,)),
}


def weight(wl: Workload, lin: Linear) -> np.ndarray:
    return heavy_tail_weight(lin.n, lin.k, lin.seed)


def activation(wl: Workload, m: int, k: int) -> np.ndarray:
    seed = wl.act_seed(m)
    if wl.act == "outlier":
        return outlier_act(m, k, seed)
    if wl.act == "swiglu":
        return swiglu_act(m, k, seed)
    return normal_act(m, k, seed)
