"""Seeded random decode shapes through every mode and weight-scale
granularity.

Every call must launch (status 0) whatever plan its shape gets -- the panel
kernel with any of its fragment counts, row groups and scale stagings, the
rows kernel, the tile kernel with or without K splits -- and its output must
lie within the GEMM tolerance of the fp64 oracle on the same codes and
scales ("Llama 3 精读" §3.1 step 3 for the three modes; the deployment
guide §4.3 for per-group scales).  The shapes are drawn once from a fixed
seed: 1 to 64 activation rows, K a multiple of 512 from 2048 (the panel
kernel's range) or ragged, N from 16 to 6000 (at most 12.6M weights).
"""
import numpy as np
import pytest

import workloads
from helpers import assert_gemm_close, dev_bf16, dev_u8, host_bf16_as_f64, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _shapes(count: int = 60, seed: int = 2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        m = int(rng.choice([1, 2, 4, 5, 8, 12, 16, 17, 24, 31, 32, 33, 40, 48, 64]))
        k = int(rng.choice([2048, 2560, 3072, 4096, 4608, 6144, 8192, 2048, 4096, 1000, 1536,
                            2100]))
        cap = min(6000, (12 << 20) // k)
        n = int(rng.integers(1024, cap) if rng.random() < 0.75 else rng.integers(16, 1024))
        mode = int(rng.integers(0, 3))
        group = int(rng.choice([0, 64, 128, 256, 512]))
        out.append((i, m, n, k, mode, group))
    return out


SHAPES = _shapes()


@pytest.fixture(scope="module")
def fq():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import fp8_weight_quantized_amd as fq
    fq.library_path()
    return fq


def _padded(a: np.ndarray, multiple: int) -> np.ndarray:
    """a copy with the row stride rounded up to a multiple (the ABI's rule)"""
    rows, cols = a.shape
    out = np.zeros((rows, -(-cols // multiple) * multiple), a.dtype)
    out[:, :cols] = a
    return out


def _dev_x(mode: int, x: np.ndarray):
    k = x.shape[1]
    if mode == 0:
        return dev_bf16(_padded(x, 8))[:, :k]
    if mode == 2:
        return torch.from_numpy(_padded(x, 8).view(np.float16)).cuda()[:, :k]
    return dev_u8(_padded(x, 16))[:, :k]


@pytest.mark.parametrize("case", SHAPES, ids=[f"{i}-m{m}-n{n}-k{k}-mode{md}-g{g}"
                                             for i, m, n, k, md, g in SHAPES])
def test_random_decode_shape(fq, orc, case):
    i, m, n, k, mode, group = case
    w = workloads.heavy_tail_weight(n, k, 900 + i)
    if group:
        wq, ws, _ = orc.quantize_weight_grouped(w, group)
    else:
        wq, ws, _ = orc.quantize_weight(w)
    xs = None
    if mode == 1:
        x, xs, _ = orc.quantize_act(workloads.outlier_act(m, k, 950 + i))
        xs = np.float32(xs)
    else:
        x = workloads.outlier_act(m, k, 950 + i)
        if mode == 2:
            x = workloads.bf16_bits_to_f32(x).astype(np.float16).view(np.uint16)
    plan = fq.describe_linear(mode, m, n, k, group=group or None)
    say("random decode shape", i, m, n, k, mode, group, plan)
    y = fq.linear(_dev_x(mode, x), dev_u8(_padded(wq, 16))[:, :k], torch.from_numpy(ws).cuda(),
                  x_scale=None if xs is None else torch.tensor([xs], device="cuda"),
                  group=group or None)
    torch.cuda.synchronize()
    if group:
        ref = orc.linear_grouped(mode, x, wq, ws, group, x_scale=xs)
    else:
        ref = orc.linear(mode, x, wq, ws, x_scale=xs)
    assert_gemm_close(host_bf16_as_f64(y), ref, f"case {i}: {plan}")


def test_sweep_reaches_every_decode_kernel(fq):
    """The drawn shapes take the panel kernel (with and without group scales,
    both scale stagings among them), the rows kernel and the tile kernel."""
    plans = [fq.describe_linear(md, m, n, k, group=g or None) for _, m, n, k, md, g in SHAPES]
    assert any(p.startswith("k_w8a16_panel") and "scales=" not in p for p in plans)
    assert any(p.startswith("k_w8a16_panel") and "scales=preloaded" in p for p in plans)
    assert any(p.startswith("k_w8a16_rows") for p in plans)
    assert any(p.startswith("k_w8a16_tile") for p in plans)
