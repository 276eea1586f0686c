"""Pins for the oracle's per-group weight quantization and grouped linear layer.

FP8量化与长上下文实测：Llama 3 70B部署优化指南 §4.3 names per-group granularity as
the next step beyond per-channel scales; each group takes the §3.1 formula
over its own values.  Pins: the guide's recipe run group by group with torch
in fp32 (padding a ragged last group with zeros, which cannot change an
absmax); group = K reducing exactly to the pinned per-channel quantizer; the
row scale being the largest of its group scales; the guide's claim that finer
groups lose less; and an exact rational brute force of the grouped linear
layer (codes decoded by torch, not by the oracle) on tiny shapes with ragged
groups, in all three modes.
"""
from fractions import Fraction

import numpy as np
import pytest

import workloads

torch = pytest.importorskip("torch")


def torch_grouped(w_bits: np.ndarray, group: int):
    n, k = w_bits.shape
    ng = -(-k // group)
    w = np.zeros((n, ng * group), np.float32)
    w[:, :k] = workloads.bf16_bits_to_f32(w_bits)
    wt = torch.from_numpy(w).view(n, ng, group)
    s = (wt.abs().amax(dim=2, keepdim=True) / 448.0).clamp(min=1e-12)
    q = (wt / s).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    return q.reshape(n, ng * group)[:, :k].numpy(), s.reshape(n, ng).numpy()


def torch_decode(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


@pytest.mark.parametrize("n,k,group,seed", [(64, 512, 128, 0), (33, 1024, 64, 1), (7, 4096, 512, 2),
                                            (9, 300, 128, 3), (5, 77, 64, 4), (3, 8, 3, 5),
                                            (16, 1000, 256, 6)])
def test_matches_page_recipe_per_group(orc, n, k, group, seed):
    w = workloads.heavy_tail_weight(n, k, seed)
    q, s, nf = orc.quantize_weight_grouped(w, group)
    qr, sr = torch_grouped(w, group)
    assert not nf
    assert (s.view(np.uint32) == sr.view(np.uint32)).all()
    assert (q == qr).all()


@pytest.mark.parametrize("k,group", [(512, 512), (300, 300), (300, 1000)])
def test_one_group_is_per_channel(orc, k, group):
    w = workloads.heavy_tail_weight(20, k, 7)
    q, s, _ = orc.quantize_weight_grouped(w, group)
    qc, sc, _ = orc.quantize_weight(w)
    assert s.shape == (20, 1)
    assert (q == qc).all() and (s[:, 0].view(np.uint32) == sc.view(np.uint32)).all()


def test_row_scale_is_largest_group_scale(orc):
    """absmax/448 is monotone in absmax, so the per-channel scale of a row is the
    largest of its group scales, bit for bit."""
    w = workloads.heavy_tail_weight(50, 1024, 8)
    _, s, _ = orc.quantize_weight_grouped(w, 128)
    _, sc, _ = orc.quantize_weight(w)
    assert (s.max(axis=1).view(np.uint32) == sc.view(np.uint32)).all()


def test_finer_groups_lose_less(orc):
    """The guide's reason for per-group scales: a smaller reconstruction error."""
    w = workloads.heavy_tail_weight(128, 4096, 9)
    wf = workloads.bf16_bits_to_f32(w).astype(np.float64)
    q, s, _ = orc.quantize_weight(w)
    err_row = ((torch_decode(q) * s[:, None] - wf) ** 2).mean()
    prev = err_row
    for group in (512, 128, 64):
        qg, sg, _ = orc.quantize_weight_grouped(w, group)
        deq = torch_decode(qg) * np.repeat(sg, group, axis=1)[:, :4096]
        err = ((deq - wf) ** 2).mean()
        assert err < prev, (group, err, prev)
        prev = err


def exact_grouped(mode, x, wq, w_scale, group, x_scale=None):
    m, k = x.shape
    n = wq.shape[0]
    wd = torch_decode(wq)
    if mode == 0:
        xd = workloads.bf16_bits_to_f32(x).astype(np.float64)
    elif mode == 2:
        xd = np.ascontiguousarray(x, dtype=np.uint16).view(np.float16).astype(np.float64)
    else:
        xd = torch_decode(x)
    y = np.empty((m, n))
    for i in range(m):
        for j in range(n):
            tot = Fraction(0)
            for g0 in range(0, k, group):
                acc = sum((Fraction(float(xd[i, c])) * Fraction(float(wd[j, c]))
                           for c in range(g0, min(k, g0 + group))), Fraction(0))
                tot += acc * Fraction(float(w_scale[j, g0 // group]))
            if mode == 1:
                tot *= Fraction(float(np.float32(x_scale)))
            y[i, j] = float(tot)
    return y


def random_codes(rng, shape):
    c = rng.integers(0, 256, shape, dtype=np.uint16).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3C
    return c


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("m,n,k,group,seed", [(3, 5, 7, 3, 0), (2, 4, 16, 8, 1), (4, 3, 10, 4, 2),
                                              (1, 6, 9, 9, 3)])
def test_grouped_linear_brute_force(orc, mode, m, n, k, group, seed):
    rng = np.random.default_rng(seed)
    wq = random_codes(rng, (n, k))
    ng = -(-k // group)
    ws = rng.uniform(0.001, 0.05, (n, ng)).astype(np.float32)
    xs = None
    if mode == 0:
        x = workloads.f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    elif mode == 2:
        x = rng.standard_normal((m, k)).astype(np.float16).view(np.uint16)
    else:
        x = random_codes(rng, (m, k))
        xs = np.float32(0.0123)
    got = orc.linear_grouped(mode, x, wq, ws, group, x_scale=xs)
    ref = exact_grouped(mode, x, wq, ws, group, x_scale=xs)
    # fp64 sums of at most 16 terms: within a few ulp of the exact value
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-300), (got, ref)


@pytest.mark.parametrize("mode", [0, 1])
def test_grouped_linear_one_group_is_per_channel(orc, mode):
    rng = np.random.default_rng(5)
    w = workloads.heavy_tail_weight(40, 256, 10)
    wq, ws, _ = orc.quantize_weight(w)
    xb = workloads.outlier_act(6, 256, 11)
    if mode == 0:
        x, xs = xb, None
    else:
        x, xs, _ = orc.quantize_act(xb)
    ref = orc.linear(mode, x, wq, ws, x_scale=xs)
    got = orc.linear_grouped(mode, x, wq, ws[:, None], 256, x_scale=xs)
    assert np.allclose(got, ref, rtol=1e-14, atol=0)
    rows = np.array([5, 0, 3])
    assert np.allclose(orc.linear_grouped(mode, x, wq, ws[:, None], 256, x_scale=xs, rows=rows),
                       ref[rows], rtol=1e-14, atol=0)
    del rng
