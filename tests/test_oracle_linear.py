"""Pins for the oracle's scaled linear layer (fp64).

The three FP8 MatMul modes of Llama 3 精读 §3.1 step 3 -- fp8_w_bf16_a,
fp8_w_fp8_a and fp8_w_fp16_a -- with the per-channel weight scale and
per-tensor activation scale of FP8量化与长上下文实测 §1.2.  The weight keeps the [out, in] layout of
a linear layer, so Y = X W^T.

Pins: exact rational brute force (fractions.Fraction, decoding codes with
torch's float8 decoder, not the oracle's) on tiny shapes, closed forms, and
the row-selection path.  A transposed operand, a dropped scale, a wrong index
or a lost term each break the brute-force comparison; the shapes are
non-square so a transpose cannot pass by symmetry.
"""
from fractions import Fraction

import numpy as np
import pytest

import workloads

torch = pytest.importorskip("torch")


def torch_decode(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def exact_linear(mode, x, wq, w_scale, x_scale=None):
    m, k = x.shape
    n = wq.shape[0]
    wd = torch_decode(wq)
    if mode == 0:
        xd = workloads.bf16_bits_to_f32(x).astype(np.float64)
    elif mode == 2:
        xd = np.ascontiguousarray(x, dtype=np.uint16).view(np.float16).astype(np.float64)
    else:
        xd = torch_decode(x)
    y = [[None] * n for _ in range(m)]
    for i in range(m):
        for j in range(n):
            acc = sum((Fraction(float(xd[i, c])) * Fraction(float(wd[j, c])) for c in range(k)),
                      Fraction(0))
            sc = Fraction(float(w_scale[j]))
            if mode == 1:
                sc *= Fraction(float(np.float32(x_scale)))
            y[i][j] = acc * sc
    return y


def random_codes(rng, shape):
    c = rng.integers(0, 256, shape, dtype=np.uint16).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3C                     # no NaN codes
    return c


@pytest.mark.parametrize("m,n,k,seed", [(3, 5, 7, 0), (1, 4, 8, 1), (6, 2, 3, 2), (4, 7, 1, 3)])
def test_w8a8_brute_force_exact(orc, m, n, k, seed):
    rng = np.random.default_rng(seed)
    xq = random_codes(rng, (m, k))
    wq = random_codes(rng, (n, k))
    ws = (rng.random(n).astype(np.float32) + np.float32(0.01))
    xs = np.float32(0.0371)
    got = orc.linear(1, xq, wq, ws, xs)
    ref = exact_linear(1, xq, wq, ws, xs)
    for i in range(m):
        for j in range(n):
            # the fp64 sum is exact; only the final product by the scales rounds
            assert abs(Fraction(got[i, j]) - ref[i][j]) <= abs(ref[i][j]) * Fraction(1, 2 ** 52)


@pytest.mark.parametrize("m,n,k,seed", [(3, 5, 7, 0), (2, 6, 8, 4), (5, 3, 2, 5)])
def test_w8a16_brute_force(orc, m, n, k, seed):
    rng = np.random.default_rng(seed)
    x = workloads.normal_act(m, k, seed)
    wq = random_codes(rng, (n, k))
    ws = rng.random(n).astype(np.float32) + np.float32(0.01)
    got = orc.linear(0, x, wq, ws)
    ref = exact_linear(0, x, wq, ws)
    xd = np.abs(workloads.bf16_bits_to_f32(x).astype(np.float64))
    wd = np.abs(torch_decode(wq))
    for i in range(m):
        for j in range(n):
            mag = float(np.dot(xd[i], wd[j])) * float(ws[j])
            assert abs(Fraction(got[i, j]) - ref[i][j]) <= Fraction(k + 2) * Fraction(2.0 ** -53) * Fraction(mag) + Fraction(0)


def f16_bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float16).view(np.uint16)


@pytest.mark.parametrize("m,n,k,seed", [(3, 5, 7, 0), (2, 6, 8, 4), (5, 3, 2, 5), (1, 4, 9, 6)])
def test_w8a16_f16_brute_force(orc, m, n, k, seed):
    """fp8_w_fp16_a: activations decoded by numpy's float16, not the oracle."""
    rng = np.random.default_rng(seed)
    x = f16_bits(rng.standard_normal((m, k)) * 3.0)
    x[0, 0] = 0x0001                       # a subnormal (2^-24)
    wq = random_codes(rng, (n, k))
    ws = rng.random(n).astype(np.float32) + np.float32(0.01)
    got = orc.linear(2, x, wq, ws)
    ref = exact_linear(2, x, wq, ws)
    xd = np.abs(x.view(np.float16).astype(np.float64))
    wd = np.abs(torch_decode(wq))
    for i in range(m):
        for j in range(n):
            mag = float(np.dot(xd[i], wd[j])) * float(ws[j])
            assert abs(Fraction(got[i, j]) - ref[i][j]) <= Fraction(k + 2) * Fraction(2.0 ** -53) * Fraction(mag)


def test_modes_read_activation_bits_differently(orc):
    """The same 16-bit pattern 0x3C00 is 1.0 in fp16 and 2^-7 in bf16: a
    one-hot X picks one weight column, scaled accordingly."""
    wq = random_codes(np.random.default_rng(9), (5, 6))
    ws = np.ones(5, np.float32)
    x = np.zeros((1, 6), np.uint16)
    x[0, 4] = 0x3C00
    col = torch_decode(wq)[:, 4]
    assert np.array_equal(orc.linear(2, x, wq, ws)[0], col)
    assert np.array_equal(orc.linear(0, x, wq, ws)[0], col * 2.0 ** -7)


def test_row_sums_closed_form(orc):
    """All weight codes 1.0 (0x38) and unit scales: Y is the row sums of X."""
    x = workloads.normal_act(4, 96, 3)
    wq = np.full((3, 96), 0x38, np.uint8)
    y = orc.linear(0, x, wq, np.ones(3, np.float32))
    xs = workloads.bf16_bits_to_f32(x).astype(np.float64)
    for i in range(4):
        exact = float(sum(Fraction(float(v)) for v in xs[i]))
        assert np.all(np.abs(y[i] - exact) <= 96 * 2.0 ** -53 * np.abs(xs[i]).sum())


def test_identity_weight_closed_form(orc):
    """W = c I quantizes to 0x7E on the diagonal with s = fl32(c / 448), so Y = 448 s X."""
    c = np.float32(0.75)
    k = 32
    w = np.zeros((k, k), np.uint16)
    w[np.arange(k), np.arange(k)] = workloads.f32_to_bf16_bits(np.array([c]))[0]
    wq, ws, _ = orc.quantize_weight(w)
    assert (np.diag(wq) == 0x7E).all() and (ws == c / np.float32(448.0)).all()
    x = workloads.normal_act(5, k, 8)
    y = orc.linear(0, x, wq, ws)
    xd = workloads.bf16_bits_to_f32(x).astype(np.float64)
    assert (y == xd * 448.0 * np.float64(ws[0])).all()


def test_rank_one_closed_form(orc):
    """Equal rows of X and equal rows of W give one value u . v everywhere."""
    rng = np.random.default_rng(2)
    u = random_codes(rng, (1, 64))
    v = random_codes(rng, (1, 64))
    xq = np.repeat(u, 4, axis=0)
    wq = np.repeat(v, 6, axis=0)
    y = orc.linear(1, xq, wq, np.ones(6, np.float32), np.float32(1.0))
    dot = float(np.dot(torch_decode(u[0]), torch_decode(v[0])))
    assert (y == dot).all()


def test_row_selection(orc):
    x = workloads.normal_act(9, 40, 1)
    wq, ws, _ = orc.quantize_weight(workloads.heavy_tail_weight(11, 40, 2))
    full = orc.linear(0, x, wq, ws)
    sel = orc.linear(0, x, wq, ws, rows=np.array([7, 0, 3]))
    assert (sel == full[[7, 0, 3]]).all()


def test_transpose_is_wrong(orc):
    """Guard against an operand swap: X W^T differs from the swapped product."""
    x = workloads.normal_act(3, 3, 4)
    wq, ws, _ = orc.quantize_weight(workloads.heavy_tail_weight(3, 3, 5))
    y = orc.linear(0, x, wq, ws)
    xd = workloads.bf16_bits_to_f32(x).astype(np.float64)
    wd = torch_decode(wq) * ws[:, None]
    assert np.allclose(y, xd @ wd.T, rtol=1e-12, atol=0)
    assert not np.allclose(y, (wd @ xd.T), rtol=1e-6, atol=0)
