"""Pins for the oracle's weight (per-channel) and activation (per-tensor) quantization.

The conversion recipe of FP8量化与长上下文实测：Llama 3 70B部署优化指南 §3.1
(absmax over each output row / 448, clamp the scale at 1e-12, divide, cast
to float8_e4m3fn), executed with torch in fp32 -- a library special case
that shares nothing with the C oracle -- must give the oracle's codes and
scales bit for bit.  Invariants I1-I7 of the method add pins that a wrong
axis, a reciprocal multiply, a bf16 scale, single rounding or a lost sign
would each break.
"""
import numpy as np
import pytest

import workloads

torch = pytest.importorskip("torch")

FLOOR = np.float32(1e-12)


def torch_recipe_rows(w_bits: np.ndarray):
    """Per-row recipe in fp32 torch ops (per-channel: one scale per output row)."""
    w = torch.from_numpy(workloads.bf16_bits_to_f32(w_bits))
    s = (w.abs().amax(dim=1, keepdim=True) / 448.0).clamp(min=1e-12)
    q = (w / s).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    return q.numpy(), s.reshape(-1).numpy()


def torch_recipe_tensor(x_bits: np.ndarray):
    x = torch.from_numpy(workloads.bf16_bits_to_f32(x_bits))
    s = (x.abs().amax() / 448.0).clamp(min=1e-12)
    q = (x / s).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    return q.numpy(), np.float32(s.item())


CASES = [(256, 512, 0), (64, 4096, 1), (33, 1000, 2), (7, 13, 3), (1, 1, 4), (300, 8, 5)]


@pytest.mark.parametrize("n,k,seed", CASES)
def test_weight_matches_page_recipe(orc, n, k, seed):
    w = workloads.heavy_tail_weight(n, k, seed)
    q, s, nf = orc.quantize_weight(w)
    qr, sr = torch_recipe_rows(w)
    assert not nf
    assert (s.view(np.uint32) == sr.view(np.uint32)).all()
    assert (q == qr).all()


@pytest.mark.parametrize("m,k,seed", [(16, 512, 0), (8, 4096, 1), (5, 77, 2)])
def test_act_matches_page_recipe(orc, m, k, seed):
    x = workloads.outlier_act(m, k, seed)
    q, s, nf = orc.quantize_act(x)
    qr, sr = torch_recipe_tensor(x)
    assert not nf
    assert np.float32(s).view(np.uint32) == sr.view(np.uint32)
    assert (q == qr).all()


def test_act_is_weight_on_one_row(orc):
    """Per-tensor scaling is per-channel scaling of the tensor viewed as one row."""
    x = workloads.swiglu_act(24, 96, 9)
    q, s, _ = orc.quantize_act(x)
    q1, s1, _ = orc.quantize_weight(np.ascontiguousarray(x.reshape(1, -1)))
    assert s1[0] == s and (q1.reshape(q.shape) == q).all()


def test_strided_input(orc):
    w = workloads.heavy_tail_weight(40, 200, 3)
    big = np.zeros((40, 256), np.uint16)
    big[:, :200] = w
    q1, s1, _ = orc.quantize_weight(w)
    q2, s2, _ = orc.quantize_weight(big[:, :200])
    assert (q1 == q2).all() and (s1 == s2).all()


def test_scale_bits(orc):
    rng = np.random.default_rng(5)
    a = np.abs(rng.standard_normal(5000).astype(np.float32)) * np.float32(4.0)
    for v in a[:500]:
        assert orc.scale_from_amax(v) == np.float32(v) / np.float32(448.0)      # I2
    assert orc.scale_from_amax(0.0).view(np.uint32) == 0x2B8CBCCC               # clamp = 1e-12f
    assert orc.scale_from_amax(448.0 * 1e-12 * 0.5) == FLOOR


def test_I1_max_code_is_448(orc):
    tab = orc.e4m3_table()
    w = workloads.heavy_tail_weight(512, 1024, 8)
    q, s, _ = orc.quantize_weight(w)
    assert (np.abs(tab[q]).max(axis=1) == 448.0).all()


def test_I3_no_nan_codes(orc):
    w = workloads.heavy_tail_weight(128, 777, 12)
    q, _, _ = orc.quantize_weight(w)
    assert not ((q & 0x7F) == 0x7F).any()


def test_I4_zero_rows(orc):
    w = np.zeros((3, 64), np.uint16)
    w[1, :] = 0x8000                       # -0.0
    w[2, 5] = 0x0001                       # smallest bf16 subnormal: clamp engages
    q, s, _ = orc.quantize_weight(w)
    assert (s.view(np.uint32) == 0x2B8CBCCC).all()
    assert (q[0] == 0).all() and (q[1] == 0x80).all()
    assert (q[2, :5] == 0).all() and q[2, 5] == 0  # 9.2e-41 / 1e-12 rounds to 0


def test_I5_power_of_two_scaling(orc):
    w = workloads.heavy_tail_weight(64, 256, 4)
    f = workloads.bf16_bits_to_f32(w)
    for j in (-3, 5):
        w2 = workloads.f32_to_bf16_bits(f * np.float32(2.0 ** j))
        q1, s1, _ = orc.quantize_weight(w)
        q2, s2, _ = orc.quantize_weight(w2)
        assert (q1 == q2).all()
        assert (s2 == s1 * np.float32(2.0 ** j)).all()


def test_I6_error_bound(orc):
    tab = orc.e4m3_table()
    w = workloads.heavy_tail_weight(128, 512, 6)
    q, s, _ = orc.quantize_weight(w)
    f = workloads.bf16_bits_to_f32(w).astype(np.float64)
    deq = tab[q] * s[:, None].astype(np.float64)
    bound = 2.0 ** -4 * np.abs(f) * (1 + 2.0 ** -19) + 2.0 ** -10 * s[:, None]
    assert (np.abs(deq - f) <= bound).all()


def test_I7_permutation_and_concatenation(orc):
    x = workloads.normal_act(8, 128, 21)
    q, s, _ = orc.quantize_act(x)
    perm = np.random.default_rng(1).permutation(x.size)
    xp = x.reshape(-1)[perm].reshape(x.shape)
    qp, sp, _ = orc.quantize_act(np.ascontiguousarray(xp))
    assert sp == s and (qp.reshape(-1) == q.reshape(-1)[perm]).all()
    g = workloads.heavy_tail_weight(48, 64, 30)
    u = workloads.heavy_tail_weight(40, 64, 31)
    qg, sg, _ = orc.quantize_weight(g)
    qu, su, _ = orc.quantize_weight(u)
    qc, sc, _ = orc.quantize_weight(np.concatenate([g, u]))
    assert (qc == np.concatenate([qg, qu])).all() and (sc == np.concatenate([sg, su])).all()


def test_double_rounding_reading(orc):
    """The quotient is rounded to fp32 first, then to E4M3 (two roundings).

    w = 0.087890625, s = fl32(0.087890625 * 2 / 21) lands fl32(w / s) exactly on
    10.5, which rounds to even (10); rounding the exact quotient once would
    have given 11.
    """
    w = np.float32(0.087890625)
    s = np.float32(0.0083705354)
    t = w / s
    assert t == np.float32(10.5)
    assert float(w) / float(s) > 10.5
    assert orc.cast_e4m3(t) == 0x52       # 10.0


def test_nonfinite_flag(orc):
    w = workloads.heavy_tail_weight(4, 16, 0)
    w[2, 3] = 0x7F80                       # +inf
    _, _, nf = orc.quantize_weight(w)
    assert nf
    x = workloads.normal_act(2, 8, 0)
    x[1, 1] = 0x7FC0                       # NaN
    _, _, nf = orc.quantize_act(x)
    assert nf
