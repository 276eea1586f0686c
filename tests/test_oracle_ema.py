"""Pins for the oracle's static and EMA-scaled activation quantization.

Static scale: the conversion of FP8量化与长上下文实测：Llama 3 70B部署优化指南
§3.1 with the per-tensor scale given instead of recomputed (§1.2), run with
torch in fp32 -- a library route that shares nothing with the C oracle --
must give the same codes, including the saturation that a held scale makes
reachable.

EMA scale: "Llama 3 精读" FP8 + 128K write-up §3.1 step 2 (decay 0.9999) and
§5.3 tip 2 (temperature term).  The update is pinned by closed forms: the
special decays 0 and 1, exactly representable steps, the geometric approach
to the fixed point s_new * (1 + 0.1 T) with its fp32 error bound, and the
1e-12 floor.  The call semantics (delayed scale, seeding) are pinned against
the already pinned dynamic and static quantizers.
"""
import numpy as np
import pytest

import workloads

torch = pytest.importorskip("torch")


def torch_static(x_bits: np.ndarray, s: float) -> np.ndarray:
    x = torch.from_numpy(workloads.bf16_bits_to_f32(x_bits))
    q = (x / torch.tensor(np.float32(s))).clamp(-448.0, 448.0)
    return q.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def f32(v) -> float:
    return float(np.float32(v))


# ------------------------------------------------------------------ static --
@pytest.mark.parametrize("m,k,seed", [(16, 512, 0), (5, 77, 1), (64, 4096, 2)])
@pytest.mark.parametrize("frac", [1.0, 0.25, 0.013, 3.7])
def test_static_matches_page_recipe(orc, m, k, seed, frac):
    """Held scale = frac * dynamic scale; frac < 1 forces saturation."""
    x = workloads.outlier_act(m, k, seed)
    _, s_dyn, _ = orc.quantize_act(x)
    s = np.float32(s_dyn * np.float32(frac))
    q, nf = orc.quantize_act_static(x, s)
    assert not nf
    assert (q == torch_static(x, s)).all()
    if frac < 1.0:
        sat = (q & 0x7F) == 0x7E
        assert sat.sum() > 0           # the held scale really clips something


def test_static_at_dynamic_scale_is_dynamic(orc):
    x = workloads.outlier_act(33, 1000, 7)
    q_dyn, s_dyn, _ = orc.quantize_act(x)
    q, _ = orc.quantize_act_static(x, s_dyn)
    assert (q == q_dyn).all()


def test_static_saturation_values(orc):
    """Beyond 448 * s every value maps to +-448 (codes 0x7E / 0xFE), sign kept."""
    vals = np.array([[1000.0, -1000.0, 449.0, -465.0, 3e38, -3e38, 448.0, 0.0, -0.0]], np.float32)
    x = workloads.f32_to_bf16_bits(vals)
    q, _ = orc.quantize_act_static(x, 1.0)
    assert q.tolist() == [[0x7E, 0xFE, 0x7E, 0xFE, 0x7E, 0xFE, 0x7E, 0x00, 0x80]]


def test_static_power_of_two_scale_is_exact_shift(orc):
    """s = 2^j: X / s is exact, so the codes are the bare cast of X * 2^-j."""
    x = workloads.outlier_act(8, 256, 3)
    xf = workloads.bf16_bits_to_f32(x)
    for j in (-3, 0, 2, 5):
        q, _ = orc.quantize_act_static(x, 2.0 ** j)
        ref = orc.cast_e4m3_array((xf * np.float32(2.0 ** -j)).astype(np.float32))
        assert (q == ref).all(), j


def test_static_nonfinite_flag(orc):
    x = workloads.outlier_act(4, 64, 4)
    x[2, 5] = 0x7F80                   # +inf
    _, nf = orc.quantize_act_static(x, 1.0)
    assert nf


# --------------------------------------------------------------- EMA update --
def test_ema_decay_one_freezes(orc):
    for s_old, s_new in [(0.5, 9.0), (3e-5, 1e-12), (7.25, 7.25)]:
        for t in (0.0, 0.1, 1.0):
            assert orc.ema_scale(s_old, s_new, 1.0, t) == np.float32(s_old)


def test_ema_decay_zero_follows(orc):
    for s_old, s_new in [(0.5, 9.0), (3e-5, 0.37), (7.25, 1e-12)]:
        assert orc.ema_scale(s_old, s_new, 0.0, 0.0) == np.float32(s_new)


def test_ema_exact_steps(orc):
    # 0.75 * 2 + 0.25 * 4 = 2.5, every intermediate exact in fp32
    assert orc.ema_scale(2.0, 4.0, 0.75, 0.0) == np.float32(2.5)
    # T = 10: 1 + 0.1 * 10 rounds to exactly 2 in fp32, so the new term doubles
    assert orc.ema_scale(2.0, 4.0, 0.75, 10.0) == np.float32(3.5)
    # d = 0.5, T = 5: heat = 1 + fl(0.1f * 5) = 1.5 exactly
    assert orc.ema_scale(1.0, 8.0, 0.5, 5.0) == np.float32(0.5 + 4.0 * 1.5)


def test_ema_page_decay_one_step(orc):
    """d = 0.9999 against the exact real-number update of the fp32 inputs."""
    rng = np.random.default_rng(11)
    d = np.float32(0.9999)
    for _ in range(200):
        s_old = np.float32(rng.uniform(1e-3, 1.0))
        s_new = np.float32(s_old * np.float32(rng.uniform(0.2, 5.0)))
        t = np.float32(rng.choice([0.0, 0.1, 1.0]))
        heat = 1.0 + float(np.float32(np.float32(0.1) * t))
        exact = float(d) * float(s_old) + (1.0 - float(d)) * float(s_new) * heat
        got = float(orc.ema_scale(s_old, s_new, d, t))
        # five fp32 roundings, each within half an ulp of its result
        assert abs(got - exact) <= 4 * np.finfo(np.float32).eps * exact


@pytest.mark.parametrize("d,t", [(0.5, 0.0), (0.9, 0.0), (0.5, 1.0), (0.75, 0.1)])
def test_ema_geometric_approach(orc, d, t):
    """Constant input: s_t - s* = d^t (s_0 - s*), s* = s_new (1 + 0.1 T)."""
    s0, s_new = 0.02, 0.3
    heat = 1.0 + float(np.float32(np.float32(0.1) * np.float32(t)))
    star = float(np.float32(s_new)) * heat
    s = np.float32(s0)
    for step in range(1, 61):
        s = orc.ema_scale(s, s_new, d, t)
        want = star + d ** step * (float(np.float32(s0)) - star)
        # errors do not grow: each step damps the earlier ones by d
        bound = 6 * np.finfo(np.float32).eps * star / (1.0 - d)
        assert abs(float(s) - want) <= bound, (step, float(s), want)


def test_ema_floor(orc):
    tiny = np.float32(1e-12)
    assert orc.ema_scale(tiny, tiny, 0.9999, 0.0) >= tiny
    assert orc.ema_scale(tiny, tiny, 0.3, 0.0) >= tiny
    assert orc.ema_scale(tiny, tiny, 0.9999, 0.0) == tiny


# ------------------------------------------------------------ EMA call ----
def test_ema_call_sequence(orc):
    """Seed = dynamic; each later call casts with the previous state."""
    xs = [workloads.outlier_act(12, 300, 20 + i) for i in range(5)]
    xs[3] = (workloads.bf16_bits_to_f32(xs[3]) * 8).astype(np.float32)
    xs[3] = workloads.f32_to_bf16_bits(xs[3])   # a jump in range: saturation on this call
    d, t = 0.9, 0.1
    q0, used0, st, nf = orc.quantize_act_ema(xs[0], 0.0, d, t, seed=True)
    qd, sd, _ = orc.quantize_act(xs[0])
    assert (q0 == qd).all() and used0 == sd and st == sd and not nf
    for x in xs[1:]:
        prev = st
        q, used, st, nf = orc.quantize_act_ema(x, prev, d, t)
        q_static, _ = orc.quantize_act_static(x, prev)
        _, s_dyn, _ = orc.quantize_act(x)
        assert used == prev
        assert (q == q_static).all()
        assert st == orc.ema_scale(prev, s_dyn, d, t)


def test_ema_call_page_decay_barely_moves(orc):
    """With d = 0.9999 a tenfold jump moves the scale by about 0.1 %."""
    x = workloads.outlier_act(8, 512, 30)
    _, _, s, _ = orc.quantize_act_ema(x, 0.0, 0.9999, 0.0, seed=True)
    big = workloads.f32_to_bf16_bits(workloads.bf16_bits_to_f32(x) * 10)
    _, used, s2, _ = orc.quantize_act_ema(big, s, 0.9999, 0.0)
    assert used == s
    assert 1.0008 < float(s2) / float(s) < 1.0010


def test_ema_call_empty_tensor(orc):
    """An empty tensor has maximum 0: one step towards the 1e-12 floor, no codes."""
    x = np.zeros((0, 64), np.uint16)
    q, used, st, nf = orc.quantize_act_ema(x, 0.25, 0.5, 0.0)
    assert q.shape == (0, 64) and not nf
    assert used == np.float32(0.25)
    assert st == orc.ema_scale(0.25, 1e-12, 0.5, 0.0)
    assert abs(float(st) - (0.125 + 0.5e-12)) <= 1e-7 * 0.125
