"""GPU parity of static and EMA-scaled activation quantization against the oracle.

Static: the per-tensor cast of FP8量化与长上下文实测：Llama 3 70B部署优化指南
§3.1 / §1.2 with a held scale.  EMA: the moving-average activation scale of
the "Llama 3 精读" write-up (§3.1 step 2, decay 0.9999; §5.3 tip 2,
temperature).  Codes, the scale each call used and the state after each call
are compared bit for bit with the oracle over call sequences, in all three
memory layouts, on the full prefill activation, through the W8A8 GEMM, and
under HIP graph replay (the write-up runs its FP8 kernels in CUDA graphs).
"""
import numpy as np
import pytest

import workloads
from helpers import assert_gemm_close, dev_bf16, dev_u8, host_bf16_as_f64, host_f32, host_u8, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fq():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import fp8_weight_quantized_amd as fq
    fq.library_path()
    return fq


def bits(v) -> int:
    return int(np.float32(v).view(np.uint32))


def dev_scalar(v) -> "torch.Tensor":
    return torch.tensor([np.float32(v)], dtype=torch.float32, device="cuda")


def assert_codes(qg: np.ndarray, qr: np.ndarray, what):
    bad = np.argwhere(qg != qr)
    assert bad.size == 0, (what, bad[:5].tolist(),
                           [(int(qg[tuple(i)]), int(qr[tuple(i)])) for i in bad[:5]])


# ------------------------------------------------------------------ static --
def check_static(fq, orc, x_bits: np.ndarray, s, what, x_dev=None):
    say("quantize_act_static", what, x_bits.shape, float(s))
    xd = dev_bf16(x_bits) if x_dev is None else x_dev
    q = fq.quantize_act_static(xd, dev_scalar(s))
    torch.cuda.synchronize()
    qr, _ = orc.quantize_act_static(x_bits, s)
    assert_codes(host_u8(q), qr, what)
    return qr


@pytest.mark.parametrize("m,k,seed", [(16, 512, 0), (5, 77, 1), (1, 4096, 2), (64, 4096, 3),
                                      (12, 8192, 4), (1, 8, 5), (3, 13, 6), (257, 1032, 7)])
@pytest.mark.parametrize("frac", [1.0, 0.37, 0.02, 2.5])
def test_static_shapes(fq, orc, m, k, seed, frac):
    x = workloads.outlier_act(m, k, seed)
    _, s_dyn, _ = orc.quantize_act(x)
    s = np.float32(s_dyn * np.float32(frac))
    qr = check_static(fq, orc, x, s, f"outlier seed {seed} frac {frac}")
    if frac < 1.0:
        assert ((qr & 0x7F) == 0x7E).any()     # saturation reached on this case


def test_static_layouts(fq, orc):
    x = workloads.normal_act(9, 200, 4)
    big = np.zeros((9, 256), np.uint16)
    big[:, :200] = x
    # rows layout: 16-byte aligned rows with a row stride above k
    check_static(fq, orc, x, 0.004, "rows layout", dev_bf16(big)[:, :200])
    # element layout: a row stride that is not a multiple of 8
    odd = np.zeros((9, 203), np.uint16)
    odd[:, :200] = x
    check_static(fq, orc, x, 0.004, "element layout", dev_bf16(odd)[:, :200])


def test_static_every_bf16_numerator(fq, orc):
    """Every finite bf16 value, cast with held scales that clip most of them.
    Scales 1 and 2^-20 put quotients exactly on E4M3 midpoints (the cast's
    exact-division fallback); 1e38, 3e38 and 2^-126 have a reciprocal outside
    the range where the reciprocal product is used, so every element takes
    the exact division."""
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = allbits[(allbits & 0x7F80) != 0x7F80]
    x = finite.reshape(-1, 8)
    for s in (1.0, 3.7e-3, 2.0 ** -20, 1.234e5, 1e-12, 7.1e30, 1e38, 3e38, 2.0 ** -126):
        check_static(fq, orc, x, np.float32(s), f"all bf16, scale {s!r}")


def test_static_empty_and_flag(fq, orc):
    q = fq.quantize_act_static(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"),
                               dev_scalar(1.0))
    assert q.shape == (0, 64)
    x = workloads.normal_act(4, 256, 1)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    fq.quantize_act_static(dev_bf16(x), dev_scalar(0.01), nonfinite_flag=flag)
    assert int(flag.item()) == 0
    x[3, 255] = 0xFF80                              # -inf
    fq.quantize_act_static(dev_bf16(x), dev_scalar(0.01), nonfinite_flag=flag)
    assert int(flag.item()) == 1


# --------------------------------------------------------------------- EMA --
def ema_sequence(fq, orc, xs, decay, temperature, what, x_devs=None):
    """Run one EMA state over the tensors xs on both sides; compare every call."""
    ema = fq.EmaActScale("cuda", decay, temperature)
    state = np.float32(0.0)
    outs = []
    for i, x in enumerate(xs):
        say("quantize_act_ema", what, i, x.shape, decay, temperature)
        xd = dev_bf16(x) if x_devs is None else x_devs[i]
        q, used = ema(xd)
        torch.cuda.synchronize()
        qr, used_r, state, _ = orc.quantize_act_ema(x, state, decay, temperature, seed=(i == 0))
        assert_codes(host_u8(q), qr, (what, i))
        assert bits(host_f32(used)[0]) == bits(used_r), (what, i, host_f32(used)[0], used_r)
        assert bits(host_f32(ema.state)[0]) == bits(state), (what, i, host_f32(ema.state)[0], state)
        outs.append((q, used, qr, used_r))
    return outs


def mixed_inputs(k: int, base_seed: int):
    xs = [workloads.outlier_act(m, k, base_seed + i) for i, m in enumerate((64, 1, 8, 64, 33, 1))]
    # a tenfold jump in range on call 3 and a collapse on call 5
    xs[3] = workloads.f32_to_bf16_bits(workloads.bf16_bits_to_f32(xs[3]) * 10)
    xs[5] = workloads.f32_to_bf16_bits(workloads.bf16_bits_to_f32(xs[5]) * 0.01)
    return xs


@pytest.mark.parametrize("decay,temperature", [(0.9999, 0.0), (0.9999, 0.1), (0.9999, 1.0),
                                               (0.9, 0.0), (0.5, 1.0), (0.0, 0.0), (1.0, 0.0)])
def test_ema_sequence(fq, orc, decay, temperature):
    ema_sequence(fq, orc, mixed_inputs(4096, 100), decay, temperature, "mixed")


@pytest.mark.parametrize("k", [77, 1032, 8192])
def test_ema_ragged_k(fq, orc, k):
    ema_sequence(fq, orc, mixed_inputs(k, 200), 0.9, 0.1, f"k={k}")


def test_ema_layouts(fq, orc):
    xs = [workloads.normal_act(9, 200, 10 + i) for i in range(4)]
    xs[2] = workloads.f32_to_bf16_bits(workloads.bf16_bits_to_f32(xs[2]) * 6)
    for ld, name in ((256, "rows layout"), (203, "element layout")):
        devs = []
        for x in xs:
            big = np.zeros((9, ld), np.uint16)
            big[:, :200] = x
            devs.append(dev_bf16(big)[:, :200])
        ema_sequence(fq, orc, xs, 0.8, 0.0, name, devs)


def test_ema_empty_tensor(fq, orc):
    """An empty tensor is a tensor whose maximum is 0: the state moves towards 1e-12."""
    xs = [workloads.outlier_act(4, 64, 1), np.zeros((0, 64), np.uint16),
          workloads.outlier_act(4, 64, 2)]
    ema_sequence(fq, orc, xs, 0.5, 0.0, "empty")


def test_ema_full_prefill_activation(fq, orc):
    wl = workloads.WORKLOADS["mlp_prefill"]
    lin = wl.linears[0]
    x0 = workloads.activation(wl, wl.ms[0], lin.k)
    x1 = workloads.outlier_act(wl.ms[0], lin.k, 77)
    ema_sequence(fq, orc, [x0, x1], 0.9999, 0.1, "mlp_prefill X[8192,4096]")


def test_ema_nonfinite_flag(fq):
    st = torch.zeros(1, dtype=torch.float32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    x = workloads.normal_act(4, 256, 1)
    fq.quantize_act_ema(dev_bf16(x), st, seed=True, nonfinite_flag=flag)
    fq.quantize_act_ema(dev_bf16(x), st, nonfinite_flag=flag)
    assert int(flag.item()) == 0
    x[0, 0] = 0x7FC0
    fq.quantize_act_ema(dev_bf16(x), st, nonfinite_flag=flag)
    assert int(flag.item()) == 1


@pytest.mark.parametrize("m", [1, 64, 300])
def test_ema_codes_through_w8a8(fq, orc, m):
    """The EMA codes and the scale they were made with drive fp8_w_fp8_a."""
    n, k = 512, 4096
    wq, ws, _ = orc.quantize_weight(workloads.heavy_tail_weight(n, k, 5))
    xs = [workloads.outlier_act(m, k, 300 + i) for i in range(3)]
    outs = ema_sequence(fq, orc, xs, 0.9, 0.0, f"w8a8 m={m}")
    wd, wsd = dev_u8(wq), torch.from_numpy(ws).cuda()
    for i, (q, used, qr, used_r) in enumerate(outs):
        say("linear w8a8 after ema", m, i)
        y = fq.linear(q, wd, wsd, x_scale=used)
        torch.cuda.synchronize()
        ref = orc.linear(1, qr, wq, ws, x_scale=used_r)
        assert_gemm_close(host_bf16_as_f64(y), ref, f"ema w8a8 m={m} call {i}")


def test_ema_graph_replay(fq, orc):
    """Captured once, replayed: every replay takes one EMA step, as eager calls do."""
    m, k = 64, 4096
    xs = [workloads.outlier_act(m, k, 400 + i) for i in range(5)]
    xs[2] = workloads.f32_to_bf16_bits(workloads.bf16_bits_to_f32(xs[2]) * 4)
    decay, temp = 0.9, 0.1
    ema = fq.EmaActScale("cuda", decay, temp)
    xbuf = dev_bf16(xs[0])
    ema(xbuf)                                         # seeded eagerly
    torch.cuda.synchronize()
    _, _, state, _ = orc.quantize_act_ema(xs[0], 0.0, decay, temp, seed=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    say("ema graph capture")
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            q, used = ema(xbuf)
    torch.cuda.current_stream().wait_stream(s)
    # capturing enqueues nothing: the state is still the seeded one
    torch.cuda.synchronize()
    assert bits(host_f32(ema.state)[0]) == bits(state)
    for i, x in enumerate(xs[1:], start=1):
        say("ema graph replay", i)
        xbuf.copy_(dev_bf16(x))
        g.replay()
        torch.cuda.synchronize()
        qr, used_r, state, _ = orc.quantize_act_ema(x, state, decay, temp)
        assert_codes(host_u8(q), qr, ("replay", i))
        assert bits(host_f32(used)[0]) == bits(used_r), ("replay", i)
        assert bits(host_f32(ema.state)[0]) == bits(state), ("replay", i)
        torch.zeros(1 << 20, device="cuda").sum()     # unrelated eager work between replays
