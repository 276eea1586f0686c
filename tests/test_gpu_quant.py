"""GPU parity of the quantizers against the oracle: codes and scales bit-exact.

Covers the E4M3 cast on every fp32 bit pattern, per-channel weight
quantization (FP8量化与长上下文实测：Llama 3 70B部署优化指南 §3.1) and dynamic
per-tensor activation quantization (§1.2) on ragged shapes, special rows and
every full-size workload, through the C ABI (via the thin binding).
"""
import numpy as np
import pytest

import workloads
from helpers import dev_bf16, host_f32, host_u8, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fq():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import fp8_weight_quantized_amd as fq
    fq.library_path()
    return fq


def same_bits_f32(a: np.ndarray, b: np.ndarray) -> bool:
    return a.shape == b.shape and bool((a.view(np.uint32) == b.view(np.uint32)).all())


def check_weight(fq, orc, w_bits: np.ndarray, what: str):
    say("quantize_weight", what, w_bits.shape)
    q, s = fq.quantize_weight(dev_bf16(w_bits))
    torch.cuda.synchronize()
    qr, sr, _ = orc.quantize_weight(w_bits)
    qg = host_u8(q)
    sg = host_f32(s)
    assert same_bits_f32(sg, sr), (what, np.flatnonzero(sg.view(np.uint32) != sr.view(np.uint32))[:5])
    bad = np.argwhere(qg != qr)
    assert bad.size == 0, (what, bad[:5].tolist(), [(int(qg[tuple(i)]), int(qr[tuple(i)])) for i in bad[:5]])


def check_act(fq, orc, x_bits: np.ndarray, what: str):
    say("quantize_act", what, x_bits.shape)
    q, s = fq.quantize_act(dev_bf16(x_bits))
    torch.cuda.synchronize()
    qr, sr, _ = orc.quantize_act(x_bits)
    assert host_f32(s)[0].view(np.uint32) == np.float32(sr).view(np.uint32), what
    qg = host_u8(q)
    bad = np.argwhere(qg != qr)
    assert bad.size == 0, (what, bad[:5].tolist())


def test_cast_every_fp32_pattern(fq, orc):
    """The device cast equals the oracle on all 2^32 fp32 inputs (NaN inputs excluded)."""
    chunk = 1 << 28
    idx = np.arange(chunk, dtype=np.uint32)
    for first in range(0, 1 << 32, chunk):
        say("cast chunk", hex(first))
        base = first if first < (1 << 31) else first - (1 << 32)
        vals = (torch.arange(chunk, dtype=torch.int32, device="cuda") + base).view(torch.float32)
        got = host_u8(fq.cast_f32_to_e4m3(vals))
        ref = orc.cast_e4m3_bits(first, chunk)
        nan = np.isnan((idx + np.uint32(first)).view(np.float32))
        bad = np.flatnonzero((got != ref) & ~nan)
        assert bad.size == 0, [(hex(first + int(i)), int(got[i]), int(ref[i])) for i in bad[:8]]


@pytest.mark.parametrize("n,k,seed", [
    (256, 512, 0), (33, 1000, 1), (7, 13, 2), (1, 1, 3), (300, 8, 4), (64, 4096, 6),
    (3, 7, 9), (130, 2056, 10),
    (5, 40000, 5),        # rows longer than the register-resident path: streamed twice
    (16, 32776, 7),
])
def test_weight_shapes(fq, orc, n, k, seed):
    check_weight(fq, orc, workloads.heavy_tail_weight(n, k, seed), f"heavy-tail seed {seed}")


def test_weight_strided(fq, orc):
    w = workloads.heavy_tail_weight(40, 1000, 3)
    big = np.zeros((40, 1024), np.uint16)
    big[:, :1000] = w
    dev = dev_bf16(big)[:, :1000]
    say("quantize_weight strided")
    q, s = fq.quantize_weight(dev)
    qr, sr, _ = orc.quantize_weight(w)
    assert (host_u8(q) == qr).all() and same_bits_f32(host_f32(s), sr)


def test_weight_special_rows(fq, orc):
    k = 96
    rows = []
    rows.append(np.zeros(k, np.uint16))                              # all +0: scale clamps
    rows.append(np.full(k, 0x8000, np.uint16))                       # all -0: codes 0x80
    r = np.zeros(k, np.uint16); r[7] = 0x0001; rows.append(r)        # bf16 subnormal only
    r = workloads.f32_to_bf16_bits(np.linspace(-3e38, 3e38, k)); rows.append(r)   # huge
    r = workloads.f32_to_bf16_bits(np.linspace(-1e-30, 1e-30, k)); rows.append(r)  # tiny
    r = workloads.f32_to_bf16_bits(np.full(k, 448.0)); rows.append(r)   # constant rows
    r = workloads.f32_to_bf16_bits(np.full(k, -0.0625)); rows.append(r)
    rng = np.random.default_rng(0)
    r = rng.integers(0, 1 << 16, k).astype(np.uint16)
    r[(r & 0x7F80) == 0x7F80] = 0x3F80                              # random finite bit patterns
    rows.append(r)
    check_weight(fq, orc, np.stack(rows), "special rows")


def test_weight_nonfinite_flag(fq):
    w = workloads.heavy_tail_weight(8, 64, 1)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    fq.quantize_weight(dev_bf16(w), nonfinite_flag=flag)
    assert int(flag.item()) == 0
    w[3, 9] = 0x7F80
    fq.quantize_weight(dev_bf16(w), nonfinite_flag=flag)
    assert int(flag.item()) == 1


WEIGHT_CONFIGS = [(wl.key, lin) for wl in workloads.WORKLOADS.values() for lin in wl.linears]


@pytest.mark.parametrize("key,lin", WEIGHT_CONFIGS, ids=[f"{k}-{l.name}" for k, l in WEIGHT_CONFIGS])
def test_weight_full_workloads(fq, orc, key, lin):
    wl = workloads.WORKLOADS[key]
    check_weight(fq, orc, workloads.weight(wl, lin), f"{key}/{lin.name}")


@pytest.mark.parametrize("m,k,seed", [(16, 512, 0), (5, 77, 1), (1, 4096, 2), (64, 4096, 3),
                                      (12, 8192, 4), (1, 8, 5), (3, 13, 6), (257, 1032, 7)])
def test_act_shapes(fq, orc, m, k, seed):
    check_act(fq, orc, workloads.outlier_act(m, k, seed), f"outlier seed {seed}")


def test_act_empty_and_zero(fq, orc):
    say("quantize_act empty")
    q, s = fq.quantize_act(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"))
    assert q.shape == (0, 64)
    assert host_f32(s)[0].view(np.uint32) == 0x2B8CBCCC
    check_act(fq, orc, np.zeros((4, 64), np.uint16), "all zero")
    check_act(fq, orc, np.full((4, 64), 0x8000, np.uint16), "all -0")


def test_act_strided(fq, orc):
    x = workloads.normal_act(9, 200, 4)
    big = np.zeros((9, 256), np.uint16)
    big[:, :200] = x
    say("quantize_act strided")
    q, s = fq.quantize_act(dev_bf16(big)[:, :200])
    qr, sr, _ = orc.quantize_act(x)
    assert (host_u8(q) == qr).all() and host_f32(s)[0] == sr


def test_act_nonfinite_flag(fq):
    x = workloads.normal_act(4, 256, 1)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    fq.quantize_act(dev_bf16(x), nonfinite_flag=flag)
    assert int(flag.item()) == 0
    x[2, 100] = 0x7FC0
    fq.quantize_act(dev_bf16(x), nonfinite_flag=flag)
    assert int(flag.item()) == 1


@pytest.mark.parametrize("key", ["mlp_prefill", "down_prefill_70b"])
def test_act_full_workloads(fq, orc, key):
    wl = workloads.WORKLOADS[key]
    lin = wl.linears[0]
    check_act(fq, orc, workloads.activation(wl, wl.ms[0], lin.k), key)


def test_division_every_bf16_numerator(fq, orc):
    """For 160 scales, every finite bf16 value up to the tensor's absmax is divided
    and cast: the quotient rounding (IEEE fp32 division, then RNE to E4M3) is
    exercised on all numerators."""
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = allbits[(allbits & 0x7F80) != 0x7F80]
    mags = workloads.bf16_bits_to_f32(finite)
    rng = np.random.default_rng(42)
    picks = list(rng.choice(np.abs(mags[mags != 0]), 120, replace=False))
    picks += [2.0 ** e for e in range(-133, 128, 7)]
    picks += [448.0, 1.0, 3.0e-10, 1.0e-38]
    for j, amax in enumerate(picks[:160]):
        amax = np.float32(amax)
        sel = finite[np.abs(mags) <= amax]
        if sel.size == 0:
            continue
        pad = (-sel.size) % 8
        x = np.concatenate([sel, np.zeros(pad, np.uint16)]).reshape(-1, 8)
        check_act(fq, orc, x, f"division sweep {j} amax={float(amax)!r}")
