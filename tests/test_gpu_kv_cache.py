"""GPU parity of the FP8 KV-cache write against the oracle, bit for bit.

FP8量化与长上下文实测：Llama 3 70B部署优化指南 §3.2: each attention layer keeps
a running maximum that prefill (calibrating) batches raise and decode reads
as it stands.  Whole caches, running maxima, scales and flags are compared
after every call: calibrating prefill chunks of several sizes, a warm-up then
decode sequence, head counts and widths, K/V slices of a fused QKV output,
bad slots, non-finite input, an empty batch, the Llama-3-70B prefill chunk
at full size, and HIP graph replay of a decode write.
"""
import numpy as np
import pytest

import workloads
from helpers import dev_bf16, dev_u8, host_f32, host_u8, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SENTINEL = 0x5A


@pytest.fixture(scope="module")
def fq():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import fp8_weight_quantized_amd as fq
    fq.library_path()
    return fq


class Layer:
    """One layer's caches and running maxima, on the device and in the oracle."""

    def __init__(self, heads, slots, head_dim):
        self.h, self.s, self.d = heads, slots, head_dim
        self.kc = np.full((heads, slots, head_dim), SENTINEL, np.uint8)
        self.vc = self.kc.copy()
        self.run = np.zeros(2, np.float32)
        self.kc_d, self.vc_d = dev_u8(self.kc), dev_u8(self.vc)
        self.run_d = torch.zeros(2, dtype=torch.float32, device="cuda")

    def write(self, fq, orc, k, v, slot, calibrate, what, k_dev=None, v_dev=None):
        say("kv_cache_write", what, k.shape, self.h, self.s, self.d, calibrate)
        flags = torch.zeros(1, dtype=torch.int32, device="cuda")
        sc = fq.kv_cache_write(dev_bf16(k) if k_dev is None else k_dev,
                               dev_bf16(v) if v_dev is None else v_dev,
                               torch.from_numpy(np.asarray(slot, np.int64)).cuda(),
                               self.kc_d, self.vc_d, self.run_d, calibrate, flags=flags)
        torch.cuda.synchronize()
        self.run, sc_r, fl_r = orc.kv_cache_write(k, v, self.h, np.asarray(slot, np.int64), self.kc,
                                                  self.vc, self.run, calibrate)
        self.check(what)
        assert (host_f32(sc).view(np.uint32) == sc_r.view(np.uint32)).all(), (what, host_f32(sc), sc_r)
        assert int(flags.item()) == fl_r, (what, int(flags.item()), fl_r)
        return sc_r, fl_r

    def check(self, what):
        for name, dev, ref in (("k", self.kc_d, self.kc), ("v", self.vc_d, self.vc)):
            got = host_u8(dev)
            bad = np.argwhere(got != ref)
            assert bad.size == 0, (what, name, bad[:5].tolist())
        assert (host_f32(self.run_d).view(np.uint32) == self.run.view(np.uint32)).all(), \
            (what, host_f32(self.run_d), self.run)


def kv_batch(t, width, seed, k_gain=1.0, v_gain=0.3):
    k = workloads.outlier_act(t, width, seed)
    v = workloads.normal_act(t, width, seed + 1)
    scale = lambda a, g: workloads.f32_to_bf16_bits(workloads.bf16_bits_to_f32(a) * np.float32(g))  # noqa: E731
    return scale(k, k_gain), scale(v, v_gain)


@pytest.mark.parametrize("t,s_rows", [(1, 16), (16, 64), (77, 300), (300, 300), (2048, 4096)])
def test_calibrating_prefill(fq, orc, t, s_rows):
    L = Layer(8, s_rows, 128)
    k, v = kv_batch(t, 8 * 128, t)
    slot = np.random.default_rng(t).permutation(s_rows)[:t]
    L.write(fq, orc, k, v, slot, True, f"prefill t={t}")


def test_warmup_then_decode(fq, orc):
    """Warm-up prefill batches raise the maxima; decode steps saturate beyond them."""
    L = Layer(8, 2048, 128)
    pos = 0
    for i, (t, g) in enumerate([(256, 1.0), (128, 2.5), (512, 0.7)]):
        k, v = kv_batch(t, 1024, 10 + i, k_gain=g, v_gain=0.3 * g)
        L.write(fq, orc, k, v, np.arange(pos, pos + t), True, f"warm-up {i}")
        pos += t
    for step in range(4):
        # a batch of 12 sequences, one new token each, some well beyond the range
        k, v = kv_batch(12, 1024, 50 + step, k_gain=1.0 + 2 * step, v_gain=0.5)
        slot = pos + np.arange(12) * 40 + step
        L.write(fq, orc, k, v, slot, False, f"decode {step}")
    assert ((L.kc[:, pos:, :] & 0x7F) == 0x7E).any()     # decode saturated somewhere


def test_held_arbitrary_running_max(fq, orc):
    """Running maxima set by the caller to fp32 values no bf16 maximum gives
    (so the scale r / 448 is not of the dynamic form), on a write large
    enough (32 heads x 128, 2048 tokens: 4 chunks per thread) for the cast to
    take one reciprocal and two FMA correction steps per value: every code
    must still equal the oracle's, which divides."""
    L = Layer(32, 2048, 128)
    L.run = np.array([np.float32(2.7182817), np.float32(0.33333334)], np.float32)
    L.run_d.copy_(torch.from_numpy(L.run.copy()))
    k, v = kv_batch(2048, 32 * 128, 7, k_gain=0.5, v_gain=0.1)
    L.write(fq, orc, k, v, np.arange(2048), False, "held, arbitrary running max")
    # a calibrating write whose maxima stay below the running maxima keeps them
    k, v = kv_batch(2048, 32 * 128, 8, k_gain=0.01, v_gain=0.001)
    L.write(fq, orc, k, v, np.arange(2048)[::-1].copy(), True, "calibrating, maxima below")
    assert (L.run == np.array([np.float32(2.7182817), np.float32(0.33333334)], np.float32)).all()


@pytest.mark.parametrize("heads,head_dim", [(1, 8), (4, 64), (32, 128), (2, 136), (8, 256)])
def test_head_shapes(fq, orc, heads, head_dim):
    L = Layer(heads, 96, head_dim)
    k, v = kv_batch(40, heads * head_dim, heads * 1000 + head_dim)
    L.write(fq, orc, k, v, np.arange(40) * 2, True, "shape calibrate")
    k, v = kv_batch(5, heads * head_dim, heads * 1000 + head_dim + 7, k_gain=3.0)
    L.write(fq, orc, k, v, [1, 3, 5, 95, 7], False, "shape decode")


def test_slices_of_fused_qkv(fq, orc):
    """K and V as column slices of a fused QKV projection output (Llama-3-70B:
    64 query heads, 8 KV heads, head_dim 128; row stride 10240)."""
    t, hq, hkv, d = 33, 64, 8, 128
    width = (hq + 2 * hkv) * d
    qkv = workloads.outlier_act(t, width, 5)
    q_end, k_end = hq * d, (hq + hkv) * d
    k, v = np.ascontiguousarray(qkv[:, q_end:k_end]), np.ascontiguousarray(qkv[:, k_end:])
    qkv_d = dev_bf16(qkv)
    L = Layer(hkv, 64, d)
    L.write(fq, orc, k, v, np.arange(t), True, "fused qkv", qkv_d[:, q_end:k_end], qkv_d[:, k_end:])


def test_bad_slots(fq, orc):
    L = Layer(8, 10, 128)
    k, v = kv_batch(6, 1024, 60)
    _, fl = L.write(fq, orc, k, v, [3, -1, 10, 9, 1 << 40, 0], True, "bad slots")
    assert fl == 2


def test_nonfinite_input(fq, orc):
    L = Layer(8, 10, 128)
    k, v = kv_batch(4, 1024, 70)
    L.write(fq, orc, k, v, np.arange(4), True, "finite")
    v[2, 300] = 0x7F80
    _, fl = L.write(fq, orc, k, v, np.arange(4, 8), False, "inf in v (decode)")
    assert fl == 1


def test_empty_batch(fq, orc):
    L = Layer(8, 10, 128)
    k, v = kv_batch(4, 1024, 80)
    L.write(fq, orc, k, v, np.arange(4), True, "before")
    e = np.zeros((0, 1024), np.uint16)
    sc, fl = L.write(fq, orc, e, e, np.zeros(0, np.int64), True, "empty calibrating")
    assert fl == 0


def test_full_70b_prefill_chunk(fq, orc):
    """Llama-3-70B layer: 8 KV heads x 128, an 8192-token prefill chunk into an
    8192-row cache, then a 12-token decode step."""
    L = Layer(8, 8192, 128)
    k, v = kv_batch(8192, 1024, 90)
    L.write(fq, orc, k, v, np.arange(8192), True, "70b prefill 8192")
    k, v = kv_batch(12, 1024, 91, k_gain=1.5)
    L.write(fq, orc, k, v, np.arange(8000, 8012), False, "70b decode 12")


def test_decode_graph_replay(fq, orc):
    """A decode write captured once and replayed with new tokens and slots."""
    L = Layer(8, 512, 128)
    k, v = kv_batch(256, 1024, 100)
    L.write(fq, orc, k, v, np.arange(256), True, "graph warm-up")
    kb = torch.empty((12, 1024), dtype=torch.bfloat16, device="cuda")
    vb = torch.empty_like(kb)
    sb = torch.zeros(12, dtype=torch.int64, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    say("kv graph capture")
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            sc = fq.kv_cache_write(kb, vb, sb, L.kc_d, L.vc_d, L.run_d, False)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    L.check("after capture")                          # capture wrote nothing
    for i in range(4):
        say("kv graph replay", i)
        k, v = kv_batch(12, 1024, 110 + i, k_gain=1.0 + i)
        slot = 256 + np.arange(12) * 20 + i
        kb.copy_(dev_bf16(k))
        vb.copy_(dev_bf16(v))
        sb.copy_(torch.from_numpy(slot.astype(np.int64)))
        g.replay()
        torch.cuda.synchronize()
        L.run, sc_r, _ = orc.kv_cache_write(k, v, 8, slot.astype(np.int64), L.kc, L.vc, L.run, False)
        L.check(f"replay {i}")
        assert (host_f32(sc).view(np.uint32) == sc_r.view(np.uint32)).all()
        torch.zeros(1 << 20, device="cuda").sum()
