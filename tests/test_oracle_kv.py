"""Pins for the oracle's FP8 KV-cache write with a running-max scale.

FP8量化与长上下文实测：Llama 3 70B部署优化指南 §3.2: each attention layer keeps a
running maximum that prefill batches raise and that decode reads as it stands;
the scale and cast are those of §3.1.  The cache layout is the contiguous
[kv_heads, seq_len, head_dim] of one layer ("Some Technical Notes About
Llama 3" commentary, §3.2).  The expected caches are built here with torch's
fp32 recipe and numpy indexing -- a route that shares nothing with the C
oracle -- and the running maximum with numpy's max.
"""
import numpy as np
import pytest

import workloads

torch = pytest.importorskip("torch")

H, D = 8, 128
SENTINEL = 0x5A


def amax_bits(x_bits: np.ndarray) -> np.float32:
    return np.float32(np.abs(workloads.bf16_bits_to_f32(x_bits)).max(initial=0.0))


def torch_scale(amax) -> np.float32:
    return np.float32((torch.tensor(np.float32(amax)) / 448.0).clamp(min=1e-12).item())


def torch_codes(x_bits: np.ndarray, s) -> np.ndarray:
    x = torch.from_numpy(workloads.bf16_bits_to_f32(x_bits))
    q = (x / torch.tensor(np.float32(s))).clamp(-448.0, 448.0)
    return q.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def expected_cache(cache: np.ndarray, x_bits: np.ndarray, s, slot: np.ndarray) -> np.ndarray:
    out = cache.copy()
    codes = torch_codes(x_bits, s).reshape(len(slot), H, D)
    ok = (slot >= 0) & (slot < cache.shape[1])
    out[:, slot[ok], :] = codes[ok].transpose(1, 0, 2)
    return out


def new_caches(s_rows: int):
    return (np.full((H, s_rows, D), SENTINEL, np.uint8), np.full((H, s_rows, D), SENTINEL, np.uint8))


def kv_pair(t: int, seed: int, v_gain: float = 0.3):
    k = workloads.outlier_act(t, H * D, seed)
    v = workloads.f32_to_bf16_bits(workloads.bf16_bits_to_f32(workloads.normal_act(t, H * D, seed + 1))
                                   * np.float32(v_gain))
    return k, v


@pytest.mark.parametrize("t,s_rows,seed", [(16, 64, 0), (5, 5, 1), (1, 40, 2), (77, 300, 3)])
def test_calibrating_write_matches_recipe(orc, t, s_rows, seed):
    k, v = kv_pair(t, seed)
    rng = np.random.default_rng(seed)
    slot = rng.permutation(s_rows)[:t].astype(np.int64)
    kc, vc = new_caches(s_rows)
    run, sc, fl = orc.kv_cache_write(k, v, H, slot, kc, vc, [0.0, 0.0], calibrate=True)
    assert fl == 0
    assert run[0] == amax_bits(k) and run[1] == amax_bits(v)
    assert sc[0] == torch_scale(run[0]) and sc[1] == torch_scale(run[1])
    kc0, vc0 = new_caches(s_rows)
    assert (kc == expected_cache(kc0, k, sc[0], slot)).all()
    assert (vc == expected_cache(vc0, v, sc[1], slot)).all()


def test_running_max_over_prefill_batches(orc):
    kc, vc = new_caches(512)
    run = np.zeros(2, np.float32)
    seen_k, seen_v = np.float32(0), np.float32(0)
    pos = 0
    for i, (t, gain) in enumerate([(64, 1.0), (32, 3.0), (100, 0.5), (7, 2.0)]):
        k, v = kv_pair(t, 10 + i, v_gain=gain)
        k = workloads.f32_to_bf16_bits(workloads.bf16_bits_to_f32(k) * np.float32(gain))
        slot = np.arange(pos, pos + t, dtype=np.int64)
        pos += t
        before_k, before_v = kc.copy(), vc.copy()
        run, sc, fl = orc.kv_cache_write(k, v, H, slot, kc, vc, run, calibrate=True)
        seen_k, seen_v = max(seen_k, amax_bits(k)), max(seen_v, amax_bits(v))
        assert fl == 0 and run[0] == seen_k and run[1] == seen_v, i
        # the batch is cast with the raised maximum, so nothing saturates in prefill
        assert (kc == expected_cache(before_k, k, torch_scale(seen_k), slot)).all(), i
        assert (vc == expected_cache(before_v, v, torch_scale(seen_v), slot)).all(), i


def test_decode_reads_scale_as_it_stands(orc):
    kc, vc = new_caches(64)
    k, v = kv_pair(32, 20)
    run, sc, _ = orc.kv_cache_write(k, v, H, np.arange(32), kc, vc, [0.0, 0.0], calibrate=True)
    # a decode batch four times larger: same scales, the excess saturates
    k2, v2 = kv_pair(3, 21, v_gain=1.2)
    k2 = workloads.f32_to_bf16_bits(workloads.bf16_bits_to_f32(k2) * 4)
    slot = np.array([40, 33, 63], np.int64)
    before_k, before_v = kc.copy(), vc.copy()
    run2, sc2, fl = orc.kv_cache_write(k2, v2, H, slot, kc, vc, run, calibrate=False)
    assert fl == 0 and (run2 == run).all() and (sc2 == sc).all()
    assert (kc == expected_cache(before_k, k2, sc[0], slot)).all()
    assert (vc == expected_cache(before_v, v2, sc[1], slot)).all()
    assert ((kc[:, slot, :] & 0x7F) == 0x7E).any()


def test_cold_start_saturates(orc):
    """Before any calibrating call the maximum is 0, the scale is the 1e-12 floor,
    and every non-zero value saturates: the page's reason for a warm-up."""
    kc, vc = new_caches(4)
    k, v = kv_pair(2, 30)
    _, sc, _ = orc.kv_cache_write(k, v, H, np.array([0, 1]), kc, vc, [0.0, 0.0], calibrate=False)
    assert sc[0] == np.float32(1e-12) and sc[1] == np.float32(1e-12)
    nz = workloads.bf16_bits_to_f32(k).reshape(2, H, D).transpose(1, 0, 2) != 0
    assert ((kc[:, :2, :] & 0x7F)[nz] == 0x7E).all()


def test_bad_slots_skipped_and_flagged(orc):
    kc, vc = new_caches(10)
    k, v = kv_pair(4, 40)
    slot = np.array([3, -1, 10, 9], np.int64)
    _, sc, fl = orc.kv_cache_write(k, v, H, slot, kc, vc, [0.0, 0.0], calibrate=True)
    assert fl == 2
    kc0, vc0 = new_caches(10)
    assert (kc == expected_cache(kc0, k, sc[0], slot)).all()
    untouched = [r for r in range(10) if r not in (3, 9)]
    assert (kc[:, untouched, :] == SENTINEL).all() and (vc[:, untouched, :] == SENTINEL).all()


def test_nonfinite_flag(orc):
    kc, vc = new_caches(4)
    k, v = kv_pair(2, 50)
    v[1, 7] = 0x7F80
    _, _, fl = orc.kv_cache_write(k, v, H, np.array([0, 1]), kc, vc, [1.0, 1.0], calibrate=False)
    assert fl & 1


def test_k_and_v_are_independent(orc):
    k, v = kv_pair(9, 60, v_gain=0.05)
    slot = np.arange(9, dtype=np.int64)
    a = new_caches(9)
    b = new_caches(9)
    ra, sa, _ = orc.kv_cache_write(k, v, H, slot, a[0], a[1], [0.5, 0.0], calibrate=True)
    rb, sb, _ = orc.kv_cache_write(v, k, H, slot, b[0], b[1], [0.0, 0.5], calibrate=True)
    assert (ra == rb[::-1]).all() and (sa == sb[::-1]).all()
    assert (a[0] == b[1]).all() and (a[1] == b[0]).all()


def test_strided_rows(orc):
    k, v = kv_pair(6, 70)
    kk = np.zeros((6, H * D + 64), np.uint16)
    vv = np.zeros((6, H * D + 64), np.uint16)
    kk[:, :H * D], vv[:, :H * D] = k, v
    slot = np.array([5, 0, 2, 1, 4, 3], np.int64)
    a, b = new_caches(6), new_caches(6)
    r1 = orc.kv_cache_write(k, v, H, slot, a[0], a[1], [0.0, 0.0], calibrate=True)
    r2 = orc.kv_cache_write(kk[:, :H * D], vv[:, :H * D], H, slot, b[0], b[1], [0.0, 0.0],
                            calibrate=True)
    assert (r1[0] == r2[0]).all() and (a[0] == b[0]).all() and (a[1] == b[1]).all()
