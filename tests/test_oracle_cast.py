"""Pins for the oracle's fp32 -> E4M3 cast (round to nearest even, saturating).

What pins it, independently of the oracle's own code:
  * hand-worked cases from the format (tests/golden/cast_examples.json);
  * a second route inside the oracle (linear arg-min scan) on every boundary;
  * torch's float8_e4m3fn cast after a clamp to [-448, 448] -- a library
    special case -- on every finite fp32 bit pattern;
  * the textbook properties: round-trip error bound, saturation, monotonicity
    and odd symmetry.
The pages ask for the RNE cast of torch.float8_e4m3fn
(FP8量化与长上下文实测：Llama 3 70B部署优化指南 §3.1) within the symmetric
[-448, 448] range (Llama 3 精读 §2.1).
"""
import json
import os

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden", "cast_examples.json")


def test_golden_cases(orc):
    with open(GOLD) as f:
        cases = json.load(f)["cases"]
    for value, code, why in cases:
        assert orc.cast_e4m3(value) == code, (value, why)
        assert orc.cast_e4m3_scan(value) == code, (value, why)


def _boundary_inputs(orc):
    """Every representable value and every midpoint, +-3 fp32 ulps, both signs."""
    tab = orc.e4m3_table()[:0x7F]
    mids = (tab[:-1] + tab[1:]) / 2.0
    pts = np.concatenate([tab, mids, [464.0, 480.0, 2.0 ** -10, 2.0 ** -11]]).astype(np.float32)
    out = []
    for p in pts:
        b = np.array([p], np.float32).view(np.int32)[0]
        for d in range(-3, 4):
            out.append(np.int32(b + d))
    arr = np.array(out, np.int32)
    arr = arr[arr >= 0].view(np.float32)
    return np.concatenate([arr, -arr])


def test_search_equals_scan_on_boundaries(orc):
    for t in _boundary_inputs(orc):
        assert orc.cast_e4m3(t) == orc.cast_e4m3_scan(t), float(t)


def test_search_equals_scan_random(orc):
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32)
    vals = bits.view(np.float32)
    vals = vals[~np.isnan(vals)]
    for t in vals:
        assert orc.cast_e4m3(t) == orc.cast_e4m3_scan(t)


def _torch_cast(torch, vals: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(vals).clamp_(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_matches_torch_on_every_fp32_pattern(orc):
    """All 2^32 bit patterns (NaNs excluded: out of domain), in chunks."""
    torch = pytest.importorskip("torch")
    chunk = 1 << 26
    for first in range(0, 1 << 32, chunk):
        got = orc.cast_e4m3_bits(first, chunk)
        vals = (np.arange(chunk, dtype=np.uint32) + np.uint32(first)).view(np.float32)
        ref = _torch_cast(torch, vals)
        ok = (got == ref) | np.isnan(vals)
        if not ok.all():
            bad = np.flatnonzero(~ok)[:5]
            raise AssertionError([(hex(first + int(i)), int(got[i]), int(ref[i])) for i in bad])


def test_round_trip_bound(orc):
    tab = orc.e4m3_table()
    rng = np.random.default_rng(11)
    mags = np.exp2(rng.uniform(-14.0, np.log2(448.0), 200000)).astype(np.float32)
    vals = mags * np.where(rng.random(mags.size) < 0.5, -1, 1).astype(np.float32)
    codes = orc.cast_e4m3_array(vals)
    dec = tab[codes]
    a = np.abs(vals.astype(np.float64))
    err = np.abs(dec - vals.astype(np.float64))
    normal = a >= 2.0 ** -6
    # half a unit in the last place of E4M3: 2^(floor(log2|t|) - 4) for normals,
    # 2^-10 in the subnormal range
    bound = np.where(normal, np.exp2(np.floor(np.log2(np.maximum(a, 1e-30))) - 4.0), 2.0 ** -10)
    assert (err <= bound).all()


def test_saturation(orc):
    for t in [448.0, 448.5, 463.9, 464.0, 1000.0, 3.4e38, float("inf")]:
        assert orc.cast_e4m3(t) == 0x7E
        assert orc.cast_e4m3(-t) == 0xFE


def test_monotone_and_odd(orc):
    tab = orc.e4m3_table()
    rng = np.random.default_rng(3)
    vals = np.sort(rng.uniform(-600.0, 600.0, 100000).astype(np.float32))
    vals = np.concatenate([vals, np.sort(rng.uniform(-0.05, 0.05, 50000).astype(np.float32))])
    codes = orc.cast_e4m3_array(vals)
    for seg in (slice(0, 100000), slice(100000, None)):
        dec = tab[codes[seg]]
        assert (np.diff(dec) >= 0).all()
    neg = orc.cast_e4m3_array(-vals)
    assert (neg == (codes ^ 0x80)).all()
