"""Pins for the oracle's E4M3 decode table.

The pages fix the format (FP8量化与长上下文实测：Llama 3 70B部署优化指南 §1.1:
4 exponent bits, 3 mantissa bits, largest value about 448, smallest non-zero
about 2^-9; Llama 3 精读 §2.1: range [-448, 448]).  These facts leave exactly
one 256-code table; the tests check the oracle's decoder against the stated
facts, against the structure they force, and against torch's own
float8_e4m3fn decoder (a library special case, independent of the oracle).
"""
import json
import math
import os

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden", "e4m3_format.json")


@pytest.fixture(scope="module")
def table(orc):
    return orc.e4m3_table()


@pytest.fixture(scope="module")
def facts():
    with open(GOLD) as f:
        return json.load(f)


def test_page_facts(table, facts):
    finite = table[np.isfinite(table)]
    assert finite.max() == facts["max_value"]
    assert finite.min() == facts["range"][0]
    assert finite.max() == facts["range"][1]
    assert finite[finite > 0].min() == facts["min_positive_value"]
    assert not np.isinf(table).any()          # e4m3fn has no infinities
    # 4 exponent bits + 3 mantissa bits: 2^7 magnitudes, one of them NaN
    assert len(set(np.abs(finite).tolist())) == 2 ** (facts["exponent_bits"] + facts["mantissa_bits"]) - 1


def test_structure(table):
    assert np.isnan(table[0x7F]) and np.isnan(table[0xFF])
    assert np.isfinite(table).sum() == 254
    pos = table[:0x7F]
    assert (np.diff(pos) > 0).all()            # strictly increasing 0x00 .. 0x7E
    assert pos[0] == 0.0 and math.copysign(1.0, table[0x80]) == -1.0
    for c in range(0x7F):                      # odd symmetry: sign bit only
        assert table[c | 0x80] == -table[c]
    assert table[0x7E] == 448.0
    assert table[0x01] == 2.0 ** -9            # smallest subnormal
    assert table[0x07] == 7 * 2.0 ** -9        # largest subnormal
    assert table[0x08] == 2.0 ** -6            # smallest normal
    assert table[0x38] == 1.0                  # bias 7
    assert table[0x78] == 256.0                # all-ones exponent is finite


def test_spacing(table):
    # within a binade the 8 mantissa steps are equal; subnormals step by 2^-9
    pos = table[:0x7F]
    for e in range(1, 16):
        lo = e * 8
        hi = min(lo + 8, 0x7F)
        step = np.diff(pos[lo:hi])
        assert np.all(step == 2.0 ** (e - 7 - 3))
    assert np.all(np.diff(pos[:9]) == 2.0 ** -9)


def test_matches_torch_decoder(table):
    torch = pytest.importorskip("torch")
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert (nan == np.isnan(table)).all()
    assert (ref[~nan] == table[~nan]).all()
    # signed zero
    assert math.copysign(1.0, ref[0x80]) == math.copysign(1.0, table[0x80])


def test_f16_decode_every_pattern(orc):
    """IEEE binary16 decode (the fp8_w_fp16_a activations) against numpy's
    float16 on all 65536 bit patterns, plus the landmarks of the format."""
    import numpy as np
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.f16_value(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert orc.f16_value(0x3C00) == 1.0
    assert orc.f16_value(0x7BFF) == 65504.0
    assert orc.f16_value(0x0001) == 2.0 ** -24
    assert orc.f16_value(0x0400) == 2.0 ** -14
    assert orc.f16_value(0x8000) == 0.0 and np.signbit(orc.f16_value(0x8000))
