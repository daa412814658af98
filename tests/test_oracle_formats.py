"""Pins of the oracle's element codecs against the format definitions.

Each check uses something other than the oracle's own code: the E2M1 bit-field
definition, torch's float8_e4m3fn conversion (a library routine), a threshold
formulation of E2M1 rounding, and the golden tie table.
"""
import json
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f32_from_bits(bits):
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


def _bits(f):
    return np.asarray(f, dtype=np.float32).view(np.uint32)


def test_format_constants(orc):
    g = json.load(open(os.path.join(GOLDEN, "format_constants.json")))
    assert g["global_scale_divisor"] == 6 * 448
    assert orc.e2m1_value(7) == g["e2m1_max"]
    assert orc.e4m3_value(0x7E) == g["e4m3_max"]
    # 0x7E is the largest finite E4M3 byte: 0x7F is NaN
    assert np.isnan(orc.e4m3_value(0x7F)) and np.isnan(orc.e4m3_value(0xFF))


def test_e2m1_decode_exhaustive(orc):
    """All 16 codes against the E2M1 bit fields: sign | 2-bit exponent (bias 1)
    | 1-bit mantissa, exponent 0 subnormal with step 0.5."""
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        mag = m * 0.5 if e == 0 else (1 + m / 2) * 2.0 ** (e - 1)
        want = -mag if s else mag
        got = orc.e2m1_value(c)
        assert got == want and np.signbit(got) == bool(s), c
    assert sorted({abs(orc.e2m1_value(c)) for c in range(16)}) == [0, .5, 1, 1.5, 2, 3, 4, 6]


def test_e4m3_decode_exhaustive(orc):
    """All 256 bytes against torch's float8_e4m3fn decode."""
    lib = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    for b in range(256):
        got = orc.e4m3_value(b)
        if np.isnan(lib[b]):
            assert np.isnan(got), hex(b)
        else:
            assert got == lib[b] and np.signbit(got) == np.signbit(lib[b]), hex(b)


def _e4m3_probe_values():
    """Non-negative floats below 480 concentrated where E4M3 rounding decides:
    +-300 ulps around every grid value and midpoint, a strided sweep of all
    float32 bit patterns in [0, 480) and random floats."""
    grid = np.zeros(1, np.float64)
    vals = torch.arange(0, 127, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    mids = (vals[:-1] + vals[1:]) / 2
    centres = np.concatenate([vals, mids, [464.0]]).astype(np.float32)
    cb = _bits(centres).astype(np.int64)
    nb = (cb[:, None] + np.arange(-300, 301)[None, :]).ravel()
    nb = nb[(nb >= 0)]
    top = int(_bits(np.float32(480.0)))
    stride = np.arange(0, top, 4099, dtype=np.int64)
    rnd = np.random.default_rng(7).random(200_000).astype(np.float32) * np.float32(479.0)
    allv = np.concatenate([_f32_from_bits(nb.astype(np.uint32)), _f32_from_bits(stride.astype(np.uint32)), rnd, grid.astype(np.float32)])
    # torch's conversion is RNE without saturation (above 464 it gives NaN),
    # so the comparison stops at 464, the tie that still rounds to 448
    allv = allv[(allv >= 0) & (allv <= 464.0)]
    return np.unique(allv)


def test_e4m3_encode_matches_torch(orc):
    """RNE to E4M3 against torch's float32 -> float8_e4m3fn conversion (ties to
    even, 464 -> 448) on ~1.5 M probe values in [0, 464]."""
    v = _e4m3_probe_values()
    got = orc.e4m3_encode_array(v)
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(v[i]), int(got[i]), int(want[i])) for i in bad[:10]]


def test_e4m3_encode_saturates(orc):
    for f in [448.0, 464.0, 480.0, 1000.0, 3.0e38, float("inf")]:
        assert orc.e4m3_encode(f) == 0x7E
    # subnormal steps and their ties (2^-10 -> 0, 1.5 * 2^-9 -> 2^-8, 7.5 * 2^-9 -> 2^-6)
    assert orc.e4m3_encode(2.0 ** -10) == 0x00
    assert orc.e4m3_encode(float(np.nextafter(np.float32(2.0 ** -10), np.float32(1)))) == 0x01
    assert orc.e4m3_encode(1.5 * 2.0 ** -9) == 0x02
    assert orc.e4m3_encode(7.5 * 2.0 ** -9) == 0x08


def _e2m1_by_thresholds(v):
    """E2M1 RNE-sat magnitude code as a count of midpoint thresholds crossed
    (strict above a midpoint whose lower neighbour has the even code)."""
    v = np.asarray(v, np.float64)
    return ((v > 0.25).astype(np.int32) + (v >= 0.75) + (v > 1.25) + (v >= 1.75)
            + (v > 2.5) + (v >= 3.5) + (v > 5.0)).astype(np.uint8)


@pytest.mark.slow
def test_e2m1_encode_bruteforce(orc):
    """Every 37th float32 bit pattern in [0, 16] plus +-5000 ulps around each
    grid value and midpoint, against the threshold formulation."""
    top = int(_bits(np.float32(16.0)))
    pats = np.arange(0, top + 1, 37, dtype=np.uint32)
    centres = np.array([0.25, 0.5, 0.75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6, 7], np.float32)
    nb = (_bits(centres).astype(np.int64)[:, None] + np.arange(-5000, 5001)[None, :]).ravel()
    v = np.concatenate([_f32_from_bits(pats), _f32_from_bits(nb.astype(np.uint32))])
    got = orc.e2m1_encode_mag_array(v)
    want = _e2m1_by_thresholds(v)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(v[i]), int(got[i]), int(want[i])) for i in bad[:10]]


def test_e2m1_ties_golden(orc):
    rows = [l.split() for l in open(os.path.join(GOLDEN, "e2m1_ties.txt")) if l.strip() and not l.startswith("#")]
    for mag, code, val in rows:
        c = orc.e2m1_encode_mag(float(mag))
        assert c == int(code), mag
        assert orc.e2m1_value(c) == float(val)


def test_bf16_rounding_matches_torch(orc):
    rng = np.random.default_rng(11)
    f = (rng.standard_normal(200_000) * np.exp(rng.uniform(-30, 30, 200_000))).astype(np.float32)
    # exact bf16 midpoints (ties) and their neighbours
    base = rng.integers(0, 0x7F00, 5000, dtype=np.uint32) << 16
    ties = _f32_from_bits(base | 0x8000)
    f = np.concatenate([f, ties, -ties, _f32_from_bits(base | 0x7FFF), _f32_from_bits(base | 0x8001)])
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(orc.f32_to_bf16(f), want)


def test_f64_to_bf16_direct_rounding(orc):
    """Rounding a double straight to bf16 differs from double -> float -> bf16
    only at fp32-induced ties; check both kinds against exact definitions."""
    one_plus_half_ulp = 1.0 + 2.0 ** -8          # exact bf16 tie between 1 and 1 + 2^-7
    assert orc.f64_to_bf16_scalar(one_plus_half_ulp) == 0x3F80
    just_above = 1.0 + 2.0 ** -8 + 2.0 ** -40   # rounds to float as the tie, but is above it
    assert orc.f64_to_bf16_scalar(just_above) == 0x3F81
    assert orc.f64_to_bf16_scalar(-just_above) == 0xBF81
    assert orc.f64_to_bf16_scalar(0.0) == 0x0000
