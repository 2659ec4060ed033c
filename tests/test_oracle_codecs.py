"""Pins for the oracle's codecs (CPU only).

Each test checks the oracle against something other than itself: the OCP
bit-field definitions of E2M1 / E4M3, torch's own float8_e4m3fn and bfloat16
casts, exact rational rounding, and hand-worked edge values.
"""
import math
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


# ------------------------------------------------------------------ E4M3
def test_e4m3_decode_matches_torch_for_all_256_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).tolist()
    for c in range(256):
        got = oracle.e4m3_decode(c)
        if c in (0x7F, 0xFF):
            assert math.isnan(got) and math.isnan(ref[c])
        else:
            assert got == ref[c], (hex(c), got, ref[c])
            assert math.copysign(1.0, got) == math.copysign(1.0, ref[c])


@pytest.mark.parametrize("code,value", [
    (0x7E, 448.0), (0x08, 2.0 ** -6), (0x01, 2.0 ** -9), (0x38, 1.0),
    (0x40, 2.0), (0x30, 0.5), (0x2F, 0.46875), (0x07, 7 * 2.0 ** -9),
    (0xB8, -1.0), (0x80, -0.0)])
def test_e4m3_decode_spot_values(code, value):
    got = oracle.e4m3_decode(code)
    assert got == value and math.copysign(1, got) == math.copysign(1, value)


def _e4m3_probe_values():
    """Every grid point, every midpoint between neighbours, one binary32 ulp
    either side of each, plus random log-spread values, all below 464."""
    grid = sorted({abs(oracle.e4m3_decode(c)) for c in range(0x7F)})
    vals = []
    for a, b in zip(grid, grid[1:]):
        mid = np.float32((a + b) / 2)        # exact: midpoint has 5 bits
        for v in (np.float32(a), mid):
            vals += [v, np.nextafter(v, np.float32(0)), np.nextafter(v, np.float32(1e9))]
    rng = np.random.default_rng(7)
    vals += list((10.0 ** rng.uniform(-12, math.log10(460), 20000)).astype(np.float32))
    vals = np.array(vals, dtype=np.float32)
    vals = vals[vals < 464]
    return np.concatenate([vals, -vals])


def test_e4m3_encode_matches_torch_cast_below_464():
    # torch's cast rounds to nearest even over the finite grid (it does not
    # saturate, so it is only a reference below 464).
    vals = _e4m3_probe_values()
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(v)) for v in vals], dtype=np.uint8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(vals[i]), hex(got[i]), hex(ref[i])) for i in bad[:10]]


@pytest.mark.parametrize("y,code", [
    (448.0, 0x7E), (455.0, 0x7E), (463.99, 0x7E), (464.0, 0x7E), (480.0, 0x7E),
    (500.0, 0x7E), (1e30, 0x7E), (-500.0, 0xFE), (-448.0, 0xFE),
    (2.0 ** -10, 0x00), (1.5 * 2.0 ** -10, 0x01), (-(2.0 ** -10), 0x80),
    (0.0, 0x00), (-0.0, 0x80), (1e-30, 0x00)])
def test_e4m3_encode_saturation_and_zero(y, code):
    assert oracle.e4m3_encode(y) == code


def test_e4m3_roundtrip_every_finite_code():
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert oracle.e4m3_encode(oracle.e4m3_decode(c)) == c, hex(c)


# ------------------------------------------------------------------ E2M1
def _e2m1_bitfield(c):
    """OCP MX E2M1: sign, 2-bit exponent (bias 1), 1-bit mantissa."""
    s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
    v = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
    return -v if s else v


def test_e2m1_decode_matches_bitfield_definition():
    for c in range(16):
        got, ref = oracle.e2m1_decode(c), _e2m1_bitfield(c)
        assert got == ref and math.copysign(1, got) == math.copysign(1, ref), c
    assert [oracle.e2m1_decode(c) for c in range(8)] == [0, .5, 1, 1.5, 2, 3, 4, 6]


def _e2m1_round_by_binade(y):
    """Independent route: round |y| to the E2M1 spacing of its binade with
    Python's round() (ties to even), saturate at 6, map value -> code."""
    a = abs(y)
    step = 0.5 if a < 2 else (1.0 if a < 4 else 2.0)
    v = round(a / step) * step
    v = min(v, 6.0)
    code = [0, .5, 1, 1.5, 2, 3, 4, 6].index(v)
    return code | (8 if math.copysign(1, y) < 0 else 0)


def test_e2m1_encode_matches_binade_rounding():
    rng = np.random.default_rng(3)
    vals = list(np.float32(rng.uniform(-8, 8, 20000)))
    for g in [0, .25, .5, .75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6, 7]:
        f = np.float32(g)
        vals += [f, np.nextafter(f, np.float32(-1)), np.nextafter(f, np.float32(9))]
    vals += [-v for v in vals]
    for v in vals:
        assert oracle.e2m1_encode(float(v)) == _e2m1_round_by_binade(float(v)), float(v)


@pytest.mark.parametrize("y,code", [
    (0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6),
    (6.0, 7), (7.0, 7), (100.0, 7), (-0.1, 8), (-0.0, 8), (-5.0, 14), (-2.5, 12)])
def test_e2m1_encode_ties_even_and_saturation(y, code):
    assert oracle.e2m1_encode(y) == code


# ------------------------------------------------------------------ int8
def test_int8_encode_matches_numpy_rint_and_clip():
    rng = np.random.default_rng(5)
    v = np.float32(rng.uniform(-140, 140, 20000))
    halves = np.arange(-130, 131, dtype=np.float32) + np.float32(0.5)
    v = np.concatenate([v, halves, -halves]).astype(np.float32)
    ref = np.clip(np.rint(v), -127, 127).astype(np.int8)
    got = np.array([oracle.int8_encode(float(x)) for x in v], dtype=np.int8)
    assert np.array_equal(got, ref)
    assert oracle.int8_encode(-1000.0) == -127 and oracle.int8_encode(126.5) == 126


# ------------------------------------------------------------------ BF16
def test_bf16_rounding_matches_torch_for_f32_values():
    rng = np.random.default_rng(11)
    v = (rng.standard_normal(20000) * 10.0 ** rng.uniform(-30, 30, 20000)).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_from_double(float(x)) for x in v], dtype=np.uint16)
    assert np.array_equal(got, ref)


def _bf16_exact(x: Fraction) -> int:
    """Exact rational RNE to BF16 (normal range)."""
    if x == 0:
        return 0
    sign = 0x8000 if x < 0 else 0
    a = abs(x)
    e = math.floor(math.log2(a))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = a / Fraction(2) ** (e - 7)                  # in [128, 256)
    r = math.floor(q)
    rem = q - r
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and r % 2 == 1):
        r += 1
    val = Fraction(r) * Fraction(2) ** (e - 7)
    bits = np.array([float(val)], dtype=np.float32).view(np.uint32)[0] >> 16
    return int(bits) | sign


def test_bf16_rounding_of_doubles_is_single_rounding():
    # Values close to BF16 midpoints, where rounding f64 -> f32 -> bf16 would
    # double-round; the oracle must round once.
    rng = np.random.default_rng(13)
    for _ in range(3000):
        base = float(np.float32(rng.uniform(1, 2)))
        b = oracle.bf16_from_double(base)
        lo = oracle.bf16_to_float(b & 0xFFFF)
        up = oracle.bf16_to_float((b + 1) & 0xFFFF)
        mid = (Fraction(lo) + Fraction(up)) / 2
        for d in (Fraction(1, 2 ** 40), -Fraction(1, 2 ** 40), Fraction(0)):
            x = mid + d
            assert oracle.bf16_from_double(float(x)) == _bf16_exact(x)
