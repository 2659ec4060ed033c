"""The quotient shortcut the quantizer kernels use for their scales, checked
exhaustively on the CPU (no GPU, no HIP code: the arithmetic is restated
here with exact binary64 steps).

The kernels form fl(amax / 127) and fl(amax / 448) as
    q0 = RN(a * r),  t = RN(q0 * b - a),  q = RN(q0 - t * r),
with r = RN(1/b) and every RN a binary32 rounding (two FMAs after the
multiply), in place of the IEEE division.  Scaling a by a power of two
scales every step exactly as long as nothing under- or overflows, so the
check over every binary32 significand in [1, 2) covers every a in the
range the kernels allow (2^-100 .. 2^126).  The same holds for the
divisions by a stored scale, whose reciprocal is an IEEE division; those
are covered by the GPU parity tests instead, value by value.
"""
import numpy as np
import pytest

RCP = {127: np.float32(float.fromhex("0x1.020408p-7")), 448: np.float32(float.fromhex("0x1.24924ap-9"))}


def _rn32(x64):
    return x64.astype(np.float32).astype(np.float64)


def _rn32_of_sum(a64, b64):
    """RN to binary32 of the exact a + b (a, b binary64 values): the binary64
    sum s is exact up to its rounding error e (TwoSum); rounding s to
    binary32 could only go wrong (a second rounding) where s is exactly a
    binary32 midpoint, and there the sign of e decides."""
    s = a64 + b64
    bb = s - a64
    e = (a64 - (s - bb)) + (b64 - bb)
    r = _rn32(s)
    m, ex = np.frexp(s)
    scaled = np.ldexp(m, 25)             # the 25th significant bit is the half-ulp of binary32
    mid = (scaled == np.floor(scaled)) & (np.mod(scaled, 2) == 1) & (e != 0)
    if mid.any():
        r0 = s[mid].astype(np.float32)   # one of the two neighbours (the even one)
        above = r0.astype(np.float64) > s[mid]
        hi = np.where(above, r0, np.nextafter(r0, np.float32(np.inf)))
        lo = np.where(above, np.nextafter(r0, np.float32(-np.inf)), r0)
        r[mid] = np.where(e[mid] > 0, hi, lo).astype(np.float64)
    return r


@pytest.mark.parametrize("b", [127, 448])
def test_constant_division_shortcut_is_the_ieee_quotient_for_every_significand(b):
    a32 = (np.arange(1 << 23, dtype=np.uint32) | np.uint32(0x3F800000)).view(np.float32)
    a = a32.astype(np.float64)
    r = np.float64(RCP[b])
    assert RCP[b] == np.float32(1.0) / np.float32(b)          # r = RN(1/b)
    q0 = _rn32(a * r)                     # a * r is exact in binary64 (24 + 24 bits)
    t = _rn32(q0 * b - a)                 # exact in binary64, and in fact in binary32
    assert np.array_equal(t, q0 * b - a)
    q = _rn32_of_sum(q0, -(t * r))        # t * r exact in binary64
    ieee = (a32 / np.float32(b)).astype(np.float64)
    bad = np.flatnonzero(q != ieee)
    assert bad.size == 0, f"{bad.size} differ, first a = {a32[bad[0]]!r}"


def test_the_checker_sees_a_wrong_reciprocal():
    """The same steps with a reciprocal 2^-10 (relative) off do disagree with the
    IEEE quotient somewhere, so the test above can fail."""
    a32 = (np.arange(1 << 23, dtype=np.uint32) | np.uint32(0x3F800000)).view(np.float32)
    a = a32.astype(np.float64)
    r = np.float64(np.float32(RCP[127]) * np.float32(1 + 2.0 ** -10))
    q0 = _rn32(a * r)
    t = q0 * 127 - a
    q = _rn32_of_sum(q0, -(_rn32(t) * r))
    assert np.any(q != (a32 / np.float32(127)).astype(np.float64))
