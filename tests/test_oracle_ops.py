"""Pins for the oracle's quantizers and contractions (CPU only).

Pins used: the hand-worked blocks in tests/golden (derived from the format
definitions), exact rational brute force on tiny shapes, special cases that
reduce to numpy's integer / binary64 matmul, and the invariants the pages
state (row-wise passthrough, batched GEMV == per-row GEMV) or that follow
from the rounding rules (error bounds, zero blocks, idempotence).
"""
import configparser
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_blocks.ini")


def _cases():
    cp = configparser.ConfigParser()
    cp.read(GOLDEN)
    return cp


def _bf16(vals):
    return torch.tensor([float(v) for v in vals], dtype=torch.float32) \
        .to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _hexbytes(s):
    return np.array([int(t, 16) for t in s.split()], dtype=np.uint8)


def _f32hex(h):
    return np.array([int(h, 16)], dtype=np.uint32).view(np.float32)[0]


# ------------------------------------------------------- hand-worked blocks
def test_hw1_hw2_quantize_bf16_nvfp4():
    cp = _cases()
    for name in ("HW1", "HW2"):
        c = cp[name]
        x = _bf16(c["x"].split())[None, :]
        packed, sc = oracle.quantize_bf16_nvfp4(x, float(c["scale2"]))
        assert sc[0, 0] == int(c["expect_scale"], 16), name
        assert np.array_equal(packed[0], _hexbytes(c["expect_packed"])), (name, packed)


def test_hw3_requant_w_nvfp4_int8():
    c = _cases()["HW3"]
    codes = [int(t) for t in c["codes"].split()]
    packed = np.array([[codes[2 * i] | (codes[2 * i + 1] << 4) for i in range(16)]], np.uint8)
    sc = _hexbytes(c["scales16"])[None, :]
    q, s = oracle.requant_w_nvfp4_int8(packed, sc, float(c["scale2"]))
    assert np.array_equal(q[0], np.array(c["expect_q"].split(), dtype=np.int8))
    assert s[0, 0] == _f32hex(c["expect_scale_hex"])


def test_hw4_requant_a_bf16_int8():
    c = _cases()["HW4"]
    q, s = oracle.requant_a_bf16_int8(_bf16(c["x"].split())[None, :])
    assert np.array_equal(q[0], np.array(c["expect_q"].split(), dtype=np.int8))
    assert s[0, 0] == _f32hex(c["expect_scale_hex"])


def test_hw5_quant_rowwise_fp8():
    c = _cases()["HW5"]
    q, s = oracle.quant_rowwise_fp8(_bf16(c["x"].split())[None, :])
    assert np.array_equal(q[0], _hexbytes(c["expect_q"]))
    assert s[0] == _f32hex(c["expect_scale_hex"])


def test_hw8_int8_divides_by_the_stored_scale():
    """HW8: the int8 code of 0.28125 in a block of absmax 0.5625 is 63 when
    the element is divided by the stored binary32 scale, and 64 under the
    other reading (rounding the exact quotient 63.5).  The second assertion
    recomputes that other reading with exact rationals, so the fixture
    provably tells the two apart."""
    c = _cases()["HW8"]
    x = [float(t) for t in c["x"].split()]
    q, s = oracle.requant_a_bf16_int8(_bf16(x)[None, :])
    expect = np.array(c["expect_q"].split(), dtype=np.int8)
    assert np.array_equal(q[0], expect)
    assert s[0, 0] == _f32hex(c["expect_scale_hex"])
    exact = Fraction(127) * Fraction(x[1]) / Fraction(max(abs(v) for v in x))
    assert exact == Fraction(127, 2)                       # a midpoint
    alt = round(exact)                                      # Python rounds ties to even
    assert alt == int(c["exact_quotient_q1"]) != expect[1]


def test_hw9_e4m3_row_divides_by_the_stored_scale():
    """HW9: the E4M3 code of 1.453125 in a row of absmax 3.875 is 0x73 when
    divided by the stored scale (quotient 168 + 2^-16), and 0x72 when the
    exact quotient 168 (a midpoint of 160 and 176) is rounded instead."""
    c = _cases()["HW9"]
    x = [float(t) for t in c["x"].split()]
    q, s = oracle.quant_rowwise_fp8(_bf16(x)[None, :])
    expect = _hexbytes(c["expect_q"])
    assert np.array_equal(q[0], expect)
    assert s[0] == _f32hex(c["expect_scale_hex"])
    exact = Fraction(448) * Fraction(x[1]) / Fraction(max(abs(v) for v in x))
    assert exact == 168                                     # midpoint of 160 and 176
    # torch's E4M3 cast rounds a binary32 to nearest-even; 168.0 is exact in it
    alt = int(torch.tensor([float(exact)]).to(torch.float8_e4m3fn).view(torch.uint8)[0])
    assert alt == int(c["exact_quotient_code1"], 16) != expect[1]


def test_hw6_blockfp8_bf16_intermediate():
    c = _cases()["HW6"]
    code = int(c["code"], 16)
    w = np.full((128, 128), code, np.uint8)
    grid = np.full((1, 1), float(c["block_scale"]), np.float32)
    q, s = oracle.requant_w_blockfp8_rowwise(w, grid)
    y = oracle.bf16_to_float(int(c["expect_bf16_hex"], 16))
    assert y == 4.46875
    assert np.all(q == 0x7E)
    assert s[0] == np.float32(y) / np.float32(448)


def test_hw7_e4m3_encode_edges():
    c = _cases()["HW7"]
    ys = [float(t) for t in c["y"].split()]
    assert [oracle.e4m3_encode(y) for y in ys] == list(_hexbytes(c["expect"]))


# ------------------------------------------------------------- quantizers
def _dec4(codes):
    return np.vectorize(oracle.e4m3_decode)(codes.astype(np.int64))


def _dec2(codes):
    return np.vectorize(oracle.e2m1_decode)(codes.astype(np.int64))


def _unpack(packed):
    lo = packed & 15
    hi = packed >> 4
    return np.stack([lo, hi], axis=-1).reshape(packed.shape[0], -1)


def test_requant_a_error_bound_and_absmax_code():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((8, 256)).astype(np.float32)
    x[0, :32] = 0.0                     # a zero block
    x[1, 5] = 40.0                      # an outlier
    xb = _bf16(x.ravel()).reshape(8, 256)
    xf = oracle.bf16_bits_to_f32(xb).astype(np.float64)
    q, s = oracle.requant_a_bf16_int8(xb)
    blocks = xf.reshape(8, 8, 32)
    qb = q.reshape(8, 8, 32).astype(np.float64)
    assert s[0, 0] == 0 and np.all(q[0, :32] == 0)          # zero block
    for r in range(8):
        for b in range(8):
            amax = np.abs(blocks[r, b]).max()
            if amax == 0:
                continue
            assert np.isclose(s[r, b] * 127, amax, rtol=2 ** -22)
            assert np.abs(qb[r, b]).max() == 127             # absmax -> 127
            err = np.abs(blocks[r, b] - qb[r, b] * s[r, b])
            assert np.all(err <= s[r, b] * (0.5 + 2 ** -20))
    assert np.all(np.abs(q) <= 127)


def test_requant_w_nibble_order_and_reblocking():
    # One nonzero nibble at a time: the int8 output is nonzero exactly there,
    # and the 32-block's scale comes from the right pair of 16-blocks.
    k = 64
    for pos in (0, 1, 15, 16, 17, 31, 32, 63):
        packed = np.zeros((1, k // 2), np.uint8)
        code = 7
        packed[0, pos // 2] = code if pos % 2 == 0 else code << 4
        sc = np.full((1, k // 16), 0x38, np.uint8)        # all sub-scales 1.0
        sc[0, pos // 16] = 0x40                             # 2.0 where the value is
        q, s = oracle.requant_w_nvfp4_int8(packed, sc, 1.0)
        nz = np.nonzero(q[0])[0]
        assert list(nz) == [pos] and q[0, pos] == 127
        b = pos // 32
        assert s[0, b] == np.float32(12.0) / np.float32(127)
        assert s[0, 1 - b] == 0


def test_requant_w_scale2_is_a_multiplier():
    # Scaling scale2 by a power of two leaves codes unchanged and scales s.
    rng = np.random.default_rng(2)
    packed = rng.integers(0, 256, (4, 64), dtype=np.uint8)
    sc = rng.integers(0x20, 0x50, (4, 8), dtype=np.uint8)
    q1, s1 = oracle.requant_w_nvfp4_int8(packed, sc, 1.0)
    q2, s2 = oracle.requant_w_nvfp4_int8(packed, sc, 0.25)
    assert np.array_equal(q1, q2) and np.array_equal(s2, s1 * np.float32(0.25))


def test_nvfp4_requantizing_a_dequantized_block_is_idempotent():
    # A block holding a +-6 code at scale2 = 1 dequantises to values whose
    # absmax gives back the same E4M3 scale; re-quantising returns the codes.
    rng = np.random.default_rng(4)
    for _ in range(200):
        codes = rng.integers(0, 16, 16)
        codes[rng.integers(0, 16)] = 7 | (8 * rng.integers(0, 2))
        sb = int(rng.integers(0x10, 0x70))
        vals = _dec2(codes) * oracle.e4m3_decode(sb)
        xb = _bf16(vals)
        assert np.array_equal(oracle.bf16_bits_to_f32(xb), vals.astype(np.float32))
        packed, sc = oracle.quantize_bf16_nvfp4(xb[None, :], 1.0)
        assert sc[0, 0] == sb
        got = _unpack(packed)[0]
        # -0 codes may come back as +0 only where the value is zero
        exp = np.where(_dec2(codes) == 0, got, codes)
        assert np.array_equal(got, exp)


def test_nvfp4_error_bound_and_zero_block():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((4, 64)) * 0.02).astype(np.float32)
    x[2, 16:32] = 0.0
    xb = _bf16(x.ravel()).reshape(4, 64)
    xf = oracle.bf16_bits_to_f32(xb).astype(np.float64)
    s2 = float(np.float32(np.abs(xf).max()) / np.float32(448))
    packed, sc = oracle.quantize_bf16_nvfp4(xb, s2)
    assert sc[2, 1] == 0 and np.all(_unpack(packed)[2, 16:32] == 0)
    d = _dec4(sc).astype(np.float64) * s2
    v = _dec2(_unpack(packed)) * np.repeat(d, 16, axis=1)
    # half the local E2M1 spacing (1 at the top binade) times the scale
    dd = np.repeat(d, 16, axis=1)
    r = np.abs(v) / np.where(dd == 0, 1, dd)
    step = np.where(r >= 4, 2.0, np.where(r >= 2, 1.0, 0.5))
    assert np.all(np.abs(v - xf) <= 0.5 * step * dd * (1 + 1e-6) + 1e-30)


def test_rowwise_fp8_relative_error_and_passthrough_of_rowwise_weight():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((16, 512)) * 0.02).astype(np.float32)
    xb = _bf16(x.ravel()).reshape(16, 512)
    q, s = oracle.quant_rowwise_fp8(xb)
    xf = oracle.bf16_bits_to_f32(xb).astype(np.float64)
    v = _dec4(q) * s[:, None]
    normal = np.abs(xf) >= s[:, None] * 2.0 ** -6
    rel = np.abs(v - xf)[normal] / np.abs(xf)[normal]
    assert rel.max() <= 2.0 ** -4 * (1 + 1e-5)
    assert np.all(np.max(np.abs(_dec4(q)), axis=1) == 448.0)


def test_blockfp8_with_unit_scales_requantizes_to_identical_codes():
    # Block FP8 whose scales are all 1.0 and whose every row holds a +-448:
    # the BF16 step is exact, the row scale is 448/448 = 1, codes come back.
    rng = np.random.default_rng(9)
    w = rng.integers(0, 0x7F, (128, 256), dtype=np.uint8)
    w |= (rng.integers(0, 2, w.shape, dtype=np.uint8) << 7)
    w[np.arange(128), rng.integers(0, 256, 128)] = 0x7E
    grid = np.ones((1, 2), np.float32)
    q, s = oracle.requant_w_blockfp8_rowwise(w, grid)
    assert np.all(s == 1.0)
    same = np.where(np.vectorize(oracle.e4m3_decode)(w.astype(np.int64)) == 0, q, w)
    assert np.array_equal(q, same)


def test_blockfp8_grid_indexing():
    # A grid with one distinct block: only the rows and columns of that block
    # change, and the BF16-rounded value sets their codes.
    w = np.full((256, 256), 0x38, np.uint8)            # every weight 1.0
    grid = np.ones((2, 2), np.float32)
    grid[1, 0] = 2.0 ** -3
    q, s = oracle.requant_w_blockfp8_rowwise(w, grid)
    # rows 128..255: values 1/8 in columns 0..127, 1 elsewhere -> amax 1
    assert np.all(s == np.float32(1.0) / np.float32(448))
    assert np.all(q[128:, :128] == oracle.e4m3_encode(448.0 / 8))
    assert np.all(q[128:, 128:] == 0x7E) and np.all(q[:128] == 0x7E)


# ------------------------------------------------------------ contractions
def _bf16_exact(x: Fraction) -> int:
    from tests.test_oracle_codecs import _bf16_exact as f
    return f(x)


def test_int8_block_partials_match_numpy_int64():
    rng = np.random.default_rng(10)
    a = rng.integers(-127, 128, (5, 96), dtype=np.int8)
    w = rng.integers(-127, 128, (7, 96), dtype=np.int8)
    p = oracle.int8_block_partials(a, w)
    ref = np.einsum("mbk,nbk->mnb", a.reshape(5, 3, 32).astype(np.int64),
                    w.reshape(7, 3, 32).astype(np.int64))
    assert np.array_equal(p, ref)
    # extreme partial: every product 127*127
    full = np.full((1, 32), 127, np.int8)
    assert oracle.int8_block_partials(full, full)[0, 0, 0] == 32 * 127 * 127


def test_int8_gemm_unit_scales_is_bf16_of_integer_matmul():
    rng = np.random.default_rng(12)
    a = rng.integers(-127, 128, (6, 128), dtype=np.int8)
    w = rng.integers(-127, 128, (5, 128), dtype=np.int8)
    ones_a = np.ones((6, 4), np.float32)
    ones_w = np.ones((5, 4), np.float32)
    c = oracle.int8_gemm_blockscaled(a, w, ones_a, ones_w)
    ref = a.astype(np.int64) @ w.astype(np.int64).T
    exp = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)   # |ref| < 2^24: exact in f32
    assert np.array_equal(c, exp)


def test_int8_gemm_brute_force_rational():
    rng = np.random.default_rng(14)
    m, n, k = 3, 4, 64
    a = rng.integers(-127, 128, (m, k), dtype=np.int8)
    w = rng.integers(-127, 128, (n, k), dtype=np.int8)
    sa = rng.uniform(0.001, 0.1, (m, 2)).astype(np.float32)
    sw = rng.uniform(0.0001, 0.01, (n, 2)).astype(np.float32)
    c = oracle.int8_gemm_blockscaled(a, w, sa, sw)
    for i in range(m):
        for j in range(n):
            tot = Fraction(0)
            for b in range(2):
                pb = sum(int(a[i, t]) * int(w[j, t]) for t in range(32 * b, 32 * b + 32))
                tot += Fraction(pb) * Fraction(float(sa[i, b])) * Fraction(float(sw[j, b]))
            assert c[i, j] == _bf16_exact(tot)


def test_w4a4_unit_scales_is_bf16_of_e2m1_matmul():
    rng = np.random.default_rng(15)
    m, n, k = 4, 6, 64
    ap = rng.integers(0, 256, (m, k // 2), dtype=np.uint8)
    wp = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    one_a = np.full((m, k // 16), 0x38, np.uint8)
    one_w = np.full((n, k // 16), 0x38, np.uint8)
    c = oracle.w4a4_gemm(ap, one_a, wp, one_w, 1.0, 1.0)
    ref = _dec2(_unpack(ap)) @ _dec2(_unpack(wp)).T          # exact in f64
    exp = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(c, exp)


def test_w4a4_brute_force_rational_with_scales():
    rng = np.random.default_rng(16)
    m, n, k = 2, 3, 32
    ap = rng.integers(0, 256, (m, k // 2), dtype=np.uint8)
    wp = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    asc = rng.integers(0x08, 0x70, (m, 2), dtype=np.uint8)
    wsc = rng.integers(0x08, 0x70, (n, 2), dtype=np.uint8)
    sa2, sw2 = 1.0, float(np.float32(0.37))
    c = oracle.w4a4_gemm(ap, asc, wp, wsc, sa2, sw2)
    au, wu = _unpack(ap), _unpack(wp)
    for i in range(m):
        for j in range(n):
            tot = Fraction(0)
            for b in range(2):
                pb = sum(Fraction(oracle.e2m1_decode(au[i, t])) * Fraction(oracle.e2m1_decode(wu[j, t]))
                         for t in range(16 * b, 16 * b + 16))
                tot += Fraction(oracle.e4m3_decode(asc[i, b])) * Fraction(oracle.e4m3_decode(wsc[j, b])) * pb
            assert c[i, j] == _bf16_exact(Fraction(sa2) * Fraction(sw2) * tot)


def test_fp8_gemv_matches_f64_matmul_and_rational():
    rng = np.random.default_rng(17)
    m, n, k = 3, 9, 48
    x = _bf16(rng.standard_normal(m * k)).reshape(m, k)
    w = rng.integers(0, 0x7F, (n, k), dtype=np.uint8) | \
        (rng.integers(0, 2, (n, k), dtype=np.uint8) << 7)
    rs = rng.uniform(1e-5, 1e-3, n).astype(np.float32)
    c = oracle.fp8_gemv_rowscale(x, w, rs)
    xf = oracle.bf16_bits_to_f32(x).astype(np.float64)
    for i in range(m):
        for j in range(n):
            tot = sum(Fraction(float(xf[i, t])) * Fraction(oracle.e4m3_decode(w[j, t])) for t in range(k))
            assert c[i, j] == _bf16_exact(Fraction(float(rs[j])) * tot)


def test_fp8_gemv_batched_rows_equal_single_row_calls():
    # The pages' invariant for the batched GEMV: each row is bit-identical
    # to an M=1 call on that row.
    rng = np.random.default_rng(18)
    x = _bf16(rng.standard_normal(16 * 256)).reshape(16, 256)
    w = rng.integers(0, 0x7F, (33, 256), dtype=np.uint8)
    rs = rng.uniform(1e-4, 1e-2, 33).astype(np.float32)
    full = oracle.fp8_gemv_rowscale(x, w, rs)
    for i in range(16):
        assert np.array_equal(full[i:i + 1], oracle.fp8_gemv_rowscale(x[i:i + 1], w, rs))


def test_fp8_gemm_rowscale_rational_and_zero_rows():
    rng = np.random.default_rng(19)
    m, n, k = 3, 4, 32
    a = rng.integers(0, 0x7F, (m, k), dtype=np.uint8)
    w = rng.integers(0, 0x7F, (n, k), dtype=np.uint8) | 0x80
    sa = rng.uniform(1e-3, 1e-2, m).astype(np.float32)
    sw = rng.uniform(1e-4, 1e-3, n).astype(np.float32)
    sa[2] = 0.0                                 # a zero-scale row contributes 0
    c = oracle.fp8_gemm_rowscale(a, sa, w, sw)
    assert np.all((c[2] & 0x7FFF) == 0)           # +0 or -0
    for i in range(2):
        for j in range(n):
            tot = sum(Fraction(oracle.e4m3_decode(a[i, t])) * Fraction(oracle.e4m3_decode(w[j, t]))
                      for t in range(k))
            assert c[i, j] == _bf16_exact(Fraction(float(sa[i])) * Fraction(float(sw[j])) * tot)


# ---------------------------------------------------------------------------
# Block-scaled FP8 GEMV (fp8_gemv_batch.rs, w8a16_gemv / _batch2 / _batch4):
# C[i,j] = bf16(sum_t x[i,t] * e4m3(w[j,t]) * s[j/128, t/128]).
def _blockscale_case(seed, m, n, k):
    rng = np.random.default_rng(seed)
    x = _bf16(rng.standard_normal(m * k)).reshape(m, k)
    w = rng.integers(0, 0x7F, (n, k), dtype=np.uint8) | \
        (rng.integers(0, 2, (n, k), dtype=np.uint8) << 7)
    s = rng.uniform(1e-3, 1e-1, (n // 128, k // 128)).astype(np.float32)
    return x, w, s


def test_fp8_gemv_blockscale_rational():
    # Exact rationals: every product carries the scale of its own 128 x 128
    # block (two N blocks, two K blocks, all four scales distinct).
    x, w, s = _blockscale_case(21, 2, 256, 256)
    c = oracle.fp8_gemv_blockscale(x, w, s)
    xf = oracle.bf16_bits_to_f32(x).astype(np.float64)
    for i in range(2):
        for j in (0, 1, 63, 127, 128, 200, 255):
            tot = sum(Fraction(float(xf[i, t])) * Fraction(oracle.e4m3_decode(w[j, t])) *
                      Fraction(float(s[j // 128, t // 128])) for t in range(256))
            assert c[i, j] == _bf16_exact(tot)


def test_fp8_gemv_blockscale_unit_grid_is_bf16_of_f64_matmul():
    # With every block scale 1 the GEMV is a plain product: numpy's f64
    # matmul of the decoded operands, rounded to BF16 (its summation order
    # differs, so allow one BF16 ulp on the rare value next to a tie).
    x, w, _ = _blockscale_case(22, 4, 128, 384)
    s = np.ones((1, 3), np.float32)
    c = oracle.fp8_gemv_blockscale(x, w, s).astype(np.int64)
    wf = np.vectorize(oracle.e4m3_decode)(w).astype(np.float64)
    ref = oracle.bf16_bits_to_f32(x).astype(np.float64) @ wf.T
    ref_bits = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    ref_bits = ref_bits.astype(np.int64) & 0xFFFF
    diff = np.abs(c - ref_bits)
    assert diff.max() <= 1 and np.mean(diff == 0) > 0.99


def test_fp8_gemv_blockscale_single_live_k_block_is_a_row_scaled_slice():
    # A grid that is zero outside K block 1 computes that block's 128-column
    # slice alone, with the block's scale acting as a row scale (the
    # row-scaled GEMV, pinned separately above, on the slice).
    x, w, s = _blockscale_case(23, 3, 256, 384)
    s[:, 0] = 0.0
    s[:, 2] = 0.0
    c = oracle.fp8_gemv_blockscale(x, w, s)
    rs = np.repeat(s[:, 1], 128).astype(np.float32)
    ref = oracle.fp8_gemv_rowscale(np.ascontiguousarray(x[:, 128:256]),
                                   np.ascontiguousarray(w[:, 128:256]), rs)
    assert np.array_equal(c, ref)


def test_fp8_gemv_blockscale_power_of_two_grid_scales_exactly():
    # Doubling every block scale doubles every output exactly (no overflow
    # at these magnitudes): BF16 exponent + 1, same mantissa.
    x, w, s = _blockscale_case(24, 2, 128, 256)
    c1 = oracle.fp8_gemv_blockscale(x, w, s).astype(np.int64)
    c2 = oracle.fp8_gemv_blockscale(x, w, (s * 2).astype(np.float32)).astype(np.int64)
    nz = (c1 & 0x7FFF) != 0
    assert np.array_equal(c2[nz], c1[nz] + (1 << 7))


def test_fp8_gemv_blockscale_batched_rows_equal_single_row_calls():
    # The pages' invariant (w8a16_gemv_batch4 is bit-identical per row to
    # w8a16_gemv).
    x, w, s = _blockscale_case(25, 4, 128, 256)
    full = oracle.fp8_gemv_blockscale(x, w, s)
    for i in range(4):
        assert np.array_equal(full[i:i + 1], oracle.fp8_gemv_blockscale(x[i:i + 1], w, s))


# ---------------------------------------------------------------------------
# NVFP4-weight GEMV (W4A16; fp8_gemv_batch.rs names w4a16_gemv_batch8_rt2):
# C[i,j] = bf16(scale2 * sum_t x[i,t] * e2m1(w[j,t]) * e4m3(s[j,t/16])).
def _e2m1_ocp(code: int) -> Fraction:
    """OCP MX FP4 (E2M1) from its bit fields: sign, 2-bit exponent (bias 1),
    1-bit mantissa; exponent 0 is subnormal (0 or 0.5)."""
    sign = -1 if code & 8 else 1
    e, mb = (code >> 1) & 3, code & 1
    mag = Fraction(mb, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(mb, 2))
    return sign * mag


def _e4m3_torch(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn) \
        .to(torch.float64).numpy()


def _w4a16_case(seed, m, n, k):
    rng = np.random.default_rng(seed)
    x = _bf16(rng.standard_normal(m * k)).reshape(m, k)
    wp = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    # E4M3 block scales over subnormal and normal codes, no NaN
    ws = rng.integers(0x01, 0x7F, (n, k // 16), dtype=np.uint8)
    return x, wp, ws


def test_w4a16_gemv_rational():
    x, wp, ws = _w4a16_case(31, 2, 3, 64)
    ws[0, 0], ws[1, 1], ws[2, 2] = 0x01, 0x07, 0x7E     # 2^-9, subnormal max, 448
    scale2 = np.float32(0.37)
    c = oracle.w4a16_gemv(x, wp, ws, scale2)
    xf = oracle.bf16_bits_to_f32(x).astype(np.float64)
    sf = _e4m3_torch(ws)
    for i in range(2):
        for j in range(3):
            tot = Fraction(0)
            for t in range(64):
                code = (wp[j, t // 2] >> (4 * (t % 2))) & 15
                tot += Fraction(float(xf[i, t])) * _e2m1_ocp(int(code)) * Fraction(float(sf[j, t // 16]))
            assert c[i, j] == _bf16_exact(Fraction(float(scale2)) * tot), (i, j)


def test_w4a16_gemv_unit_scales_is_bf16_of_f64_matmul():
    # E4M3 code 0x38 is 1.0; with scale2 = 1 the GEMV is x @ e2m1(W)^T, which
    # numpy's f64 matmul forms exactly here (sums of bf16 x small halves), so
    # only the single BF16 rounding differs, at most on a tie.
    x, wp, _ = _w4a16_case(32, 4, 16, 256)
    ws = np.full((16, 256 // 16), 0x38, np.uint8)
    c = oracle.w4a16_gemv(x, wp, ws, 1.0).astype(np.int64)
    lo = np.vectorize(lambda b: float(_e2m1_ocp(int(b) & 15)))(wp)
    hi = np.vectorize(lambda b: float(_e2m1_ocp(int(b) >> 4)))(wp)
    wf = np.stack([lo, hi], axis=2).reshape(16, 256)
    ref = oracle.bf16_bits_to_f32(x).astype(np.float64) @ wf.T
    ref_bits = np.array([[_bf16_exact(Fraction(float(v))) for v in row] for row in ref], np.int64)
    assert np.array_equal(c, ref_bits)


def test_w4a16_gemv_nibble_order_and_block_indexing():
    # A weight with one nonzero code picks exactly one activation column:
    # element t sits in byte t/2 (low nibble for even t) and takes the scale
    # of block t/16.
    rng = np.random.default_rng(33)
    m, k = 3, 64
    x = _bf16(rng.standard_normal(m * k)).reshape(m, k)
    xf = oracle.bf16_bits_to_f32(x).astype(np.float64)
    ws = np.array([[0x30, 0x38, 0x40, 0x48]], np.uint8)          # 0.5, 1, 2, 4
    sf = _e4m3_torch(ws)[0]
    for t, code in [(0, 0x3), (1, 0xD), (17, 0x7), (46, 0x5), (63, 0xA)]:
        wp = np.zeros((1, k // 2), np.uint8)
        wp[0, t // 2] = code << (4 * (t % 2))
        c = oracle.w4a16_gemv(x, wp, ws, 1.5)
        for i in range(m):
            want = Fraction(3, 2) * Fraction(float(xf[i, t])) * _e2m1_ocp(code) * \
                Fraction(float(sf[t // 16]))
            assert c[i, 0] == _bf16_exact(want), (t, i)


def test_w4a16_gemv_batched_rows_equal_single_row_calls():
    x, wp, ws = _w4a16_case(34, 4, 8, 128)
    full = oracle.w4a16_gemv(x, wp, ws, 0.01)
    for i in range(4):
        assert np.array_equal(full[i:i + 1], oracle.w4a16_gemv(x[i:i + 1], wp, ws, 0.01))
