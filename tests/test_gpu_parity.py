"""HIP path vs the CPU oracle, element by element, at sizes the oracle
finishes in seconds: several tiles plus ragged tails, and the edge cases of
each format (zero blocks, saturation, exact ties, subnormal scales).

Codes, scales and int32 block partials must be bit-exact; BF16 contraction
outputs must meet the stated tolerances (tests/gpu_util.py).
"""
import numpy as np
import pytest
import torch

import gemv_nvfp4_int8_amd as qp
import oracle
import synth
from tests.gpu_util import (assert_gemm_close, assert_gemv_close, bits,
                            copy_from_address, dev, empty, filled, host)

pytestmark = pytest.mark.gpu


def _bf16_rows(shape, seed, std=1.0, outliers=0.0):
    return synth.bf16_normal(shape, std, seed, "cpu", outlier_frac=outliers,
                             outlier_mult=20.0)


def _with_edges(x: torch.Tensor) -> torch.Tensor:
    """Plant edge blocks: an all-zero 32-block, a block of tiny values, a
    block holding exact ties, a saturating spike."""
    x = x.clone()
    k = x.shape[1]
    x[0, :32] = 0.0
    if x.shape[0] > 1:
        x[1, :32] = torch.tensor([1e-30] * 32)
    if x.shape[0] > 2 and k >= 64:
        t = torch.tensor([1, -2, 3, 0.25, 12, 0.75, -5, 2.5] * 4, dtype=torch.float32)
        x[2, 32:64] = t.to(torch.bfloat16)
    if x.shape[0] > 3:
        x[3, k - 1] = 3.0e4
    # signed zeros and tiny negatives keep their sign through every encoder
    x[-1, 1::7] = -0.0
    x[-1, 3::11] = -1e-30
    return x


# ------------------------------------------------------------- quantizers
@pytest.mark.parametrize("m,k", [(1, 32), (16, 512), (37, 160), (130, 1024)])
def test_requant_a_bf16_int8_bit_exact(m, k):
    a = _with_edges(_bf16_rows((m, k), 11 + m, outliers=0.01))
    q, s = empty((m, k), torch.int8), empty((m, k // 32), torch.float32)
    qp.requant_a_bf16_int8(dev(a), q, s)
    oq, os_ = oracle.requant_a_bf16_int8(bits(a))
    assert np.array_equal(host(q), oq)
    assert np.array_equal(host(s).view(np.uint32), os_.view(np.uint32))


@pytest.mark.parametrize("n,k,scale2", [(256, 512, 1.0), (33, 96, 0.0173), (300, 64, 2.0 ** -9)])
def test_requant_w_nvfp4_int8_bit_exact(n, k, scale2):
    c = synth.w4a8_tiny("cpu", m=1, n=n, k=k)
    sc = c.w_e4m3.clone()
    every = torch.arange(256, dtype=torch.int32)
    every[(every & 0x7F) == 0x7F] = 0x7E               # every finite E4M3 code
    cnt = min(256, sc.numel())
    sc.view(-1)[:cnt] = every[:cnt].to(torch.uint8)
    q, s = empty((n, k), torch.int8), empty((n, k // 32), torch.float32)
    qp.requant_w_nvfp4_int8(dev(c.w_packed), dev(sc), scale2, q, s)
    oq, os_ = oracle.requant_w_nvfp4_int8(bits(c.w_packed), bits(sc), scale2)
    assert np.array_equal(host(q), oq)
    assert np.array_equal(host(s).view(np.uint32), os_.view(np.uint32))


@pytest.mark.parametrize("rows,k,scale2", [(16, 512, 1.0), (33, 96, 1.0), (64, 256, None), (5, 4096, 0.37)])
def test_quantize_bf16_nvfp4_bit_exact(rows, k, scale2):
    x = _with_edges(_bf16_rows((rows, k), 21 + rows, std=0.02 if scale2 is None else 1.0))
    if scale2 is None:
        scale2 = synth.per_tensor_scale2(x)
    p, s = empty((rows, k // 2), torch.uint8), empty((rows, k // 16), torch.uint8)
    qp.quantize_bf16_nvfp4(dev(x), p, s, scale2)
    op, os_ = oracle.quantize_bf16_nvfp4(bits(x), scale2)
    assert np.array_equal(host(s), os_)
    assert np.array_equal(host(p), op)


# k / 8 chunks of 16 bytes per row select the kernel: one wave per row with
# up to 1, 2, 4, 6, 8, 10, 12 or 16 chunks per lane, a workgroup per row with
# up to 8 chunks per thread, or the two-pass long-row loop; each is run
# full and ragged (k = 1552, 2064, 6160, 12304 leave part of the last round
# empty), with row counts that leave the last workgroup's waves partly idle.
# Thousands of rows (the activation shapes) run with every workgroup resident
# at once; 4099 and 4133 rows leave the last workgroup partly idle, and
# k = 1008 and 5136 leave lanes without a chunk.
@pytest.mark.parametrize("rows,k", [(1, 16), (7, 48), (5, 1024), (6, 1552), (9, 2064),
                                    (4, 4096), (40, 5120), (3, 6144), (2, 6160), (3, 8192),
                                    (2, 12304), (3, 16384), (3, 20000), (4096, 512),
                                    (4099, 1008), (4133, 5136), (8192, 5120)])
def test_quant_rowwise_fp8_bit_exact(rows, k):
    x = _with_edges(_bf16_rows((rows, k), 31 + rows, std=0.02))
    q, s = empty((rows, k), torch.uint8), empty((rows,), torch.float32)
    qp.quant_rowwise_fp8(dev(x), q, s)
    oq, os_ = oracle.quant_rowwise_fp8(bits(x))
    assert np.array_equal(host(s).view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(host(q), oq)


@pytest.mark.parametrize("n,k", [(128, 128), (256, 384), (384, 5120), (1152, 1024),
                                 (640, 8192), (256, 2176), (256, 5888), (128, 8320),
                                 (128, 16384), (128, 16512), (256, 24576)])
def test_requant_blockfp8_rowwise_bit_exact(n, k):
    # k / 16 chunks per row select a one-wave-per-row kernel with up to 2, 4,
    # 5, 6, 8, 12 or 16 chunks per lane (k = 128 and 384 leave most lanes
    # idle, 2176, 5888 and 8320 part of the last round) or, past 16384, the
    # two-pass workgroup-per-row loop (16512, 24576).
    cse = synth.fp8_block("cpu", m=1, n=n, k=k)
    w, grid = cse.w_block.clone(), cse.block_grid
    w[1, ::5] = 0x80                     # -0.0 codes
    w[2, ::3] = 0x81                     # smallest negative subnormal
    wo, so = empty((n, k), torch.uint8), empty((n,), torch.float32)
    wres, sres = qp.requant_w_blockfp8_rowwise(qp.QP_FP8_BLOCK128, dev(w), dev(grid), wo, so)
    assert (wres, sres) == (wo.data_ptr(), so.data_ptr())
    oq, os_ = oracle.requant_w_blockfp8_rowwise(bits(w), grid.numpy())
    assert np.array_equal(host(so).view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(host(wo), oq)


def test_rowwise_weight_passes_through_without_launch_or_write():
    n, k = 256, 512
    w = dev(synth.uniform_bytes((n, k), 5))
    s = dev(torch.rand(n))
    wo, so = filled((n, k), torch.uint8), filled((n,), torch.float32)
    before = qp.launch_count()
    wres, sres = qp.requant_w_blockfp8_rowwise(qp.QP_FP8_PER_ROW, w, s, wo, so)
    assert (wres, sres) == (w.data_ptr(), s.data_ptr())
    assert qp.launch_count() == before
    assert bool((wo == 0xA5).all()) and bool((so.view(torch.uint8) == 0xA5).all())


# ------------------------------------------------------------ contractions
@pytest.mark.parametrize("m,n,k", [(16, 256, 512), (130, 200, 96), (1, 129, 32)])
def test_int8_block_partials_bit_exact(m, n, k):
    g = torch.Generator().manual_seed(m * 1000 + n)
    a = torch.randint(-127, 128, (m, k), generator=g, dtype=torch.int8)
    w = torch.randint(-127, 128, (n, k), generator=g, dtype=torch.int8)
    a[0, :32] = 127
    w[0, :32] = 127                                        # extreme partial 516128
    p = filled((m, n, k // 32), torch.int32)
    qp.int8_gemm_block_partials(dev(a), dev(w), p)
    assert np.array_equal(host(p), oracle.int8_block_partials(a.numpy(), w.numpy()))


def test_w4a8_tiny_pipeline_matches_oracle():
    """The W4A8 tiny workload (NVFP4 256x512 -> int8/per-32, BF16 acts 16x512)."""
    c = synth.w4a8_tiny("cpu")
    n, k, m = c.n, c.k, c.m
    w_i8, w_s = empty((n, k), torch.int8), empty((n, k // 32), torch.float32)
    a_i8, a_s = empty((m, k), torch.int8), empty((m, k // 32), torch.float32)
    out = filled((m, n), torch.bfloat16)
    qp.requant_w_nvfp4_int8(dev(c.w_packed), dev(c.w_e4m3), c.scale2, w_i8, w_s)
    qp.int8_w4a8_prefill(dev(c.a_bf16), w_i8, w_s, a_i8, a_s, out)
    ow, ows = oracle.requant_w_nvfp4_int8(bits(c.w_packed), bits(c.w_e4m3), c.scale2)
    oa, oas = oracle.requant_a_bf16_int8(bits(c.a_bf16))
    assert np.array_equal(host(w_i8), ow) and np.array_equal(host(w_s), ows)
    assert np.array_equal(host(a_i8), oa) and np.array_equal(host(a_s), oas)
    p = empty((m, n, k // 32), torch.int32)
    qp.int8_gemm_block_partials(a_i8, w_i8, p)
    assert np.array_equal(host(p), oracle.int8_block_partials(oa, ow))
    assert_gemm_close(host(out), oracle.int8_gemm_blockscaled(oa, ow, oas, ows), "w4a8 tiny")


# Ragged M and N tails, one and several tiles, K of one block up to the
# prefill's 5120.
@pytest.mark.parametrize("m,n,k", [(130, 200, 96), (256, 384, 1024), (7, 64, 5120),
                                   (256, 128, 64), (300, 200, 640), (513, 161, 192),
                                   (1024, 1056, 2048)])
def test_int8_gemm_blockscaled_ragged(m, n, k):
    a = _bf16_rows((m, k), 41 + m, outliers=0.01)
    w = _bf16_rows((n, k), 42 + n, std=0.02)
    oa, oas = oracle.requant_a_bf16_int8(bits(a))
    ow, ows = oracle.requant_a_bf16_int8(bits(w))
    out = filled((m, n), torch.bfloat16)
    qp.int8_gemm_blockscaled(dev(torch.from_numpy(oa)), dev(torch.from_numpy(ow)),
                             dev(torch.from_numpy(oas)), dev(torch.from_numpy(ows)), out)
    assert_gemm_close(host(out), oracle.int8_gemm_blockscaled(oa, ow, oas, ows), f"int8 {m}x{n}x{k}")


def _fold_in_f32(p, sa, sw):
    """The GEMM's F32 fold of exact block partials p [m, n, nb], written out:
    acc = fma(P_b, fl(a_s * w_s), acc) for b = 0, 1, ... in K order, each FMA
    one binary32 rounding (emulated exactly: P_b * sc is exact in binary64,
    and the sum is rounded once with a midpoint correction), then BF16."""
    from tests.test_division_shortcut import _rn32_of_sum
    m, n, nb = p.shape
    acc = np.zeros((m, n), np.float64)
    for b in range(nb):
        sc = (sa[:, b][:, None] * sw[:, b][None, :]).astype(np.float32)
        acc = _rn32_of_sum(p[:, :, b].astype(np.float64) * sc.astype(np.float64), acc)
    return bits(torch.from_numpy(acc.astype(np.float32)).to(torch.bfloat16))


@pytest.mark.parametrize("m,n,k", [(130, 200, 96), (256, 128, 128), (300, 200, 640),
                                   (513, 161, 384)])
def test_int8_gemm_is_the_f32_fold_of_the_exact_partials(m, n, k):
    """The GEMM (int8 MFMA) and its operand-route ablation (FP16 MFMA on
    converted operands, for K % 128 == 0) both return, bit for bit, bf16 of
    the F32 FMA chain over the exact int32 block partials in K order, with
    each scale product a binary32 multiply."""
    a = _bf16_rows((m, k), 61 + m, outliers=0.01)
    w = _bf16_rows((n, k), 62 + n, std=0.02)
    oa, oas = oracle.requant_a_bf16_int8(bits(a))
    ow, ows = oracle.requant_a_bf16_int8(bits(w))
    t = lambda x: dev(torch.from_numpy(x))
    p = empty((m, n, k // 32), torch.int32)
    qp.int8_gemm_block_partials(t(oa), t(ow), p)
    pp = host(p)
    assert np.array_equal(pp, oracle.int8_block_partials(oa, ow))
    want = _fold_in_f32(pp, oas, ows)
    out = filled((m, n), torch.bfloat16)
    qp.int8_gemm_blockscaled(t(oa), t(ow), t(oas), t(ows), out)
    assert np.array_equal(host(out), want)
    if k % 128 == 0:
        # the operand-route ablation (FP16 MFMA on converted operands)
        out = filled((m, n), torch.bfloat16)
        qp.int8_gemm_blockscaled_f16ops(t(oa), t(ow), t(oas), t(ows), out)
        assert np.array_equal(host(out), want)


# Shapes cover both kernels: the 128 x 128 one and the 256 x 160 one (M >= 256,
# N >= 160, K % 256 == 0) with one tile (256, 160), shifted last tiles
# (300 x 330, 520 x 500), one stage, an even and an odd stage count, and
# N % 4 != 0 (element-wise epilogue).  With N % 8 == 0 every tile stores
# through the LDS-staged epilogue, shifted ones with a row / 8-column test
# (256 x 160; 520 x 488 shifted in M and N, 520 x 480 in M only, 512 x 488 in
# N only).  The output starts filled with a sentinel, so a skipped store fails.
@pytest.mark.parametrize("m,n,k", [(64, 96, 256), (33, 70, 160), (200, 300, 1024), (5, 130, 4096),
                                   (256, 160, 256), (300, 330, 512), (520, 500, 1280), (257, 162, 768),
                                   (520, 488, 512), (520, 480, 512), (512, 488, 512)])
def test_w4a4_gemm_matches_oracle(m, n, k):
    a = _bf16_rows((m, k), 51 + m)
    w = _bf16_rows((n, k), 52 + n, std=0.02)
    sw2 = synth.per_tensor_scale2(w)
    ap, asc = oracle.quantize_bf16_nvfp4(bits(a), 1.0)
    wp, wsc = oracle.quantize_bf16_nvfp4(bits(w), sw2)
    out = filled((m, n), torch.bfloat16)
    t = lambda x: dev(torch.from_numpy(x))
    qp.w4a4_gemm(t(ap), t(asc), t(wp), t(wsc), out, 1.0, sw2)
    assert_gemm_close(host(out), oracle.w4a4_gemm(ap, asc, wp, wsc, 1.0, sw2), f"w4a4 {m}x{n}x{k}")


# The W4A4 GEMM runs a last round that is at most half full as 128 x 160 half
# tiles (one workgroup per CU).  Each output keeps its K sum order, so an
# M = 2304 or 2200 call (9 x 32 tiles: the last 32 split on 256 CUs) must
# equal, bit for bit, the same rows of an M = 3328 call (13 x 32 tiles, last
# round 160 > 128: no split).  M = 2200 shifts the last half tile;
# N = 5122 (33 column tiles, N % 4 != 0) takes the element-wise epilogue.
@pytest.mark.parametrize("m,n", [(2304, 5120), (2200, 5120), (2304, 5122)])
def test_w4a4_gemm_half_tile_tail_is_bit_identical(m, n):
    k, mref = 512, 3328
    cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    tiles = lambda mm: -(-mm // 256) * -(-n // 160)
    splits = lambda mm: 0 < tiles(mm) % cus <= cus // 2
    if not (splits(m) and not splits(mref)):
        pytest.skip(f"{cus} CUs: these shapes do not separate split and unsplit grids")
    a = _bf16_rows((mref, k), 91)
    w = _bf16_rows((n, k), 92, std=0.02)
    sw2 = synth.per_tensor_scale2(w)
    ap, asc = oracle.quantize_bf16_nvfp4(bits(a), 1.0)
    wp, wsc = oracle.quantize_bf16_nvfp4(bits(w), sw2)
    t = lambda x: dev(torch.from_numpy(np.ascontiguousarray(x)))
    ref = filled((mref, n), torch.bfloat16)
    qp.w4a4_gemm(t(ap), t(asc), t(wp), t(wsc), ref, 1.0, sw2)
    out = filled((m, n), torch.bfloat16)
    qp.w4a4_gemm(t(ap[:m]), t(asc[:m]), t(wp), t(wsc), out, 1.0, sw2)
    assert np.array_equal(host(out), host(ref)[:m])
    rng = np.random.default_rng(m + n)
    ri = np.union1d(rng.choice(m, 24, replace=False), np.arange(m - 8, m))
    ci = np.union1d(rng.choice(n, 64, replace=False), np.arange(n - 200, n))
    assert_gemm_close(host(out)[np.ix_(ri, ci)],
                      oracle.w4a4_gemm(ap[ri], asc[ri], wp[ci], wsc[ci], 1.0, sw2), f"w4a4 {m}x{n}")


@pytest.mark.parametrize("m,n,k", [(32, 128, 256), (256, 160, 512)])
def test_w4a4_every_scale_code_and_nibble(m, n, k):
    # All 16 E2M1 codes against all finite E4M3 scale codes, on both kernels.
    g = torch.Generator().manual_seed(3)
    ap = torch.randint(0, 256, (m, k // 2), generator=g, dtype=torch.int32).to(torch.uint8)
    wp = torch.randint(0, 256, (n, k // 2), generator=g, dtype=torch.int32).to(torch.uint8)
    codes = torch.arange(256, dtype=torch.int32)
    codes = codes[(codes & 0x7F) != 0x7F].to(torch.uint8)
    asc = codes[torch.randint(0, codes.numel(), (m, k // 16), generator=g)]
    wsc = codes[torch.randint(0, codes.numel(), (n, k // 16), generator=g)]
    out = filled((m, n), torch.bfloat16)
    qp.w4a4_gemm(dev(ap), dev(asc), dev(wp), dev(wsc), out, 1.0, 1.0)
    ref = oracle.w4a4_gemm(ap.numpy(), asc.numpy(), wp.numpy(), wsc.numpy(), 1.0, 1.0)
    assert_gemm_close(host(out), ref, "w4a4 all codes")


# Shapes cover both kernels: the 128 x 128 one (small M or N, K % 128 != 0)
# and the 256 x 256 one (M, N >= 256, K % 128 == 0) with a whole number of
# its 5-stage unroll (K = 640), a tail of 1 and of 2 stages (K = 128, 896),
# last tiles shifted back (M = 300, 260; N = 520, 514) and N % 4 != 0 (514:
# element-wise epilogue everywhere), and whole multiples of the unroll with
# shifted last tiles and N % 8 != 0 (K = 1280, 2560: 16-byte stores need
# N % 8 == 0, so N = 516 stores element-wise).
@pytest.mark.parametrize("m,n,k", [(130, 200, 272), (256, 384, 1024), (3, 70, 5120), (300, 520, 640),
                                   (512, 256, 128), (260, 514, 896), (300, 520, 1280),
                                   (512, 768, 2560), (260, 516, 1280)])
def test_fp8_gemm_rowscale_matches_oracle(m, n, k):
    a = _bf16_rows((m, k), 61 + m)
    w = _bf16_rows((n, k), 62 + n, std=0.02)
    oa, oas = oracle.quant_rowwise_fp8(bits(a))
    ow, ows = oracle.quant_rowwise_fp8(bits(w))
    out = filled((m, n), torch.bfloat16)
    t = lambda x: dev(torch.from_numpy(x))
    qp.fp8_gemm_rowscale(t(oa), t(oas), t(ow), t(ows), out)
    assert_gemm_close(host(out), oracle.fp8_gemm_rowscale(oa, oas, ow, ows), f"fp8 {m}x{n}x{k}")


# More 256 x 256 tiles than compute units (289 tiles: a second wave of 33
# workgroups; 289 % 8 = 1 leaves one tile outside the XCD remap); shifted last
# tiles with N % 8 != 0 (element-wise epilogue) and with N % 8 == 0 (staged
# epilogue with a row / 8-column guard), shifted in M, in N or in both.  The
# output starts filled with a sentinel, so a skipped store fails.  The
# oracle computes a sample of rows and columns (each output depends only on
# its own row pair): random ones plus every row and column of the last two
# tile rows and columns.
@pytest.mark.parametrize("m,n,k", [(4352, 4352, 640), (4200, 4100, 640), (4200, 4104, 1280),
                                   (4200, 4352, 640), (4352, 4104, 640)])
def test_fp8_gemm_rowscale_many_tiles_matches_oracle(m, n, k):
    a = _bf16_rows((m, k), 63 + m)
    w = _bf16_rows((n, k), 64 + n, std=0.02)
    oa, oas = oracle.quant_rowwise_fp8(bits(a))
    ow, ows = oracle.quant_rowwise_fp8(bits(w))
    out = filled((m, n), torch.bfloat16)
    t = lambda x: dev(torch.from_numpy(x))
    qp.fp8_gemm_rowscale(t(oa), t(oas), t(ow), t(ows), out)
    rng = np.random.default_rng(m + n + k)
    ri = np.union1d(rng.choice(m - 512, 96, replace=False), np.arange(m - 512, m))
    ci = np.union1d(rng.choice(n - 512, 96, replace=False), np.arange(n - 512, n))
    ref = oracle.fp8_gemm_rowscale(oa[ri], oas[ri], ow[ci], ows[ci])
    assert_gemm_close(host(out)[np.ix_(ri, ci)], ref, f"fp8 {m}x{n}x{k}")


# One workgroup runs per CU, so a grid whose last round is at most half full
# runs that round's tiles as 256 x 128 half tiles.  Each output still takes its
# whole K sum in the same order, so results must not depend on the split: an
# M = 2048 or 1900 call (8 x 48 tiles, the last 128 of the banded order split
# into halves on 256 CUs) must equal, bit for bit, the same rows of an
# M = 2304 call (9 x 48 tiles, last round 176 > 128: no split).  N = 12200
# shifts the last half tile; N = 12196 (N % 8 != 0) takes the element-wise
# epilogue; M = 1900 shifts the last tile row.
@pytest.mark.parametrize("m,n", [(2048, 12200), (1900, 12200), (2048, 12196)])
def test_fp8_gemm_half_tile_tail_is_bit_identical(m, n):
    k, mref = 1280, 2304
    cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    tiles = lambda mm: -(-mm // 256) * -(-n // 256)
    splits = lambda mm: 0 < tiles(mm) % cus <= cus // 2
    if not (splits(m) and not splits(mref)):
        pytest.skip(f"{cus} CUs: these shapes do not separate split and unsplit grids")
    a = _bf16_rows((mref, k), 81)
    w = _bf16_rows((n, k), 82, std=0.02)
    oa, oas = oracle.quant_rowwise_fp8(bits(a))
    ow, ows = oracle.quant_rowwise_fp8(bits(w))
    t = lambda x: dev(torch.from_numpy(np.ascontiguousarray(x)))
    ref = filled((mref, n), torch.bfloat16)
    qp.fp8_gemm_rowscale(t(oa), t(oas), t(ow), t(ows), ref)
    out = filled((m, n), torch.bfloat16)
    qp.fp8_gemm_rowscale(t(oa[:m]), t(oas[:m]), t(ow), t(ows), out)
    assert np.array_equal(host(out), host(ref)[:m])
    rng = np.random.default_rng(m + n)
    ri = np.union1d(rng.choice(m, 24, replace=False), np.arange(m - 8, m))
    ci = np.union1d(rng.choice(n, 64, replace=False), np.arange(n - 300, n))
    assert_gemm_close(host(out)[np.ix_(ri, ci)],
                      oracle.fp8_gemm_rowscale(oa[ri], oas[ri], ow[ci], ows[ci]), f"fp8 {m}x{n}")


def test_fp8_rowwise_proj_block_and_passthrough():
    m, n, k = 70, 256, 512
    cse = synth.fp8_block("cpu", m=m, n=n, k=k)
    t = lambda x: dev(torch.from_numpy(x))
    # block-scaled layer: requant + activation quant + GEMM in one call
    wr, wrs = empty((n, k), torch.uint8), empty((n,), torch.float32)
    aq, asc = empty((m, k), torch.uint8), empty((m,), torch.float32)
    out = filled((m, n), torch.bfloat16)
    qp.fp8_rowwise_proj(qp.QP_FP8_BLOCK128, dev(cse.w_block), dev(cse.block_grid),
                        wr, wrs, dev(cse.a_bf16), aq, asc, out)
    ow, ows = oracle.requant_w_blockfp8_rowwise(bits(cse.w_block), cse.block_grid.numpy())
    oa, oas = oracle.quant_rowwise_fp8(bits(cse.a_bf16))
    assert np.array_equal(host(wr), ow) and np.array_equal(host(aq), oa)
    assert_gemm_close(host(out), oracle.fp8_gemm_rowscale(oa, oas, ow, ows), "proj block")
    # already row-wise layer: passthrough, no requant launch
    pw, pws = oracle.quant_rowwise_fp8(bits(cse.w_rowwise_bf16))
    out2 = filled((m, n), torch.bfloat16)
    before = qp.launch_count()
    qp.fp8_rowwise_proj(qp.QP_FP8_PER_ROW, t(pw), t(pws), None, None,
                        dev(cse.a_bf16), aq, asc, out2)
    assert qp.launch_count() - before == 2            # act quant + GEMM only
    assert_gemm_close(host(out2), oracle.fp8_gemm_rowscale(oa, oas, pw, pws), "proj rowwise")


@pytest.mark.parametrize("n,k", [(37, 512), (200, 48), (6144, 5120)])
def test_fp8_gemv_rowscale_all_m(n, k):
    w = synth.gemv_weight_bf16(n, k, "cpu")
    ow, ows = oracle.quant_rowwise_fp8(bits(w))
    wq, ws = dev(torch.from_numpy(ow)), dev(torch.from_numpy(ows))
    x = synth.gemv_acts_bf16(16, k, "cpu")
    for m in range(1, 17):
        out = filled((m, n), torch.bfloat16)
        qp.fp8_gemv_rowscale(dev(x[:m].contiguous()), wq, ws, out)
        assert_gemv_close(host(out), oracle.fp8_gemv_rowscale(bits(x[:m]), ow, ows), f"gemv m={m}")


# N >= 65536 runs the row-owning kernel above M = 2 and the K-split kernel
# at M <= 2, so there the invariant also holds across the two kernels: K =
# 2560 gives four non-empty K quarters (the last short), 1040 a partial last
# segment and an empty last quarter, 256 three empty quarters.
@pytest.mark.parametrize("n,k", [(300, 512), (17408, 5120), (65552, 2560), (65552, 1040),
                                 (65600, 256)])
def test_fp8_gemv_batched_rows_bit_identical_to_single_row(n, k):
    """The pages' invariant for the batched GEMV (fp8_gemv_batch.rs,
    dense_gemv_fp8w_batch2): each row of an M-row call equals, bit for bit,
    an M = 1 call on that row."""
    w = synth.gemv_weight_bf16(n, k, "cpu", shape_id=1)
    ow, ows = oracle.quant_rowwise_fp8(bits(w))
    wq, ws = dev(torch.from_numpy(ow)), dev(torch.from_numpy(ows))
    x = dev(synth.gemv_acts_bf16(16, k, "cpu", shape_id=1))
    singles = []
    for i in range(16):
        o = empty((1, n), torch.bfloat16)
        qp.fp8_gemv_rowscale(x[i:i + 1], wq, ws, o)
        singles.append(o)
    single = torch.cat(singles)
    for m in (2, 3, 8, 16):
        o = empty((m, n), torch.bfloat16)
        qp.fp8_gemv_rowscale(x[:m], wq, ws, o)
        assert torch.equal(o.view(torch.int16), single[:m].view(torch.int16)), m


# Both FP8 GEMV kernels sum every row in the same order (K quarters ending on
# 256-element boundaries, added in order), so a weight row's output does not
# depend on N either: the first 17408 rows of a wide weight (row-owning
# kernel above M = 2) equal, bit for bit, the same rows run as a narrow
# weight (K-split kernel).
@pytest.mark.parametrize("k", [2560, 1040, 256])
def test_fp8_gemv_wide_and_narrow_kernels_agree_bit_for_bit(k):
    n, nn = 65552, 17408
    w = synth.gemv_weight_bf16(n, k, "cpu", shape_id=6)
    ow, ows = oracle.quant_rowwise_fp8(bits(w))
    wq, ws = dev(torch.from_numpy(ow)), dev(torch.from_numpy(ows))
    x = dev(synth.gemv_acts_bf16(16, k, "cpu", shape_id=6))
    for m in (1, 2, 3, 8, 16):
        wide, narrow = empty((m, n), torch.bfloat16), empty((m, nn), torch.bfloat16)
        qp.fp8_gemv_rowscale(x[:m], wq, ws, wide)
        qp.fp8_gemv_rowscale(x[:m], wq[:nn], ws[:nn], narrow)
        assert torch.equal(wide[:, :nn].view(torch.int16), narrow.view(torch.int16)), m


@pytest.mark.parametrize("n,k", [(70000, 512), (65552, 1040), (37, 1040), (12300, 1040)])
def test_fp8_gemv_wide_and_partial_segments(n, k):
    # n >= 65536 takes the row-split kernel; k = 1040 ends 16 elements into a
    # 256-element segment; n = 70000 / 65552 leave ragged row tiles; n = 12300
    # takes the K-split kernel with two segments in flight, ragged against
    # both its 8- and 16-row units, and its last wave gets no segment.
    w = synth.gemv_weight_bf16(n, k, "cpu", shape_id=2)
    ow, ows = oracle.quant_rowwise_fp8(bits(w))
    wq, ws = dev(torch.from_numpy(ow)), dev(torch.from_numpy(ows))
    x = synth.gemv_acts_bf16(16, k, "cpu", shape_id=2)
    for m in (1, 3, 16):
        out = filled((m, n), torch.bfloat16)
        qp.fp8_gemv_rowscale(dev(x[:m].contiguous()), wq, ws, out)
        assert_gemv_close(host(out), oracle.fp8_gemv_rowscale(bits(x[:m]), ow, ows), f"gemv {n}x{k} m={m}")


# Narrow weights above M = 2 take a whole number of workgroups per CU, each
# with ceil(N / workgroups) live rows inside a capacity of 16 to 80 rows.  On
# a 256-CU part these N reach every capacity: 12288 (48 rows at M > 8),
# 16384 (64), 17408 (68 live of 80 at M > 8, 34 of 48 at M <= 8, 14 of 16
# at M <= 4), 20481 (41 of 48, ragged last workgroup), 40000 (79 of 80).  The
# whole output is checked against the oracle, and every row of an M-row call
# equals the M = 1 call on that row bit for bit.
@pytest.mark.parametrize("n", [12288, 16384, 17408, 20481, 40000])
def test_fp8_gemv_balanced_row_split(n):
    k = 1040
    w = synth.gemv_weight_bf16(n, k, "cpu", shape_id=3)
    ow, ows = oracle.quant_rowwise_fp8(bits(w))
    wq, ws = dev(torch.from_numpy(ow)), dev(torch.from_numpy(ows))
    x = synth.gemv_acts_bf16(16, k, "cpu", shape_id=3)
    xd = dev(x)
    singles = []
    for i in range(16):
        o = empty((1, n), torch.bfloat16)
        qp.fp8_gemv_rowscale(xd[i:i + 1], wq, ws, o)
        singles.append(o)
    single = torch.cat(singles)
    for m in (3, 5, 8, 9, 16):
        out = filled((m, n), torch.bfloat16)
        qp.fp8_gemv_rowscale(xd[:m], wq, ws, out)
        assert_gemv_close(host(out), oracle.fp8_gemv_rowscale(bits(x[:m]), ow, ows), f"gemv {n} m={m}")
        assert torch.equal(out.view(torch.int16), single[:m].view(torch.int16)), m


# ---------------------------------------------------------------------------
# Block-scaled FP8 GEMV (fp8_gemv_batch.rs, w8a16_gemv_batch4 / _batch2).
@pytest.mark.parametrize("n,k", [(128, 128), (256, 384), (384, 1152), (6144, 5120),
                                 (12416, 1152), (65664, 640)])
def test_fp8_gemv_blockscale_all_m(n, k):
    # k = 384 and 1152 end half-way through a 256-element segment; k = 1152
    # leaves the last K-split wave without a segment; n = 12416 takes the
    # K-split kernel with two segments in flight; n = 65664 takes the
    # row-split kernel.
    w, grid = synth.gemv_block_weight(n, k, "cpu", shape_id=0)
    x = synth.gemv_acts_bf16(16, k, "cpu", shape_id=3)
    wd, gd = dev(w), dev(grid)
    for m in (range(1, 17) if n * k < 6144 * 5120 else (1, 3, 16)):
        out = filled((m, n), torch.bfloat16)
        qp.fp8_gemv_blockscale(dev(x[:m].contiguous()), wd, gd, out)
        assert_gemv_close(host(out), oracle.fp8_gemv_blockscale(bits(x[:m]), w.numpy(), grid.numpy()),
                          f"block gemv {n}x{k} m={m}")


@pytest.mark.parametrize("n,k", [(256, 512), (65536, 256)])
def test_fp8_gemv_blockscale_every_code_and_extreme_scales(n, k):
    # Every finite E4M3 code (subnormals included) appears in every row, and
    # the grid mixes zero blocks with power-of-two scales from 2^-30 to 2^10.
    g = np.random.default_rng(5)
    w = g.integers(0, 256, (n, k), dtype=np.uint8)
    w[:, :256] = np.arange(256, dtype=np.uint8)[None, :]
    w[(w & 0x7F) == 0x7F] = 0x00
    grid = np.exp2(g.integers(-30, 11, (n // 128, k // 128))).astype(np.float32)
    grid[g.random(grid.shape) < 0.2] = 0.0
    x = synth.gemv_acts_bf16(4, k, "cpu", shape_id=4)
    out = filled((4, n), torch.bfloat16)
    qp.fp8_gemv_blockscale(dev(x), dev(torch.from_numpy(w)), dev(torch.from_numpy(grid)), out)
    assert_gemv_close(host(out), oracle.fp8_gemv_blockscale(bits(x), w, grid), "block gemv codes")


@pytest.mark.parametrize("n,k", [(384, 640), (17408, 5120), (65536, 5120), (65664, 640)])
def test_fp8_gemv_blockscale_batched_rows_bit_identical_to_single_row(n, k):
    """The pages' invariant for w8a16_gemv_batch4 (fp8_gemv_batch.rs): each
    row of an M-row call equals, bit for bit, the single-row call."""
    w, grid = synth.gemv_block_weight(n, k, "cpu", shape_id=1)
    wd, gd = dev(w), dev(grid)
    x = dev(synth.gemv_acts_bf16(16, k, "cpu", shape_id=5))
    singles = []
    for i in range(16):
        o = empty((1, n), torch.bfloat16)
        qp.fp8_gemv_blockscale(x[i:i + 1], wd, gd, o)
        singles.append(o)
    single = torch.cat(singles)
    for m in (2, 3, 4, 16):
        o = empty((m, n), torch.bfloat16)
        qp.fp8_gemv_blockscale(x[:m], wd, gd, o)
        assert torch.equal(o.view(torch.int16), single[:m].view(torch.int16)), m


# The block-scaled form's kernels also share every row's summation order:
# the first 12416 rows of a wide weight equal the same rows run narrow
# (K = 640: an odd number of 128-blocks, an empty last K quarter).
@pytest.mark.parametrize("k", [5120, 640])
def test_fp8_gemv_blockscale_wide_and_narrow_kernels_agree_bit_for_bit(k):
    n, nn = 65664, 12416
    w, grid = synth.gemv_block_weight(n, k, "cpu", shape_id=2)
    wd, gd = dev(w), dev(grid)
    x = dev(synth.gemv_acts_bf16(16, k, "cpu", shape_id=7))
    for m in (1, 2, 3, 8, 16):
        wide, narrow = empty((m, n), torch.bfloat16), empty((m, nn), torch.bfloat16)
        qp.fp8_gemv_blockscale(x[:m], wd, gd, wide)
        qp.fp8_gemv_blockscale(x[:m], wd[:nn], gd[:nn // 128], narrow)
        assert torch.equal(wide[:, :nn].view(torch.int16), narrow.view(torch.int16)), m


# ---------------------------------------------------------------------------
# NVFP4-weight GEMV, W4A16 (fp8_gemv_batch.rs names w4a16_gemv_batch8_rt2).
@pytest.mark.parametrize("n,k", [(64, 64), (256, 96), (200, 352), (384, 1216), (5000, 224),
                                 (3000, 2048), (6144, 5120), (17408, 512), (65600, 448),
                                 (65664, 1600)])
def test_w4a16_gemv_all_m(n, k):
    # k = 96 / 352 / 1216 / 224 / 448 / 1600 end 96 / 352 / 192 / 224 / 448 /
    # 64 elements into a 512-element window; k = 1216 (3 windows) ends on an
    # odd window.  Narrow n take 4 rows per wave (17408) or 3 live rows of
    # 4 (6144, and 5000 with a ragged last workgroup, and the small n);
    # n >= 65536 takes 8 rows per wave (ragged last tiles), whose staged scale
    # pieces straddle the end of a row's scales at k = 448 and 1600.  m <= 4
    # and m > 4 take the one- and two-group kernels; at m <= 4 the small
    # narrow grids (all but n = 17408) run four register stages, with 1, 3,
    # 4 (k = 2048) and 10 windows.
    wp, ws, s2 = synth.gemv_nvfp4_weight(n, k, "cpu", shape_id=0)
    x = synth.gemv_acts_bf16(8, k, "cpu", shape_id=6)
    wpd, wsd = dev(wp), dev(ws)
    for m in (range(1, 9) if n * k < 6144 * 5120 else (1, 3, 5, 8)):
        out = filled((m, n), torch.bfloat16)
        qp.w4a16_gemv(dev(x[:m].contiguous()), wpd, wsd, s2, out)
        assert_gemv_close(host(out), oracle.w4a16_gemv(bits(x[:m]), wp.numpy(), ws.numpy(), s2),
                          f"w4a16 {n}x{k} m={m}")


@pytest.mark.parametrize("n,k", [(256, 512), (65536, 256)])
def test_w4a16_gemv_every_code_and_scale(n, k):
    # Every byte value (so every nibble pair) in every row, and every finite
    # E4M3 scale code of either sign across the blocks.
    g = np.random.default_rng(6)
    wp = g.integers(0, 256, (n, k // 2), dtype=np.uint8)
    wp[:, :128] = np.arange(256, dtype=np.uint8)[:128][None, :] + \
        (np.arange(n, dtype=np.uint8)[:, None] & 1) * 128
    ws = g.integers(0, 256, (n, k // 16), dtype=np.uint8)
    ws[(ws & 0x7F) == 0x7F] = 0x38
    ws.reshape(-1)[:254] = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    x = synth.gemv_acts_bf16(4, k, "cpu", shape_id=7)
    out = filled((4, n), torch.bfloat16)
    qp.w4a16_gemv(dev(x), dev(torch.from_numpy(wp)), dev(torch.from_numpy(ws)), 0.75, out)
    assert_gemv_close(host(out), oracle.w4a16_gemv(bits(x), wp, ws, 0.75), "w4a16 codes")


@pytest.mark.parametrize("n,k", [(384, 640), (17408, 5120), (65536, 5120)])
def test_w4a16_gemv_batched_rows_bit_identical_to_single_row(n, k):
    """Each row of an M-row call equals, bit for bit, the single-row call
    (the batched GEMV family's invariant, fp8_gemv_batch.rs)."""
    wp, ws, s2 = synth.gemv_nvfp4_weight(n, k, "cpu", shape_id=1)
    wpd, wsd = dev(wp), dev(ws)
    x = dev(synth.gemv_acts_bf16(8, k, "cpu", shape_id=8))
    singles = []
    for i in range(8):
        o = empty((1, n), torch.bfloat16)
        qp.w4a16_gemv(x[i:i + 1], wpd, wsd, s2, o)
        singles.append(o)
    single = torch.cat(singles)
    for m in (2, 4, 5, 8):
        o = empty((m, n), torch.bfloat16)
        qp.w4a16_gemv(x[:m], wpd, wsd, s2, o)
        assert torch.equal(o.view(torch.int16), single[:m].view(torch.int16)), m


# ---------------------------------------------------------------------------
# Derived-weight cache (dispatch_proj_rowwise.rs, requant_weight_rowwise_fp8_
# cached and DerivedWeights; gemm_dense_int8.rs, lazy first-use requant).
def test_cache_derives_once_and_matches_the_oracle():
    m, n, k = 64, 256, 384
    cse = synth.fp8_block("cpu", m, n, k)
    w, g = dev(cse.w_block), dev(cse.block_grid)
    c = qp.DerivedWeights()
    try:
        before = qp.launch_count()
        p1 = c.requant_w_blockfp8_rowwise(qp.QP_FP8_BLOCK128, w, g)
        assert qp.launch_count() == before + 1
        assert c.stats() == (1, n * k + 4 * n)
        p2 = c.requant_w_blockfp8_rowwise(qp.QP_FP8_BLOCK128, w, g)
        assert p2 == p1 and qp.launch_count() == before + 1          # a hit: no launch
        ow, ows = oracle.requant_w_blockfp8_rowwise(bits(cse.w_block), cse.block_grid.numpy())
        wq = copy_from_address(p1[0], (n, k), torch.uint8)
        ws = copy_from_address(p1[1], (n,), torch.float32)
        assert np.array_equal(host(wq), ow) and np.array_equal(host(ws), ows)
        # the same address asked for with other sizes holds another weight
        with pytest.raises(qp.QProjError) as err:
            c.requant_w_blockfp8_rowwise(qp.QP_FP8_BLOCK128, w[:128], g[:1])
        assert err.value.status == qp.QP_ERR_SHAPE
        # a second weight is a second entry; eviction drops only the first
        w2 = w.clone()
        c.requant_w_blockfp8_rowwise(qp.QP_FP8_BLOCK128, w2, g)
        assert c.stats() == (2, 2 * (n * k + 4 * n))
        c.evict(w)
        assert c.stats() == (1, n * k + 4 * n)
        before = qp.launch_count()
        c.requant_w_blockfp8_rowwise(qp.QP_FP8_BLOCK128, w, g)
        assert qp.launch_count() == before + 1                        # derived again
        # a per-row weight passes through untouched
        assert c.requant_w_blockfp8_rowwise(qp.QP_FP8_PER_ROW, wq, ws) == (wq.data_ptr(), ws.data_ptr())
        assert c.stats() == (2, 2 * (n * k + 4 * n))
    finally:
        c.close()


def test_cache_concurrent_requests_derive_once():
    """Eight host threads ask for the same weight at once (ctypes releases
    the GIL inside the call): the miss holds the cache's lock, so exactly
    one derivation is launched and every thread gets the same buffers."""
    import threading
    m, n, k = 64, 256, 384
    cse = synth.fp8_block("cpu", m, n, k)
    w, g = dev(cse.w_block), dev(cse.block_grid)
    c = qp.DerivedWeights()
    try:
        torch.cuda.synchronize()
        before = qp.launch_count()
        got, errs = [], []
        go = threading.Barrier(8)

        def ask():
            try:
                go.wait()
                got.append(c.requant_w_blockfp8_rowwise(qp.QP_FP8_BLOCK128, w, g))
            except Exception as e:          # reported below
                errs.append(e)

        ts = [threading.Thread(target=ask) for _ in range(8)]
        for t in ts:
            t.start()
        for t in ts:
            t.join()
        assert not errs, errs
        assert len(got) == 8 and len(set(got)) == 1
        assert qp.launch_count() == before + 1
        assert c.stats() == (1, n * k + 4 * n)
        ow, ows = oracle.requant_w_blockfp8_rowwise(bits(cse.w_block), cse.block_grid.numpy())
        wq = copy_from_address(got[0][0], (n, k), torch.uint8)
        assert np.array_equal(host(wq), ow)
    finally:
        torch.cuda.synchronize()
        c.close()


def test_cached_projection_equals_stateless_across_streams():
    """Derive on a side stream, then use the hit on the current stream
    without synchronising the side stream: the hit orders the projection
    after the derivation."""
    m, n, k = 130, 384, 640
    cse = synth.fp8_block("cpu", m, n, k)
    w, g, a = dev(cse.w_block), dev(cse.block_grid), dev(cse.a_bf16)
    aq, asc = empty((m, k), torch.uint8), empty((m,), torch.float32)
    ref = filled((m, n), torch.bfloat16)
    wr, wrs = empty((n, k), torch.uint8), empty((n,), torch.float32)
    qp.fp8_rowwise_proj(qp.QP_FP8_BLOCK128, w, g, wr, wrs, a, aq, asc, ref)
    c = qp.DerivedWeights()
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        c.requant_w_blockfp8_rowwise(qp.QP_FP8_BLOCK128, w, g, stream=side)
        out = filled((m, n), torch.bfloat16)
        aq2, asc2 = empty((m, k), torch.uint8), empty((m,), torch.float32)
        c.fp8_rowwise_proj(qp.QP_FP8_BLOCK128, w, g, a, aq2, asc2, out)
        assert torch.equal(host_t(out), host_t(ref))
        assert c.stats()[0] == 1
    finally:
        torch.cuda.synchronize()
        c.close()


def test_cached_int8_prefill_equals_stateless():
    m, n, k = 96, 320, 512
    cse = synth.w4a8_prefill("cpu", m, n, k)
    wb, a = dev(cse.w_bf16), dev(cse.a_bf16)
    wp, we = empty((n, k // 2), torch.uint8), empty((n, k // 16), torch.uint8)
    qp.quantize_bf16_nvfp4(wb, wp, we, cse.scale2)
    wi8, wsc = empty((n, k), torch.int8), empty((n, k // 32), torch.float32)
    qp.requant_w_nvfp4_int8(wp, we, cse.scale2, wi8, wsc)
    ai8, asc = empty((m, k), torch.int8), empty((m, k // 32), torch.float32)
    ref = filled((m, n), torch.bfloat16)
    qp.int8_w4a8_prefill(a, wi8, wsc, ai8, asc, ref)
    c = qp.DerivedWeights()
    try:
        out = filled((m, n), torch.bfloat16)
        c.int8_w4a8_prefill(a, wp, we, cse.scale2, ai8, asc, out)
        before = qp.launch_count()
        c.int8_w4a8_prefill(a, wp, we, cse.scale2, ai8, asc, out)
        assert qp.launch_count() == before + 2                        # act requant + GEMM only
        assert torch.equal(host_t(out), host_t(ref))
        p = c.requant_w_nvfp4_int8(wp, we, cse.scale2)
        assert torch.equal(host_t(copy_from_address(p[0], (n, k), torch.int8)), host_t(wi8))
        assert torch.equal(host_t(copy_from_address(p[1], (n, k // 32), torch.float32)), host_t(wsc))
        with pytest.raises(qp.QProjError) as err:                     # another scale2: another weight
            c.requant_w_nvfp4_int8(wp, we, cse.scale2 * 2)
        assert err.value.status == qp.QP_ERR_SHAPE
    finally:
        c.close()


def host_t(t):
    torch.cuda.synchronize()
    return t.cpu().view(torch.uint8) if t.dtype != torch.uint8 else t.cpu()


@pytest.mark.parametrize("m,n,k", [(520, 500, 1280), (200, 300, 96)])
def test_w4a4_tile_orders_agree_bit_for_bit(m, n, k):
    """The tile-order ablation (gemm_fp4.rs, w4a4_gemm against
    w4a4_gemm_mfast) changes only which workgroup computes which tile."""
    a = _bf16_rows((m, k), 71)
    w = _bf16_rows((n, k), 72, std=0.02)
    ap, asc = empty((m, k // 2), torch.uint8), empty((m, k // 16), torch.uint8)
    wp, wsc = empty((n, k // 2), torch.uint8), empty((n, k // 16), torch.uint8)
    qp.quantize_bf16_nvfp4(dev(a), ap, asc, 1.0)
    qp.quantize_bf16_nvfp4(dev(w), wp, wsc, 0.01)
    outs = []
    for order in (qp.QP_TILES_BANDED, qp.QP_TILES_MFAST, qp.QP_TILES_NFAST):
        o = filled((m, n), torch.bfloat16)
        qp.w4a4_gemm(ap, asc, wp, wsc, o, 1.0, 0.01, tile_order=order)
        outs.append(host(o))
    ref = oracle.w4a4_gemm(host(ap), host(asc), host(wp), host(wsc), 1.0, 0.01)
    assert_gemm_close(outs[0], ref, "w4a4 banded")
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
