"""The degenerate shapes each entry point allows: one output row or column,
the smallest legal K (a single scale block, or a single partial segment of
a GEMV), and the wide GEMV kernels at their smallest K, against the CPU
oracle.  Codes and scales bit-exact, contractions to the same bounds as the
other parity tests.
"""
import numpy as np
import pytest
import torch

import gemv_nvfp4_int8_amd as qp
import oracle
import synth
from tests.gpu_util import assert_gemm_close, assert_gemv_close, bits, dev, empty, filled, host

pytestmark = pytest.mark.gpu


def _bf16(shape, seed, std=1.0):
    return synth.bf16_normal(shape, std, seed, "cpu")


def _t(x):
    return dev(torch.from_numpy(x))


@pytest.mark.parametrize("n,k", [(1, 32), (1, 64), (3, 32)])
def test_requant_w_nvfp4_int8_one_row_and_one_block(n, k):
    c = synth.w4a8_tiny("cpu", m=1, n=n, k=k)
    q, s = empty((n, k), torch.int8), empty((n, k // 32), torch.float32)
    qp.requant_w_nvfp4_int8(dev(c.w_packed), dev(c.w_e4m3), 0.5, q, s)
    oq, os_ = oracle.requant_w_nvfp4_int8(bits(c.w_packed), bits(c.w_e4m3), 0.5)
    assert np.array_equal(host(q), oq)
    assert np.array_equal(host(s).view(np.uint32), os_.view(np.uint32))


@pytest.mark.parametrize("rows,k", [(1, 32), (2, 32), (1, 96)])
def test_quantize_bf16_nvfp4_one_row(rows, k):
    x = _bf16((rows, k), 701 + rows + k)
    p, s = empty((rows, k // 2), torch.uint8), empty((rows, k // 16), torch.uint8)
    qp.quantize_bf16_nvfp4(dev(x), p, s, 1.0)
    op, os_ = oracle.quantize_bf16_nvfp4(bits(x), 1.0)
    assert np.array_equal(host(s), os_)
    assert np.array_equal(host(p), op)


@pytest.mark.parametrize("m,n,k", [(1, 1, 32), (1, 33, 32), (33, 1, 64), (2, 3, 32), (1, 1, 5120)])
def test_int8_gemm_single_rows_columns_and_block(m, n, k):
    a = _bf16((m, k), 711 + m)
    w = _bf16((n, k), 712 + n, std=0.02)
    oa, oas = oracle.requant_a_bf16_int8(bits(a))
    ow, ows = oracle.requant_a_bf16_int8(bits(w))
    out = filled((m, n), torch.bfloat16)
    qp.int8_gemm_blockscaled(_t(oa), _t(ow), _t(oas), _t(ows), out)
    assert_gemm_close(host(out), oracle.int8_gemm_blockscaled(oa, ow, oas, ows), f"int8 {m}x{n}x{k}")
    p = empty((m, n, k // 32), torch.int32)
    qp.int8_gemm_block_partials(_t(oa), _t(ow), p)
    assert np.array_equal(host(p), oracle.int8_block_partials(oa, ow))


@pytest.mark.parametrize("m,n,k", [(1, 1, 32), (1, 40, 32), (17, 1, 64), (1, 1, 4096)])
def test_w4a4_gemm_single_rows_columns_and_block(m, n, k):
    a = _bf16((m, k), 721 + m)
    w = _bf16((n, k), 722 + n, std=0.02)
    sw2 = synth.per_tensor_scale2(w)
    ap, asc = oracle.quantize_bf16_nvfp4(bits(a), 1.0)
    wp, wsc = oracle.quantize_bf16_nvfp4(bits(w), sw2)
    out = filled((m, n), torch.bfloat16)
    qp.w4a4_gemm(_t(ap), _t(asc), _t(wp), _t(wsc), out, 1.0, sw2)
    assert_gemm_close(host(out), oracle.w4a4_gemm(ap, asc, wp, wsc, 1.0, sw2), f"w4a4 {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(1, 1, 16), (1, 300, 16), (5, 1, 48), (1, 1, 5120)])
def test_fp8_gemm_single_rows_columns_and_k16(m, n, k):
    a = _bf16((m, k), 731 + m)
    w = _bf16((n, k), 732 + n, std=0.02)
    oa, oas = oracle.quant_rowwise_fp8(bits(a))
    ow, ows = oracle.quant_rowwise_fp8(bits(w))
    out = filled((m, n), torch.bfloat16)
    qp.fp8_gemm_rowscale(_t(oa), _t(oas), _t(ow), _t(ows), out)
    assert_gemm_close(host(out), oracle.fp8_gemm_rowscale(oa, oas, ow, ows), f"fp8 {m}x{n}x{k}")


# n = 1 and 7 take the narrow kernel with one workgroup; n = 65537 the wide
# one with a ragged last workgroup; k = 16 is a single partial segment.
@pytest.mark.parametrize("n,k", [(1, 16), (1, 5120), (7, 16), (65537, 16)])
def test_fp8_gemv_one_output_row_and_k16(n, k):
    w = synth.gemv_weight_bf16(n, k, "cpu", shape_id=8)
    ow, ows = oracle.quant_rowwise_fp8(bits(w))
    x = synth.gemv_acts_bf16(16, k, "cpu", shape_id=8)
    wq, ws = _t(ow), _t(ows)
    for m in (1, 2, 16):
        out = filled((m, n), torch.bfloat16)
        qp.fp8_gemv_rowscale(dev(x[:m].contiguous()), wq, ws, out)
        assert_gemv_close(host(out), oracle.fp8_gemv_rowscale(bits(x[:m]), ow, ows), f"gemv {n}x{k} m={m}")


@pytest.mark.parametrize("n,k", [(128, 128), (65536, 128)])
def test_fp8_gemv_blockscale_one_block_column(n, k):
    w, grid = synth.gemv_block_weight(n, k, "cpu", shape_id=9)
    x = synth.gemv_acts_bf16(16, k, "cpu", shape_id=9)
    for m in (1, 16):
        out = filled((m, n), torch.bfloat16)
        qp.fp8_gemv_blockscale(dev(x[:m].contiguous()), dev(w), dev(grid), out)
        assert_gemv_close(host(out), oracle.fp8_gemv_blockscale(bits(x[:m]), w.numpy(), grid.numpy()),
                          f"block gemv {n}x{k} m={m}")


@pytest.mark.parametrize("n,k", [(1, 32), (1, 5120), (5, 32), (65540, 32)])
def test_w4a16_gemv_one_output_row_and_k32(n, k):
    wp, ws, s2 = synth.gemv_nvfp4_weight(n, k, "cpu", shape_id=10)
    x = synth.gemv_acts_bf16(8, k, "cpu", shape_id=10)
    for m in (1, 5, 8):
        out = filled((m, n), torch.bfloat16)
        qp.w4a16_gemv(dev(x[:m].contiguous()), dev(wp), dev(ws), s2, out)
        assert_gemv_close(host(out), oracle.w4a16_gemv(bits(x[:m]), wp.numpy(), ws.numpy(), s2),
                          f"w4a16 {n}x{k} m={m}")


# k / 16 % 4 == 2 on the row-split kernel: the dword holding the matrix's
# last two scale bytes reaches past the end of the scale buffer, and a load
# that does so reads that whole dword as zero.  At k = 32, 160 and 2080 the
# two bytes open the first dword of the last piece (which starts at byte 0,
# 8 and 128 of the row's scales); at k = 96 and 224 they open its second
# dword.  The last rows carry the check.
@pytest.mark.parametrize("n,k", [(65540, 32), (65536, 160), (65544, 2080), (65536, 96),
                                 (65539, 224)])
def test_w4a16_gemv_wide_scale_row_end(n, k):
    wp, ws, s2 = synth.gemv_nvfp4_weight(n, k, "cpu", shape_id=11)
    x = synth.gemv_acts_bf16(8, k, "cpu", shape_id=11)
    for m in (1, 8):
        out = filled((m, n), torch.bfloat16)
        qp.w4a16_gemv(dev(x[:m].contiguous()), dev(wp), dev(ws), s2, out)
        ref = oracle.w4a16_gemv(bits(x[:m]), wp.numpy(), ws.numpy(), s2)
        assert_gemv_close(host(out), ref, f"w4a16 {n}x{k} m={m}")


@pytest.mark.parametrize("m,n,k", [(1, 1, 32), (1, 33, 64), (3, 1, 32)])
def test_int8_w4a8_prefill_single_rows_columns(m, n, k):
    """The fused prefill (activation requant, then the int8 GEMM) at one row
    or column and one scale block: its activation codes and scales bit-exact,
    its output to the GEMM bound."""
    a = _bf16((m, k), 741 + m)
    w = _bf16((n, k), 742 + n, std=0.02)
    ow, ows = oracle.requant_a_bf16_int8(bits(w))
    aq, asc = empty((m, k), torch.int8), empty((m, k // 32), torch.float32)
    out = filled((m, n), torch.bfloat16)
    qp.int8_w4a8_prefill(dev(a), _t(ow), _t(ows), aq, asc, out)
    oa, oas = oracle.requant_a_bf16_int8(bits(a))
    assert np.array_equal(host(aq), oa)
    assert np.array_equal(host(asc).view(np.uint32), oas.view(np.uint32))
    assert_gemm_close(host(out), oracle.int8_gemm_blockscaled(oa, ow, oas, ows), f"prefill {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(1, 128, 128), (3, 128, 256)])
def test_fp8_rowwise_proj_single_row_one_block(m, n, k):
    """The fused block-FP8 projection (weight requant, activation quant, GEMM)
    at one activation row and a single 128 x 128 scale block or row of them."""
    cse = synth.fp8_block("cpu", m=m, n=n, k=k)
    wr, wrs = empty((n, k), torch.uint8), empty((n,), torch.float32)
    aq, asc = empty((m, k), torch.uint8), empty((m,), torch.float32)
    out = filled((m, n), torch.bfloat16)
    qp.fp8_rowwise_proj(qp.QP_FP8_BLOCK128, dev(cse.w_block), dev(cse.block_grid), wr, wrs,
                        dev(cse.a_bf16), aq, asc, out)
    ow, ows = oracle.requant_w_blockfp8_rowwise(bits(cse.w_block), cse.block_grid.numpy())
    oa, oas = oracle.quant_rowwise_fp8(bits(cse.a_bf16))
    assert np.array_equal(host(wr), ow) and np.array_equal(host(aq), oa)
    assert_gemm_close(host(out), oracle.fp8_gemm_rowscale(oa, oas, ow, ows), f"proj {m}x{n}x{k}")
