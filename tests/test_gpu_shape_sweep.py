"""Seeded random shapes through every entry point, against the oracle.

The parity tests pick their shapes by hand, one per kernel path and edge;
this sweep draws shapes at random (fixed seed, so the cases are the same on
every run) within each entry point's legal range, so that combinations
nobody picked (tile remainders against stage counts, row groups against
segment tails, grids of a few workgroups) are exercised too.  Codes and
scales must be bit-exact, contractions within the stated tolerances
(tests/gpu_util.py).
"""
import numpy as np
import pytest
import torch

import gemv_nvfp4_int8_amd as qp
import oracle
import synth
from tests.gpu_util import (assert_gemm_close, assert_gemv_close, bits, dev, empty,
                            filled, host)

pytestmark = pytest.mark.gpu

_rng = np.random.default_rng(0x5EED5)


def _draw(n, make):
    return [make() for _ in range(n)]


def _i(lo, hi):
    return int(_rng.integers(lo, hi + 1))


def _acts(shape, seed, std=1.0):
    return synth.bf16_normal(shape, std, seed, "cpu", outlier_frac=0.01, outlier_mult=20.0)


# ------------------------------------------------------------- quantizers
@pytest.mark.parametrize("m,k", _draw(6, lambda: (_i(1, 300), 32 * _i(1, 64))))
def test_sweep_requant_a_bf16_int8(m, k):
    a = _acts((m, k), 1000 + m + k)
    q, s = empty((m, k), torch.int8), empty((m, k // 32), torch.float32)
    qp.requant_a_bf16_int8(dev(a), q, s)
    oq, os_ = oracle.requant_a_bf16_int8(bits(a))
    assert np.array_equal(host(q), oq)
    assert np.array_equal(host(s).view(np.uint32), os_.view(np.uint32))


@pytest.mark.parametrize("n,k,scale2", _draw(6, lambda: (_i(1, 300), 32 * _i(1, 64),
                                                         float(_rng.choice([1.0, 0.37, 2.0 ** -7])))))
def test_sweep_requant_w_nvfp4_int8(n, k, scale2):
    c = synth.w4a8_tiny("cpu", m=1, n=n, k=k)
    q, s = empty((n, k), torch.int8), empty((n, k // 32), torch.float32)
    qp.requant_w_nvfp4_int8(dev(c.w_packed), dev(c.w_e4m3), scale2, q, s)
    oq, os_ = oracle.requant_w_nvfp4_int8(bits(c.w_packed), bits(c.w_e4m3), scale2)
    assert np.array_equal(host(q), oq)
    assert np.array_equal(host(s).view(np.uint32), os_.view(np.uint32))


@pytest.mark.parametrize("rows,k", _draw(6, lambda: (_i(1, 300), 32 * _i(1, 64))))
def test_sweep_quantize_bf16_nvfp4(rows, k):
    x = _acts((rows, k), 2000 + rows + k)
    p, s = empty((rows, k // 2), torch.uint8), empty((rows, k // 16), torch.uint8)
    qp.quantize_bf16_nvfp4(dev(x), p, s, 1.0)
    op, os_ = oracle.quantize_bf16_nvfp4(bits(x), 1.0)
    assert np.array_equal(host(s), os_)
    assert np.array_equal(host(p), op)


@pytest.mark.parametrize("rows,k", _draw(8, lambda: (_i(1, 300), 16 * _i(1, 600))))
def test_sweep_quant_rowwise_fp8(rows, k):
    x = _acts((rows, k), 3000 + rows + k, std=0.02)
    q, s = empty((rows, k), torch.uint8), empty((rows,), torch.float32)
    qp.quant_rowwise_fp8(dev(x), q, s)
    oq, os_ = oracle.quant_rowwise_fp8(bits(x))
    assert np.array_equal(host(s).view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(host(q), oq)


@pytest.mark.parametrize("n,k", _draw(6, lambda: (128 * _i(1, 4), 128 * _i(1, 40))))
def test_sweep_requant_blockfp8_rowwise(n, k):
    cse = synth.fp8_block("cpu", m=1, n=n, k=k)
    w, grid = cse.w_block, cse.block_grid
    wo, so = empty((n, k), torch.uint8), empty((n,), torch.float32)
    qp.requant_w_blockfp8_rowwise(qp.QP_FP8_BLOCK128, dev(w), dev(grid), wo, so)
    oq, os_ = oracle.requant_w_blockfp8_rowwise(bits(w), grid.numpy())
    assert np.array_equal(host(so).view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(host(wo), oq)


# ------------------------------------------------------------- GEMMs
@pytest.mark.parametrize("m,n,k", _draw(6, lambda: (_i(1, 600), _i(1, 700), 32 * _i(1, 48))))
def test_sweep_int8_gemm_blockscaled(m, n, k):
    oa, oas = oracle.requant_a_bf16_int8(bits(_acts((m, k), 4000 + m)))
    ow, ows = oracle.requant_a_bf16_int8(bits(_acts((n, k), 4001 + n, std=0.02)))
    out = filled((m, n), torch.bfloat16)
    t = lambda x: dev(torch.from_numpy(x))
    qp.int8_gemm_blockscaled(t(oa), t(ow), t(oas), t(ows), out)
    assert_gemm_close(host(out), oracle.int8_gemm_blockscaled(oa, ow, oas, ows), f"int8 {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", _draw(6, lambda: (_i(1, 600), _i(1, 700), 32 * _i(1, 48))))
def test_sweep_w4a4_gemm(m, n, k):
    w = _acts((n, k), 5001 + n, std=0.02)
    sw2 = synth.per_tensor_scale2(w)
    ap, asc = oracle.quantize_bf16_nvfp4(bits(_acts((m, k), 5000 + m)), 1.0)
    wp, wsc = oracle.quantize_bf16_nvfp4(bits(w), sw2)
    out = filled((m, n), torch.bfloat16)
    t = lambda x: dev(torch.from_numpy(x))
    qp.w4a4_gemm(t(ap), t(asc), t(wp), t(wsc), out, 1.0, sw2)
    assert_gemm_close(host(out), oracle.w4a4_gemm(ap, asc, wp, wsc, 1.0, sw2), f"w4a4 {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", _draw(6, lambda: (_i(1, 600), _i(1, 700), 16 * _i(1, 100))))
def test_sweep_fp8_gemm_rowscale(m, n, k):
    oa, oas = oracle.quant_rowwise_fp8(bits(_acts((m, k), 6000 + m)))
    ow, ows = oracle.quant_rowwise_fp8(bits(_acts((n, k), 6001 + n, std=0.02)))
    out = filled((m, n), torch.bfloat16)
    t = lambda x: dev(torch.from_numpy(x))
    qp.fp8_gemm_rowscale(t(oa), t(oas), t(ow), t(ows), out)
    assert_gemm_close(host(out), oracle.fp8_gemm_rowscale(oa, oas, ow, ows), f"fp8 {m}x{n}x{k}")


# ------------------------------------------------------------- GEMVs
# N up to 20000 reaches the narrow kernels' two-segments-in-flight form
# (N >= 12288); M is drawn over the whole range of each entry point.
@pytest.mark.parametrize("m,n,k", _draw(8, lambda: (_i(1, 16), _i(1, 20000), 16 * _i(1, 400))))
def test_sweep_fp8_gemv_rowscale(m, n, k):
    ow, ows = oracle.quant_rowwise_fp8(bits(_acts((n, k), 7000 + n, std=0.02)))
    x = _acts((m, k), 7001 + m)
    out = filled((m, n), torch.bfloat16)
    t = lambda a: dev(torch.from_numpy(a))
    qp.fp8_gemv_rowscale(dev(x), t(ow), t(ows), out)
    assert_gemv_close(host(out), oracle.fp8_gemv_rowscale(bits(x), ow, ows), f"gemv {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", _draw(6, lambda: (_i(1, 16), 128 * _i(1, 120), 128 * _i(1, 20))))
def test_sweep_fp8_gemv_blockscale(m, n, k):
    w, grid = synth.gemv_block_weight(n, k, "cpu", shape_id=0)
    x = _acts((m, k), 8000 + m)
    out = filled((m, n), torch.bfloat16)
    qp.fp8_gemv_blockscale(dev(x), dev(w), dev(grid), out)
    assert_gemv_close(host(out), oracle.fp8_gemv_blockscale(bits(x), w.numpy(), grid.numpy()),
                      f"block gemv {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", _draw(6, lambda: (_i(1, 8), _i(1, 20000), 32 * _i(1, 200))))
def test_sweep_w4a16_gemv(m, n, k):
    wp, ws, s2 = synth.gemv_nvfp4_weight(n, k, "cpu", shape_id=0)
    x = _acts((m, k), 9000 + m)
    out = filled((m, n), torch.bfloat16)
    qp.w4a16_gemv(dev(x), dev(wp), dev(ws), s2, out)
    assert_gemv_close(host(out), oracle.w4a16_gemv(bits(x), wp.numpy(), ws.numpy(), s2),
                      f"w4a16 {m}x{n}x{k}")
