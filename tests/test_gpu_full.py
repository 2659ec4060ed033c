"""Full-size parity: every workload at its real shape, run through the same
entry points and launch configurations the benchmark times, checked on
sampled rows / outputs that the CPU oracle computes from the same synthetic
inputs (the oracle quantizes its own copy of the sampled rows; every
quantizer here is row-local, so sampling rows loses nothing).

Codes and scales: bit-exact on the sampled rows.  BF16 contraction outputs:
the stated tolerances (tests/gpu_util.py).
"""
import numpy as np
import pytest
import torch

import gemv_nvfp4_int8_amd as qp
import oracle
import synth
from tests.gpu_util import (DEV, assert_gemm_close, assert_gemv_close, bits,
                            empty, host)

pytestmark = pytest.mark.gpu


def _rows(n, count, seed):
    g = np.random.default_rng(seed)
    idx = np.sort(g.choice(n, size=min(count, n), replace=False))
    # always include the first and the last row (tile edges, ragged tail)
    return np.unique(np.concatenate([[0, n - 1], idx]))


@pytest.mark.parametrize("sid,n,k", [(0, 6144, 5120), (1, 17408, 5120), (2, 152064, 5120)])
def test_gemv_decode_shapes(sid, n, k):
    """FP8 row-scaled GEMV decode/verify: weight from BF16 N(0,0.02) row-absmax
    quantized, per-row F32 scale; BF16 acts N(0,1); M in {1,2,8,16}."""
    wb = synth.gemv_weight_bf16(n, k, DEV, shape_id=sid)
    wq, ws = empty((n, k), torch.uint8), empty((n,), torch.float32)
    qp.quant_rowwise_fp8(wb, wq, ws)
    x = synth.gemv_acts_bf16(16, k, DEV, shape_id=sid)
    rows = _rows(n, 384, 100 + sid)
    ridx = torch.from_numpy(rows).to(DEV)
    ow, ows = oracle.quant_rowwise_fp8(bits(wb.index_select(0, ridx)))
    assert np.array_equal(host(wq.index_select(0, ridx)), ow)
    assert np.array_equal(host(ws.index_select(0, ridx)).view(np.uint32), ows.view(np.uint32))
    xb = bits(x)
    full16 = None
    for m in (1, 2, 8, 16):
        out = empty((m, n), torch.bfloat16)
        qp.fp8_gemv_rowscale(x[:m], wq, ws, out)
        got = host(out)[:, rows]
        assert_gemv_close(got, oracle.fp8_gemv_rowscale(xb[:m], ow, ows), f"N={n} M={m}")
        if m == 16:
            full16 = out
    # batched rows equal single-row calls, bit for bit, over the whole output
    for i in (0, 7, 15):
        o1 = empty((1, n), torch.bfloat16)
        qp.fp8_gemv_rowscale(x[i:i + 1], wq, ws, o1)
        assert torch.equal(o1.view(torch.int16), full16[i:i + 1].view(torch.int16))


@pytest.mark.parametrize("sid,n,k", [(0, 6144, 5120), (1, 17408, 5120), (2, 152064, 5120)])
def test_block_scaled_gemv_decode_shapes(sid, n, k):
    """Block-scaled FP8 GEMV (w8a16_gemv_batch4 / _batch2) at the decode
    shapes, M in {1, 2, 4}: E4M3 weight with 128 x 128 F32 block scales,
    BF16 acts N(0,1).  Three whole 128-row blocks (the first, the last and
    one drawn) are checked against the oracle, and every row of the M = 4
    call against its single-row call."""
    w, grid = synth.gemv_block_weight(n, k, DEV, shape_id=sid)
    x = synth.gemv_acts_bf16(4, k, DEV, shape_id=sid)
    nb = n // 128
    blocks = sorted({0, nb - 1, int(np.random.default_rng(200 + sid).integers(1, nb - 1))})
    wh, gh, xb = host(w), host(grid), bits(x)
    for m in (1, 2, 4):
        out = empty((m, n), torch.bfloat16)
        qp.fp8_gemv_blockscale(x[:m], w, grid, out)
        got = host(out)
        for b in blocks:
            ref = oracle.fp8_gemv_blockscale(xb[:m], np.ascontiguousarray(wh[128 * b:128 * (b + 1)]),
                                             np.ascontiguousarray(gh[b:b + 1]))
            assert_gemv_close(got[:, 128 * b:128 * (b + 1)], ref, f"N={n} M={m} block {b}")
        if m == 4:
            for i in range(4):
                o1 = empty((1, n), torch.bfloat16)
                qp.fp8_gemv_blockscale(x[i:i + 1], w, grid, o1)
                assert torch.equal(o1.view(torch.int16), out[i:i + 1].view(torch.int16)), i


@pytest.mark.parametrize("sid,n,k", [(0, 6144, 5120), (1, 17408, 5120), (2, 152064, 5120)])
def test_w4a16_gemv_decode_shapes(sid, n, k):
    """NVFP4-weight GEMV at the decode shapes, M in {1, 2, 8}: the weight is
    a BF16 N(0,0.02) draw quantised to NVFP4 by quantize_bf16_nvfp4 (scale2 =
    max|W|/448), the acts BF16 N(0,1).  Sampled rows are checked against the
    oracle on the same codes, and the M = 8 rows against single-row calls."""
    wb = synth.gemv_weight_bf16(n, k, DEV, shape_id=sid)
    s2 = synth.per_tensor_scale2(wb)
    wp, ws = empty((n, k // 2), torch.uint8), empty((n, k // 16), torch.uint8)
    qp.quantize_bf16_nvfp4(wb, wp, ws, s2)
    del wb
    x = synth.gemv_acts_bf16(8, k, DEV, shape_id=sid)
    rows = _rows(n, 384, 300 + sid)
    ridx = torch.from_numpy(rows).to(DEV)
    owp, ows = host(wp.index_select(0, ridx)), host(ws.index_select(0, ridx))
    xb = bits(x)
    for m in (1, 2, 8):
        out = empty((m, n), torch.bfloat16)
        qp.w4a16_gemv(x[:m], wp, ws, s2, out)
        got = host(out)[:, rows]
        assert_gemv_close(got, oracle.w4a16_gemv(xb[:m], owp, ows, s2), f"N={n} M={m}")
        if m == 8:
            for i in (0, 7):
                o1 = empty((1, n), torch.bfloat16)
                qp.w4a16_gemv(x[i:i + 1], wp, ws, s2, o1)
                assert torch.equal(o1.view(torch.int16), out[i:i + 1].view(torch.int16)), i


def test_w4a8_prefill_full():
    """W4A8 prefill: NVFP4 weight 17408x5120 (from BF16 N(0,0.02), scale2 =
    max|W|/448) -> int8 per-32; BF16 acts 2048x5120 with 1% outliers x20."""
    m, n, k = 2048, 17408, 5120
    c = synth.w4a8_prefill(DEV, m, n, k)
    wp, we = empty((n, k // 2), torch.uint8), empty((n, k // 16), torch.uint8)
    qp.quantize_bf16_nvfp4(c.w_bf16, wp, we, c.scale2)
    w_i8, w_s = empty((n, k), torch.int8), empty((n, k // 32), torch.float32)
    qp.requant_w_nvfp4_int8(wp, we, c.scale2, w_i8, w_s)
    a_i8, a_s = empty((m, k), torch.int8), empty((m, k // 32), torch.float32)
    out = empty((m, n), torch.bfloat16)
    qp.int8_w4a8_prefill(c.a_bf16, w_i8, w_s, a_i8, a_s, out)

    # activations: the whole requant, bit-exact
    oa, oas = oracle.requant_a_bf16_int8(bits(c.a_bf16))
    assert np.array_equal(host(a_i8), oa)
    assert np.array_equal(host(a_s).view(np.uint32), oas.view(np.uint32))
    # weight: sampled rows through the oracle's own NVFP4 -> int8 chain
    wr = _rows(n, 256, 7)
    widx = torch.from_numpy(wr).to(DEV)
    owp, owe = oracle.quantize_bf16_nvfp4(bits(c.w_bf16.index_select(0, widx)), c.scale2)
    assert np.array_equal(host(wp.index_select(0, widx)), owp)
    assert np.array_equal(host(we.index_select(0, widx)), owe)
    ow, ows = oracle.requant_w_nvfp4_int8(owp, owe, c.scale2)
    assert np.array_equal(host(w_i8.index_select(0, widx)), ow)
    assert np.array_equal(host(w_s.index_select(0, widx)).view(np.uint32), ows.view(np.uint32))
    # GEMM on sampled outputs
    ar = _rows(m, 64, 8)
    ref = oracle.int8_gemm_blockscaled(oa[ar], ow, oas[ar], ows)
    got = host(out)[np.ix_(ar, wr)]
    assert_gemm_close(got, ref, "w4a8 prefill")


def test_w4a4_prefill_full():
    """W4A4 prefill: BF16 acts 4096x17408 -> NVFP4 (scale2 1.0); NVFP4 weight
    5120x17408 from N(0,0.02); NVFP4 x NVFP4 GEMM -> BF16 [4096, 5120]."""
    m, n, k = 4096, 5120, 17408
    c = synth.w4a4_prefill(DEV, m, n, k)
    ap_, as_ = empty((m, k // 2), torch.uint8), empty((m, k // 16), torch.uint8)
    wp, ws = empty((n, k // 2), torch.uint8), empty((n, k // 16), torch.uint8)
    qp.quantize_bf16_nvfp4(c.a_bf16, ap_, as_, 1.0)
    qp.quantize_bf16_nvfp4(c.w_bf16, wp, ws, c.scale_w2)
    out = empty((m, n), torch.bfloat16)
    qp.w4a4_gemm(ap_, as_, wp, ws, out, 1.0, c.scale_w2)
    ar, wr = _rows(m, 48, 9), _rows(n, 96, 10)
    aidx, widx = torch.from_numpy(ar).to(DEV), torch.from_numpy(wr).to(DEV)
    oap, oas = oracle.quantize_bf16_nvfp4(bits(c.a_bf16.index_select(0, aidx)), 1.0)
    owp, ows = oracle.quantize_bf16_nvfp4(bits(c.w_bf16.index_select(0, widx)), c.scale_w2)
    assert np.array_equal(host(ap_.index_select(0, aidx)), oap)
    assert np.array_equal(host(as_.index_select(0, aidx)), oas)
    assert np.array_equal(host(wp.index_select(0, widx)), owp)
    assert np.array_equal(host(ws.index_select(0, widx)), ows)
    ref = oracle.w4a4_gemm(oap, oas, owp, ows, 1.0, c.scale_w2)
    got = host(out)[np.ix_(ar, wr)]
    assert_gemm_close(got, ref, "w4a4 prefill")


def test_blockfp8_rowwise_requant_and_gemm_full():
    """Block-FP8 -> row-wise FP8 requant + GEMM: E4M3 weight 12288x5120 with
    128x128 F32 block scales (log-uniform 1e-4..1e-2), requantised via BF16;
    a second layer already row-wise passes through; BF16 acts M=8192."""
    m, n, k = 8192, 12288, 5120
    c = synth.fp8_block(DEV, m, n, k)
    wq, wsr = empty((n, k), torch.uint8), empty((n,), torch.float32)
    aq, asr = empty((m, k), torch.uint8), empty((m,), torch.float32)
    out = empty((m, n), torch.bfloat16)
    qp.fp8_rowwise_proj(qp.QP_FP8_BLOCK128, c.w_block, c.block_grid, wq, wsr,
                        c.a_bf16, aq, asr, out)
    # the already row-wise layer: its own pair, no requant launch
    pw, pws = empty((n, k), torch.uint8), empty((n,), torch.float32)
    qp.quant_rowwise_fp8(c.w_rowwise_bf16, pw, pws)
    out2 = empty((m, n), torch.bfloat16)
    before = qp.launch_count()
    qp.fp8_rowwise_proj(qp.QP_FP8_PER_ROW, pw, pws, None, None, c.a_bf16, aq, asr, out2)
    assert qp.launch_count() - before == 2

    wr = _rows(n, 256, 11)      # rows from many 128-row scale blocks
    widx = torch.from_numpy(wr).to(DEV)
    grid = c.block_grid.cpu().numpy()
    # the oracle requantises whole 128-row groups (the grid is per block) and
    # keeps the sampled rows
    groups = np.unique(wr // 128)
    ow_rows, ows_rows = [], []
    for gi in groups:
        gq, gs = oracle.requant_w_blockfp8_rowwise(
            bits(c.w_block[gi * 128:(gi + 1) * 128]), grid[gi:gi + 1])
        sel = wr[(wr // 128) == gi] - gi * 128
        ow_rows.append(gq[sel])
        ows_rows.append(gs[sel])
    ow, ows = np.concatenate(ow_rows), np.concatenate(ows_rows)
    assert np.array_equal(host(wq.index_select(0, widx)), ow)
    assert np.array_equal(host(wsr.index_select(0, widx)).view(np.uint32), ows.view(np.uint32))
    ar = _rows(m, 48, 12)
    aidx = torch.from_numpy(ar).to(DEV)
    oa, oas = oracle.quant_rowwise_fp8(bits(c.a_bf16.index_select(0, aidx)))
    assert np.array_equal(host(aq.index_select(0, aidx)), oa)
    assert_gemm_close(host(out)[np.ix_(ar, wr)], oracle.fp8_gemm_rowscale(oa, oas, ow, ows),
                      "fp8 block -> rowwise GEMM")
    opw, opws = oracle.quant_rowwise_fp8(bits(c.w_rowwise_bf16.index_select(0, widx)))
    assert np.array_equal(host(pw.index_select(0, widx)), opw)
    assert_gemm_close(host(out2)[np.ix_(ar, wr)], oracle.fp8_gemm_rowscale(oa, oas, opw, opws),
                      "fp8 passthrough GEMM")
