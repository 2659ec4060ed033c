"""Parity at the largest extents the ABI accepts.

Every entry point takes tensors of up to 2^31 - 1 elements, and the kernels
address them with 32-bit offsets.  Each case here puts its largest tensor just
under that bound (ragged against the kernels' tiles where the entry point
allows it), so real rows sit next to the offsets' limit.  Inputs are seeded and
generated on the device; the oracle checks sampled rows -- the first, the
middle and the last ones (whole 128-row blocks where a scale grid spans them)
-- from host copies of just those rows.  Byte outputs must match bit for bit,
contractions within the bounds of the other parity tests.
"""
import numpy as np
import pytest
import torch

import gemv_nvfp4_int8_amd as qp
import oracle
import synth
from tests.gpu_util import assert_gemm_close, assert_gemv_close, bits, empty, filled, host

pytestmark = pytest.mark.gpu

LIMIT = (1 << 31) - 1
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _rows(n):
    return [0, 1, n // 2, n - 2, n - 1]


def _blocks(n):
    """Row indices of the first, a middle and the last 128-row block."""
    mid = (n // 256) * 128
    return list(range(0, 128)) + list(range(mid, mid + 128)) + list(range(n - 128, n))


def _e4m3(shape, seed):
    b = synth.uniform_bytes(shape, seed, DEV)
    b[(b & 0x7F) == 0x7F] = 0x7E             # finite codes only
    return b


def _cpu(t, idx):
    return t[idx].cpu().numpy()


@pytest.mark.parametrize("n,k,ms", [(419428, 5120, (3,)),          # row-split kernel
                                    (65535, 32768, (1, 16))])     # K-split kernel
def test_fp8_gemv_rowscale_largest(n, k, ms):
    assert n * k <= LIMIT
    w = _e4m3((n, k), 901)
    s = synth.loguniform((n,), 1e-4, 1e-2, 902, DEV)
    x = synth.gemv_acts_bf16(16, k, DEV, shape_id=9)
    rows = _rows(n)
    for m in ms:
        out = filled((m, n), torch.bfloat16)
        qp.fp8_gemv_rowscale(x[:m], w, s, out)
        ref = oracle.fp8_gemv_rowscale(bits(x[:m].cpu()), _cpu(w, rows), _cpu(s, rows))
        assert_gemv_close(host(out)[:, rows], ref, f"gemv {n}x{k} m={m}")


@pytest.mark.parametrize("n,k", [(419328, 5120), (65408, 32768)])
def test_fp8_gemv_blockscale_largest(n, k):
    assert n * k <= LIMIT
    w = _e4m3((n, k), 903)
    grid = synth.loguniform((n // 128, k // 128), 1e-4, 1e-2, 904, DEV)
    x = synth.gemv_acts_bf16(4, k, DEV, shape_id=10)
    out = filled((4, n), torch.bfloat16)
    qp.fp8_gemv_blockscale(x, w, grid, out)
    rows = _blocks(n)
    g = grid[[0, (n // 256), n // 128 - 1]].cpu().numpy()
    ref = oracle.fp8_gemv_blockscale(bits(x.cpu()), _cpu(w, rows), g)
    assert_gemv_close(host(out)[:, rows], ref, f"block gemv {n}x{k}")


@pytest.mark.parametrize("n,k,m", [(419428, 5120, 2), (65535, 32768, 8)])
def test_w4a16_gemv_largest(n, k, m):
    assert n * k <= LIMIT
    wp = synth.uniform_bytes((n, k // 2), 905, DEV)
    ws = _e4m3((n, k // 16), 906)
    ws &= 0x7F                                  # non-negative block scales
    x = synth.gemv_acts_bf16(m, k, DEV, shape_id=11)
    out = filled((m, n), torch.bfloat16)
    qp.w4a16_gemv(x, wp, ws, 1.0 / 64, out)
    rows = _rows(n)
    ref = oracle.w4a16_gemv(bits(x.cpu()), _cpu(wp, rows), _cpu(ws, rows), 1.0 / 64)
    assert_gemv_close(host(out)[:, rows], ref, f"w4a16 {n}x{k} m={m}")


def _bf16_rows(rows, k, seed):
    assert rows * k <= LIMIT
    return synth.bf16_normal((rows, k), 1.0, seed, DEV)


def test_quant_rowwise_fp8_largest():
    rows, k = 419428, 5120
    x = _bf16_rows(rows, k, 907)
    q, s = empty((rows, k), torch.uint8), empty((rows,), torch.float32)
    qp.quant_rowwise_fp8(x, q, s)
    idx = _rows(rows)
    rq, rs = oracle.quant_rowwise_fp8(bits(x[idx].cpu()))
    torch.cuda.synchronize()
    assert np.array_equal(_cpu(q, idx), rq)
    assert np.array_equal(_cpu(s, idx).view(np.uint32), rs.view(np.uint32))


def test_requant_a_bf16_int8_largest():
    m, k = 419428, 5120
    a = _bf16_rows(m, k, 908)
    q, s = empty((m, k), torch.int8), empty((m, k // 32), torch.float32)
    qp.requant_a_bf16_int8(a, q, s)
    idx = _rows(m)
    rq, rs = oracle.requant_a_bf16_int8(bits(a[idx].cpu()))
    torch.cuda.synchronize()
    assert np.array_equal(_cpu(q, idx), rq)
    assert np.array_equal(_cpu(s, idx).view(np.uint32), rs.view(np.uint32))


def test_quantize_bf16_nvfp4_largest():
    rows, k = 419428, 5120
    x = _bf16_rows(rows, k, 909)
    p, s = empty((rows, k // 2), torch.uint8), empty((rows, k // 16), torch.uint8)
    qp.quantize_bf16_nvfp4(x, p, s, 1.0)
    idx = _rows(rows)
    rp, rs = oracle.quantize_bf16_nvfp4(bits(x[idx].cpu()), 1.0)
    torch.cuda.synchronize()
    assert np.array_equal(_cpu(p, idx), rp)
    assert np.array_equal(_cpu(s, idx), rs)


def test_requant_w_nvfp4_int8_largest():
    n, k = 419428, 5120
    assert n * k <= LIMIT
    wp = synth.uniform_bytes((n, k // 2), 910, DEV)
    we = _e4m3((n, k // 16), 911)
    q, s = empty((n, k), torch.int8), empty((n, k // 32), torch.float32)
    qp.requant_w_nvfp4_int8(wp, we, 0.75, q, s)
    idx = _rows(n)
    rq, rs = oracle.requant_w_nvfp4_int8(_cpu(wp, idx), _cpu(we, idx), 0.75)
    torch.cuda.synchronize()
    assert np.array_equal(_cpu(q, idx), rq)
    assert np.array_equal(_cpu(s, idx).view(np.uint32), rs.view(np.uint32))


def test_requant_w_blockfp8_rowwise_largest():
    n, k = 419328, 5120
    assert n * k <= LIMIT
    w = _e4m3((n, k), 912)
    grid = synth.loguniform((n // 128, k // 128), 1e-4, 1e-2, 913, DEV)
    q, s = empty((n, k), torch.uint8), empty((n,), torch.float32)
    qp.requant_w_blockfp8_rowwise(qp.QP_FP8_BLOCK128, w, grid, q, s)
    idx = _blocks(n)
    g = grid[[0, n // 256, n // 128 - 1]].cpu().numpy()
    rq, rs = oracle.requant_w_blockfp8_rowwise(_cpu(w, idx), g)
    torch.cuda.synchronize()
    assert np.array_equal(_cpu(q, idx), rq)
    assert np.array_equal(_cpu(s, idx).view(np.uint32), rs.view(np.uint32))


def test_int8_gemm_blockscaled_largest_k():
    # M*K just under 2^31 with a ragged last M tile and a partial last K stage
    m, n, k = 4095, 256, 524384
    assert m * k <= LIMIT and k % 32 == 0
    g = torch.Generator(device=DEV)
    g.manual_seed(synth.seed_of(14, 0))
    a = torch.randint(-127, 128, (m, k), generator=g, device=DEV, dtype=torch.int8)
    w = torch.randint(-127, 128, (n, k), generator=g, device=DEV, dtype=torch.int8)
    sa = synth.loguniform((m, k // 32), 1e-3, 1e-2, 914, DEV)
    sw = synth.loguniform((n, k // 32), 1e-3, 1e-2, 915, DEV)
    out = filled((m, n), torch.bfloat16)
    qp.int8_gemm_blockscaled(a, w, sa, sw, out)
    ri, cj = _rows(m), _rows(n)
    ref = oracle.int8_gemm_blockscaled(_cpu(a, ri), _cpu(w, cj), _cpu(sa, ri), _cpu(sw, cj))
    assert_gemm_close(host(out)[ri][:, cj], ref, "int8 largest K")


def test_fp8_gemm_rowscale_largest_k():
    m, n, k = 4096, 256, 524160
    assert m * k <= LIMIT and k % 128 == 0
    a, w = _e4m3((m, k), 916), _e4m3((n, k), 917)
    sa = synth.loguniform((m,), 1e-4, 1e-2, 918, DEV)
    sw = synth.loguniform((n,), 1e-4, 1e-2, 919, DEV)
    out = filled((m, n), torch.bfloat16)
    qp.fp8_gemm_rowscale(a, sa, w, sw, out)
    ri, cj = _rows(m), _rows(n)
    ref = oracle.fp8_gemm_rowscale(_cpu(a, ri), _cpu(sa, ri), _cpu(w, cj), _cpu(sw, cj))
    assert_gemm_close(host(out)[ri][:, cj], ref, "fp8 largest K")


def test_w4a4_gemm_largest_k():
    m, n, k = 512, 320, 4194048
    assert m * k <= LIMIT and k % 256 == 0
    ap, wp = synth.uniform_bytes((m, k // 2), 920, DEV), synth.uniform_bytes((n, k // 2), 921, DEV)
    sa, sw = _e4m3((m, k // 16), 922) & 0x7F, _e4m3((n, k // 16), 923) & 0x7F
    out = filled((m, n), torch.bfloat16)
    qp.w4a4_gemm(ap, sa, wp, sw, out, 1.0, 0.5)
    ri, cj = _rows(m), _rows(n)
    ref = oracle.w4a4_gemm(_cpu(ap, ri), _cpu(sa, ri), _cpu(wp, cj), _cpu(sw, cj), 1.0, 0.5)
    assert_gemm_close(host(out)[ri][:, cj], ref, "w4a4 largest K")
