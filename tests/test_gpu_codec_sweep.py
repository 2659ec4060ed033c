"""Every BF16 input of each quantizer's rounding domain, through the kernels.

The activation quantizers round fl(x / s) onto a grid with the gfx950
converters (int8 through the packed u8 converter, E4M3 through the packed
FP8 converter, E2M1 through the packed FP4 converter).  Built so that the
stored scale is exactly 1, a block's quotients are its inputs themselves, so
the codes the kernel writes are the converters' (and the surrounding
arithmetic's) answer for every BF16 value of the domain: every grid point,
every midpoint between neighbours (ties to even), the BF16 neighbours on
either side of each, subnormals, signed zeros, both signs.  The oracle
encodes the same inputs with its own grid search, so the comparison is bit
for bit against definitions the kernels share nothing with.

  int8   (gemm_dense_int8.rs, int8_gemm_faith2_prefill, first launch): each
         32-block leads with +-127, so s = fl(127/127) = 1; every |x| <= 127.
  E4M3   (dispatch_proj_rowwise.rs, quant_rowwise_fp8): each row leads with
         +-448, so s = fl(448/448) = 1; every |x| <= 448.
  E2M1   (gemm_fp4.rs, quantize_bf16_to_nvfp4, scale2 = 1): each 16-block
         leads with +-6, so the E4M3 block scale encodes fl(6/6) = 1 and
         d = 1; every |x| <= 6.

The hand-worked blocks of tests/golden run through the kernels as well, and
are compared with their hand-derived codes and scales directly.
"""
import configparser
import os

import numpy as np
import pytest
import torch

import gemv_nvfp4_int8_amd as qp
import oracle
from tests.gpu_util import dev, empty, host

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_blocks.ini")


def _bf16_domain(limit: float) -> np.ndarray:
    """Bit patterns of every BF16 value v with |v| <= limit (limit itself a
    BF16 value), both signs, +-0 included."""
    top = int(np.array([limit], np.float32).view(np.uint32)[0] >> 16)
    pos = np.arange(0, top + 1, dtype=np.uint16)
    return np.concatenate([pos, pos | np.uint16(0x8000)])


def _lead_blocks(vals: np.ndarray, lead: float, bsz: int, per_row: int) -> np.ndarray:
    """Blocks of bsz BF16 values, each opening with +-lead (alternating) and
    then bsz - 1 domain values; rows of per_row blocks (tail blocks padded
    with zeros)."""
    body = bsz - 1
    nblk = -(-len(vals) // body)
    nblk = -(-nblk // per_row) * per_row
    padded = np.zeros(nblk * body, np.uint16)
    padded[:len(vals)] = vals
    lead_bits = int(np.array([lead], np.float32).view(np.uint32)[0] >> 16)
    leads = np.where(np.arange(nblk) % 2 == 0, lead_bits, lead_bits | 0x8000).astype(np.uint16)
    blocks = np.concatenate([leads[:, None], padded.reshape(nblk, body)], axis=1)
    return blocks.reshape(nblk // per_row, per_row * bsz)


def _t(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def test_int8_codes_over_every_bf16_input_at_unit_scale():
    x = _lead_blocks(_bf16_domain(127.0), 127.0, 32, 32)          # rows of k = 1024
    m, k = x.shape
    q, s = empty((m, k), torch.int8), empty((m, k // 32), torch.float32)
    qp.requant_a_bf16_int8(dev(_t(x)), q, s)
    oq, os_ = oracle.requant_a_bf16_int8(x)
    assert np.all(os_ == 1.0)
    assert np.array_equal(host(s).view(np.uint32), os_.view(np.uint32))
    got = host(q)
    bad = np.argwhere(got != oq)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[0]}: " \
        f"x bits {x[tuple(bad[0])]:#06x} got {got[tuple(bad[0])]} oracle {oq[tuple(bad[0])]}"


def test_e4m3_codes_over_every_bf16_input_at_unit_scale():
    x = _lead_blocks(_bf16_domain(448.0), 448.0, 4096, 1)        # rows of k = 4096
    rows, k = x.shape
    q, s = empty((rows, k), torch.uint8), empty((rows,), torch.float32)
    qp.quant_rowwise_fp8(dev(_t(x)), q, s)
    oq, os_ = oracle.quant_rowwise_fp8(x)
    assert np.all(os_ == 1.0)
    assert np.array_equal(host(s).view(np.uint32), os_.view(np.uint32))
    got = host(q)
    bad = np.argwhere(got != oq)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[0]}: " \
        f"x bits {x[tuple(bad[0])]:#06x} got {got[tuple(bad[0])]:#04x} oracle {oq[tuple(bad[0])]:#04x}"


def test_e2m1_codes_over_every_bf16_input_at_unit_scale():
    x = _lead_blocks(_bf16_domain(6.0), 6.0, 16, 64)              # rows of k = 1024
    rows, k = x.shape
    p, s = empty((rows, k // 2), torch.uint8), empty((rows, k // 16), torch.uint8)
    qp.quantize_bf16_nvfp4(dev(_t(x)), p, s, 1.0)
    op, os_ = oracle.quantize_bf16_nvfp4(x, 1.0)
    assert np.all(os_ == 0x38)                                     # E4M3 1.0
    assert np.array_equal(host(s), os_)
    got = host(p)
    bad = np.argwhere(got != op)
    assert bad.size == 0, f"{len(bad)} bytes differ, first at {bad[0]}: " \
        f"got {got[tuple(bad[0])]:#04x} oracle {op[tuple(bad[0])]:#04x}"


# ---------------------------------------- the encoders on binary32 values
# The quotients the kernels encode are arbitrary binary32 values, so the
# device encoders are also driven directly (test export qproj_encode_test):
# every binary32 value within 64 ulps of each grid point and each midpoint,
# a strided sample (every 997th bit pattern) of the whole domain, both
# signs and both zeros, against the oracle's encoders.
def _f32_bits(v):
    return np.asarray(v, np.float32).view(np.uint32).astype(np.int64)


def _around(points, ulps=64):
    """Every non-negative binary32 within `ulps` of each point."""
    u = _f32_bits(points)[:, None] + np.arange(-ulps, ulps + 1)[None, :]
    u = u[(u >= 0) & (u < 0x7F800000)]
    return np.unique(u).astype(np.uint32).view(np.float32)


def _domain(grid, limit, strict):
    """Grid points, midpoints, their neighbourhoods and a strided sample of
    [0, limit) (or [0, limit]), both signs."""
    g = np.asarray(grid, np.float64)
    pts = np.concatenate([g, (g[:-1] + g[1:]) / 2, [limit]])
    vals = np.concatenate([_around(pts.astype(np.float32)),
                           np.arange(0, int(_f32_bits([limit])[0]), 997,
                                     dtype=np.int64).astype(np.uint32).view(np.float32)])
    vals = vals[(vals < limit) if strict else (vals <= limit)]
    vals = np.unique(vals)
    vals = np.concatenate([vals, -vals, np.array([-0.0], np.float32)])
    pad = (-len(vals)) % 8
    return np.concatenate([vals, np.zeros(pad, np.float32)]).astype(np.float32)


E4M3_GRID = [oracle.e4m3_decode(c) for c in range(0x7F)]
E2M1_GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
INT8_GRID = list(range(128))


@pytest.mark.parametrize("kind,okind,grid,limit,strict", [
    (qp.QP_ENC_E4M3_NOSAT, oracle.ENC_E4M3, E4M3_GRID, 464.0, True),
    (qp.QP_ENC_E4M3, oracle.ENC_E4M3, E4M3_GRID + [464.0, 480.0, 1e6], 3.0e38, False),
    (qp.QP_ENC_E2M1_NOSAT, oracle.ENC_E2M1, E2M1_GRID + [8.0], 8.0, False),
    (qp.QP_ENC_E2M1, oracle.ENC_E2M1, E2M1_GRID + [8.0, 1e3], 3.0e38, False),
    (qp.QP_ENC_INT8, oracle.ENC_INT8, INT8_GRID, 127.5, True),
    (qp.QP_ENC_E4M3_SCALE, oracle.ENC_E4M3, E4M3_GRID + [464.0, 1e6], 3.0e38, False),
], ids=["e4m3", "e4m3_sat", "e2m1", "e2m1_sat", "int8", "e4m3_scale"])
def test_device_encoders_on_binary32_boundaries(kind, okind, grid, limit, strict):
    y = _domain(grid, limit, strict)
    if kind == qp.QP_ENC_E4M3_SCALE:
        y = np.abs(y)                    # block scales are never negative
    out = empty((len(y),), torch.uint8)
    qp.encode_test(kind, dev(torch.from_numpy(y)), out)
    got = host(out)
    want = oracle.encode_array(okind, y)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} of {len(y)} differ; first y = {y[bad[0]]!r} " \
        f"({_f32_bits([y[bad[0]]])[0]:#010x}): got {got[bad[0]]:#04x}, oracle {want[bad[0]]:#04x}"


# ------------------------------------------------- hand-worked blocks on the GPU
def _cases():
    cp = configparser.ConfigParser()
    cp.read(GOLDEN)
    return cp


def _bf16(vals, pad_to=None):
    v = [float(t) for t in vals]
    if pad_to:
        v += [0.0] * (pad_to - len(v))
    return torch.tensor(v, dtype=torch.float32).to(torch.bfloat16)[None, :]


def _hexbytes(s):
    return np.array([int(t, 16) for t in s.split()], dtype=np.uint8)


def _f32hex(h):
    return np.array([int(h, 16)], dtype=np.uint32).view(np.float32)[0]


@pytest.mark.parametrize("name", ["HW1", "HW2"])
def test_hand_worked_nvfp4_blocks_on_gpu(name):
    c = _cases()[name]
    x = _bf16(c["x"].split(), pad_to=32)               # k % 32 == 0; block 2 all zero
    p, s = empty((1, 16), torch.uint8), empty((1, 2), torch.uint8)
    qp.quantize_bf16_nvfp4(dev(x), p, s, float(c["scale2"]))
    assert host(s)[0, 0] == int(c["expect_scale"], 16) and host(s)[0, 1] == 0
    assert np.array_equal(host(p)[0, :8], _hexbytes(c["expect_packed"]))
    assert np.all(host(p)[0, 8:] == 0)


def test_hand_worked_int8_weight_block_on_gpu():
    c = _cases()["HW3"]
    codes = [int(t) for t in c["codes"].split()]
    packed = torch.tensor([[codes[2 * i] | (codes[2 * i + 1] << 4) for i in range(16)]],
                          dtype=torch.uint8)
    sc = torch.from_numpy(_hexbytes(c["scales16"])[None, :])
    q, s = empty((1, 32), torch.int8), empty((1, 1), torch.float32)
    qp.requant_w_nvfp4_int8(dev(packed), dev(sc), float(c["scale2"]), q, s)
    assert np.array_equal(host(q)[0], np.array(c["expect_q"].split(), dtype=np.int8))
    assert host(s)[0, 0] == _f32hex(c["expect_scale_hex"])


@pytest.mark.parametrize("name", ["HW4", "HW8"])
def test_hand_worked_int8_activation_blocks_on_gpu(name):
    c = _cases()[name]
    q, s = empty((1, 32), torch.int8), empty((1, 1), torch.float32)
    qp.requant_a_bf16_int8(dev(_bf16(c["x"].split())), q, s)
    assert np.array_equal(host(q)[0], np.array(c["expect_q"].split(), dtype=np.int8))
    assert host(s)[0, 0] == _f32hex(c["expect_scale_hex"])


@pytest.mark.parametrize("name", ["HW5", "HW9"])
def test_hand_worked_e4m3_rows_on_gpu(name):
    c = _cases()[name]
    q, s = empty((1, 16), torch.uint8), empty((1,), torch.float32)
    qp.quant_rowwise_fp8(dev(_bf16(c["x"].split())), q, s)
    assert np.array_equal(host(q)[0], _hexbytes(c["expect_q"]))
    assert host(s)[0] == _f32hex(c["expect_scale_hex"])


def test_hand_worked_blockfp8_intermediate_on_gpu():
    c = _cases()["HW6"]
    w = torch.full((128, 128), int(c["code"], 16), dtype=torch.uint8)
    grid = torch.full((1, 1), float(c["block_scale"]), dtype=torch.float32)
    wo, so = empty((128, 128), torch.uint8), empty((128,), torch.float32)
    qp.requant_w_blockfp8_rowwise(qp.QP_FP8_BLOCK128, dev(w), dev(grid), wo, so)
    y = np.float32(oracle.bf16_to_float(int(c["expect_bf16_hex"], 16)))
    assert np.all(host(wo) == 0x7E)
    assert np.all(host(so) == y / np.float32(448))
