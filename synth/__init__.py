"""Seeded synthetic inputs for the quantized dense projection.

This module only draws random numbers and lays them out in the storage
formats the entry points take (BF16 tensors, E4M3 / packed E2M1 bytes, F32
scale grids).  It holds none of the method's arithmetic: no absmax scaling,
no code rounding and no contraction.  Where an input is itself stored in an
8-bit float format (the E4M3 sub-block scales of the tiny W4A8 case and the
block-scaled FP8 weight) the bytes come from torch's own float8_e4m3fn cast of
a plain random draw, so that the generator owns no codec.

Both the HIP path and the CPU oracle take their inputs from here; nothing in
here depends on either.  Every tensor is produced by a torch.Generator seeded
with ``0x5EED0000 + 16 * case + tensor_id``, on the device asked for (the
draws differ between CPU and GPU generators, but each is deterministic, and
every comparison feeds the same bytes to both sides).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

SEED_BASE = 0x5EED0000

# Shapes of the five workloads (tokens M, output features N, reduction K).
W4A8_TINY = dict(n=256, k=512, m=16)
GEMV_SHAPES = [(6144, 5120), (17408, 5120), (152064, 5120)]   # (N, K)
GEMV_MS = [1, 2, 8, 16]
W4A8_PREFILL = dict(m=2048, n=17408, k=5120)
W4A4_PREFILL = dict(m=4096, n=5120, k=17408)
FP8_BLOCK = dict(m=8192, n=12288, k=5120)


def seed_of(case: int, tensor_id: int) -> int:
    return SEED_BASE + 16 * case + tensor_id


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal_f32(shape, std: float, seed: int, device="cpu") -> torch.Tensor:
    g = _gen(seed, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return x * std if std != 1.0 else x


def bf16_normal(shape, std: float, seed: int, device="cpu",
                outlier_frac: float = 0.0, outlier_mult: float = 1.0) -> torch.Tensor:
    """BF16 N(0, std^2); optionally a seeded fraction of entries times a
    multiplier (before the single BF16 rounding)."""
    g = _gen(seed, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    if outlier_frac > 0.0:
        mask = torch.rand(shape, generator=g, device=device) < outlier_frac
        x = torch.where(mask, x * outlier_mult, x)
    return x.to(torch.bfloat16)


def uniform_bytes(shape, seed: int, device="cpu") -> torch.Tensor:
    g = _gen(seed, device)
    return torch.randint(0, 256, shape, generator=g, device=device,
                         dtype=torch.int32).to(torch.uint8)


def e4m3_bytes_of(x: torch.Tensor) -> torch.Tensor:
    """torch's float8_e4m3fn cast of a plain draw, as raw bytes."""
    return x.to(torch.float8_e4m3fn).view(torch.uint8)


def loguniform(shape, lo: float, hi: float, seed: int, device="cpu") -> torch.Tensor:
    g = _gen(seed, device)
    u = torch.rand(shape, generator=g, device=device, dtype=torch.float64)
    import math
    lg_lo, lg_hi = math.log10(lo), math.log10(hi)
    return torch.pow(10.0, lg_lo + (lg_hi - lg_lo) * u).to(torch.float32)


def per_tensor_scale2(w_bf16: torch.Tensor) -> float:
    """The per-tensor NVFP4 scale2 the weight workloads are built with:
    binary32 max|W| / 448 (a checkpoint-side constant handed to the method)."""
    mx = w_bf16.abs().max().to(torch.float32).cpu()
    return float(mx / torch.tensor(448.0, dtype=torch.float32))


# --------------------------------------------------------------- workloads
@dataclass
class W4A8Tiny:
    """NVFP4 weight N=256,K=512 (uniform random E2M1 nibbles, E4M3 per-16
    scales from |N(0,1)|*0.05, scale2 = 1) and BF16 activations M=16, K=512."""
    w_packed: torch.Tensor
    w_e4m3: torch.Tensor
    scale2: float
    a_bf16: torch.Tensor
    m: int = 16
    n: int = 256
    k: int = 512


def w4a8_tiny(device="cpu", m=16, n=256, k=512) -> W4A8Tiny:
    case = 0
    w_packed = uniform_bytes((n, k // 2), seed_of(case, 0), device)
    z = normal_f32((n, k // 16), 1.0, seed_of(case, 1), device)
    w_e4m3 = e4m3_bytes_of(z.abs() * 0.05)
    a = bf16_normal((m, k), 1.0, seed_of(case, 2), device)
    return W4A8Tiny(w_packed, w_e4m3, 1.0, a, m, n, k)


def gemv_weight_bf16(n: int, k: int, device="cpu", shape_id: int = 0) -> torch.Tensor:
    """BF16 N(0, 0.02^2) weight of the decode GEMV (row-quantised by the method)."""
    return bf16_normal((n, k), 0.02, seed_of(1, 2 * shape_id), device)


def gemv_acts_bf16(m: int, k: int, device="cpu", shape_id: int = 0) -> torch.Tensor:
    return bf16_normal((m, k), 1.0, seed_of(1, 2 * shape_id + 1), device)


def gemv_block_weight(n: int, k: int, device="cpu", shape_id: int = 0):
    """Block-scaled FP8 decode weight: E4M3 codes of a N(0,1) draw times 64
    (most of the E4M3 range, no saturation) and an F32 grid [N/128, K/128]
    of 128 x 128 block scales log-uniform in [1e-4, 1e-2]."""
    case = 5
    z = normal_f32((n, k), 1.0, seed_of(case, 2 * shape_id), device)
    w = e4m3_bytes_of((z * 64.0).clamp(-448.0, 448.0))
    grid = loguniform((n // 128, k // 128), 1e-4, 1e-2, seed_of(case, 2 * shape_id + 1), device)
    return w, grid


def gemv_nvfp4_weight(n: int, k: int, device="cpu", shape_id: int = 0):
    """NVFP4 decode weight drawn over every code: uniform random packed E2M1
    bytes [N, K/2], E4M3 block scales = cast(|N(0,1)| * 0.05) [N, K/16]
    (about a quarter subnormal, a few zero) and scale2 = 1/64."""
    case = 6
    wp = uniform_bytes((n, k // 2), seed_of(case, 2 * shape_id), device)
    z = normal_f32((n, k // 16), 1.0, seed_of(case, 2 * shape_id + 1), device)
    return wp, e4m3_bytes_of(z.abs() * 0.05), 1.0 / 64


@dataclass
class W4A8Prefill:
    w_bf16: torch.Tensor
    scale2: float
    a_bf16: torch.Tensor


def w4a8_prefill(device="cpu", m=2048, n=17408, k=5120) -> W4A8Prefill:
    """BF16 weight N(0,0.02) (quantised to NVFP4 by the method, scale2 =
    max|W|/448) and BF16 activations N(0,1) with 1% outliers times 20."""
    case = 2
    w = bf16_normal((n, k), 0.02, seed_of(case, 0), device)
    a = bf16_normal((m, k), 1.0, seed_of(case, 1), device,
                    outlier_frac=0.01, outlier_mult=20.0)
    return W4A8Prefill(w, per_tensor_scale2(w), a)


@dataclass
class W4A4Prefill:
    a_bf16: torch.Tensor
    w_bf16: torch.Tensor
    scale_w2: float
    scale_a2: float = 1.0


def w4a4_prefill(device="cpu", m=4096, n=5120, k=17408) -> W4A4Prefill:
    """BF16 activations N(0,1) (NVFP4 with scale2 = 1) and a BF16 weight
    N(0,0.02) (NVFP4 with scale2 = max|W|/448)."""
    case = 3
    a = bf16_normal((m, k), 1.0, seed_of(case, 0), device)
    w = bf16_normal((n, k), 0.02, seed_of(case, 1), device)
    return W4A4Prefill(a, w, per_tensor_scale2(w))


@dataclass
class Fp8BlockCase:
    w_block: torch.Tensor        # E4M3 bytes [N, K]
    block_grid: torch.Tensor     # F32 [N/128, K/128]
    w_rowwise_bf16: torch.Tensor  # BF16 [N, K]: the already-row-wise layer's source
    a_bf16: torch.Tensor         # BF16 [M, K]


def fp8_block(device="cpu", m=8192, n=12288, k=5120) -> Fp8BlockCase:
    """Block-scaled FP8 weight (E4M3 codes of a N(0,1) draw times 64, which
    spans most of the E4M3 range without saturating; F32 128x128 block scales
    log-uniform in [1e-4, 1e-2]); a second layer of the same shape that
    arrives already row-wise (its BF16 source is N(0,0.02)); BF16
    activations N(0,1)."""
    case = 4
    z = normal_f32((n, k), 1.0, seed_of(case, 0), device)
    w_block = e4m3_bytes_of((z * 64.0).clamp(-448.0, 448.0))
    grid = loguniform((n // 128, k // 128), 1e-4, 1e-2, seed_of(case, 1), device)
    w_row = bf16_normal((n, k), 0.02, seed_of(case, 2), device)
    a = bf16_normal((m, k), 1.0, seed_of(case, 3), device)
    return Fp8BlockCase(w_block, grid, w_row, a)


def to_numpy_bits(x: torch.Tensor):
    """Host numpy view of a tensor's raw bits (BF16 -> uint16)."""
    import numpy as np
    x = x.detach().contiguous().cpu()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view(np.uint16)
    if x.dtype == torch.uint8:
        return x.numpy()
    if x.dtype == torch.int8:
        return x.numpy()
    return x.numpy()
