"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
import numpy as np
import torch

import oracle
from synth import to_numpy_bits as bits

DEV = "cuda:0"


def dev(t):
    return t.to(DEV)


_hip = None


def copy_from_address(ptr: int, shape, dtype) -> torch.Tensor:
    """A device tensor holding a copy of `prod(shape)` elements at device
    address `ptr` (memory a library cache owns), made with the HIP runtime's
    hipMemcpy after a device synchronisation."""
    import ctypes
    import os
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
        _hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        _hip.hipMemcpy.restype = ctypes.c_int
    t = torch.empty(shape, dtype=dtype, device=DEV)
    torch.cuda.synchronize()
    rc = _hip.hipMemcpy(t.data_ptr(), ptr, t.numel() * t.element_size(), 3)   # device to device
    assert rc == 0, f"hipMemcpy failed ({rc})"
    return t


def empty(shape, dtype):
    return torch.empty(shape, dtype=dtype, device=DEV)


def filled(shape, dtype, byte=0xA5):
    """Output buffer pre-filled with a canary so unwritten elements show."""
    t = torch.empty(shape, dtype=dtype, device=DEV)
    t.view(torch.uint8).fill_(byte)
    return t


def host(t):
    torch.cuda.synchronize()
    return bits(t)


def bf16_f64(b):
    return oracle.bf16_bits_to_f32(np.asarray(b, dtype=np.uint16)).astype(np.float64)


def assert_gemm_close(got_bits, ref_bits, what=""):
    """GEMM bound: max|C_gpu - C_ref| <= 1e-2 * max|C_ref| per matrix, the
    tolerance stated for the block-scaled contractions.  A second, tighter
    bound (F32 accumulation differs from the binary64 oracle only by
    rounding order, so nearly every element lands on the same or the
    neighbouring BF16) guards against small systematic slips that the loose
    bound would let through."""
    g, r = bf16_f64(got_bits), bf16_f64(ref_bits)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - r)
    mx = np.abs(r).max()
    assert err.max() <= 1e-2 * mx, f"{what}: max err {err.max():.4g} vs max|C| {mx:.4g}"
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(r), 1e-30))) - 7)
    tight = err <= 2 * ulp + 1e-5 * mx
    assert tight.mean() >= 0.999, f"{what}: only {tight.mean():.5f} within 2 ulp"


def assert_gemv_close(got_bits, ref_bits, what=""):
    """FP8 GEMV bound (row- or block-scaled): 2 BF16 ulp of |C_ref|, with a
    floor of 2^-14 * rms(C_ref[m, :]) for outputs near zero.  The kernels
    form exact products and sum them in F32 (K <= 2^16 terms, F32 error
    <= ~2^-24 * K * max term, far below the floor at these shapes); the one
    BF16 rounding accounts for the first ulp, F32 summation-order effects
    on a value next to a BF16 tie for the second."""
    g, r = bf16_f64(got_bits), bf16_f64(ref_bits)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(r), 1e-38))) - 7)
    rms = np.sqrt(np.mean(r * r, axis=1, keepdims=True))
    tol = np.maximum(2 * ulp, 2.0 ** -14 * rms)
    bad = np.abs(g - r) > tol
    assert not bad.any(), f"{what}: {bad.sum()} outside 2 ulp; worst {np.abs(g - r)[bad].max():.4g}"
