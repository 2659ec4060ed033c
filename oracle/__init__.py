"""CPU oracle for the quantized dense projection (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product library never loads it, and it shares no
code with the HIP path: the arithmetic lives in ``oracle.c`` (plain C,
binary32 steps with no FMA contraction, binary64 sums, OpenMP over rows) and
this module only marshals numpy arrays into it.

Every function follows one item of the documentation pages on the method; the
citation sits on the C function.  All arrays are C-contiguous numpy arrays;
BF16 tensors travel as ``uint16`` bit patterns, E4M3 / packed E2M1 as
``uint8``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# Compiler line: no fast-math, no FMA contraction (each binary32 step rounds
# once), OpenMP for the row loops.
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared",
          "-fPIC", "-std=gnu11", "-Wall"]


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc; returns the path."""
    if force or not os.path.exists(_LIB) or \
            os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or \
                os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        F = ctypes.c_float
        L.oracle_e2m1_decode.restype = ctypes.c_double
        L.oracle_e2m1_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e2m1_encode.restype = ctypes.c_uint8
        L.oracle_e2m1_encode.argtypes = [F]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_encode.argtypes = [F]
        L.oracle_int8_encode.restype = ctypes.c_int8
        L.oracle_int8_encode.argtypes = [F]
        L.oracle_bf16_from_double.restype = ctypes.c_uint16
        L.oracle_bf16_from_double.argtypes = [ctypes.c_double]
        L.oracle_bf16_to_float.restype = F
        L.oracle_bf16_to_float.argtypes = [ctypes.c_uint16]
        L.oracle_encode_array.argtypes = [ctypes.c_int, P, P, I]
        L.oracle_requant_a_bf16_int8.argtypes = [P, P, P, I, I]
        L.oracle_requant_w_nvfp4_int8.argtypes = [P, P, F, P, P, I, I]
        L.oracle_quantize_bf16_nvfp4.argtypes = [P, P, P, F, I, I]
        L.oracle_quant_rowwise_fp8.argtypes = [P, P, P, I, I]
        L.oracle_requant_w_blockfp8_rowwise.argtypes = [P, P, P, P, I, I]
        L.oracle_int8_block_partials.argtypes = [P, P, P, I, I, I]
        L.oracle_int8_gemm_blockscaled.argtypes = [P, P, P, P, P, I, I, I]
        L.oracle_w4a4_gemm.argtypes = [P, P, P, P, P, F, F, I, I, I]
        L.oracle_fp8_gemv_rowscale.argtypes = [P, P, P, P, I, I, I]
        L.oracle_fp8_gemv_blockscale.argtypes = [P, P, P, P, I, I, I]
        L.oracle_w4a16_gemv.argtypes = [P, P, P, F, P, I, I, I]
        L.oracle_fp8_gemm_rowscale.argtypes = [P, P, P, P, P, I, I, I]
        L.oracle_num_threads.restype = ctypes.c_int
        for fn in ("oracle_requant_a_bf16_int8", "oracle_requant_w_nvfp4_int8",
                   "oracle_quantize_bf16_nvfp4", "oracle_quant_rowwise_fp8",
                   "oracle_requant_w_blockfp8_rowwise",
                   "oracle_int8_block_partials", "oracle_int8_gemm_blockscaled",
                   "oracle_w4a4_gemm", "oracle_fp8_gemv_rowscale",
                   "oracle_fp8_gemv_blockscale", "oracle_w4a16_gemv",
                   "oracle_fp8_gemm_rowscale"):
            getattr(L, fn).restype = None
        _lib = L
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops run on."""
    return int(lib().oracle_num_threads())


# ----------------------------------------------------------------- codecs
def e2m1_decode(c: int) -> float:
    return lib().oracle_e2m1_decode(int(c))


def e4m3_decode(c: int) -> float:
    return lib().oracle_e4m3_decode(int(c))


def e2m1_encode(y: float) -> int:
    return int(lib().oracle_e2m1_encode(float(y)))


def e4m3_encode(y: float) -> int:
    return int(lib().oracle_e4m3_encode(float(y)))


def int8_encode(y: float) -> int:
    return int(lib().oracle_int8_encode(float(y)))


ENC_E4M3, ENC_E2M1, ENC_INT8 = 0, 1, 2


def encode_array(kind: int, y) -> np.ndarray:
    """The scalar encoders over a float32 array: E4M3 (kind 0) or E2M1
    (kind 1) code bytes, or int8 codes as their two's-complement bytes
    (kind 2)."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, np.uint8)
    lib().oracle_encode_array(int(kind), y.ctypes.data, out.ctypes.data, y.size)
    return out


def bf16_from_double(x: float) -> int:
    return int(lib().oracle_bf16_from_double(float(x)))


def bf16_to_float(b: int) -> float:
    return float(lib().oracle_bf16_to_float(int(b)))


# ------------------------------------------------------------- quantizers
def requant_a_bf16_int8(a_bf16: np.ndarray):
    """BF16 bits [m,k] -> (int8 [m,k], f32 scale [m,k/32])."""
    a = _c(a_bf16, np.uint16)
    m, k = a.shape
    assert k % 32 == 0
    q = np.empty((m, k), np.int8)
    s = np.empty((m, k // 32), np.float32)
    lib().oracle_requant_a_bf16_int8(_p(a), _p(q), _p(s), m, k)
    return q, s


def requant_w_nvfp4_int8(packed: np.ndarray, sc16: np.ndarray, scale2: float):
    """NVFP4 ([n,k/2] packed, [n,k/16] E4M3, scale2) -> (int8 [n,k], f32 [n,k/32])."""
    packed = _c(packed, np.uint8)
    sc16 = _c(sc16, np.uint8)
    n, kh = packed.shape
    k = kh * 2
    assert k % 32 == 0 and sc16.shape == (n, k // 16)
    q = np.empty((n, k), np.int8)
    s = np.empty((n, k // 32), np.float32)
    lib().oracle_requant_w_nvfp4_int8(_p(packed), _p(sc16), float(scale2),
                                      _p(q), _p(s), n, k)
    return q, s


def quantize_bf16_nvfp4(x_bf16: np.ndarray, scale2: float = 1.0):
    """BF16 bits [r,k] -> (packed E2M1 [r,k/2], E4M3 scales [r,k/16])."""
    x = _c(x_bf16, np.uint16)
    r, k = x.shape
    assert k % 16 == 0
    packed = np.empty((r, k // 2), np.uint8)
    sc = np.empty((r, k // 16), np.uint8)
    lib().oracle_quantize_bf16_nvfp4(_p(x), _p(packed), _p(sc), float(scale2), r, k)
    return packed, sc


def quant_rowwise_fp8(x_bf16: np.ndarray):
    """BF16 bits [r,k] -> (E4M3 [r,k], f32 row scale [r])."""
    x = _c(x_bf16, np.uint16)
    r, k = x.shape
    q = np.empty((r, k), np.uint8)
    s = np.empty((r,), np.float32)
    lib().oracle_quant_rowwise_fp8(_p(x), _p(q), _p(s), r, k)
    return q, s


def requant_w_blockfp8_rowwise(w: np.ndarray, grid: np.ndarray):
    """Block-scaled E4M3 [n,k] + f32 grid [n/128,k/128] -> (E4M3 [n,k], f32 [n])."""
    w = _c(w, np.uint8)
    grid = _c(grid, np.float32)
    n, k = w.shape
    assert n % 128 == 0 and k % 128 == 0 and grid.shape == (n // 128, k // 128)
    q = np.empty((n, k), np.uint8)
    s = np.empty((n,), np.float32)
    lib().oracle_requant_w_blockfp8_rowwise(_p(w), _p(grid), _p(q), _p(s), n, k)
    return q, s


# ----------------------------------------------------------- contractions
def int8_block_partials(a: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Exact int32 partial sum per 32-K block, shape [m, n, k/32]."""
    a = _c(a, np.int8)
    w = _c(w, np.int8)
    m, k = a.shape
    n = w.shape[0]
    assert w.shape[1] == k and k % 32 == 0
    p = np.empty((m, n, k // 32), np.int32)
    lib().oracle_int8_block_partials(_p(a), _p(w), _p(p), m, n, k)
    return p


def int8_gemm_blockscaled(a, w, a_scale, w_scale) -> np.ndarray:
    """int8 [m,k] x int8 [n,k] with per-32 F32 scales -> BF16 bits [m,n]."""
    a = _c(a, np.int8)
    w = _c(w, np.int8)
    a_scale = _c(a_scale, np.float32)
    w_scale = _c(w_scale, np.float32)
    m, k = a.shape
    n = w.shape[0]
    assert w.shape[1] == k and a_scale.shape == (m, k // 32) \
        and w_scale.shape == (n, k // 32)
    out = np.empty((m, n), np.uint16)
    lib().oracle_int8_gemm_blockscaled(_p(a), _p(w), _p(a_scale), _p(w_scale),
                                       _p(out), m, n, k)
    return out


def w4a4_gemm(a_packed, a_scale, w_packed, w_scale, scale_a2, scale_w2):
    """NVFP4 [m,k] x NVFP4 [n,k] -> BF16 bits [m,n]."""
    a_packed = _c(a_packed, np.uint8)
    a_scale = _c(a_scale, np.uint8)
    w_packed = _c(w_packed, np.uint8)
    w_scale = _c(w_scale, np.uint8)
    m, kh = a_packed.shape
    n = w_packed.shape[0]
    k = kh * 2
    assert w_packed.shape[1] == kh and a_scale.shape == (m, k // 16) \
        and w_scale.shape == (n, k // 16)
    out = np.empty((m, n), np.uint16)
    lib().oracle_w4a4_gemm(_p(a_packed), _p(a_scale), _p(w_packed), _p(w_scale),
                           _p(out), float(scale_a2), float(scale_w2), m, n, k)
    return out


def fp8_gemv_rowscale(x_bf16, w, row_scale) -> np.ndarray:
    """BF16 [m,k] x E4M3 [n,k] with F32 row scale [n] -> BF16 bits [m,n]."""
    x = _c(x_bf16, np.uint16)
    w = _c(w, np.uint8)
    row_scale = _c(row_scale, np.float32)
    m, k = x.shape
    n = w.shape[0]
    assert w.shape[1] == k and row_scale.shape == (n,)
    out = np.empty((m, n), np.uint16)
    lib().oracle_fp8_gemv_rowscale(_p(x), _p(w), _p(row_scale), _p(out), m, n, k)
    return out


def fp8_gemv_blockscale(x_bf16, w, block_scale) -> np.ndarray:
    """BF16 [m,k] x E4M3 [n,k] with F32 block scales [n/128, k/128] -> BF16 bits [m,n]."""
    x = _c(x_bf16, np.uint16)
    w = _c(w, np.uint8)
    block_scale = _c(block_scale, np.float32)
    m, k = x.shape
    n = w.shape[0]
    assert w.shape[1] == k and n % 128 == 0 and k % 128 == 0
    assert block_scale.shape == (n // 128, k // 128)
    out = np.empty((m, n), np.uint16)
    lib().oracle_fp8_gemv_blockscale(_p(x), _p(w), _p(block_scale), _p(out), m, n, k)
    return out


def w4a16_gemv(x_bf16, w_packed, w_scale, scale2) -> np.ndarray:
    """BF16 [m,k] x NVFP4 (packed [n,k/2], E4M3 per-16 scales [n,k/16],
    per-tensor scale2) -> BF16 bits [m,n]."""
    x = _c(x_bf16, np.uint16)
    wp = _c(w_packed, np.uint8)
    ws = _c(w_scale, np.uint8)
    m, k = x.shape
    n = wp.shape[0]
    assert k % 16 == 0 and wp.shape == (n, k // 2) and ws.shape == (n, k // 16)
    out = np.empty((m, n), np.uint16)
    lib().oracle_w4a16_gemv(_p(x), _p(wp), _p(ws), float(scale2), _p(out), m, n, k)
    return out


def fp8_gemm_rowscale(a, a_scale, w, w_scale) -> np.ndarray:
    """E4M3 [m,k] (+[m] F32) x E4M3 [n,k] (+[n] F32) -> BF16 bits [m,n]."""
    a = _c(a, np.uint8)
    w = _c(w, np.uint8)
    a_scale = _c(a_scale, np.float32)
    w_scale = _c(w_scale, np.float32)
    m, k = a.shape
    n = w.shape[0]
    assert w.shape[1] == k and a_scale.shape == (m,) and w_scale.shape == (n,)
    out = np.empty((m, n), np.uint16)
    lib().oracle_fp8_gemm_rowscale(_p(a), _p(a_scale), _p(w), _p(w_scale),
                                   _p(out), m, n, k)
    return out


# ---------------------------------------------------------------- helpers
def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Reinterpret BF16 bit patterns as float32 values (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)
