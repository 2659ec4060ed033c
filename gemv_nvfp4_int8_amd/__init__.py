"""Python binding of libqproj, the gfx950 quantized dense projection library.

Argument marshalling only: each function takes torch tensors (device memory
owned by the caller), checks their dtypes and shapes so that no kernel can
be handed a buffer smaller than it will touch, and calls the C entry point of
the same name with raw pointers, sizes and torch's current HIP stream.
Every step of the computation runs in the library's HIP kernels; there is no
fallback.  If ``libqproj.so`` has not been built, the first call into the
library raises ImportError (build it with ``__graft_entry__.build()`` or
``python -m gemv_nvfp4_int8_amd._build``).

The operations and their rounding rules are documented in include/qproj.h.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqproj.so")

QP_OK = 0
QP_ERR_NULL = -1
QP_ERR_SHAPE = -2
QP_ERR_RANGE = -3
QP_ERR_FORMAT = -4
QP_ERR_HIP = -5
QP_ERR_ALIGN = -6
QP_ERR_ALLOC = -7
QP_ERR_SCRATCH = -8

QP_FP8_PER_ROW = 0
QP_FP8_BLOCK128 = 1
QP_FP8_SINGLE_SCALE = 2
QP_BF16 = 3
QP_NVFP4 = 4

QP_TILES_BANDED = 0
QP_TILES_MFAST = 1
QP_TILES_NFAST = 2


class QProjError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_string(status)} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libqproj.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"libqproj.so not found at {LIB_PATH}: the HIP library must be "
                "built (python -m gemv_nvfp4_int8_amd._build) -- there is no "
                "fallback path")
        L = ctypes.CDLL(LIB_PATH)
        P, U, F, I = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_float, ctypes.c_int
        PP = ctypes.POINTER(ctypes.c_void_p)
        sig = {
            "requant_w_nvfp4_int8": [P, P, F, P, P, U, U, P],
            "requant_a_bf16_int8": [P, P, P, U, U, P],
            "int8_gemm_blockscaled": [P, P, P, P, P, U, U, U, P],
            "int8_gemm_blockscaled_f16ops": [P, P, P, P, P, U, U, U, P],
            "int8_w4a8_prefill": [P, P, P, P, P, P, U, U, U, P],
            "int8_w4a8_prefill_noalloc": [P, P, P, P, U, U, U, P],
            "qproj_encode_test": [I, P, P, U, P],
            "int8_gemm_block_partials": [P, P, P, U, U, U, P],
            "quantize_bf16_nvfp4": [P, P, P, F, U, U, P],
            "w4a4_gemm": [P, P, P, P, P, F, F, U, U, U, P],
            "w4a4_gemm_tiles": [P, P, P, P, P, F, F, U, U, U, I, P],
            "requant_w_blockfp8_rowwise": [I, P, P, P, P, PP, PP, U, U, P],
            "quant_rowwise_fp8": [P, P, P, U, U, P],
            "fp8_gemm_rowscale": [P, P, P, P, P, U, U, U, P],
            "fp8_rowwise_proj": [I, P, P, P, P, P, P, P, P, U, U, U, P],
            "fp8_gemv_rowscale": [P, P, P, P, U, U, U, P],
            "fp8_gemv_blockscale": [P, P, P, P, U, U, U, P],
            "w4a16_gemv": [P, P, P, F, P, U, U, U, P],
            "qproj_cache_create": [PP],
            "qproj_cache_destroy": [P],
            "qproj_cache_evict": [P, P],
            "qproj_cache_stats": [P, ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(ctypes.c_uint64)],
            "requant_w_blockfp8_rowwise_cached": [P, I, P, P, U, U, PP, PP, P],
            "requant_w_nvfp4_int8_cached": [P, P, P, F, U, U, PP, PP, P],
            "fp8_rowwise_proj_cached": [P, I, P, P, P, P, P, P, U, U, U, P],
            "int8_w4a8_prefill_cached": [P, P, P, P, F, P, P, P, U, U, U, P],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.qproj_launch_count.restype = ctypes.c_uint64
        L.qproj_launch_count.argtypes = []
        L.qproj_status_string.restype = ctypes.c_char_p
        L.qproj_status_string.argtypes = [ctypes.c_int]
        L.qproj_noalloc_scratch_bytes.restype = ctypes.c_uint64
        L.qproj_noalloc_scratch_bytes.argtypes = []
        L.qproj_abi_version.restype = ctypes.c_int
        L.qproj_abi_version.argtypes = []
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().qproj_status_string(int(status)).decode()


def launch_count() -> int:
    return int(lib().qproj_launch_count())


def abi_version() -> int:
    return int(lib().qproj_abi_version())


# ------------------------------------------------------------------ helpers
# torch's current stream of the current device, as a raw handle.  The
# private accessor costs ~0.1 us against ~2.7 us for building a Stream object
# (per-call overhead matters: a narrow GEMV runs in a few microseconds).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream):
    if stream is None:
        if _raw_stream is not None:
            return _raw_stream(torch._C._cuda_getDevice())
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: torch.Tensor):
    return t.data_ptr()


def _need(t: torch.Tensor, name: str, dtypes, shape):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.shape != shape:
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")


def _check(fn: str, status: int):
    if status != QP_OK:
        raise QProjError(fn, status)


BF16 = (torch.bfloat16, torch.int16, torch.uint16) if hasattr(torch, "uint16") \
    else (torch.bfloat16, torch.int16)
U8 = (torch.uint8, torch.float8_e4m3fn)
I8 = (torch.int8,)
F32 = (torch.float32,)
I32 = (torch.int32,)


# --------------------------------------------------------------- entry points
def requant_w_nvfp4_int8(w_packed, w_e4m3, scale2, w_i8, w_scale, stream=None):
    n, kh = w_packed.shape
    k = 2 * kh
    _need(w_packed, "w_packed", U8, (n, kh))
    _need(w_e4m3, "w_e4m3", U8, (n, k // 16))
    _need(w_i8, "w_i8", I8, (n, k))
    _need(w_scale, "w_scale", F32, (n, k // 32))
    _check("requant_w_nvfp4_int8", lib().requant_w_nvfp4_int8(
        _ptr(w_packed), _ptr(w_e4m3), float(scale2), _ptr(w_i8), _ptr(w_scale),
        n, k, _stream(stream)))


def requant_a_bf16_int8(a, a_i8, a_scale, stream=None):
    m, k = a.shape
    _need(a, "a", BF16, (m, k))
    _need(a_i8, "a_i8", I8, (m, k))
    _need(a_scale, "a_scale", F32, (m, k // 32))
    _check("requant_a_bf16_int8", lib().requant_a_bf16_int8(
        _ptr(a), _ptr(a_i8), _ptr(a_scale), m, k, _stream(stream)))


def int8_gemm_blockscaled(a_i8, w_i8, a_scale, w_scale, out, stream=None):
    m, k = a_i8.shape
    n = w_i8.shape[0]
    _need(a_i8, "a_i8", I8, (m, k))
    _need(w_i8, "w_i8", I8, (n, k))
    _need(a_scale, "a_scale", F32, (m, k // 32))
    _need(w_scale, "w_scale", F32, (n, k // 32))
    _need(out, "out", BF16, (m, n))
    _check("int8_gemm_blockscaled", lib().int8_gemm_blockscaled(
        _ptr(a_i8), _ptr(w_i8), _ptr(a_scale), _ptr(w_scale), _ptr(out),
        m, n, k, _stream(stream)))


def int8_gemm_blockscaled_f16ops(a_i8, w_i8, a_scale, w_scale, out, stream=None):
    """The operand-route ablation of int8_gemm_blockscaled (FP16 MFMA on
    converted operands; bit-identical output; k % 128 == 0)."""
    m, k = a_i8.shape
    n = w_i8.shape[0]
    _need(a_i8, "a_i8", I8, (m, k))
    _need(w_i8, "w_i8", I8, (n, k))
    _need(a_scale, "a_scale", F32, (m, k // 32))
    _need(w_scale, "w_scale", F32, (n, k // 32))
    _need(out, "out", BF16, (m, n))
    _check("int8_gemm_blockscaled_f16ops", lib().int8_gemm_blockscaled_f16ops(
        _ptr(a_i8), _ptr(w_i8), _ptr(a_scale), _ptr(w_scale), _ptr(out),
        m, n, k, _stream(stream)))


def int8_w4a8_prefill(a_bf16, w_i8, w_scale, a_i8_scratch, a_scale_scratch,
                      out, stream=None):
    m, k = a_bf16.shape
    n = w_i8.shape[0]
    _need(a_bf16, "a_bf16", BF16, (m, k))
    _need(w_i8, "w_i8", I8, (n, k))
    _need(w_scale, "w_scale", F32, (n, k // 32))
    _need(a_i8_scratch, "a_i8_scratch", I8, (m, k))
    _need(a_scale_scratch, "a_scale_scratch", F32, (m, k // 32))
    _need(out, "out", BF16, (m, n))
    _check("int8_w4a8_prefill", lib().int8_w4a8_prefill(
        _ptr(a_bf16), _ptr(w_i8), _ptr(w_scale), _ptr(a_i8_scratch),
        _ptr(a_scale_scratch), _ptr(out), m, n, k, _stream(stream)))


QP_ENC_E4M3_NOSAT, QP_ENC_E2M1_NOSAT, QP_ENC_INT8 = 0, 1, 2
QP_ENC_E4M3, QP_ENC_E2M1, QP_ENC_E4M3_SCALE = 3, 4, 5


def encode_test(kind, y, out, stream=None):
    """Test export: the kernels' device encoder `kind` on float32 values y
    (a 1-D tensor, length a multiple of 8), one code byte per value in out."""
    n = y.numel()
    _need(y, "y", F32, (n,))
    _need(out, "out", U8, (n,))
    _check("qproj_encode_test", lib().qproj_encode_test(int(kind), _ptr(y), _ptr(out), n,
                                                        _stream(stream)))


def noalloc_scratch_bytes() -> int:
    return int(lib().qproj_noalloc_scratch_bytes())


def int8_w4a8_prefill_noalloc(a_bf16, w_i8, w_scale, out, stream=None):
    """int8_w4a8_prefill with the activation scratch held inside the library
    (a fixed per-GPU array): allocates nothing; calls on one GPU must not
    overlap."""
    m, k = a_bf16.shape
    n = w_i8.shape[0]
    _need(a_bf16, "a_bf16", BF16, (m, k))
    _need(w_i8, "w_i8", I8, (n, k))
    _need(w_scale, "w_scale", F32, (n, k // 32))
    _need(out, "out", BF16, (m, n))
    _check("int8_w4a8_prefill_noalloc", lib().int8_w4a8_prefill_noalloc(
        _ptr(a_bf16), _ptr(w_i8), _ptr(w_scale), _ptr(out), m, n, k, _stream(stream)))


def int8_gemm_block_partials(a_i8, w_i8, p, stream=None):
    m, k = a_i8.shape
    n = w_i8.shape[0]
    _need(a_i8, "a_i8", I8, (m, k))
    _need(w_i8, "w_i8", I8, (n, k))
    _need(p, "p", I32, (m, n, k // 32))
    _check("int8_gemm_block_partials", lib().int8_gemm_block_partials(
        _ptr(a_i8), _ptr(w_i8), _ptr(p), m, n, k, _stream(stream)))


def quantize_bf16_nvfp4(x, packed, scale, scale2=1.0, stream=None):
    rows, k = x.shape
    _need(x, "x", BF16, (rows, k))
    _need(packed, "packed", U8, (rows, k // 2))
    _need(scale, "scale", U8, (rows, k // 16))
    _check("quantize_bf16_nvfp4", lib().quantize_bf16_nvfp4(
        _ptr(x), _ptr(packed), _ptr(scale), float(scale2), rows, k,
        _stream(stream)))


def w4a4_gemm(a_packed, a_scale, w_packed, w_scale, out, scale_a2, scale_w2,
              stream=None, tile_order=None):
    """tile_order: None (w4a4_gemm) or one of QP_TILES_* (w4a4_gemm_tiles)."""
    m, kh = a_packed.shape
    n = w_packed.shape[0]
    k = 2 * kh
    _need(a_packed, "a_packed", U8, (m, kh))
    _need(a_scale, "a_scale", U8, (m, k // 16))
    _need(w_packed, "w_packed", U8, (n, kh))
    _need(w_scale, "w_scale", U8, (n, k // 16))
    _need(out, "out", BF16, (m, n))
    if tile_order is None:
        _check("w4a4_gemm", lib().w4a4_gemm(
            _ptr(a_packed), _ptr(a_scale), _ptr(w_packed), _ptr(w_scale), _ptr(out),
            float(scale_a2), float(scale_w2), m, n, k, _stream(stream)))
    else:
        _check("w4a4_gemm_tiles", lib().w4a4_gemm_tiles(
            _ptr(a_packed), _ptr(a_scale), _ptr(w_packed), _ptr(w_scale), _ptr(out),
            float(scale_a2), float(scale_w2), m, n, k, int(tile_order), _stream(stream)))


def requant_w_blockfp8_rowwise(fmt, w, scale, w_out=None, scale_out=None,
                               stream=None):
    """Returns the (weight_ptr, scale_ptr) pair the row-wise GEMM should read:
    the inputs' own pointers for QP_FP8_PER_ROW, w_out / scale_out after the
    requant for QP_FP8_BLOCK128."""
    n, k = w.shape
    _need(w, "w", U8, (n, k))
    if fmt == QP_FP8_BLOCK128:
        _need(scale, "scale", F32, (n // 128, k // 128))
        _need(w_out, "w_out", U8, (n, k))
        _need(scale_out, "scale_out", F32, (n,))
    elif fmt == QP_FP8_PER_ROW:
        _need(scale, "scale", F32, (n,))
    wres, sres = ctypes.c_void_p(), ctypes.c_void_p()
    _check("requant_w_blockfp8_rowwise", lib().requant_w_blockfp8_rowwise(
        int(fmt), _ptr(w), _ptr(scale),
        _ptr(w_out) if w_out is not None else None,
        _ptr(scale_out) if scale_out is not None else None,
        ctypes.byref(wres), ctypes.byref(sres), n, k, _stream(stream)))
    return wres.value, sres.value


def quant_rowwise_fp8(x, q, scale, stream=None):
    rows, k = x.shape
    _need(x, "x", BF16, (rows, k))
    _need(q, "q", U8, (rows, k))
    _need(scale, "scale", F32, (rows,))
    _check("quant_rowwise_fp8", lib().quant_rowwise_fp8(
        _ptr(x), _ptr(q), _ptr(scale), rows, k, _stream(stream)))


def fp8_gemm_rowscale(a, a_scale, w, w_scale, out, stream=None):
    m, k = a.shape
    n = w.shape[0]
    _need(a, "a", U8, (m, k))
    _need(a_scale, "a_scale", F32, (m,))
    _need(w, "w", U8, (n, k))
    _need(w_scale, "w_scale", F32, (n,))
    _need(out, "out", BF16, (m, n))
    _check("fp8_gemm_rowscale", lib().fp8_gemm_rowscale(
        _ptr(a), _ptr(a_scale), _ptr(w), _ptr(w_scale), _ptr(out), m, n, k,
        _stream(stream)))


def fp8_rowwise_proj(fmt, w, w_scale, w_rowwise, w_rowwise_scale, act, act_q,
                     act_scale, out, stream=None):
    n, k = w.shape
    m = act.shape[0]
    _need(w, "w", U8, (n, k))
    _need(act, "act", BF16, (m, k))
    _need(act_q, "act_q", U8, (m, k))
    _need(act_scale, "act_scale", F32, (m,))
    _need(out, "out", BF16, (m, n))
    if fmt == QP_FP8_BLOCK128:
        _need(w_scale, "w_scale", F32, (n // 128, k // 128))
        _need(w_rowwise, "w_rowwise", U8, (n, k))
        _need(w_rowwise_scale, "w_rowwise_scale", F32, (n,))
    else:
        _need(w_scale, "w_scale", F32, (n,))
    _check("fp8_rowwise_proj", lib().fp8_rowwise_proj(
        int(fmt), _ptr(w), _ptr(w_scale),
        _ptr(w_rowwise) if w_rowwise is not None else None,
        _ptr(w_rowwise_scale) if w_rowwise_scale is not None else None,
        _ptr(act), _ptr(act_q), _ptr(act_scale), _ptr(out), m, n, k,
        _stream(stream)))


def fp8_gemv_rowscale(x, w, row_scale, out, stream=None):
    m, k = x.shape
    n = w.shape[0]
    _need(x, "x", BF16, (m, k))
    _need(w, "w", U8, (n, k))
    _need(row_scale, "row_scale", F32, (n,))
    _need(out, "out", BF16, (m, n))
    _check("fp8_gemv_rowscale", lib().fp8_gemv_rowscale(
        _ptr(x), _ptr(w), _ptr(row_scale), _ptr(out), m, n, k, _stream(stream)))


def fp8_gemv_blockscale(x, w, block_scale, out, stream=None):
    m, k = x.shape
    n = w.shape[0]
    _need(x, "x", BF16, (m, k))
    _need(w, "w", U8, (n, k))
    _need(block_scale, "block_scale", F32, (n // 128, k // 128))
    _need(out, "out", BF16, (m, n))
    _check("fp8_gemv_blockscale", lib().fp8_gemv_blockscale(
        _ptr(x), _ptr(w), _ptr(block_scale), _ptr(out), m, n, k, _stream(stream)))


def w4a16_gemv(x, w_packed, w_e4m3, scale2, out, stream=None):
    m, k = x.shape
    n = w_packed.shape[0]
    _need(x, "x", BF16, (m, k))
    _need(w_packed, "w_packed", U8, (n, k // 2))
    _need(w_e4m3, "w_e4m3", U8, (n, k // 16))
    _need(out, "out", BF16, (m, n))
    _check("w4a16_gemv", lib().w4a16_gemv(
        _ptr(x), _ptr(w_packed), _ptr(w_e4m3), float(scale2), _ptr(out), m, n, k,
        _stream(stream)))


class DerivedWeights:
    """A derived-weight cache (the library's qp_cache): weights requantised on
    first use and kept, keyed by the source weight's device address
    (dispatch_proj_rowwise.rs, requant_weight_rowwise_fp8_cached and its
    DerivedWeights cache).  The cache owns the derived device buffers; the
    requant methods return their device addresses as ints.  close() (or
    garbage collection) frees them: no kernel reading one may be pending."""

    def __init__(self):
        h = ctypes.c_void_p()
        _check("qproj_cache_create", lib().qproj_cache_create(ctypes.byref(h)))
        self._h = h

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().qproj_cache_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def stats(self):
        """(entries, bytes) held by the cache."""
        e, b = ctypes.c_uint64(), ctypes.c_uint64()
        _check("qproj_cache_stats", lib().qproj_cache_stats(self._h, ctypes.byref(e), ctypes.byref(b)))
        return int(e.value), int(b.value)

    def evict(self, w):
        _check("qproj_cache_evict", lib().qproj_cache_evict(self._h, _ptr(w)))

    def requant_w_blockfp8_rowwise(self, fmt, w, scale, stream=None):
        """Row-wise FP8 copy of a block-scaled weight (passthrough for
        QP_FP8_PER_ROW): returns (weight address, scale address)."""
        n, k = w.shape
        _need(w, "w", U8, (n, k))
        if fmt == QP_FP8_BLOCK128:
            _need(scale, "scale", F32, (n // 128, k // 128))
        wq, sq = ctypes.c_void_p(), ctypes.c_void_p()
        _check("requant_w_blockfp8_rowwise_cached", lib().requant_w_blockfp8_rowwise_cached(
            self._h, int(fmt), _ptr(w), _ptr(scale), n, k, ctypes.byref(wq), ctypes.byref(sq),
            _stream(stream)))
        return wq.value, sq.value

    def requant_w_nvfp4_int8(self, w_packed, w_e4m3, scale2, stream=None):
        """int8 copy [n,k] and F32 per-32 scales [n,k/32] of an NVFP4 weight:
        returns (weight address, scale address)."""
        n, kh = w_packed.shape
        k = 2 * kh
        _need(w_packed, "w_packed", U8, (n, k // 2))
        _need(w_e4m3, "w_e4m3", U8, (n, k // 16))
        wq, sq = ctypes.c_void_p(), ctypes.c_void_p()
        _check("requant_w_nvfp4_int8_cached", lib().requant_w_nvfp4_int8_cached(
            self._h, _ptr(w_packed), _ptr(w_e4m3), float(scale2), n, k, ctypes.byref(wq),
            ctypes.byref(sq), _stream(stream)))
        return wq.value, sq.value

    def fp8_rowwise_proj(self, fmt, w, w_scale, act, act_q, act_scale, out, stream=None):
        m, k = act.shape
        n = w.shape[0]
        _need(w, "w", U8, (n, k))
        _need(w_scale, "w_scale", F32, (n,) if fmt == QP_FP8_PER_ROW else (n // 128, k // 128))
        _need(act, "act", BF16, (m, k))
        _need(act_q, "act_q", U8, (m, k))
        _need(act_scale, "act_scale", F32, (m,))
        _need(out, "out", BF16, (m, n))
        _check("fp8_rowwise_proj_cached", lib().fp8_rowwise_proj_cached(
            self._h, int(fmt), _ptr(w), _ptr(w_scale), _ptr(act), _ptr(act_q), _ptr(act_scale),
            _ptr(out), m, n, k, _stream(stream)))

    def int8_w4a8_prefill(self, a, w_packed, w_e4m3, scale2, a_i8, a_scale, out, stream=None):
        m, k = a.shape
        n = w_packed.shape[0]
        _need(a, "a", BF16, (m, k))
        _need(w_packed, "w_packed", U8, (n, k // 2))
        _need(w_e4m3, "w_e4m3", U8, (n, k // 16))
        _need(a_i8, "a_i8", I8, (m, k))
        _need(a_scale, "a_scale", F32, (m, k // 32))
        _need(out, "out", BF16, (m, n))
        _check("int8_w4a8_prefill_cached", lib().int8_w4a8_prefill_cached(
            self._h, _ptr(a), _ptr(w_packed), _ptr(w_e4m3), float(scale2), _ptr(a_i8),
            _ptr(a_scale), _ptr(out), m, n, k, _stream(stream)))


__all__ = [
    "requant_w_nvfp4_int8", "requant_a_bf16_int8", "int8_gemm_blockscaled",
    "int8_w4a8_prefill", "int8_gemm_block_partials", "quantize_bf16_nvfp4",
    "w4a4_gemm", "requant_w_blockfp8_rowwise", "quant_rowwise_fp8",
    "fp8_gemm_rowscale", "fp8_rowwise_proj", "fp8_gemv_rowscale",
    "fp8_gemv_blockscale", "w4a16_gemv", "DerivedWeights",
    "launch_count", "status_string", "abi_version", "lib", "QProjError",
]
