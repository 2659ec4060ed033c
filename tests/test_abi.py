"""C-ABI contract tests that need no GPU.

The library must export every function include/qproj.h declares, and every
argument check must happen on the host before any HIP call, so these tests
call the entry points with bad arguments (and with fake, never dereferenced
device addresses) and expect the documented error codes.  The row-wise
passthrough is pure pointer logic (dispatch_proj_rowwise.rs,
rowwise_pair_passthrough and its tests) and is checked here too, including
that it launches nothing (the analogue of the pages' alloc_count() == 0).
"""
import ctypes
import os
import re
import subprocess

import pytest

import gemv_nvfp4_int8_amd as qp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qproj.h")

FAKE = 0x10000          # aligned, never dereferenced
FAKE2 = 0x20000


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z0-9_]+\s*\**\s*([a-z_0-9]+)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ["requant_w_nvfp4_int8", "requant_a_bf16_int8", "int8_gemm_blockscaled",
              "quantize_bf16_nvfp4", "w4a4_gemm", "requant_w_blockfp8_rowwise",
              "fp8_gemv_rowscale", "quant_rowwise_fp8", "fp8_gemm_rowscale",
              "int8_gemm_block_partials", "fp8_gemv_blockscale", "w4a16_gemv",
              "qproj_launch_count"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", qp.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    missing = [n for n in _declared_functions() if n not in exported]
    assert not missing, missing
    L = qp.lib()
    for n in _declared_functions():
        assert hasattr(L, n)


def test_abi_version_and_status_strings():
    assert qp.abi_version() == 1
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert qp.status_string(code) != "unknown status"
    assert qp.status_string(-99) == "unknown status"


L = qp.lib()


def test_gemv_m_range_and_k_multiple():
    for m in (0, 17, 100):
        assert L.fp8_gemv_rowscale(FAKE, FAKE, FAKE, FAKE, m, 64, 64, None) == qp.QP_ERR_RANGE
    assert L.fp8_gemv_rowscale(FAKE, FAKE, FAKE, FAKE, 4, 64, 40, None) == qp.QP_ERR_SHAPE
    assert L.fp8_gemv_rowscale(FAKE, FAKE, FAKE, FAKE, 4, 0, 64, None) == qp.QP_ERR_SHAPE
    assert L.fp8_gemv_rowscale(None, FAKE, FAKE, FAKE, 4, 64, 64, None) == qp.QP_ERR_NULL
    assert L.fp8_gemv_rowscale(FAKE + 4, FAKE, FAKE, FAKE, 4, 64, 64, None) == qp.QP_ERR_ALIGN


def test_block_scaled_gemv_needs_128_multiples():
    # The scale grid covers whole 128 x 128 weight blocks.
    for m in (0, 17):
        assert L.fp8_gemv_blockscale(FAKE, FAKE, FAKE, FAKE, m, 128, 128, None) == qp.QP_ERR_RANGE
    for n, k in ((64, 128), (128, 64), (200, 256), (256, 192), (0, 128), (128, 0)):
        assert L.fp8_gemv_blockscale(FAKE, FAKE, FAKE, FAKE, 2, n, k, None) == qp.QP_ERR_SHAPE
    assert L.fp8_gemv_blockscale(FAKE, FAKE, None, FAKE, 2, 128, 128, None) == qp.QP_ERR_NULL
    assert L.fp8_gemv_blockscale(FAKE, FAKE, FAKE + 2, FAKE, 2, 128, 128, None) == qp.QP_ERR_ALIGN


def test_w4a16_gemv_argument_checks():
    for m in (0, 9):
        assert L.w4a16_gemv(FAKE, FAKE, FAKE, 1.0, FAKE, m, 64, 64, None) == qp.QP_ERR_RANGE
    for n, k in ((64, 16), (64, 48), (0, 64), (64, 0), (64, 1 << 27)):
        assert L.w4a16_gemv(FAKE, FAKE, FAKE, 1.0, FAKE, 2, n, k, None) == qp.QP_ERR_SHAPE
    assert L.w4a16_gemv(FAKE, None, FAKE, 1.0, FAKE, 2, 64, 64, None) == qp.QP_ERR_NULL
    assert L.w4a16_gemv(FAKE, FAKE, FAKE + 4, 1.0, FAKE, 2, 64, 64, None) == qp.QP_ERR_ALIGN


def test_int8_paths_need_k_multiple_of_32():
    assert L.requant_a_bf16_int8(FAKE, FAKE, FAKE, 4, 48, None) == qp.QP_ERR_SHAPE
    assert L.requant_w_nvfp4_int8(FAKE, FAKE, 1.0, FAKE, FAKE, 4, 16, None) == qp.QP_ERR_SHAPE
    assert L.int8_gemm_blockscaled(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 4, 80, None) == qp.QP_ERR_SHAPE
    assert L.int8_gemm_block_partials(FAKE, FAKE, None, 4, 4, 64, None) == qp.QP_ERR_NULL
    assert L.int8_w4a8_prefill(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 4, 64, None) == qp.QP_ERR_SHAPE


def test_sizes_beyond_2_pow_31_elements_are_rejected():
    assert L.requant_a_bf16_int8(FAKE, FAKE, FAKE, 1 << 20, 1 << 12, None) == qp.QP_ERR_SHAPE
    assert L.fp8_gemv_rowscale(FAKE, FAKE, FAKE, FAKE, 1, 1 << 20, 1 << 12, None) == qp.QP_ERR_SHAPE


def test_nvfp4_and_rowwise_shape_rules():
    assert L.quantize_bf16_nvfp4(FAKE, FAKE, FAKE, 1.0, 4, 16, None) == qp.QP_ERR_SHAPE
    assert L.quantize_bf16_nvfp4(FAKE, FAKE, FAKE + 1, 1.0, 4, 64, None) == qp.QP_ERR_ALIGN
    assert L.w4a4_gemm(FAKE, FAKE, FAKE, FAKE, FAKE, 1.0, 1.0, 4, 4, 48, None) == qp.QP_ERR_SHAPE
    assert L.quant_rowwise_fp8(FAKE, FAKE, FAKE, 4, 24, None) == qp.QP_ERR_SHAPE
    assert L.fp8_gemm_rowscale(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 4, 8, None) == qp.QP_ERR_SHAPE


def _requant(fmt, w, s, wo, so, n=4096, k=5120):
    wres, sres = ctypes.c_void_p(0), ctypes.c_void_p(0)
    st = L.requant_w_blockfp8_rowwise(fmt, w, s, wo, so, ctypes.byref(wres),
                                      ctypes.byref(sres), n, k, None)
    return st, wres.value, sres.value


def test_an_already_rowwise_weight_passes_through_verbatim():
    # The pages' fixture pointers 0xBEEF / 0x5CA1E, n = 4096, k = 5120.
    before = qp.launch_count()
    st, w, s = _requant(qp.QP_FP8_PER_ROW, 0xBEEF, 0x5CA1E, None, None)
    assert st == qp.QP_OK and (w, s) == (0xBEEF, 0x5CA1E)
    assert qp.launch_count() == before      # no launch, no write


def test_other_formats_are_never_passed_through():
    for fmt in (qp.QP_FP8_SINGLE_SCALE, qp.QP_BF16, qp.QP_NVFP4, 7, -1):
        st, w, s = _requant(fmt, 0xBEEF, 0x5CA1E, FAKE, FAKE2)
        assert st == qp.QP_ERR_FORMAT and (w, s) == (None, None)


def test_block_format_checks_shape_before_any_launch():
    before = qp.launch_count()
    st, w, s = _requant(qp.QP_FP8_BLOCK128, FAKE, FAKE, FAKE2, FAKE2, n=4000, k=5120)
    assert st == qp.QP_ERR_SHAPE and w is None
    st, w, s = _requant(qp.QP_FP8_BLOCK128, FAKE, FAKE, None, FAKE2)
    assert st == qp.QP_ERR_NULL
    assert L.fp8_rowwise_proj(qp.QP_BF16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                              FAKE, 4, 128, 128, None) == qp.QP_ERR_FORMAT
    assert qp.launch_count() == before


def test_passthrough_needs_only_the_pair():
    st, w, s = _requant(qp.QP_FP8_PER_ROW, 0xBEEF, None, None, None)
    assert st == qp.QP_ERR_NULL


def _cache():
    h = ctypes.c_void_p()
    assert L.qproj_cache_create(ctypes.byref(h)) == qp.QP_OK
    return h


def _stats(h):
    e, b = ctypes.c_uint64(), ctypes.c_uint64()
    assert L.qproj_cache_stats(h, ctypes.byref(e), ctypes.byref(b)) == qp.QP_OK
    return e.value, b.value


def test_cache_passthrough_needs_no_work_and_no_entry():
    """dispatch_proj_rowwise.rs, cached_requant_returns_rowwise_checkpoint_
    pointers_without_gpu_work: a per-row weight comes back as itself, with no
    launch and nothing allocated or cached."""
    h = _cache()
    try:
        wq, sq = ctypes.c_void_p(), ctypes.c_void_p()
        before = qp.launch_count()
        assert L.requant_w_blockfp8_rowwise_cached(h, qp.QP_FP8_PER_ROW, FAKE, FAKE2, 128, 128,
                                                   ctypes.byref(wq), ctypes.byref(sq), None) == qp.QP_OK
        assert (wq.value, sq.value) == (FAKE, FAKE2)
        assert qp.launch_count() == before
        assert _stats(h) == (0, 0)
    finally:
        assert L.qproj_cache_destroy(h) == qp.QP_OK


def test_cache_rejects_bad_calls_before_allocating():
    h = _cache()
    try:
        wq, sq = ctypes.c_void_p(), ctypes.c_void_p()
        r = lambda fmt, w, s, n, k: L.requant_w_blockfp8_rowwise_cached(
            h, fmt, w, s, n, k, ctypes.byref(wq), ctypes.byref(sq), None)
        before = qp.launch_count()
        assert r(7, FAKE, FAKE2, 128, 128) == qp.QP_ERR_FORMAT
        assert r(qp.QP_FP8_BLOCK128, FAKE, FAKE2, 200, 128) == qp.QP_ERR_SHAPE
        assert r(qp.QP_FP8_BLOCK128, FAKE, FAKE2, 128, 0) == qp.QP_ERR_SHAPE
        assert r(qp.QP_FP8_BLOCK128, None, FAKE2, 128, 128) == qp.QP_ERR_NULL
        assert r(qp.QP_FP8_BLOCK128, FAKE + 8, FAKE2, 128, 128) == qp.QP_ERR_ALIGN
        assert L.requant_w_blockfp8_rowwise_cached(h, qp.QP_FP8_BLOCK128, FAKE, FAKE2, 128, 128,
                                                   None, ctypes.byref(sq), None) == qp.QP_ERR_NULL
        assert L.requant_w_nvfp4_int8_cached(h, FAKE, FAKE2, 1.0, 64, 48, ctypes.byref(wq),
                                             ctypes.byref(sq), None) == qp.QP_ERR_SHAPE
        # the projections check their own arguments before deriving anything
        assert L.fp8_rowwise_proj_cached(h, qp.QP_FP8_BLOCK128, FAKE, FAKE2, None, FAKE, FAKE,
                                         FAKE, 4, 128, 128, None) == qp.QP_ERR_NULL
        assert L.int8_w4a8_prefill_cached(h, FAKE, FAKE, FAKE, 1.0, FAKE, FAKE, FAKE, 4, 64, 48,
                                          None) == qp.QP_ERR_SHAPE
        assert L.qproj_cache_evict(h, FAKE) == qp.QP_OK          # nothing to evict
        assert qp.launch_count() == before
        assert _stats(h) == (0, 0)
    finally:
        assert L.qproj_cache_destroy(h) == qp.QP_OK
    assert L.qproj_cache_create(None) == qp.QP_ERR_NULL
    assert L.qproj_cache_destroy(None) == qp.QP_ERR_NULL
    assert qp.status_string(qp.QP_ERR_ALLOC) != "unknown status"


def test_w4a4_tile_order_must_be_known():
    for order in (-1, 3, 99):
        assert L.w4a4_gemm_tiles(FAKE, FAKE, FAKE, FAKE, FAKE, 1.0, 1.0, 64, 64, 64, order,
                                 None) == qp.QP_ERR_FORMAT
    assert L.w4a4_gemm_tiles(FAKE, FAKE, FAKE, FAKE, FAKE, 1.0, 1.0, 64, 64, 48,
                             qp.QP_TILES_NFAST, None) == qp.QP_ERR_SHAPE


def _pp():
    return ctypes.byref(ctypes.c_void_p())


# Every stateless entry point with fake (never dereferenced) pointers and
# sizes that pass every check; each case zeroes one extent.
_EXTENT_CALLS = {
    "requant_w_nvfp4_int8": (lambda n, k: L.requant_w_nvfp4_int8(
        FAKE, FAKE2, 1.0, FAKE, FAKE2, n, k, None), (256, 256)),
    "requant_a_bf16_int8": (lambda m, k: L.requant_a_bf16_int8(
        FAKE, FAKE2, FAKE, m, k, None), (4, 256)),
    "int8_gemm_blockscaled": (lambda m, n, k: L.int8_gemm_blockscaled(
        FAKE, FAKE2, FAKE, FAKE2, FAKE, m, n, k, None), (4, 256, 256)),
    "int8_w4a8_prefill": (lambda m, n, k: L.int8_w4a8_prefill(
        FAKE, FAKE2, FAKE, FAKE2, FAKE, FAKE2, m, n, k, None), (4, 256, 256)),
    "int8_w4a8_prefill_noalloc": (lambda m, n, k: L.int8_w4a8_prefill_noalloc(
        FAKE, FAKE2, FAKE, FAKE2, m, n, k, None), (4, 256, 256)),
    "int8_gemm_blockscaled_f16ops": (lambda m, n, k: L.int8_gemm_blockscaled_f16ops(
        FAKE, FAKE2, FAKE, FAKE2, FAKE, m, n, k, None), (4, 256, 256)),
    "int8_gemm_block_partials": (lambda m, n, k: L.int8_gemm_block_partials(
        FAKE, FAKE2, FAKE, m, n, k, None), (4, 256, 256)),
    "quantize_bf16_nvfp4": (lambda r, k: L.quantize_bf16_nvfp4(
        FAKE, FAKE2, FAKE, 1.0, r, k, None), (4, 256)),
    "w4a4_gemm": (lambda m, n, k: L.w4a4_gemm(
        FAKE, FAKE2, FAKE, FAKE2, FAKE, 1.0, 1.0, m, n, k, None), (4, 256, 256)),
    "w4a4_gemm_tiles": (lambda m, n, k: L.w4a4_gemm_tiles(
        FAKE, FAKE2, FAKE, FAKE2, FAKE, 1.0, 1.0, m, n, k, qp.QP_TILES_BANDED, None),
        (4, 256, 256)),
    "requant_w_blockfp8_rowwise": (lambda n, k: L.requant_w_blockfp8_rowwise(
        qp.QP_FP8_BLOCK128, FAKE, FAKE2, FAKE, FAKE2, _pp(), _pp(), n, k, None), (256, 256)),
    "quant_rowwise_fp8": (lambda r, k: L.quant_rowwise_fp8(
        FAKE, FAKE2, FAKE, r, k, None), (4, 256)),
    "fp8_gemm_rowscale": (lambda m, n, k: L.fp8_gemm_rowscale(
        FAKE, FAKE2, FAKE, FAKE2, FAKE, m, n, k, None), (4, 256, 256)),
    "fp8_rowwise_proj": (lambda m, n, k: L.fp8_rowwise_proj(
        qp.QP_FP8_PER_ROW, FAKE, FAKE2, FAKE, FAKE2, FAKE, FAKE2, FAKE, FAKE2, m, n, k, None),
        (4, 256, 256)),
    "fp8_gemv_rowscale": (lambda m, n, k: L.fp8_gemv_rowscale(
        FAKE, FAKE2, FAKE, FAKE2, m, n, k, None), (4, 256, 256)),
    "fp8_gemv_blockscale": (lambda m, n, k: L.fp8_gemv_blockscale(
        FAKE, FAKE2, FAKE, FAKE2, m, n, k, None), (4, 256, 256)),
    "w4a16_gemv": (lambda m, n, k: L.w4a16_gemv(
        FAKE, FAKE2, FAKE, 1.0, FAKE2, m, n, k, None), (4, 256, 256)),
}


@pytest.mark.parametrize("name", sorted(_EXTENT_CALLS))
def test_empty_extent_is_rejected_before_any_launch(name):
    """A zero M, N, K or row count is an error (QP_ERR_SHAPE, or QP_ERR_RANGE
    where M has a documented range), returned by the host checks: the
    launch counter does not move."""
    call, sizes = _EXTENT_CALLS[name]
    for i in range(len(sizes)):
        args = list(sizes)
        args[i] = 0
        before = qp.launch_count()
        st = call(*args)
        assert st in (qp.QP_ERR_SHAPE, qp.QP_ERR_RANGE), (name, args, st)
        assert qp.launch_count() == before


def test_every_stateless_entry_point_is_in_the_extent_table():
    stateless = [n for n in _declared_functions()
                 if not n.startswith("qproj_") and not n.endswith("_cached")]
    assert sorted(stateless) == sorted(_EXTENT_CALLS)


def test_empty_extent_is_rejected_by_the_cached_entry_points():
    h = ctypes.c_void_p()
    assert L.qproj_cache_create(ctypes.byref(h)) == qp.QP_OK
    try:
        calls = [
            (lambda n, k: L.requant_w_blockfp8_rowwise_cached(
                h, qp.QP_FP8_BLOCK128, FAKE, FAKE2, n, k, _pp(), _pp(), None), (256, 256)),
            (lambda n, k: L.requant_w_nvfp4_int8_cached(
                h, FAKE, FAKE2, 1.0, n, k, _pp(), _pp(), None), (256, 256)),
            (lambda m, n, k: L.fp8_rowwise_proj_cached(
                h, qp.QP_FP8_BLOCK128, FAKE, FAKE2, FAKE, FAKE2, FAKE, FAKE2, m, n, k, None),
             (4, 256, 256)),
            (lambda m, n, k: L.int8_w4a8_prefill_cached(
                h, FAKE, FAKE2, FAKE, 1.0, FAKE2, FAKE, FAKE2, m, n, k, None), (4, 256, 256)),
        ]
        for call, sizes in calls:
            for i in range(len(sizes)):
                args = list(sizes)
                args[i] = 0
                before = qp.launch_count()
                assert call(*args) == qp.QP_ERR_SHAPE, args
                assert qp.launch_count() == before
        e, b = ctypes.c_uint64(), ctypes.c_uint64()
        assert L.qproj_cache_stats(h, ctypes.byref(e), ctypes.byref(b)) == qp.QP_OK
        assert (e.value, b.value) == (0, 0)       # nothing derived, nothing allocated
    finally:
        assert L.qproj_cache_destroy(h) == qp.QP_OK


def test_gemv_activation_bytes_limit():
    # 2*m*k must stay below 2^31 (31-bit activation offsets); n*k stays legal
    for fn in (L.fp8_gemv_rowscale, L.fp8_gemv_blockscale):
        assert fn(FAKE, FAKE2, FAKE, FAKE2, 16, 128, 1 << 26, None) == qp.QP_ERR_SHAPE
        assert fn(FAKE, FAKE2, FAKE, FAKE2, 8, 128, 1 << 27, None) == qp.QP_ERR_SHAPE


# Every device pointer of every stateless entry point, by position: call(p)
# takes the list of pointer values.  Block formats are used where a format
# tag decides which pointers are read.
_PTR_CALLS = {
    "requant_w_nvfp4_int8": (lambda p: L.requant_w_nvfp4_int8(
        p[0], p[1], 1.0, p[2], p[3], 256, 256, None), 4),
    "requant_a_bf16_int8": (lambda p: L.requant_a_bf16_int8(p[0], p[1], p[2], 4, 256, None), 3),
    "int8_gemm_blockscaled": (lambda p: L.int8_gemm_blockscaled(
        p[0], p[1], p[2], p[3], p[4], 4, 256, 256, None), 5),
    "int8_w4a8_prefill": (lambda p: L.int8_w4a8_prefill(
        p[0], p[1], p[2], p[3], p[4], p[5], 4, 256, 256, None), 6),
    "int8_w4a8_prefill_noalloc": (lambda p: L.int8_w4a8_prefill_noalloc(
        p[0], p[1], p[2], p[3], 4, 256, 256, None), 4),
    "int8_gemm_blockscaled_f16ops": (lambda p: L.int8_gemm_blockscaled_f16ops(
        p[0], p[1], p[2], p[3], p[4], 4, 256, 256, None), 5),
    "int8_gemm_block_partials": (lambda p: L.int8_gemm_block_partials(
        p[0], p[1], p[2], 4, 256, 256, None), 3),
    "quantize_bf16_nvfp4": (lambda p: L.quantize_bf16_nvfp4(p[0], p[1], p[2], 1.0, 4, 256, None), 3),
    "w4a4_gemm": (lambda p: L.w4a4_gemm(p[0], p[1], p[2], p[3], p[4], 1.0, 1.0, 4, 256, 256, None), 5),
    "w4a4_gemm_tiles": (lambda p: L.w4a4_gemm_tiles(
        p[0], p[1], p[2], p[3], p[4], 1.0, 1.0, 4, 256, 256, qp.QP_TILES_BANDED, None), 5),
    "requant_w_blockfp8_rowwise": (lambda p: L.requant_w_blockfp8_rowwise(
        qp.QP_FP8_BLOCK128, p[0], p[1], p[2], p[3], _pp(), _pp(), 256, 256, None), 4),
    "quant_rowwise_fp8": (lambda p: L.quant_rowwise_fp8(p[0], p[1], p[2], 4, 256, None), 3),
    "fp8_gemm_rowscale": (lambda p: L.fp8_gemm_rowscale(p[0], p[1], p[2], p[3], p[4], 4, 256, 256, None), 5),
    "fp8_rowwise_proj": (lambda p: L.fp8_rowwise_proj(
        qp.QP_FP8_BLOCK128, p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], 4, 256, 256, None), 8),
    "fp8_gemv_rowscale": (lambda p: L.fp8_gemv_rowscale(p[0], p[1], p[2], p[3], 4, 256, 256, None), 4),
    "fp8_gemv_blockscale": (lambda p: L.fp8_gemv_blockscale(p[0], p[1], p[2], p[3], 4, 256, 256, None), 4),
    "w4a16_gemv": (lambda p: L.w4a16_gemv(p[0], p[1], p[2], 1.0, p[3], 4, 256, 256, None), 4),
}


def test_every_stateless_entry_point_is_in_the_pointer_table():
    assert sorted(_PTR_CALLS) == sorted(_EXTENT_CALLS)


@pytest.mark.parametrize("name", sorted(_PTR_CALLS))
def test_every_pointer_is_checked_before_any_launch(name):
    """Each device pointer, in turn, null and then one byte off its
    alignment: QP_ERR_NULL and QP_ERR_ALIGN from the host checks, with the
    other pointers valid and nothing launched."""
    call, count = _PTR_CALLS[name]
    for i in range(count):
        for bad, want in ((0, qp.QP_ERR_NULL), (1, qp.QP_ERR_ALIGN)):
            p = [FAKE if j % 2 == 0 else FAKE2 for j in range(count)]
            p[i] = bad if bad == 0 else p[i] + bad
            before = qp.launch_count()
            st = call(p)
            assert st == want, (name, i, bad, st)
            assert qp.launch_count() == before


def test_noalloc_prefill_refuses_problems_beyond_its_scratch_array():
    """The no-allocation prefill keeps its activation scratch (int8 codes,
    then 256-byte aligned F32 scales) in a fixed array; a problem that needs
    more is refused on the host with QP_ERR_SCRATCH, launching nothing."""
    cap = qp.noalloc_scratch_bytes()
    assert cap == 24 << 20

    def need(m, k):
        return (m * k + 255) // 256 * 256 + 4 * m * (k // 32)

    k = 5120
    m_fit = max(m for m in range(1, 8192) if need(m, k) <= cap)
    before = qp.launch_count()
    assert L.int8_w4a8_prefill_noalloc(FAKE, FAKE2, FAKE, FAKE2, m_fit + 1, 128, k, None) \
        == qp.QP_ERR_SCRATCH
    assert L.int8_w4a8_prefill_noalloc(FAKE, FAKE2, FAKE, FAKE2, 1, 1, 32 * 800000, None) \
        == qp.QP_ERR_SCRATCH
    assert qp.launch_count() == before
    assert qp.status_string(qp.QP_ERR_SCRATCH) != "unknown status"


def test_f16_operand_route_needs_k_multiple_of_128():
    before = qp.launch_count()
    for k in (32, 64, 96, 160, 192):
        assert L.int8_gemm_blockscaled_f16ops(FAKE, FAKE2, FAKE, FAKE2, FAKE, 256, 128, k,
                                              None) == qp.QP_ERR_SHAPE
    assert qp.launch_count() == before
