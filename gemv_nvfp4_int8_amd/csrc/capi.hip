// capi.hip -- the extern "C" boundary of libqproj (declared in include/qproj.h).
//
// Every entry point validates its arguments on the host first (null
// pointers, alignment, sizes, divisibility, ranges, format tags) and returns
// a negative QP_ERR_* code before touching the HIP runtime, so a bad call
// never enqueues anything.  Valid calls enqueue their kernel(s) on the
// caller's stream and return; nothing here allocates or synchronises.
#include <atomic>

#include "qp_launch.hpp"
#include "../../include/qproj.h"

namespace qp {
static std::atomic<uint64_t> g_launches{0};
void count_launch(uint32_t n) { g_launches.fetch_add(n, std::memory_order_relaxed); }

uint32_t cu_count()
{
    constexpr int MAXDEV = 64;
    static std::atomic<uint32_t> cached[MAXDEV] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAXDEV)
        return 0;
    uint32_t c = cached[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
            return 0;
        c = (uint32_t)v;
        cached[dev].store(c, std::memory_order_relaxed);
    }
    return c;
}
} // namespace qp

namespace {

constexpr uint64_t MAX_ELEMS = (1ull << 31) - 1;   // every tensor < 2^31 elements

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int check_ptrs(std::initializer_list<const void *> ps)
{
    for (const void *p : ps)
        if (!p)
            return QP_ERR_NULL;
    for (const void *p : ps)
        if (!aligned16(p))
            return QP_ERR_ALIGN;
    return QP_OK;
}

inline bool fits(uint64_t rows, uint64_t cols) { return rows * cols <= MAX_ELEMS; }

inline int done(hipError_t e) { return e == hipSuccess ? QP_OK : QP_ERR_HIP; }

inline hipStream_t S(void *s) { return reinterpret_cast<hipStream_t>(s); }

} // namespace

extern "C" {

int qproj_abi_version(void) { return QPROJ_ABI_VERSION; }

uint64_t qproj_launch_count(void) { return qp::g_launches.load(); }

const char *qproj_status_string(int status)
{
    switch (status) {
    case QP_OK: return "ok";
    case QP_ERR_NULL: return "a required pointer is NULL";
    case QP_ERR_SHAPE: return "a size is zero, too large, or not a required multiple";
    case QP_ERR_RANGE: return "GEMV row count M outside the entry point's range";
    case QP_ERR_FORMAT: return "unsupported weight format tag";
    case QP_ERR_HIP: return "the HIP runtime rejected a kernel launch";
    case QP_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case QP_ERR_ALLOC: return "device memory for a derived weight could not be allocated";
    case QP_ERR_SCRATCH: return "the problem needs more than the fixed scratch array of the no-allocation entry point";
    default: return "unknown status";
    }
}

int requant_w_nvfp4_int8(const uint8_t *w_packed, const uint8_t *w_e4m3,
                         float scale2, int8_t *w_i8, float *w_scale,
                         uint32_t n, uint32_t k, void *stream)
{
    if (int e = check_ptrs({w_packed, w_e4m3, w_i8, w_scale}))
        return e;
    if (n == 0 || k == 0 || k % 32 != 0 || !fits(n, k))
        return QP_ERR_SHAPE;
    return done(qp::launch_requant_w_nvfp4_int8(w_packed, w_e4m3, scale2, w_i8,
                                                w_scale, n, k, S(stream)));
}

int requant_a_bf16_int8(const uint16_t *a, int8_t *a_i8, float *a_scale,
                        uint32_t m, uint32_t k, void *stream)
{
    if (int e = check_ptrs({a, a_i8, a_scale}))
        return e;
    if (m == 0 || k == 0 || k % 32 != 0 || !fits(m, k))
        return QP_ERR_SHAPE;
    return done(qp::launch_requant_a_bf16_int8(a, a_i8, a_scale, m, k, S(stream)));
}

int int8_gemm_blockscaled(const int8_t *a_i8, const int8_t *w_i8,
                          const float *a_scale, const float *w_scale,
                          uint16_t *out, uint32_t m, uint32_t n, uint32_t k,
                          void *stream)
{
    if (int e = check_ptrs({a_i8, w_i8, a_scale, w_scale, out}))
        return e;
    if (m == 0 || n == 0 || k == 0 || k % 32 != 0 || !fits(m, k) ||
        !fits(n, k) || !fits(m, n))
        return QP_ERR_SHAPE;
    return done(qp::launch_int8_gemm(a_i8, w_i8, a_scale, w_scale, out, nullptr,
                                     m, n, k, S(stream)));
}

int int8_w4a8_prefill(const uint16_t *a_bf16, const int8_t *w_i8,
                      const float *w_scale, int8_t *a_i8_scratch,
                      float *a_scale_scratch, uint16_t *out,
                      uint32_t m, uint32_t n, uint32_t k, void *stream)
{
    if (int e = check_ptrs({a_bf16, w_i8, w_scale, a_i8_scratch, a_scale_scratch, out}))
        return e;
    if (m == 0 || n == 0 || k == 0 || k % 32 != 0 || !fits(m, k) ||
        !fits(n, k) || !fits(m, n))
        return QP_ERR_SHAPE;
    if (int e = done(qp::launch_requant_a_bf16_int8(a_bf16, a_i8_scratch,
                                                    a_scale_scratch, m, k, S(stream))))
        return e;
    return done(qp::launch_int8_gemm(a_i8_scratch, w_i8, a_scale_scratch, w_scale,
                                     out, nullptr, m, n, k, S(stream)));
}

int int8_gemm_blockscaled_f16ops(const int8_t *a_i8, const int8_t *w_i8,
                                 const float *a_scale, const float *w_scale,
                                 uint16_t *out, uint32_t m, uint32_t n, uint32_t k,
                                 void *stream)
{
    if (int e = check_ptrs({a_i8, w_i8, a_scale, w_scale, out}))
        return e;
    if (m == 0 || n == 0 || k == 0 || k % 128 != 0 || !fits(m, k) || !fits(n, k) ||
        !fits(m, n))
        return QP_ERR_SHAPE;
    return done(qp::launch_int8_gemm_f16ops(a_i8, w_i8, a_scale, w_scale, out, m, n, k,
                                            S(stream)));
}

int int8_gemm_block_partials(const int8_t *a_i8, const int8_t *w_i8, int32_t *p,
                             uint32_t m, uint32_t n, uint32_t k, void *stream)
{
    if (int e = check_ptrs({a_i8, w_i8, p}))
        return e;
    if (m == 0 || n == 0 || k == 0 || k % 32 != 0 || !fits(m, k) ||
        !fits(n, k) || !fits((uint64_t)m * n, k / 32))
        return QP_ERR_SHAPE;
    return done(qp::launch_int8_gemm(a_i8, w_i8, nullptr, nullptr, nullptr, p,
                                     m, n, k, S(stream)));
}

int quantize_bf16_nvfp4(const uint16_t *x, uint8_t *packed, uint8_t *scale,
                        float scale2, uint32_t rows, uint32_t k, void *stream)
{
    if (!x || !packed || !scale)
        return QP_ERR_NULL;
    // the scale grid has k/16 bytes per row; it needs 2-byte alignment only
    if (!aligned16(x) || !aligned16(packed) || (reinterpret_cast<uintptr_t>(scale) & 1u))
        return QP_ERR_ALIGN;
    if (rows == 0 || k == 0 || k % 32 != 0 || !fits(rows, k))
        return QP_ERR_SHAPE;
    return done(qp::launch_quantize_bf16_nvfp4(x, packed, scale, scale2, rows, k,
                                               S(stream)));
}

int w4a4_gemm(const uint8_t *a_packed, const uint8_t *a_scale,
              const uint8_t *w_packed, const uint8_t *w_scale, uint16_t *out,
              float scale_a2, float scale_w2, uint32_t m, uint32_t n,
              uint32_t k, void *stream)
{
    return w4a4_gemm_tiles(a_packed, a_scale, w_packed, w_scale, out, scale_a2, scale_w2,
                           m, n, k, QP_TILES_BANDED, stream);
}

int w4a4_gemm_tiles(const uint8_t *a_packed, const uint8_t *a_scale,
                    const uint8_t *w_packed, const uint8_t *w_scale, uint16_t *out,
                    float scale_a2, float scale_w2, uint32_t m, uint32_t n,
                    uint32_t k, int tile_order, void *stream)
{
    if (tile_order != QP_TILES_BANDED && tile_order != QP_TILES_MFAST &&
        tile_order != QP_TILES_NFAST)
        return QP_ERR_FORMAT;
    if (!a_packed || !a_scale || !w_packed || !w_scale || !out)
        return QP_ERR_NULL;
    // the large-tile kernel stages scale rows with 16-byte loads, so the
    // scale grids need the same alignment as every other pointer
    if (!aligned16(a_packed) || !aligned16(w_packed) || !aligned16(out) ||
        !aligned16(a_scale) || !aligned16(w_scale))
        return QP_ERR_ALIGN;
    if (m == 0 || n == 0 || k == 0 || k % 32 != 0 || !fits(m, k) ||
        !fits(n, k) || !fits(m, n))
        return QP_ERR_SHAPE;
    return done(qp::launch_w4a4_gemm(a_packed, a_scale, w_packed, w_scale, out,
                                     scale_a2, scale_w2, m, n, k, (uint32_t)tile_order,
                                     S(stream)));
}

int requant_w_blockfp8_rowwise(int fmt, const uint8_t *w, const float *scale,
                               uint8_t *w_out, float *scale_out,
                               const uint8_t **w_res, const float **scale_res,
                               uint32_t n, uint32_t k, void *stream)
{
    if (fmt == QP_FP8_PER_ROW) {
        // Already the row-wise pair: hand back the caller's own pointers.
        if (!w || !scale)
            return QP_ERR_NULL;
        if (w_res)
            *w_res = w;
        if (scale_res)
            *scale_res = scale;
        return QP_OK;
    }
    if (fmt != QP_FP8_BLOCK128)
        return QP_ERR_FORMAT;
    if (int e = check_ptrs({w, scale, w_out, scale_out}))
        return e;
    if (n == 0 || k == 0 || n % 128 != 0 || k % 128 != 0 || !fits(n, k))
        return QP_ERR_SHAPE;
    int e = done(qp::launch_requant_blockfp8_rowwise(w, scale, w_out, scale_out,
                                                     n, k, S(stream)));
    if (e == QP_OK) {
        if (w_res)
            *w_res = w_out;
        if (scale_res)
            *scale_res = scale_out;
    }
    return e;
}

int quant_rowwise_fp8(const uint16_t *x, uint8_t *q, float *scale,
                      uint32_t rows, uint32_t k, void *stream)
{
    if (int e = check_ptrs({x, q, scale}))
        return e;
    if (rows == 0 || k == 0 || k % 16 != 0 || !fits(rows, k))
        return QP_ERR_SHAPE;
    return done(qp::launch_quant_rowwise_fp8(x, q, scale, rows, k, S(stream)));
}

int fp8_gemm_rowscale(const uint8_t *a, const float *a_scale, const uint8_t *w,
                      const float *w_scale, uint16_t *out, uint32_t m,
                      uint32_t n, uint32_t k, void *stream)
{
    if (int e = check_ptrs({a, a_scale, w, w_scale, out}))
        return e;
    if (m == 0 || n == 0 || k == 0 || k % 16 != 0 || !fits(m, k) ||
        !fits(n, k) || !fits(m, n))
        return QP_ERR_SHAPE;
    return done(qp::launch_fp8_gemm_rowscale(a, a_scale, w, w_scale, out, m, n, k,
                                             S(stream)));
}

int fp8_rowwise_proj(int fmt, const uint8_t *w, const float *w_scale,
                     uint8_t *w_rowwise, float *w_rowwise_scale,
                     const uint16_t *act, uint8_t *act_q, float *act_scale,
                     uint16_t *out, uint32_t m, uint32_t n, uint32_t k,
                     void *stream)
{
    if (fmt != QP_FP8_PER_ROW && fmt != QP_FP8_BLOCK128)
        return QP_ERR_FORMAT;
    if (int e = check_ptrs({w, w_scale, act, act_q, act_scale, out}))
        return e;
    if (m == 0 || n == 0 || k == 0 || k % 16 != 0 || !fits(m, k) ||
        !fits(n, k) || !fits(m, n))
        return QP_ERR_SHAPE;
    if (fmt == QP_FP8_BLOCK128) {
        if (int e = check_ptrs({w_rowwise, w_rowwise_scale}))
            return e;
        if (n % 128 != 0 || k % 128 != 0)
            return QP_ERR_SHAPE;
    }
    const uint8_t *wq = nullptr;
    const float *ws = nullptr;
    if (int e = requant_w_blockfp8_rowwise(fmt, w, w_scale, w_rowwise, w_rowwise_scale,
                                           &wq, &ws, n, k, stream))
        return e;
    if (int e = done(qp::launch_quant_rowwise_fp8(act, act_q, act_scale, m, k, S(stream))))
        return e;
    return done(qp::launch_fp8_gemm_rowscale(act_q, act_scale, wq, ws, out, m, n, k,
                                             S(stream)));
}

int fp8_gemv_rowscale(const uint16_t *x, const uint8_t *w,
                      const float *row_scale, uint16_t *out, uint32_t m,
                      uint32_t n, uint32_t k, void *stream)
{
    if (int e = check_ptrs({x, w, row_scale, out}))
        return e;
    if (m < 1 || m > 16)
        return QP_ERR_RANGE;
    // (the K-split kernel addresses the activations with 31-bit byte offsets)
    if (n == 0 || k == 0 || k % 16 != 0 || !fits(n, k) || !fits(m, n) ||
        (uint64_t)2 * m * k >= (1ull << 31))
        return QP_ERR_SHAPE;
    return done(qp::launch_fp8_gemv_rowscale(x, w, row_scale, out, m, n, k, S(stream)));
}

int fp8_gemv_blockscale(const uint16_t *x, const uint8_t *w,
                        const float *block_scale, uint16_t *out, uint32_t m,
                        uint32_t n, uint32_t k, void *stream)
{
    if (int e = check_ptrs({x, w, block_scale, out}))
        return e;
    if (m < 1 || m > 16)
        return QP_ERR_RANGE;
    if (n == 0 || k == 0 || n % 128 != 0 || k % 128 != 0 || !fits(n, k) || !fits(m, n) ||
        (uint64_t)2 * m * k >= (1ull << 31))
        return QP_ERR_SHAPE;
    return done(qp::launch_fp8_gemv_blockscale(x, w, block_scale, out, m, n, k, S(stream)));
}

int w4a16_gemv(const uint16_t *x, const uint8_t *w_packed, const uint8_t *w_e4m3,
               float scale2, uint16_t *out, uint32_t m, uint32_t n, uint32_t k,
               void *stream)
{
    if (int e = check_ptrs({x, w_packed, w_e4m3, out}))
        return e;
    if (m < 1 || m > 8)
        return QP_ERR_RANGE;
    // (the kernel addresses every buffer with 30-bit offsets)
    if (n == 0 || k == 0 || k % 32 != 0 || !fits(n, k) || !fits(m, n) ||
        (uint64_t)m * k * 2 >= (1u << 30))
        return QP_ERR_SHAPE;
    return done(qp::launch_w4a16_gemv(x, w_packed, w_e4m3, scale2, out, m, n, k, S(stream)));
}

} // extern "C"
