// noalloc.hip -- the W4A8 prefill call for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// int8_w4a8_prefill takes its activation scratch (int8 codes and per-32
// scales) from the caller.  This variant keeps that scratch in a file-scope
// device array instead, of a fixed size, so the caller passes only inputs
// and outputs.  Each GPU the library runs on holds its own copy of the array
// until the process ends.  In host code the array's name is not a device
// address: its address on each device is looked up once, with that device
// current, and only that looked-up pointer is handed to kernels.
//
// Every call on one GPU uses that GPU's one array, so calls that overlap on
// one GPU (two streams, two threads) race on it; the caller must order them.
// Nothing in the array needs to start at zero: the activation requant writes
// every byte the GEMM then reads.
#include <mutex>

#include "qp_launch.hpp"
#include "../../include/qproj.h"

namespace {

static __device__ __align__(256) uint8_t scratch[QP_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::once_flag g_once[MAX_DEVICES];
void *g_ptr[MAX_DEVICES];
hipError_t g_err[MAX_DEVICES];

// The array's device address on the current device (looked up once per
// device), or nullptr with the HIP error in *err.
void *scratch_ptr(hipError_t *err)
{
    int dev = -1;
    if ((*err = hipGetDevice(&dev)) != hipSuccess)
        return nullptr;
    if (dev < 0 || dev >= MAX_DEVICES) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::call_once(g_once[dev], [dev] {
        void *p = nullptr;
        g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
    });
    *err = g_err[dev];
    return g_ptr[dev];
}

constexpr uint64_t align256(uint64_t b) { return (b + 255u) & ~uint64_t(255u); }

} // namespace

extern "C" {

uint64_t qproj_noalloc_scratch_bytes(void) { return QP_NOALLOC_SCRATCH_BYTES; }

int int8_w4a8_prefill_noalloc(const uint16_t *a_bf16, const int8_t *w_i8,
                              const float *w_scale, uint16_t *out,
                              uint32_t m, uint32_t n, uint32_t k, void *stream)
{
    for (const void *p : {(const void *)a_bf16, (const void *)w_i8, (const void *)w_scale,
                          (const void *)out})
        if (!p)
            return QP_ERR_NULL;
    for (const void *p : {(const void *)a_bf16, (const void *)w_i8, (const void *)w_scale,
                          (const void *)out})
        if (reinterpret_cast<uintptr_t>(p) & 15u)
            return QP_ERR_ALIGN;
    constexpr uint64_t MAX_ELEMS = (1ull << 31) - 1;
    if (m == 0 || n == 0 || k == 0 || k % 32 != 0 || (uint64_t)m * k > MAX_ELEMS ||
        (uint64_t)n * k > MAX_ELEMS || (uint64_t)m * n > MAX_ELEMS)
        return QP_ERR_SHAPE;
    // int8 codes [m, k], then (256-byte aligned) F32 scales [m, k/32]
    const uint64_t codes = (uint64_t)m * k;
    const uint64_t need = align256(codes) + 4ull * m * (k / 32);
    if (need > QP_NOALLOC_SCRATCH_BYTES)
        return QP_ERR_SCRATCH;

    hipError_t e;
    uint8_t *base = static_cast<uint8_t *>(scratch_ptr(&e));
    if (!base)
        return QP_ERR_HIP;
    int8_t *a_i8 = reinterpret_cast<int8_t *>(base);
    float *a_scale = reinterpret_cast<float *>(base + align256(codes));
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (qp::launch_requant_a_bf16_int8(a_bf16, a_i8, a_scale, m, k, st) != hipSuccess)
        return QP_ERR_HIP;
    if (qp::launch_int8_gemm(a_i8, w_i8, a_scale, w_scale, out, nullptr, m, n, k, st) !=
        hipSuccess)
        return QP_ERR_HIP;
    return QP_OK;
}

} // extern "C"
