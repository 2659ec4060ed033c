// codec_test.hip -- test export: the device encoders the quantizer kernels
// use, applied to arbitrary binary32 values, so that a test can compare them
// with reference encoders on any input it builds (the kernels themselves
// only ever see quotients x/s of their inputs).
#include "qp_device.hpp"
#include "qp_launch.hpp"
#include "../../include/qproj.h"

namespace qp {

// One thread encodes 8 consecutive values; one code per output byte
// (E2M1 codes in the low nibble, int8 codes as two's-complement bytes).
__global__ __launch_bounds__(256) void k_encode_test(int kind, const float *__restrict__ y,
                                                     uint8_t *__restrict__ out, uint32_t n8)
{
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;
    if (i >= n8)
        return;
    const f32x4 a = *reinterpret_cast<const f32x4 *>(y + 8 * (size_t)i);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(y + 8 * (size_t)i + 4);
    const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    u32x2 o = {0, 0};
    if (kind == QP_ENC_E4M3_NOSAT || kind == QP_ENC_E4M3) {
        const bool nosat = kind == QP_ENC_E4M3_NOSAT;
        o[0] = nosat ? cvt_e4m3x4_nosat(v[0], v[1], v[2], v[3]) : cvt_e4m3x4(v[0], v[1], v[2], v[3]);
        o[1] = nosat ? cvt_e4m3x4_nosat(v[4], v[5], v[6], v[7]) : cvt_e4m3x4(v[4], v[5], v[6], v[7]);
    } else if (kind == QP_ENC_E2M1_NOSAT || kind == QP_ENC_E2M1) {
        const uint32_t c = kind == QP_ENC_E2M1_NOSAT ? cvt_e2m1x8_nosat(v) : cvt_e2m1x8(v);
        // spread the eight nibbles over eight bytes
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            lo |= ((c >> (4 * j)) & 15u) << (8 * j);
            hi |= ((c >> (16 + 4 * j)) & 15u) << (8 * j);
        }
        o = (u32x2){lo, hi};
    } else if (kind == QP_ENC_INT8) {
        o = (u32x2){pack_i8x4(&v[0]), pack_i8x4(&v[4])};
    } else {                             // QP_ENC_E4M3_SCALE
        uint32_t w[2] = {0, 0};
#pragma unroll
        for (int j = 0; j < 8; ++j)
            w[j / 4] |= enc_e4m3_scale(v[j]) << (8 * (j % 4));
        o = (u32x2){w[0], w[1]};
    }
    *reinterpret_cast<u32x2 *>(out + 8 * (size_t)i) = o;
}

} // namespace qp

extern "C" int qproj_encode_test(int kind, const float *y, uint8_t *out, uint32_t n,
                                 void *stream)
{
    if (!y || !out)
        return QP_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(y) | reinterpret_cast<uintptr_t>(out)) & 15u)
        return QP_ERR_ALIGN;
    if (kind < QP_ENC_E4M3_NOSAT || kind > QP_ENC_E4M3_SCALE)
        return QP_ERR_FORMAT;
    if (n == 0 || n % 8 != 0 || n > (1u << 30))
        return QP_ERR_SHAPE;
    const uint32_t n8 = n / 8;
    hipLaunchKernelGGL(qp::k_encode_test, dim3((n8 + 255) / 256), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), kind, y, out, n8);
    qp::count_launch();
    return hipGetLastError() == hipSuccess ? QP_OK : QP_ERR_HIP;
}
