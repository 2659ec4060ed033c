// qp_launch.hpp -- host-side launchers of the gfx950 kernels.  Arguments are
// assumed validated by the C ABI layer (capi.hip); each launcher enqueues its
// kernel(s) on `st` and returns the HIP launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qp {

hipError_t launch_requant_a_bf16_int8(const uint16_t *a, int8_t *q, float *s,
                                      uint32_t m, uint32_t k, hipStream_t st);
hipError_t launch_requant_w_nvfp4_int8(const uint8_t *packed, const uint8_t *sc16,
                                       float scale2, int8_t *q, float *s,
                                       uint32_t n, uint32_t k, hipStream_t st);
hipError_t launch_quantize_bf16_nvfp4(const uint16_t *x, uint8_t *packed,
                                      uint8_t *sc16, float scale2, uint32_t rows,
                                      uint32_t k, hipStream_t st);
hipError_t launch_quant_rowwise_fp8(const uint16_t *x, uint8_t *q, float *s,
                                    uint32_t rows, uint32_t k, hipStream_t st);
hipError_t launch_requant_blockfp8_rowwise(const uint8_t *w, const float *grid,
                                           uint8_t *q, float *s, uint32_t n,
                                           uint32_t k, hipStream_t st);
hipError_t launch_fp8_gemv_rowscale(const uint16_t *x, const uint8_t *w,
                                    const float *rs, uint16_t *out, uint32_t m,
                                    uint32_t n, uint32_t k, hipStream_t st);
hipError_t launch_fp8_gemv_blockscale(const uint16_t *x, const uint8_t *w,
                                      const float *grid, uint16_t *out, uint32_t m,
                                      uint32_t n, uint32_t k, hipStream_t st);
hipError_t launch_w4a16_gemv(const uint16_t *x, const uint8_t *wp, const uint8_t *ws,
                             float scale2, uint16_t *out, uint32_t m, uint32_t n,
                             uint32_t k, hipStream_t st);
hipError_t launch_int8_gemm(const int8_t *a, const int8_t *w, const float *as,
                            const float *ws, uint16_t *out, int32_t *partials,
                            uint32_t m, uint32_t n, uint32_t k, hipStream_t st);
// The operand-route ablation: the same GEMM on FP16 MFMA (k % 128 == 0).
hipError_t launch_int8_gemm_f16ops(const int8_t *a, const int8_t *w, const float *as,
                                   const float *ws, uint16_t *out, uint32_t m, uint32_t n,
                                   uint32_t k, hipStream_t st);
hipError_t launch_fp8_gemm_rowscale(const uint8_t *a, const float *as,
                                    const uint8_t *w, const float *ws,
                                    uint16_t *out, uint32_t m, uint32_t n,
                                    uint32_t k, hipStream_t st);
// order: the workgroup -> tile mapping (0 banded XCD-aware, 1 M-fast,
// 2 N-fast; see tile_coords_order).
hipError_t launch_w4a4_gemm(const uint8_t *ap, const uint8_t *asc,
                            const uint8_t *wp, const uint8_t *wsc, uint16_t *out,
                            float sa2, float sw2, uint32_t m, uint32_t n,
                            uint32_t k, uint32_t order, hipStream_t st);

// Counts kernel launches enqueued by the library (all launchers add to it).
void count_launch(uint32_t n = 1);

// Compute units of the current device, queried once per device; 0 if the
// query fails (launch shapes that depend on it then take a fixed default).
uint32_t cu_count();

} // namespace qp
