// gemv_fp8.hip -- row-scaled FP8 GEMV for decode / verify batches (M <= 16)
// on gfx950 (fp8_gemv_batch.rs: fp8_gemv_rowscale_batch8_rt2 /
// _batch16_rt2 / dense_gemv_fp8w_batch2).
//
//   C[i,j] = bf16( row_scale[j] * sum_t x[i,t] * e4m3(w[j,t]) )
//
// Design (MI355X-first):
//  * The contraction runs on MFMA, not on the vector ALU: at 8 TB/s an M=16
//    GEMV needs ~250 TFLOP/s, beyond the FP32 vector peak.  The E4M3 weight
//    converts exactly to BF16 (v_cvt_scalef32_pk_bf16_fp8, scale 1.0), the
//    activations already are BF16, and v_mfma_f32_16x16x32_bf16 forms exact
//    products with F32 accumulation.  The activation rows are the MFMA's 16
//    M-rows; rows >= M are zero and cost nothing in memory.
//  * Each weight byte is loaded once, with 16-byte loads straight into the
//    MFMA B-operand registers (no LDS for the weight).  A K-range that a
//    lane owns is the same in the A and B operands, so the MFMA's K order is
//    free to follow memory order.
//  * One 256-thread workgroup owns 16*T weight rows; its four waves split K
//    into interleaved 64-element steps and their partial tiles are added in
//    a fixed order through LDS.  Nothing in the reduction depends on M, so
//    every output row is bit-identical to an M = 1 call on that row.
#include "qp_device.hpp"
#include "qp_launch.hpp"

namespace qp {

// 16 E4M3 codes (one 16-byte load) -> two 8-wide BF16 MFMA operands.
__device__ __forceinline__ void fp8x16_to_bf16(u32x4 w, bf16x8 &lo, bf16x8 &hi)
{
    bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, false);
    bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, true);
    bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, false);
    bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, true);
    bf16x2 p4 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2], 1.0f, false);
    bf16x2 p5 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2], 1.0f, true);
    bf16x2 p6 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[3], 1.0f, false);
    bf16x2 p7 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[3], 1.0f, true);
    lo = (bf16x8){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    hi = (bf16x8){p4[0], p4[1], p5[0], p5[1], p6[0], p6[1], p7[0], p7[1]};
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v)
{
    return __builtin_bit_cast(bf16x8, v);
}

constexpr int GEMV_WAVES = 4;      // K-split ways inside a workgroup
constexpr int GEMV_STEP = 64;      // K elements per wave step (4 lanes x 16)
constexpr int GEMV_UNROLL = 4;     // steps in flight per wave

template <int T>
__global__ __launch_bounds__(256) void k_fp8_gemv_rowscale(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ w,
    const float *__restrict__ rs, uint16_t *__restrict__ out,
    uint32_t m, uint32_t n, uint32_t k)
{
    __shared__ f32x4 red[GEMV_WAVES - 1][T][WAVE];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int col = lane & 15;     // MFMA row of A (activation) and column of B (weight row)
    const int grp = lane >> 4;     // which 16-element slice of a 64-element step
    const uint32_t n0 = blockIdx.x * (16u * T);

    const uint8_t *wrow[T];
    bool wok[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        uint32_t nn = n0 + 16u * t + col;
        wok[t] = nn < n;
        wrow[t] = w + (size_t)(wok[t] ? nn : 0u) * k;
    }
    const bool xok = (uint32_t)col < m;
    const uint16_t *xrow = x + (size_t)(xok ? col : 0) * k;

    f32x4 acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t)
        acc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};

    const uint32_t nsteps = (k + GEMV_STEP - 1) / GEMV_STEP;
    for (uint32_t s0 = wave; s0 < nsteps; s0 += GEMV_WAVES * GEMV_UNROLL) {
        u32x4 wv[GEMV_UNROLL][T];
        u32x4 xa[GEMV_UNROLL], xb[GEMV_UNROLL];
#pragma unroll
        for (int u = 0; u < GEMV_UNROLL; ++u) {
            uint32_t s = s0 + GEMV_WAVES * u;
            uint32_t kk = s * GEMV_STEP + 16u * grp;
            bool kok = s < nsteps && kk < k;
#pragma unroll
            for (int t = 0; t < T; ++t) {
                wv[u][t] = (u32x4){0, 0, 0, 0};
                if (kok && wok[t])
                    wv[u][t] = __builtin_nontemporal_load(
                        reinterpret_cast<const u32x4 *>(wrow[t] + kk));
            }
            xa[u] = (u32x4){0, 0, 0, 0};
            xb[u] = (u32x4){0, 0, 0, 0};
            if (kok && xok) {
                const u32x4 *xp = reinterpret_cast<const u32x4 *>(xrow + kk);
                xa[u] = xp[0];
                xb[u] = xp[1];
            }
        }
#pragma unroll
        for (int u = 0; u < GEMV_UNROLL; ++u) {
#pragma unroll
            for (int t = 0; t < T; ++t) {
                bf16x8 blo, bhi;
                fp8x16_to_bf16(wv[u][t], blo, bhi);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[u]), blo, acc[t], 0, 0, 0);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xb[u]), bhi, acc[t], 0, 0, 0);
            }
        }
    }

    // Fixed-order reduction of the four K-partial tiles.
    if (wave > 0) {
#pragma unroll
        for (int t = 0; t < T; ++t)
            red[wave - 1][t][lane] = acc[t];
    }
    __syncthreads();
    if (wave != 0)
        return;
#pragma unroll
    for (int t = 0; t < T; ++t) {
        f32x4 r = acc[t];
#pragma unroll
        for (int v = 0; v < GEMV_WAVES - 1; ++v)
            r += red[v][t][lane];
        // lane holds rows 4*grp + i (i = 0..3) of column `col`
        uint32_t nn = n0 + 16u * t + col;
        if (nn < n) {
            float sc = rs[nn];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t mm = 4u * grp + i;
                if (mm < m)
                    out[(size_t)mm * n + nn] = (uint16_t)f32_to_bf16(r[i] * sc);
            }
        }
    }
}

hipError_t launch_fp8_gemv_rowscale(const uint16_t *x, const uint8_t *w,
                                    const float *rs, uint16_t *out, uint32_t m,
                                    uint32_t n, uint32_t k, hipStream_t st)
{
    // Two 16-row tiles per workgroup when there are enough rows to keep all
    // 256 CUs busy; one otherwise.  Depends on n only (never on m).
    if (n >= 32u * 1024u) {
        uint32_t grid = (n + 31) / 32;
        hipLaunchKernelGGL(k_fp8_gemv_rowscale<2>, dim3(grid), dim3(256), 0, st,
                           x, w, rs, out, m, n, k);
    } else {
        uint32_t grid = (n + 15) / 16;
        hipLaunchKernelGGL(k_fp8_gemv_rowscale<1>, dim3(grid), dim3(256), 0, st,
                           x, w, rs, out, m, n, k);
    }
    count_launch();
    return hipGetLastError();
}

} // namespace qp
