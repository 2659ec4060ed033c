// gemm_fp8.hip -- row-wise FP8 GEMM (the contraction at the end of
// dispatch_proj_rowwise.rs, cublas_fp8_rowwise_proj):
//
//   C[i,j] = bf16( a_scale[i] * w_scale[j] * sum_t e4m3(a[i,t]) * e4m3(w[j,t]) )
//
// Both operands are native FP8, so the contraction runs straight on
// v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3, unit E8M0 scales) with F32
// accumulation; the row and column scales are applied once in the epilogue.
// Any M is served: tails are zero-filled in LDS and masked at the store.
#include "gemm_common.hpp"
#include "qp_launch.hpp"

namespace qp {

constexpr int F8_BM = 128, F8_BN = 128, F8_BK = 128;
constexpr int F8_PITCH = F8_BK + 16;

__global__ __launch_bounds__(256) void k_fp8_gemm_rowscale(
    const uint8_t *__restrict__ A, const float *__restrict__ as,
    const uint8_t *__restrict__ W, const float *__restrict__ ws,
    uint16_t *__restrict__ out, uint32_t M, uint32_t N, uint32_t K,
    uint32_t mtiles, uint32_t ntiles)
{
    __shared__ __attribute__((aligned(16))) uint8_t sA[2][F8_BM * F8_PITCH];
    __shared__ __attribute__((aligned(16))) uint8_t sW[2][F8_BN * F8_PITCH];

    uint32_t tm, tn;
    tile_coords(mtiles, ntiles, tm, tn);
    const uint32_t m0 = tm * F8_BM, n0 = tn * F8_BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave & 1, wn = wave >> 1;

    StageLoader<F8_BM, F8_BK> la;
    StageLoader<F8_BN, F8_BK> lw;

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.0f;

    const uint32_t nst = (K + F8_BK - 1) / F8_BK;
    la.load(A, K, m0, M, 0, K);
    lw.load(W, K, n0, N, 0, K);
    la.store(sA[0]);
    lw.store(sW[0]);
    __syncthreads();

    const int arow = wm * 64 + (lane & 31);
    const int wrow = wn * 64 + (lane & 31);
    const int koff = 32 * (lane >> 5);

    for (uint32_t st = 0; st < nst; ++st) {
        const int buf = st & 1;
        if (st + 1 < nst) {
            la.load(A, K, m0, M, (st + 1) * F8_BK, K);
            lw.load(W, K, n0, N, (st + 1) * F8_BK, K);
        }
#pragma unroll
        for (int ks = 0; ks < F8_BK / 64; ++ks) {
            i32x8 fa[2], fw[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const uint8_t *pa = &sA[buf][(arow + 32 * t) * F8_PITCH + ks * 64 + koff];
                const uint8_t *pw = &sW[buf][(wrow + 32 * t) * F8_PITCH + ks * 64 + koff];
                i32x4 a0 = *reinterpret_cast<const i32x4 *>(pa);
                i32x4 a1 = *reinterpret_cast<const i32x4 *>(pa + 16);
                i32x4 w0 = *reinterpret_cast<const i32x4 *>(pw);
                i32x4 w1 = *reinterpret_cast<const i32x4 *>(pw + 16);
                fa[t] = (i32x8){a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
                fw[t] = (i32x8){w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
            }
#pragma unroll
            for (int ti = 0; ti < 2; ++ti)
#pragma unroll
                for (int tj = 0; tj < 2; ++tj)
                    acc[ti][tj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        fa[ti], fw[tj], acc[ti][tj], 0, 0, 0, 127, 0, 127);
        }
        if (st + 1 < nst) {
            la.store(sA[buf ^ 1]);
            lw.store(sW[buf ^ 1]);
        }
        __syncthreads();
    }

#pragma unroll
    for (int tj = 0; tj < 2; ++tj) {
        uint32_t gj = n0 + wn * 64 + 32 * tj + (lane & 31);
        float swj = gj < N ? ws[gj] : 0.0f;
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                uint32_t gi = m0 + wm * 64 + 32 * ti + mfma32_row(r, lane);
                if (gi < M && gj < N)
                    out[(size_t)gi * N + gj] =
                        (uint16_t)f32_to_bf16(acc[ti][tj][r] * (as[gi] * swj));
            }
        }
    }
}

hipError_t launch_fp8_gemm_rowscale(const uint8_t *a, const float *as,
                                    const uint8_t *w, const float *ws,
                                    uint16_t *out, uint32_t m, uint32_t n,
                                    uint32_t k, hipStream_t st)
{
    uint32_t mt = (m + F8_BM - 1) / F8_BM, nt = (n + F8_BN - 1) / F8_BN;
    hipLaunchKernelGGL(k_fp8_gemm_rowscale, dim3(mt * nt), dim3(256), 0, st,
                       a, as, w, ws, out, m, n, k, mt, nt);
    count_launch();
    return hipGetLastError();
}

} // namespace qp
