// gemm_w4a4.hip -- NVFP4 x NVFP4 GEMM for the W4A4 prefill
// (gemm_fp4.rs, w4a4_gemm / w4a4_gemm_mfast):
//
//   C[i,j] = bf16( sA2 * sW2 * sum_b e4m3(sa[i,b]) * e4m3(sw[j,b]) * P_b )
//   P_b    = sum over 16-element block b of e2m1(a) * e2m1(w)
//
// gfx950's block-scaled FP4 MFMA takes power-of-two (E8M0) scales per 32
// elements, while NVFP4 carries an E4M3 scale per 16.  Instead of running
// FP4 MFMAs per 16-block and scaling partial sums on the vector ALU, each
// E2M1 code is multiplied by its block's E4M3 scale while it is unpacked
// from LDS into registers (E2M1 -> FP16 conversion, then a packed FP16
// multiply by the block scale).  The product has at
// most 6 significant bits and lies in [2^-10, 2688], so it is exact in FP16;
// FP16 MFMA then forms exact products of the scaled operands with F32
// accumulation, which is the block-scaled sum up to F32 rounding order.
// Operands stay packed (4 bits) in LDS; the per-tensor scales are applied
// in the epilogue.
#include "gemm_common.hpp"
#include "qp_launch.hpp"

namespace qp {

constexpr int W4_BM = 128, W4_BN = 128;
constexpr int W4_BKE = 128;              // K elements per stage
constexpr int W4_BKB = W4_BKE / 2;       // packed bytes per row per stage
constexpr int W4_PITCH = W4_BKB + 16;
constexpr int W4_NSC = W4_BKE / 16;      // scale bytes per row per stage

// Eight E2M1 codes (one dword, low nibble first) times the block scale ->
// FP16 x 8.  The converter runs with a unit scale (its scale operand is
// meant for power-of-two MX scales, so an E4M3 scale's mantissa cannot go
// through it); the E4M3 scale, exact in FP16, is applied with a packed FP16
// multiply whose result (at most 6 significant bits) is exact.
__device__ __forceinline__ f16x8 fp4x8_scaled(uint32_t d, f16x2 s)
{
    f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 0) * s;
    f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 1) * s;
    f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 2) * s;
    f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 3) * s;
    return (f16x8){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ f16x2 e4m3_to_f16x2(uint32_t byte)
{
    _Float16 h = (_Float16)dec_e4m3(byte);     // exact: E4M3 fits in FP16
    return (f16x2){h, h};
}

__global__ __launch_bounds__(256) void k_w4a4_gemm(
    const uint8_t *__restrict__ Ap, const uint8_t *__restrict__ Asc,
    const uint8_t *__restrict__ Wp, const uint8_t *__restrict__ Wsc,
    uint16_t *__restrict__ out, float s2, uint32_t M, uint32_t N, uint32_t K,
    uint32_t mtiles, uint32_t ntiles)
{
    __shared__ __attribute__((aligned(16))) uint8_t sA[2][W4_BM * W4_PITCH];
    __shared__ __attribute__((aligned(16))) uint8_t sW[2][W4_BN * W4_PITCH];
    __shared__ __attribute__((aligned(16))) uint8_t sAs[2][W4_BM * W4_NSC];
    __shared__ __attribute__((aligned(16))) uint8_t sWs[2][W4_BN * W4_NSC];

    uint32_t tm, tn;
    tile_coords(mtiles, ntiles, tm, tn);
    const uint32_t m0 = tm * W4_BM, n0 = tn * W4_BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const uint32_t kb = K / 2;        // packed bytes per row
    const uint32_t nsb = K / 16;      // scale bytes per row

    StageLoader<W4_BM, W4_BKB> la;
    StageLoader<W4_BN, W4_BKB> lw;
    uint32_t ras, rws;                // 4 scale bytes per thread per operand

    auto load_stage = [&](uint32_t kst) {
        la.load(Ap, kb, m0, M, kst * W4_BKB, kb);
        lw.load(Wp, kb, n0, N, kst * W4_BKB, kb);
        int row = threadIdx.x >> 1, half = threadIdx.x & 1;
        uint32_t s0 = kst * W4_NSC + 4 * half;
        ras = 0;
        rws = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (m0 + row < M && s0 + e < nsb)
                ras |= (uint32_t)Asc[(size_t)(m0 + row) * nsb + s0 + e] << (8 * e);
            if (n0 + row < N && s0 + e < nsb)
                rws |= (uint32_t)Wsc[(size_t)(n0 + row) * nsb + s0 + e] << (8 * e);
        }
    };
    auto store_stage = [&](int buf) {
        la.store(sA[buf]);
        lw.store(sW[buf]);
        int row = threadIdx.x >> 1, half = threadIdx.x & 1;
        *reinterpret_cast<uint32_t *>(&sAs[buf][row * W4_NSC + 4 * half]) = ras;
        *reinterpret_cast<uint32_t *>(&sWs[buf][row * W4_NSC + 4 * half]) = rws;
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.0f;

    const uint32_t nst = (K + W4_BKE - 1) / W4_BKE;
    load_stage(0);
    store_stage(0);
    __syncthreads();

    const int g = lane >> 5;                   // lane half: elements [64g, 64g+64)
    const int arow = wm * 64 + (lane & 31);
    const int wrow = wn * 64 + (lane & 31);

    for (uint32_t st = 0; st < nst; ++st) {
        const int buf = st & 1;
        if (st + 1 < nst)
            load_stage(st + 1);

        u32x4 pa[2][2], pw[2][2];
        uint32_t qa[2], qw[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint8_t *a = &sA[buf][(arow + 32 * t) * W4_PITCH + 32 * g];
            const uint8_t *w = &sW[buf][(wrow + 32 * t) * W4_PITCH + 32 * g];
            pa[t][0] = *reinterpret_cast<const u32x4 *>(a);
            pa[t][1] = *reinterpret_cast<const u32x4 *>(a + 16);
            pw[t][0] = *reinterpret_cast<const u32x4 *>(w);
            pw[t][1] = *reinterpret_cast<const u32x4 *>(w + 16);
            qa[t] = *reinterpret_cast<const uint32_t *>(&sAs[buf][(arow + 32 * t) * W4_NSC + 4 * g]);
            qw[t] = *reinterpret_cast<const uint32_t *>(&sWs[buf][(wrow + 32 * t) * W4_NSC + 4 * g]);
        }
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            f16x2 fsa[2], fsw[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                fsa[t] = e4m3_to_f16x2((qa[t] >> (8 * blk)) & 0xFFu);
                fsw[t] = e4m3_to_f16x2((qw[t] >> (8 * blk)) & 0xFFu);
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {            // two MFMAs per 16-block
                int j = 2 * blk + h;                 // dword of the lane's 32 bytes
                f16x8 fa[2], fw[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    fa[t] = fp4x8_scaled(pa[t][j / 4][j % 4], fsa[t]);
                    fw[t] = fp4x8_scaled(pw[t][j / 4][j % 4], fsw[t]);
                }
#pragma unroll
                for (int ti = 0; ti < 2; ++ti)
#pragma unroll
                    for (int tj = 0; tj < 2; ++tj)
                        acc[ti][tj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            fa[ti], fw[tj], acc[ti][tj], 0, 0, 0);
            }
        }

        if (st + 1 < nst)
            store_stage(buf ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int tj = 0; tj < 2; ++tj) {
            uint32_t gj = n0 + wn * 64 + 32 * tj + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                uint32_t gi = m0 + wm * 64 + 32 * ti + mfma32_row(r, lane);
                if (gi < M && gj < N)
                    out[(size_t)gi * N + gj] = (uint16_t)f32_to_bf16(acc[ti][tj][r] * s2);
            }
        }
}

hipError_t launch_w4a4_gemm(const uint8_t *ap, const uint8_t *asc,
                            const uint8_t *wp, const uint8_t *wsc, uint16_t *out,
                            float sa2, float sw2, uint32_t m, uint32_t n,
                            uint32_t k, hipStream_t st)
{
    uint32_t mt = (m + W4_BM - 1) / W4_BM, nt = (n + W4_BN - 1) / W4_BN;
    float s2 = sa2 * sw2;
    hipLaunchKernelGGL(k_w4a4_gemm, dim3(mt * nt), dim3(256), 0, st,
                       ap, asc, wp, wsc, out, s2, m, n, k, mt, nt);
    count_launch();
    return hipGetLastError();
}

} // namespace qp
