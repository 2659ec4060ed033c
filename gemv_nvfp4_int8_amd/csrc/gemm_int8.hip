// gemm_int8.hip -- int8 x int8 block-scaled GEMM for the W4A8 prefill
// (gemm_dense_int8.rs, int8_gemm_faith2 launched by int8_gemm_faith2_prefill).
//
//   C[i,j] = bf16( sum_b a_scale[i,b] * w_scale[j,b] * P_b[i,j] )
//   P_b    = sum over the 32-element K block b of a_i8 * w_i8   (exact int32)
//
// One v_mfma_i32_32x32x32_i8 covers exactly one 32-element K block of a
// 32x32 output tile, so P_b comes out of the matrix core exact and whole;
// the vector ALU then converts it and adds a_scale*w_scale*P_b into the F32
// accumulator.  The block scales of a stage are staged in LDS next to the
// operand tiles.  The same tile code can instead write every P_b to memory
// (the block-partials test export).
#include "gemm_common.hpp"
#include "qp_launch.hpp"

namespace qp {

constexpr int I8_BM = 128, I8_BN = 128, I8_BK = 128;   // BK in bytes = elements
constexpr int I8_KB = I8_BK / 32;                       // K blocks per stage
constexpr int I8_PITCH = I8_BK + 16;

template <bool PARTIALS>
__global__ __launch_bounds__(256) void k_int8_gemm(
    const int8_t *__restrict__ A, const int8_t *__restrict__ W,
    const float *__restrict__ as, const float *__restrict__ ws,
    uint16_t *__restrict__ out, int32_t *__restrict__ part,
    uint32_t M, uint32_t N, uint32_t K, uint32_t mtiles, uint32_t ntiles)
{
    __shared__ __attribute__((aligned(16))) uint8_t sA[2][I8_BM * I8_PITCH];
    __shared__ __attribute__((aligned(16))) uint8_t sW[2][I8_BN * I8_PITCH];
    // scales stored block-major so 4 consecutive rows are one 16-byte read
    __shared__ __attribute__((aligned(16))) float sAs[2][I8_KB][I8_BM];
    __shared__ __attribute__((aligned(16))) float sWs[2][I8_KB][I8_BN];

    uint32_t tm, tn;
    tile_coords(mtiles, ntiles, tm, tn);
    const uint32_t m0 = tm * I8_BM, n0 = tn * I8_BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const uint32_t nb = K / 32;

    StageLoader<I8_BM, I8_BK> la;
    StageLoader<I8_BN, I8_BK> lw;
    float ras[2], rws[2];   // 512 scale values per operand per stage / 256 threads

    auto load_stage = [&](uint32_t kst) {
        uint32_t k0 = kst * I8_BK;
        la.load(reinterpret_cast<const uint8_t *>(A), K, m0, M, k0, K);
        lw.load(reinterpret_cast<const uint8_t *>(W), K, n0, N, k0, K);
        if constexpr (!PARTIALS) {      // the partials export has no scales
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                int c = threadIdx.x + 256 * j;
                int row = c / I8_KB, b = c % I8_KB;
                uint32_t gb = kst * I8_KB + b;
                ras[j] = (m0 + row < M && gb < nb) ? as[(size_t)(m0 + row) * nb + gb] : 0.0f;
                rws[j] = (n0 + row < N && gb < nb) ? ws[(size_t)(n0 + row) * nb + gb] : 0.0f;
            }
        }
    };
    auto store_stage = [&](int buf) {
        la.store(sA[buf]);
        lw.store(sW[buf]);
        if constexpr (!PARTIALS) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                int c = threadIdx.x + 256 * j;
                int row = c / I8_KB, b = c % I8_KB;
                sAs[buf][b][row] = ras[j];
                sWs[buf][b][row] = rws[j];
            }
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.0f;

    const uint32_t nst = (K + I8_BK - 1) / I8_BK;
    load_stage(0);
    store_stage(0);
    __syncthreads();

    const int arow = wm * 64 + (lane & 31);     // + 32*ti
    const int wrow = wn * 64 + (lane & 31);     // + 32*tj
    const int koff = 16 * (lane >> 5);          // lane's 16 bytes of a 32-block

    for (uint32_t st = 0; st < nst; ++st) {
        const int buf = st & 1;
        if (st + 1 < nst)
            load_stage(st + 1);

        // two K blocks at a time: a full unroll keeps every block's int32
        // tile live at once and spills
#pragma unroll 2
        for (int kb = 0; kb < I8_KB; ++kb) {
            i32x4 fa[2], fw[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                fa[t] = *reinterpret_cast<const i32x4 *>(&sA[buf][(arow + 32 * t) * I8_PITCH + kb * 32 + koff]);
                fw[t] = *reinterpret_cast<const i32x4 *>(&sW[buf][(wrow + 32 * t) * I8_PITCH + kb * 32 + koff]);
            }
            const i32x16 zero = {};
            if constexpr (PARTIALS) {
                uint32_t gb = st * I8_KB + kb;
#pragma unroll
                for (int ti = 0; ti < 2; ++ti)
#pragma unroll
                    for (int tj = 0; tj < 2; ++tj) {
                        i32x16 p = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[ti], fw[tj], zero, 0, 0, 0);
                        uint32_t gj = n0 + wn * 64 + 32 * tj + (lane & 31);
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            uint32_t gi = m0 + wm * 64 + 32 * ti + mfma32_row(r, lane);
                            if (gb < nb && gi < M && gj < N)
                                part[((size_t)gi * N + gj) * nb + gb] = p[r];
                        }
                    }
            } else {
                // scale-and-add: acc += float(P) * (a_scale[row] * w_scale[col])
                float wsc[2];
#pragma unroll
                for (int tj = 0; tj < 2; ++tj)
                    wsc[tj] = sWs[buf][kb][wn * 64 + 32 * tj + (lane & 31)];
#pragma unroll
                for (int ti = 0; ti < 2; ++ti) {
                    // rows 8g + 4*(lane/32) + 0..3 of this 32-row tile, g = 0..3
                    f32x4 asc[4];
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        asc[g] = *reinterpret_cast<const f32x4 *>(
                            &sAs[buf][kb][wm * 64 + 32 * ti + 8 * g + 4 * (lane >> 5)]);
#pragma unroll
                    for (int tj = 0; tj < 2; ++tj) {
                        i32x16 p = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[ti], fw[tj], zero, 0, 0, 0);
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            acc[ti][tj][r] = __builtin_fmaf((float)p[r], asc[r >> 2][r & 3] * wsc[tj],
                                                            acc[ti][tj][r]);
                    }
                }
            }
        }

        if (st + 1 < nst)
            store_stage(buf ^ 1);
        __syncthreads();
    }

    if constexpr (!PARTIALS) {
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
#pragma unroll
            for (int tj = 0; tj < 2; ++tj) {
                uint32_t gj = n0 + wn * 64 + 32 * tj + (lane & 31);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    uint32_t gi = m0 + wm * 64 + 32 * ti + mfma32_row(r, lane);
                    if (gi < M && gj < N)
                        out[(size_t)gi * N + gj] = (uint16_t)f32_to_bf16(acc[ti][tj][r]);
                }
            }
    }
}

hipError_t launch_int8_gemm(const int8_t *a, const int8_t *w, const float *as,
                            const float *ws, uint16_t *out, int32_t *partials,
                            uint32_t m, uint32_t n, uint32_t k, hipStream_t st)
{
    uint32_t mt = (m + I8_BM - 1) / I8_BM, nt = (n + I8_BN - 1) / I8_BN;
    dim3 grid(mt * nt), block(256);
    if (partials)
        hipLaunchKernelGGL(k_int8_gemm<true>, grid, block, 0, st, a, w, as, ws,
                           out, partials, m, n, k, mt, nt);
    else
        hipLaunchKernelGGL(k_int8_gemm<false>, grid, block, 0, st, a, w, as, ws,
                           out, partials, m, n, k, mt, nt);
    count_launch();
    return hipGetLastError();
}

} // namespace qp
