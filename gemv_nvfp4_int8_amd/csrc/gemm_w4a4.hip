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

#include <type_traits>

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
    uint32_t mtiles, uint32_t ntiles, uint32_t order)
{
    __shared__ __attribute__((aligned(16))) uint8_t sA[2][W4_BM * W4_PITCH];
    __shared__ __attribute__((aligned(16))) uint8_t sW[2][W4_BN * W4_PITCH];
    __shared__ __attribute__((aligned(16))) uint8_t sAs[2][W4_BM * W4_NSC];
    __shared__ __attribute__((aligned(16))) uint8_t sWs[2][W4_BN * W4_NSC];

    uint32_t tm, tn;
    tile_coords_order(order, mtiles, ntiles, tm, tn);
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

// ---------------------------------------------------------------------------
// Large-tile variant for K % 256 == 0, M >= 256, N >= 160: 256 x 160
// workgroup tiles (M = 4096, N = 5120 makes 512 tiles, two rounds on 256
// CUs), each wave a 128 x 80 block of 8 x 5 v_mfma_f32_16x16x32_f16 tiles,
// so every converted fragment feeds 5 or 8 MFMAs.
//
// K advances in stages of 256 elements.  A stage buffer holds the packed
// A panel (256 rows x 128 bytes), the packed W panel (160 rows), and the
// 16 scale bytes of every row of both (W scale rows padded to 256 so each
// wave issues the same loads); two buffers, filled by 16-byte LDS-DMA loads
// a whole stage (~5000 MFMA cycles) ahead.  Packed rows are stored with the
// 16-byte chunks XOR-swizzled by (row / 2) % 8, so 16 consecutive rows
// reading one logical chunk hit distinct banks.
//
// K order: both operands must pair the same k, so any permutation shared by
// A and W is allowed.  Lane group g (lane / 16) reads the 16 bytes (32
// elements) at byte 64t + 16g of the stage row for four consecutive MFMA
// K steps 4t + v (t = 0, 1; v = 0 .. 3) and feeds bytes 4v .. 4v+3 to step
// 4t + v; those 8 elements lie in 16-element block 8t + 2g + v/2.
//
// The MFMAs compute C^T tiles (W fragment first): lane l holds row l % 16 of
// its C tile and four consecutive columns 4*(l/16) .. +3, written as one
// 8-byte store.  The last tile row / column is shifted back to end at M / N
// (every loaded row exists) and stores only what the previous tile did not.
// ---------------------------------------------------------------------------
constexpr int WB_TM = 256, WB_TN = 160;
constexpr int WB_KE = 256;                    // K elements per stage
constexpr int WB_KB = WB_KE / 2;              // packed bytes per row per stage
constexpr int WB_NS = WB_KE / 16;             // scale bytes per row per stage
constexpr int WB_PA = 0;                      // byte offsets in a stage buffer
constexpr int WB_PW = WB_PA + WB_TM * WB_KB;  // 32 KB
constexpr int WB_SA = WB_PW + WB_TN * WB_KB;  // + 20 KB
constexpr int WB_SW = WB_SA + WB_TM * WB_NS;  // + 4 KB
constexpr int WB_BUF = WB_SW + 256 * WB_NS;   // + 4 KB = 60 KB
constexpr int W4_EPITCH = 2 * WB_TN + 16;     // epilogue staging: bytes per output row
static_assert(128 * W4_EPITCH <= WB_BUF, "half the output tile fits one stage buffer");

// WM waves along M (2 or 4) times 2 along N: a wave owns RW = TM / WM rows
// (NA = RW / 16 MFMA tiles) by 80 columns (5 tiles).  WM = 4 runs two waves
// per SIMD (512 threads, at most 256 registers each).
//
// TM is the tile height: 256, or 128 for the half tiles of a thin last
// round.  One workgroup runs per CU, so time goes by rounds of one tile per
// CU; when the last round is at most half full, its tiles run in a second
// launch as two 128 x 160 halves each (the first half on rows m0 .. m0+127),
// on twice the CUs, with the same stage buffer layout (A rows 128-255 and
// their scales unused).  Each output keeps its whole K sum, in the same
// order, so results do not depend on the split.  The TM = 256 launch takes
// the first nfull tiles of the launch's tile order, the TM = 128 launch the
// rest, workgroups 2i and 2i + 1 the halves of tile nfull + i.
template <int WM, int TM = WB_TM>
__global__ __launch_bounds__(128 * WM, 1) void k_w4a4_gemm_big(
    const uint8_t *__restrict__ Ap, const uint8_t *__restrict__ Asc,
    const uint8_t *__restrict__ Wp, const uint8_t *__restrict__ Wsc,
    uint16_t *__restrict__ out, float s2, uint32_t M, uint32_t N, uint32_t K,
    uint32_t mtiles, uint32_t ntiles, uint32_t nfull, uint32_t order)
{
    static_assert(TM == WB_TM || TM == WB_TM / 2, "whole or half tiles");
    constexpr int NW = 2 * WM;            // waves
    constexpr int RW = TM / WM;           // rows per wave
    constexpr int NA = RW / 16;           // A tiles per wave
    constexpr int APW = TM / 8 / NW;      // A packed kilobytes per wave
    // Two stage buffers as separate LDS variables (distinct alias scopes:
    // reading one need not wait for the DMA into the other).
    __shared__ __attribute__((aligned(1024))) uint8_t B0[WB_BUF];
    __shared__ __attribute__((aligned(1024))) uint8_t B1[WB_BUF];

    uint32_t tm, tn, half = 0;
    if (TM == WB_TM) {
        tile_in_order(order, order == 0 ? xcd_remap(blockIdx.x, nfull) : blockIdx.x,
                      mtiles, ntiles, tm, tn);
    } else {
        tile_in_order(order, nfull + blockIdx.x / 2, mtiles, ntiles, tm, tn);
        half = blockIdx.x & 1;
    }
    const uint32_t m0 = tm * WB_TM + TM * half, n0 = tn * WB_TN;
    const uint32_t m0e = min(m0, M - TM), n0e = min(n0, N - WB_TN);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave % WM, wn = wave / WM;
    const uint32_t ldp = K / 2, lds_ = K / 16;         // packed / scale row strides
    const uint32_t nst = K / WB_KE;

    // ---- DMA addressing (instruction j of a wave fills one kilobyte:
    // 8 packed rows x 128 bytes, lane -> row lane/8, physical chunk lane%8
    // holding logical chunk (lane%8) ^ swz(row), swz(row) = ((kb & 1) << 2)
    // | (lane >> 4) for kilobyte kb).
    uint32_t dvo[2];
#pragma unroll
    for (int e = 0; e < 2; ++e)
        dvo[e] = (uint32_t)(lane >> 3) * ldp + 16u * ((lane & 7) ^ ((e << 2) | (lane >> 4)));
    // A kilobytes kb = APW*w + j; W kilobytes kb = w + NW*j (kb < 20; the
    // parity of kb, which picks the swizzle, is then that of j, resp. w);
    // the 4 A-scale and 4 W-scale kilobytes (64 rows each) go to waves
    // i and i + 4 (NW = 8) or both to wave i (NW = 4).
    const uint8_t *const a_rows = Ap + (size_t)(m0e + 8 * APW * wave) * ldp;
    const uint8_t *const w_rows = Wp + (size_t)(n0e + 8 * wave) * ldp;
    const int sq = wave & 3;
    // (half tiles: the scale rows past the tile's 128 land in the unused
    // half of the region; rows past M reload row M - 1, in bounds)
    const uint32_t asr = m0e + 64 * sq + lane;
    const uint8_t *const as_row = Asc + (size_t)(TM == WB_TM || asr < M ? asr : M - 1) * lds_;
    const uint32_t wsr = n0e + 64 * sq + lane;
    const uint8_t *const ws_row = Wsc + (size_t)(wsr < N ? wsr : N - 1) * lds_;
    // Stage st into buffer B (stages past the end reload the last one: in
    // bounds, never read).
    auto dma = [&](uint32_t st, uint8_t *B) {
        const uint32_t s = st < nst ? st : nst - 1;
        const uint8_t *pa = a_rows + s * WB_KB;
#pragma unroll
        for (int j = 0; j < APW; ++j)
            __builtin_amdgcn_global_load_lds(pa + (size_t)(8 * j) * ldp + dvo[j & 1],
                                             (lds_void *)(B + WB_PA + 1024 * (APW * wave + j)), 16, 0, 0);
        const uint8_t *pw = w_rows + s * WB_KB;
#pragma unroll
        for (int j = 0; j < (20 + NW - 1) / NW; ++j)
            if (wave + NW * j < 20)
                __builtin_amdgcn_global_load_lds(pw + (size_t)(8 * NW * j) * ldp + dvo[wave & 1],
                                                 (lds_void *)(B + WB_PW + 1024 * (wave + NW * j)), 16, 0, 0);
        if (NW == 4 || wave < 4)
            __builtin_amdgcn_global_load_lds(as_row + s * WB_NS, (lds_void *)(B + WB_SA + 1024 * sq), 16, 0, 0);
        if (NW == 4 || wave >= 4)
            __builtin_amdgcn_global_load_lds(ws_row + s * WB_NS, (lds_void *)(B + WB_SW + 1024 * sq), 16, 0, 0);
    };

    // ---- fragment reads: row 16*t + (lane % 16) of the wave's half, logical
    // chunk 4*tt + g (tt = 0, 1), physical chunk ^ (((lane % 16) >> 1) & 7)
    const int g = lane >> 4, r16 = lane & 15;
    uint32_t lrow[2], lsc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        lrow[tt] = r16 * WB_KB + 16 * ((4 * tt + g) ^ ((r16 >> 1) & 7));
        lsc[tt] = r16 * WB_NS + 8 * tt + 2 * g;         // the two block scales of the lane's 32
    }
    uint32_t lo[4];
    auto launder = [&]() {
        lo[0] = lrow[0];
        lo[1] = lrow[1];
        lo[2] = lsc[0];
        lo[3] = lsc[1];
        asm volatile("" : "+v"(lo[0]), "+v"(lo[1]), "+v"(lo[2]), "+v"(lo[3]));
    };

    f32x4 acc[NA][5];
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
        for (int j = 0; j < 5; ++j)
            acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // packed 16-byte reads and 2-byte scale pairs of one half-stage (tt)
    struct Half {
        u32x4 a[NA], w[5];
        uint32_t sa[NA], sw[5];
    };
    auto read_half = [&](Half &h, const uint8_t *B, int tt) {
        const uint8_t *pa = B + WB_PA + wm * RW * WB_KB + lo[tt];
        const uint8_t *pw = B + WB_PW + wn * 80 * WB_KB + lo[tt];
        const uint8_t *qa = B + WB_SA + wm * RW * WB_NS + lo[2 + tt];
        const uint8_t *qw = B + WB_SW + wn * 80 * WB_NS + lo[2 + tt];
#pragma unroll
        for (int t = 0; t < NA; ++t) {
            h.a[t] = *reinterpret_cast<const u32x4 *>(pa + 16 * WB_KB * t);
            h.sa[t] = *reinterpret_cast<const uint16_t *>(qa + 16 * WB_NS * t);
        }
#pragma unroll
        for (int t = 0; t < 5; ++t) {
            h.w[t] = *reinterpret_cast<const u32x4 *>(pw + 16 * WB_KB * t);
            h.sw[t] = *reinterpret_cast<const uint16_t *>(qw + 16 * WB_NS * t);
        }
    };
    auto sync_all = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    // Stage st from buffer cur while stage st+1 is DMA'd into nxt (free: the
    // barrier ending the previous stage came after every read of it).
    auto stage = [&](uint32_t st, const uint8_t *cur, uint8_t *nxt) {
        dma(st + 1, nxt);
        launder();
        Half h;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            read_half(h, cur, tt);
            f16x2 sca[NA], scw[5];
#pragma unroll
            for (int t = 0; t < NA; ++t)
                sca[t] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(h.sa[t], 1.0f, false);
#pragma unroll
            for (int t = 0; t < 5; ++t)
                scw[t] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(h.sw[t], 1.0f, false);
            // Software pipeline: the fragments of K step v + 1 are converted
            // while the 40 MFMAs of step v run (measured 602 -> 582 us against
            // converting each step's fragments just before its MFMAs).  sc*
            // hold the FP16 values of a fragment's two block scales (the
            // packed FP8 converter, exact for E4M3).
            f16x8 fa[2][NA], fw[2][5];
            auto conv = [&](int v, f16x8 *da, f16x8 *dw) {
#pragma unroll
                for (int t = 0; t < NA; ++t) {
                    const _Float16 sb = sca[t][v >> 1];
                    da[t] = fp4x8_scaled(h.a[t][v], (f16x2){sb, sb});
                }
#pragma unroll
                for (int t = 0; t < 5; ++t) {
                    const _Float16 sb = scw[t][v >> 1];
                    dw[t] = fp4x8_scaled(h.w[t][v], (f16x2){sb, sb});
                }
            };
            conv(0, fa[0], fw[0]);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int c = v & 1;
#pragma unroll
                for (int ti = 0; ti < NA; ++ti)
#pragma unroll
                    for (int tj = 0; tj < 5; ++tj)
                        acc[ti][tj] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fw[c][tj], fa[c][ti], acc[ti][tj], 0, 0, 0);
                if (v < 3)
                    conv(v + 1, fa[c ^ 1], fw[c ^ 1]);
            }
        }
        sync_all();
    };

    dma(0, B0);
    sync_all();
    uint32_t st = 0;
    for (; st + 2 <= nst; st += 2) {
        stage(st, B0, B1);
        stage(st + 1, B1, B0);
    }
    if (st < nst)
        stage(st, B0, B1);

    // Epilogue: C[i][j] = bf16(s2 * acc); lane row i = ib + 16*ti, columns
    // j = jb + 16*tj + c (c = 0..3).
    const uint32_t ib = m0e + wm * RW + r16;
    const uint32_t jb = n0e + wn * 80 + 4 * g;
    if (WM == 2 && N % 8 == 0 && reinterpret_cast<uintptr_t>(out) % 16 == 0) {
        // Stored from the MFMA layout, each store would put 32 bytes into
        // each of 16 rows.  Instead the workgroup stages its TM x 160 BF16
        // tile in LDS (rows of 320 bytes at a 336-byte pitch, which spreads
        // a write's 16 rows over the banks; rows 0-127 in B0, 128-255 in
        // B1: the last stage ended with every DMA landed and a barrier) and
        // stores it row-contiguously, 64 consecutive 16-byte chunks (about
        // three rows) per instruction.  A shifted tile stores only rows
        // >= m0 and chunks at columns >= n0 (with N % 8 == 0 the shift is a
        // multiple of 8 columns, so no chunk straddles n0).
        uint8_t *const ep = (wm * RW < 128 ? B0 : B1) + ((wm * RW) & 127) * W4_EPITCH;
#pragma unroll
        for (int ti = 0; ti < NA; ++ti)
#pragma unroll
            for (int tj = 0; tj < 5; ++tj) {
                const f32x4 c = acc[ti][tj];
                u32x2 pk;
                pk[0] = pk_bf16(c[0] * s2, c[1] * s2);
                pk[1] = pk_bf16(c[2] * s2, c[3] * s2);
                *reinterpret_cast<u32x2 *>(ep + (16 * ti + r16) * W4_EPITCH +
                                           2 * (wn * 80 + 16 * tj + 4 * g)) = pk;
            }
        __syncthreads();
        uint16_t *const obase = out + (size_t)m0e * N + n0e;
        // whole tiles run a copy of the loop without the row / column test
        auto store_tile = [&](auto guarded) {
#pragma unroll 4
            for (int i = 0; i < TM * (WB_TN / 8) / 256; ++i) {
                const int idx = threadIdx.x + 256 * i;  // chunk: row idx / 20, 16 bytes idx % 20
                const int row = idx / (WB_TN / 8), ch = idx % (WB_TN / 8);
                const uint8_t *src = (row < 128 ? B0 : B1) + (row & 127) * W4_EPITCH + 16 * ch;
                if (!decltype(guarded)::value || (m0e + row >= m0 && n0e + 8 * ch >= n0))
                    *reinterpret_cast<u32x4 *>(obase + (size_t)row * N + 8 * ch) =
                        *reinterpret_cast<const u32x4 *>(src);
            }
        };
        if (m0e == m0 && n0e == n0)
            store_tile(std::false_type());
        else
            store_tile(std::true_type());
        return;
    }
    const bool fast = m0e == m0 && n0e == n0 && N % 4 == 0 &&
                      reinterpret_cast<uintptr_t>(out) % 8 == 0;
#pragma unroll
    for (int ti = 0; ti < NA; ++ti) {
        const uint32_t gi = ib + 16 * ti;
#pragma unroll
        for (int tj = 0; tj < 5; ++tj) {
            const f32x4 c = acc[ti][tj];
            const uint32_t gj = jb + 16 * tj;
            if (fast) {
                u32x2 pk;
                pk[0] = pk_bf16(c[0] * s2, c[1] * s2);
                pk[1] = pk_bf16(c[2] * s2, c[3] * s2);
                *reinterpret_cast<u32x2 *>(out + (size_t)gi * N + gj) = pk;
            } else if (gi >= m0) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (gj + r >= n0)
                        out[(size_t)gi * N + gj + r] = (uint16_t)f32_to_bf16(c[r] * s2);
            }
        }
    }
}

hipError_t launch_w4a4_gemm(const uint8_t *ap, const uint8_t *asc,
                            const uint8_t *wp, const uint8_t *wsc, uint16_t *out,
                            float sa2, float sw2, uint32_t m, uint32_t n,
                            uint32_t k, uint32_t order, hipStream_t st)
{
    float s2 = sa2 * sw2;
    if (k % WB_KE == 0 && m >= (uint32_t)WB_TM && n >= (uint32_t)WB_TN) {
        const uint32_t mt = (m + WB_TM - 1) / WB_TM, nt = (n + WB_TN - 1) / WB_TN;
        const uint32_t tiles = mt * nt;
        // One tile per CU at a time: a last round at most half full runs as
        // twice as many half tiles (with the CU count unknown, no split).
        const uint32_t cus = cu_count(), tail = cus ? tiles % cus : 0;
        const uint32_t nfull = tail != 0 && 2 * tail <= cus ? tiles - tail : tiles;
        // WM = 2 (four waves, 128 x 80 each): two waves per SIMD (WM = 4)
        // measured slower at 4096 x 5120 x 17408 (778 vs 736 us)
        if (nfull) {
            hipLaunchKernelGGL(k_w4a4_gemm_big<2>, dim3(nfull), dim3(256), 0, st,
                               ap, asc, wp, wsc, out, s2, m, n, k, mt, nt, nfull, order);
            count_launch();
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess)
                return e;
        }
        if (nfull < tiles) {
            hipLaunchKernelGGL((k_w4a4_gemm_big<2, WB_TM / 2>), dim3(2 * (tiles - nfull)), dim3(256),
                               0, st, ap, asc, wp, wsc, out, s2, m, n, k, mt, nt, nfull, order);
            count_launch();
        }
        return hipGetLastError();
    } else {
        uint32_t mt = (m + W4_BM - 1) / W4_BM, nt = (n + W4_BN - 1) / W4_BN;
        hipLaunchKernelGGL(k_w4a4_gemm, dim3(mt * nt), dim3(256), 0, st,
                           ap, asc, wp, wsc, out, s2, m, n, k, mt, nt, order);
    }
    count_launch();
    return hipGetLastError();
}

} // namespace qp
