// gemv_fp8.hip -- FP8-weight GEMVs for decode / verify batches (M <= 16) on
// gfx950 (fp8_gemv_batch.rs).  Two scale layouts share the kernels:
//
//   row-scaled    (fp8_gemv_rowscale_batch8_rt2 / _batch16_rt2,
//                  dense_gemv_fp8w_batch2)
//       C[i,j] = bf16( row_scale[j] * sum_t x[i,t] * e4m3(w[j,t]) )
//   block-scaled  (w8a16_gemv / _batch2 / _batch4; one F32 scale per
//                  128 x 128 weight block, grid S[N/128, K/128])
//       C[i,j] = bf16( sum_t x[i,t] * e4m3(w[j,t]) * S[j/128, t/128] )
//
// The block-scaled form accumulates each 128-element K block of the
// contraction in a fresh F32 partial and folds it into the running sum with
// one FMA by that block's scale; a wave's rows always lie in one 128-row
// block, so the scale is a wave-uniform scalar.
//
// Design (MI355X-first):
//  * The contraction runs on MFMA, not on the vector ALU: at 8 TB/s an M=16
//    GEMV needs ~250 TFLOP/s, beyond the FP32 vector peak.  The E4M3 weight
//    converts exactly to BF16 (v_cvt_scalef32_pk_bf16_fp8 with a unit scale),
//    the activations already are BF16, and v_mfma_f32_16x16x32_bf16 forms
//    exact products with F32 accumulation.  The activation rows are the
//    MFMA's 16 M-rows, so one pass over the weight serves every row; rows
//    >= M are zero and cost no memory traffic.
//  * The weight is read once, with 64-lane loads that each cover 4 rows x
//    256 contiguous bytes: HBM3E serves such bursts at ~6.9 TB/s on this
//    part, against ~5 TB/s for the 16 rows x 64 bytes an MFMA-shaped load
//    would touch.  Each wave transposes its bytes through a private LDS tile
//    into MFMA operand layout.
//  * Two work splits (see gemv_rows): wide weights above M = 2 give each
//    wave its own rows over all of K, with the activation segment staged
//    once per workgroup in LDS and shared by its four waves; narrow weights,
//    and wide ones at M <= 2, split K over the four waves of a workgroup
//    (everything wave-private) and add the partial tiles in a fixed order.
//    The row-owning kernel sums each row in the same K quarters, added in
//    the same order, so the two kernels give identical bits.  The K-split
//    kernel's launch shape (rows per workgroup, activation rows loaded,
//    segments in flight) may follow M, but no summation order depends on M
//    or N: every output row is bit-identical to an M = 1 call on that row.
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

// ---------------------------------------------------------------------------
// Wide weights: each wave owns 16*T rows over all of K; the four waves walk K
// together in 256-element segments.  Per segment:
//   * the weight bytes are loaded with every 64-lane instruction covering 4
//     rows x 256 contiguous bytes (HBM serves such bursts far better than the
//     16 rows x 64 bytes an MFMA-shaped load would touch), written to a
//     wave-private LDS tile and read back in MFMA operand layout;
//   * the activation segment [16 x 256] BF16 is loaded once per workgroup
//     into LDS (double-buffered, one barrier per segment) and shared by the
//     four waves.
// Loads run D segments ahead of the MFMAs.
// ---------------------------------------------------------------------------
constexpr int GV_SEG = 256;                 // K elements per segment
constexpr int GV_WPITCH = GV_SEG + 16;      // LDS bytes per weight row
constexpr int GV_XPITCH = GV_SEG + 8;       // LDS bf16 per activation row

template <int T>
struct GvSeg {
    u32x4 w[4 * T];     // 4T instructions of 4 rows x 256 B
    u32x4 x[2];         // 2 x 16 B of the workgroup's activation segment
    float s[2];         // block scales of the segment's two K blocks (BS)
};

// Fold a 128-element block partial into the running sum: acc += s * p, one
// rounding per element.
__device__ __forceinline__ void fold_block(f32x4 &acc, float s, const f32x4 &p)
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
        acc[i] = __builtin_fmaf(s, p[i], acc[i]);
}

// rs: the row scale [n] (BS = false) or the block scale grid [n/128, k/128]
// (BS = true, n and k multiples of 128).
template <int T, int D, bool BS>
__global__ __launch_bounds__(256) void k_fp8_gemv_rows(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ w,
    const float *__restrict__ rs, uint16_t *__restrict__ out,
    uint32_t m, uint32_t n, uint32_t k)
{
    constexpr int ROWS = 16 * T;
    static_assert(128 % ROWS == 0, "a wave's rows must share one 128-row scale block");
    __shared__ __attribute__((aligned(16))) uint8_t sw[4][ROWS * GV_WPITCH];
    __shared__ __attribute__((aligned(16))) uint16_t sx[2][16 * GV_XPITCH];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const uint32_t row0 = blockIdx.x * (4 * ROWS) + wave * ROWS;
    const uint32_t nseg = (k + GV_SEG - 1) / GV_SEG;
    const uint32_t kbl = k / 128;
    const float *srow = rs + (size_t)((row0 < n ? row0 : n - 1) / 128) * kbl;

    // Weight loads: instruction j covers rows row0 + 4j .. + 3, lane -> row
    // 4j + grp, bytes 16*col of the segment.  Rows past n re-read row n-1.
    const uint8_t *wsrc[4 * T];
#pragma unroll
    for (int j = 0; j < 4 * T; ++j) {
        uint32_t r = row0 + 4 * j + grp;
        wsrc[j] = w + (size_t)(r < n ? r : n - 1) * k + 16 * col;
    }
    // Activation loads: 16 rows x 256 bf16 = 512 chunks of 16 B, two per
    // thread: chunk c = tid + 256 i -> row c / 32, element 8 * (c % 32).
    const uint16_t *xsrc[2];
    bool xrow_ok[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        int c = tid + 256 * i, r = c >> 5;
        xrow_ok[i] = (uint32_t)r < m;
        xsrc[i] = x + (size_t)(xrow_ok[i] ? r : 0) * k + 8 * (c & 31);
    }

    auto load = [&](GvSeg<T> &g, uint32_t seg) {
        uint32_t kb = seg * GV_SEG;
        bool full = kb + GV_SEG <= k;
        if constexpr (BS) {
            // issued ahead of the weights, so the wait at the top of the
            // segment that uses them covers them (the second index is
            // clamped in bounds; a missing block is never folded)
            g.s[0] = srow[2 * seg];
            g.s[1] = srow[min(2 * seg + 1, kbl - 1)];
        }
#pragma unroll
        for (int j = 0; j < 4 * T; ++j) {
            uint32_t kk = kb + 16 * col;
            g.w[j] = (u32x4){0, 0, 0, 0};
            if (full || kk < k)
                g.w[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(wsrc[j] + kb));
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int c = tid + 256 * i;
            uint32_t kk = kb + 8 * (c & 31);
            g.x[i] = (u32x4){0, 0, 0, 0};
            if (xrow_ok[i] && (full || kk < k))
                g.x[i] = *reinterpret_cast<const u32x4 *>(xsrc[i] + kb);
        }
    };
    auto stash = [&](const GvSeg<T> &g, int buf) {
#pragma unroll
        for (int j = 0; j < 4 * T; ++j)
            *reinterpret_cast<u32x4 *>(&sw[wave][(4 * j + grp) * GV_WPITCH + 16 * col]) = g.w[j];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int c = tid + 256 * i;
            *reinterpret_cast<u32x4 *>(&sx[buf][(c >> 5) * GV_XPITCH + 8 * (c & 31)]) = g.x[i];
        }
    };

    f32x4 acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t)
        acc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
    // BS: the last block partial not yet folded, and its scale (a zero
    // partial with scale 0 before the first segment)
    f32x4 p_pend[T];
    float s_pend = 0.f;
#pragma unroll
    for (int t = 0; t < T; ++t)
        p_pend[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
    // The K quarters of the narrow kernel (per segments each, ending on
    // 256-element boundaries): acc holds the current quarter's sum, tot the
    // closed quarters' sums added in order, ((q0 + q1) + q2) + q3, with
    // empty trailing quarters adding +0.  A row's summation order is then
    // the narrow kernel's, so its bits do not depend on which kernel runs.
    const uint32_t per = ((k + 255) / 256 + 3) / 4;
    f32x4 tot[T];
    uint32_t closed = 0, q_end = per;
    auto close_quarter = [&]() {
#pragma unroll
        for (int t = 0; t < T; ++t) {
            tot[t] = closed == 0 ? acc[t] : tot[t] + acc[t];
            acc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
        }
        ++closed;
    };

    GvSeg<T> g[D];
#pragma unroll
    for (int d = 0; d < D; ++d)
        if ((uint32_t)d < nseg)
            load(g[d], d);

    for (uint32_t seg = 0; seg < nseg; ++seg) {
        const int buf = seg & 1;
        GvSeg<T> &cur = g[0];
        stash(cur, buf);
        // The second block of a segment may lie past K (K an odd number of
        // 128-blocks); its partial is zero and it is folded with scale 0.
        const float s_lo = cur.s[0];
        const float s_hi = 2 * seg + 1 < kbl ? cur.s[1] : 0.f;
        // rotate the prefetch queue and refill its tail
#pragma unroll
        for (int d = 0; d + 1 < D; ++d)
            g[d] = g[d + 1];
        if (seg + D < nseg)
            load(g[D - 1], seg + D);
        if (seg == q_end) {
            // a new quarter: the previous one's pending block folds into
            // its own sum first
            if constexpr (BS) {
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    fold_block(acc[t], s_pend, p_pend[t]);
                    p_pend[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
                }
                s_pend = 0.f;
            }
            close_quarter();
            q_end += per;
        }
        __syncthreads();
        f32x4 p[2][T];      // partials of the segment's two K blocks (BS)
#pragma unroll
        for (int u = 0; u < GV_SEG / 64; ++u) {
            // lane (col, grp): activation row col, k = 64u + 16 grp .. +15
            const uint16_t *xp = &sx[buf][col * GV_XPITCH + 64 * u + 16 * grp];
            u32x4 xa = *reinterpret_cast<const u32x4 *>(xp);
            u32x4 xb = *reinterpret_cast<const u32x4 *>(xp + 8);
#pragma unroll
            for (int t = 0; t < T; ++t) {
                u32x4 wv = *reinterpret_cast<const u32x4 *>(
                    &sw[wave][(16 * t + col) * GV_WPITCH + 64 * u + 16 * grp]);
                bf16x8 blo, bhi;
                fp8x16_to_bf16(wv, blo, bhi);
                if constexpr (BS) {
                    f32x4 &pb = p[u / 2][t];
                    if (u % 2 == 0)
                        pb = (f32x4){0.f, 0.f, 0.f, 0.f};
                    pb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa), blo, pb, 0, 0, 0);
                    pb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xb), bhi, pb, 0, 0, 0);
                } else {
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa), blo, acc[t], 0, 0, 0);
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xb), bhi, acc[t], 0, 0, 0);
                }
            }
            if constexpr (BS) {
                // Folds trail the MFMAs that produce them by one K step, so
                // the MFMA results are not waited for: the previous
                // segment's second block after this segment's first step,
                // this segment's first block after its third step.  The
                // order of the additions is still block by block along K.
                if (u == 0)
#pragma unroll
                    for (int t = 0; t < T; ++t)
                        fold_block(acc[t], s_pend, p_pend[t]);
                if (u == 2)
#pragma unroll
                    for (int t = 0; t < T; ++t)
                        fold_block(acc[t], s_lo, p[0][t]);
            }
        }
        if constexpr (BS) {
#pragma unroll
            for (int t = 0; t < T; ++t)
                p_pend[t] = p[1][t];
            s_pend = s_hi;
        }
    }
    if constexpr (BS)
#pragma unroll
        for (int t = 0; t < T; ++t)
            fold_block(acc[t], s_pend, p_pend[t]);
    while (closed < 4)
        close_quarter();

#pragma unroll
    for (int t = 0; t < T; ++t) {
        uint32_t nn = row0 + 16u * t + col;
        if (nn < n) {
            float sc = BS ? 1.0f : rs[nn];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t mm = 4u * grp + i;
                if (mm < m)
                    out[(size_t)mm * n + nn] =
                        (uint16_t)f32_to_bf16(BS ? tot[t][i] : tot[t][i] * sc);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Narrow weights: too few rows to give every CU several workgroups, so the
// four waves of a workgroup share its rows and split K into contiguous
// quarters (ending on 256-element boundaries).  Everything is wave-private
// (the weight transpose tile and the activation segment live in the wave's
// own LDS region, so the loop has no barrier), D segments of SEG K elements
// are loaded ahead, and the four partial tiles are added in a fixed order at
// the end.
//
// A workgroup has a capacity of RC rows (8, 12, or a multiple of 16 up to
// 80: RC / 16 MFMA row tiles) of which the first rpw are live; rows past
// them read zero.  The launcher sizes rpw so that the grid is a whole number of
// workgroups per CU.  Below 16 rows (RC = 8 or 12) the MFMA's weight rows
// RC..15 read an all-zero LDS row.  XR activation rows are loaded per segment (M <= XR);
// the rows past them likewise read a zero row.  None of RC, rpw, XR, D and
// SEG changes any summation order.
//
// Every load is a raw buffer load from a 32-bit offset (n*k < 2^31,
// m*k < 2^31).  Rows past N, bytes past K, activation rows past M and
// segments outside the wave's K range take an offset past the end of the
// buffer, which reads zero without touching memory: no load sits under a
// branch, so the compiler counts the loads in flight exactly and waits only
// for the stage it is about to use.
// ---------------------------------------------------------------------------
template <int RC, int NW, int NX, int NS>
struct GvSegK {
    u32x4 w[NW];         // RC weight rows of the segment, 1 KB per instruction
    u32x4 x[NX];         // XR activation rows of the segment, 1 KB per instruction
    float s[NS][2];      // BS: per row tile, the block scales of the lane's row for
                         // the segment's two K blocks
};

template <int RC, int XR, int D, bool BS, int SEG>
__global__ __launch_bounds__(256) void k_fp8_gemv_ksplit(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ w,
    const float *__restrict__ rs, uint16_t *__restrict__ out,
    uint32_t m, uint32_t n, uint32_t k, uint32_t rpw)
{
    // RC rows of capacity per workgroup, of which the first rpw are live
    constexpr int R = RC;
    static_assert(RC == 8 || (RC == 12 && SEG == 256) || (RC % 16 == 0 && RC <= 80),
                  "8, 12 (256-element segments) or a multiple of 16 up to 80 rows");
    static_assert(XR == 2 || XR == 4 || XR == 8 || XR == 16, "2, 4, 8 or 16 activation rows");
    static_assert(SEG == 256 || (SEG == 128 && !BS), "256-element segments, or 128 without block scales");
    // MFMA weight tiles of 16 rows (R = 8: one, its rows 8..15 zero)
    constexpr int NT = R < 16 ? 1 : R / 16;
    // 16-byte chunks per weight row and 8-element chunks per activation row
    // of a segment; rows one load instruction covers
    constexpr int WCH = SEG / 16, XCH = SEG / 8;
    constexpr int WRPI = 64 / WCH, XRPI = 64 / XCH;
    constexpr int NW = R / WRPI, NX = (XR + XRPI - 1) / XRPI;
    constexpr int WPITCH = SEG + 16, XPITCH = SEG + 8;
    // per wave: R weight rows + a zero row; XR activation rows + a zero row
    constexpr int WROWS = R < 16 ? R + 1 : R, XROWS = XR < 16 ? XR + 1 : 16;
    __shared__ __attribute__((aligned(16))) uint8_t sw[4][WROWS * WPITCH];
    __shared__ __attribute__((aligned(16))) uint16_t sx[4][XROWS * XPITCH];
    __shared__ f32x4 red[3][NT][WAVE];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const uint32_t row0 = blockIdx.x * rpw;
    // K quarters end on 256-element boundaries whatever SEG is, so that a
    // row's summation order never depends on the launch shape.
    const uint32_t per = ((k + 255) / 256 + 3) / 4 * (256 / SEG);
    const uint32_t nseg = (k + SEG - 1) / SEG;
    const uint32_t s_beg = min(nseg, per * wave), s_end = min(nseg, s_beg + per);
    const uint32_t kbl = k / 128;

    constexpr uint32_t OOB = 0x80000000u;
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc((void *)w, 0, n * k, 0x00020000);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc((void *)x, 0, 2 * m * k, 0x00020000);
    const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)rs, 0, BS ? 4 * (n / 128) * kbl : 4 * n, 0x00020000);
    // BS: the scale-grid offsets of the lane's weight row in each row tile
    // (a workgroup's rows may span two 128-row scale blocks); dead rows
    // read zero scales, which multiply their zero partials.
    constexpr int NS = BS ? NT : 1;
    uint32_t sbo[NS];
#pragma unroll
    for (int t = 0; t < NS; ++t) {
        const uint32_t rl = 16 * t + col, r = row0 + rl;
        sbo[t] = BS && rl < rpw && r < n ? 4 * (r / 128) * kbl : OOB;
    }

    // weight instruction j: row WRPI j + lane / WCH, bytes 16 (lane % WCH)
    // .. +15 of the segment
    const int wc = lane % WCH, wr0 = lane / WCH;
    uint32_t wofs[NW];
#pragma unroll
    for (int j = 0; j < NW; ++j) {
        const uint32_t rl = WRPI * j + wr0, r = row0 + rl;
        wofs[j] = rl < rpw && r < n ? r * k + 16 * wc : OOB;
    }
    // activation instruction i: row XRPI i + lane / XCH, elements
    // 8 (lane % XCH) .. +7 of the segment
    const int xc = lane % XCH, xr0 = lane / XCH;
    uint32_t xofs[NX];
#pragma unroll
    for (int i = 0; i < NX; ++i) {
        const uint32_t r = XRPI * i + xr0;
        xofs[i] = r < m ? 2 * (r * k + 8 * xc) : OOB;
    }

    auto load = [&](GvSegK<RC, NW, NX, NS> &g, uint32_t seg) {
        const bool live = seg < s_end;
        const uint32_t kb = seg * SEG;
        if constexpr (BS) {
#pragma unroll
            for (int t = 0; t < NS; ++t) {
                g.s[t][0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                    sr, live ? sbo[t] + 8 * seg : OOB, 0, 0));
                g.s[t][1] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                    sr, live && 2 * seg + 1 < kbl ? sbo[t] + 8 * seg + 4 : OOB, 0, 0));
            }
        }
        const bool wlive = live && kb + 16 * wc < k;
#pragma unroll
        for (int j = 0; j < NW; ++j)
            g.w[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                wr, wlive ? wofs[j] + kb : OOB, 0, 2));
        const bool xlive = live && kb + 8 * xc < k;
#pragma unroll
        for (int i = 0; i < NX; ++i)
            g.x[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                xr, xlive ? xofs[i] + 2 * kb : OOB, 0, 0));
    };
    auto stash = [&](const GvSegK<RC, NW, NX, NS> &g) {
#pragma unroll
        for (int j = 0; j < NW; ++j)
            *reinterpret_cast<u32x4 *>(&sw[wave][(WRPI * j + wr0) * WPITCH + 16 * wc]) = g.w[j];
#pragma unroll
        for (int i = 0; i < NX; ++i)
            if (XRPI * (i + 1) <= XROWS || XRPI * i + xr0 < XROWS)
                *reinterpret_cast<u32x4 *>(&sx[wave][(XRPI * i + xr0) * XPITCH + 8 * xc]) = g.x[i];
    };
    // The lanes of a wave exchange data through its LDS region with no
    // barrier (a wave's LDS operations execute in order).  The compiler
    // does not know that other lanes wrote what a lane reads, so a
    // wavefront-scope fence (no instruction) separates each stash from the
    // reads around it: without it, where a lane skips a stash store the
    // compiler may reuse that lane's previous read of the same address.
    auto wave_fence = [] { __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront"); };
    // the zero rows (written once; stash never touches them)
    if constexpr (R < 16)
        if (lane < WPITCH / 16)
            *reinterpret_cast<u32x4 *>(&sw[wave][R * WPITCH + 16 * lane]) = (u32x4){0, 0, 0, 0};
    if constexpr (XR < 16)
        if (lane < XPITCH / 8)
            *reinterpret_cast<u32x4 *>(&sx[wave][XR * XPITCH + 8 * lane]) = (u32x4){0, 0, 0, 0};
    // the LDS rows this lane's MFMA operands come from (weight tile t: row
    // wrow + 16 t)
    const int wrow = R < 16 && col >= R ? R : col;
    const int xrow = XR < 16 && col >= XR ? XR : col;

    f32x4 acc[NT];
    // BS: the last block partial not yet folded, and its scale (a zero
    // partial with scale 0 before the first segment)
    f32x4 p_pend[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        acc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
        p_pend[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
    float s_pend[NS];
#pragma unroll
    for (int t = 0; t < NS; ++t)
        s_pend[t] = 0.f;

    // D stages in flight.  The loop is unrolled by D so every stage is a
    // statically named variable: stage d holds segment seg + d, and is
    // reloaded with segment seg + d + D as soon as it has been stashed.
    GvSegK<RC, NW, NX, NS> g[D];
#pragma unroll
    for (int d = 0; d < D; ++d)
        load(g[d], s_beg + d);

    for (uint32_t seg0 = s_beg; seg0 < s_end; seg0 += D)
#pragma unroll
    for (int d = 0; d < D; ++d) {
        const uint32_t seg = seg0 + d;
        if (seg >= s_end)
            break;
        wave_fence();
        stash(g[d]);
        wave_fence();
        // The second block of a segment may lie past K (K an odd number of
        // 128-blocks); its scale then reads zero and its zero partial adds
        // nothing.
        float s_lo[NS], s_hi[NS];
#pragma unroll
        for (int t = 0; t < NS; ++t) {
            s_lo[t] = g[d].s[t][0];
            s_hi[t] = g[d].s[t][1];
        }
        load(g[d], seg + D);
        f32x4 p[2][NT];     // partials of the segment's two K blocks (BS)
#pragma unroll
        for (int u = 0; u < SEG / 64; ++u) {
            const uint16_t *xp = &sx[wave][xrow * XPITCH + 64 * u + 16 * grp];
            const u32x4 xa = *reinterpret_cast<const u32x4 *>(xp);
            const u32x4 xb = *reinterpret_cast<const u32x4 *>(xp + 8);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const u32x4 wv = *reinterpret_cast<const u32x4 *>(
                    &sw[wave][(wrow + 16 * t) * WPITCH + 64 * u + 16 * grp]);
                bf16x8 blo, bhi;
                fp8x16_to_bf16(wv, blo, bhi);
                if constexpr (BS) {
                    f32x4 &pb = p[u / 2][t];
                    if (u % 2 == 0)
                        pb = (f32x4){0.f, 0.f, 0.f, 0.f};
                    pb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa), blo, pb, 0, 0, 0);
                    pb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xb), bhi, pb, 0, 0, 0);
                    // Folds trail the MFMAs that produce them by one K step,
                    // so the MFMA results are not waited for: the previous
                    // segment's second block after this segment's first
                    // step, this segment's first block after its third step.
                    // The order of the additions is still block by block
                    // along K.
                    if (u == 0)
                        fold_block(acc[t], s_pend[t], p_pend[t]);
                    if (u == 2)
                        fold_block(acc[t], s_lo[t], p[0][t]);
                } else {
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa), blo, acc[t], 0, 0, 0);
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xb), bhi, acc[t], 0, 0, 0);
                }
            }
        }
        if constexpr (BS) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                p_pend[t] = p[1][t];
                s_pend[t] = s_hi[t];
            }
        }
    }
    if constexpr (BS)
#pragma unroll
        for (int t = 0; t < NT; ++t)
            fold_block(acc[t], s_pend[t], p_pend[t]);

    // Fixed-order reduction of the four K-quarter partial tiles.
    if (wave > 0)
#pragma unroll
        for (int t = 0; t < NT; ++t)
            red[wave - 1][t][lane] = acc[t];
    __syncthreads();
    if (wave != 0)
        return;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int v = 0; v < 3; ++v)
            acc[t] += red[v][t][lane];
        const uint32_t nn = row0 + 16 * t + col;
        if (16 * t + col < (int)rpw && nn < n) {
            const float sc = BS ? 1.0f : rs[nn];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t mm = 4u * grp + i;
                if (mm < m)
                    out[(size_t)mm * n + nn] =
                        (uint16_t)f32_to_bf16(BS ? acc[t][i] : acc[t][i] * sc);
            }
        }
    }
}

// Rows per workgroup.  Every workgroup reads the activation rows of its K
// range once, so more rows per workgroup means fewer activation bytes per
// weight byte; but a narrow grid is short (a few microseconds), and when
// some CUs get one workgroup more than others those CUs set the time (N =
// 17408 in 32-row workgroups is 544 of them on 256 CUs: 26.0 us, against
// 20.1 us for N = 16384's 512).  So the rows follow M:
//   - M <= 2: 12 rows in a 12-row capacity (the weight dominates and the
//     activation pair is small; at 12 rows the grid fits in the workgroups
//     the CUs hold at once, where 8 rows needed a second partial round: N =
//     17408, M = 1 / 2: 16.4 / 17.1 -> 16.2 / 16.6 us, N = 6144 equal or 1%
//     faster);
// and above M = 2 the grid is a whole number j of workgroups per CU, each
// with rpw = ceil(N / (j CUs)) live rows in a capacity of 8 or a multiple of
// 16 rows (up to 80), j following M:
//   - M <= 4: about 16 rows per workgroup (N = 6144: 12 rows on 512
//     workgroups, 8.4 -> 7.9 us);
//   - M <= 8: two workgroups per CU (N = 17408: 34 rows, 21.5 -> 19.6 us;
//     N = 6144: 12 rows, 9.6 -> 9.1 us);
//   - M <= 16: one workgroup per CU while its rows fit (N = 17408: 68 rows,
//     26.0 -> 22.0 us; N = 12288: 48 rows, 18.9 -> 16.4 us).
// The block-scaled form takes the same rows (each lane reads the scales of
// its own row's 128-row block), except that above M = 4 its 256-element
// segments would double the registers of the larger workgroups: there it
// takes them only up to 16 (M <= 8) or 32 rows, else 16 or 32 rows.  (Loading the activations straight
// into MFMA operand registers instead of through LDS was slower at every
// M > 2: each load instruction then touches 16 rows.)  None of these
// choices changes any row's summation order.
struct GvSplit {
    uint32_t rc, rpw;
};
static GvSplit gemv_split(uint32_t n, uint32_t m, bool bs)
{
    const uint32_t fixed = m <= 2 ? 8 : m <= 8 ? 16 : 32;
    const uint32_t cus = cu_count();
    if (cus == 0)
        return GvSplit{fixed, fixed};
    // M <= 2: 12 rows (N = 17408: 1451 workgroups, all resident at once);
    // wide weights 16 (lm_head, M = 2: 112.1 -> 110.8 us; block-scaled
    // M = 1 / 2: 110.9 -> 109.7 / 114.4 -> 111.5 us; 32 and 48 rows slower)
    if (m <= 2)
        return n >= 65536u ? GvSplit{16, 16} : GvSplit{12, 12};
    // the largest capacity: 80 rows, or 16 / 32 for the block-scaled form
    // above M = 4
    const uint32_t cap = m <= 4 ? 16 : bs ? fixed : 80;
    const uint32_t div = cus * cap;
    uint32_t j = (n + div - 1) / div;
    if (m > 4 && m <= 8 && j < 2)
        j = 2;
    uint32_t rpw = (n + cus * j - 1) / (cus * j);
    const uint32_t lo = m <= 4 ? 8 : 12;
    rpw = rpw < lo ? lo : rpw;
    return GvSplit{rpw <= 8 ? 8 : (rpw + 15) / 16 * 16, rpw};
}

// The (capacity, activation rows) pairs gemv_split can ask for; any other
// pair is an internal error, never a silent no-op.
template <int RC, int XR, bool BS>
constexpr bool ksplit_shape_ok()
{
    if (BS && XR > 4)
        return XR == 8 ? RC == 16 : RC == 16 || RC == 32;
    return XR == 2 ? RC == 8 || RC == 12 || RC == 16 : XR == 4 ? RC == 8 || RC == 16 : RC >= 16;
}

template <int RC, int XR, int D, bool BS, int SEG>
static hipError_t launch_ksplit_rc(const uint16_t *x, const uint8_t *w, const float *rs,
                                   uint16_t *out, uint32_t m, uint32_t n, uint32_t k,
                                   uint32_t rpw, hipStream_t st)
{
    if constexpr (ksplit_shape_ok<RC, XR, BS>()) {
        hipLaunchKernelGGL((k_fp8_gemv_ksplit<RC, XR, D, BS, (BS ? 256 : SEG)>),
                           dim3((n + rpw - 1) / rpw), dim3(256), 0, st, x, w, rs, out, m, n, k, rpw);
        return hipSuccess;
    } else {
        return hipErrorInvalidConfiguration;
    }
}

template <int XR, int D, bool BS, int SEG>
static hipError_t launch_ksplit_xr(const uint16_t *x, const uint8_t *w, const float *rs,
                                   uint16_t *out, uint32_t m, uint32_t n, uint32_t k,
                                   GvSplit sp, hipStream_t st)
{
    if (sp.rpw == 0 || sp.rpw > sp.rc)
        return hipErrorInvalidConfiguration;
    switch (sp.rc) {
    case 8: return launch_ksplit_rc<8, XR, D, BS, SEG>(x, w, rs, out, m, n, k, sp.rpw, st);
    case 12:
        if constexpr (SEG == 256)
            return launch_ksplit_rc<12, XR, D, BS, SEG>(x, w, rs, out, m, n, k, sp.rpw, st);
        return hipErrorInvalidConfiguration;
    case 16: return launch_ksplit_rc<16, XR, D, BS, SEG>(x, w, rs, out, m, n, k, sp.rpw, st);
    case 32: return launch_ksplit_rc<32, XR, D, BS, SEG>(x, w, rs, out, m, n, k, sp.rpw, st);
    case 48: return launch_ksplit_rc<48, XR, D, BS, SEG>(x, w, rs, out, m, n, k, sp.rpw, st);
    case 64: return launch_ksplit_rc<64, XR, D, BS, SEG>(x, w, rs, out, m, n, k, sp.rpw, st);
    case 80: return launch_ksplit_rc<80, XR, D, BS, SEG>(x, w, rs, out, m, n, k, sp.rpw, st);
    default: return hipErrorInvalidConfiguration;
    }
}

template <int D, bool BS, int SEG_SMALL, int SEG_BIG>
static hipError_t launch_gemv_ksplit(const uint16_t *x, const uint8_t *w, const float *rs,
                                     uint16_t *out, uint32_t m, uint32_t n, uint32_t k,
                                     hipStream_t st)
{
    const GvSplit sp = gemv_split(n, m, BS);
    if (m <= 2)
        return launch_ksplit_xr<2, D, BS, SEG_SMALL>(x, w, rs, out, m, n, k, sp, st);
    if (m <= 4)
        return launch_ksplit_xr<4, D, BS, SEG_SMALL>(x, w, rs, out, m, n, k, sp, st);
    if (m <= 8)
        return launch_ksplit_xr<8, D, BS, SEG_BIG>(x, w, rs, out, m, n, k, sp, st);
    return launch_ksplit_xr<16, D, BS, SEG_BIG>(x, w, rs, out, m, n, k, sp, st);
}

template <int T, int D, bool BS>
static void launch_gemv_rows(const uint16_t *x, const uint8_t *w, const float *rs,
                             uint16_t *out, uint32_t m, uint32_t n, uint32_t k,
                             hipStream_t st)
{
    constexpr uint32_t rows_wg = 64 * T;
    uint32_t grid = (n + rows_wg - 1) / rows_wg;
    hipLaunchKernelGGL((k_fp8_gemv_rows<T, D, BS>), dim3(grid), dim3(256), 0, st,
                       x, w, rs, out, m, n, k);
}

// Work-split choice.  Wide weights (lm_head-class) give every CU several
// row-split workgroups; narrow ones split K inside the workgroup to keep
// enough waves streaming.  The two kernels sum every row in the same order,
// so the choice, which may follow m, never changes a row's bits.
static bool gemv_wide(uint32_t n) { return n >= 65536u; }
// The row-owning kernel serves wide weights except at M <= 2, where the
// K-split kernel reads them faster (lm_head, M = 1 / 2: 115.4 -> 110.1 /
// 116.0 -> 112.5 us row-scaled, 116.3 -> 111.4 / 116.6 -> 114.6 us
// block-scaled; at M = 4 and 8 it is slower, its many small workgroups each
// reading the activation rows).  Both kernels sum every row in the same
// order, so the choice changes no bits.
static bool gemv_rows(uint32_t n, uint32_t m) { return gemv_wide(n) && m > 2; }

// Segments in flight per wave for the K-split kernel: two once the grid has
// several workgroups per CU (measured: N = 17408 gains 4-5% at every M,
// N = 6144 loses 0-3%), together with 128-element segments above M = 4
// (half the LDS per workgroup, so more workgroups stay resident: N = 17408,
// M = 16 26.9 -> 25.9 us; at N = 6144 and at M <= 4 they measured equal or
// slower).  Neither the depth nor the segment size changes any summation
// order.
template <bool BS>
static hipError_t launch_gemv_narrow(const uint16_t *x, const uint8_t *w, const float *rs,
                                     uint16_t *out, uint32_t m, uint32_t n, uint32_t k,
                                     hipStream_t st)
{
    if (n >= 12288u)
        return launch_gemv_ksplit<2, BS, 256, 128>(x, w, rs, out, m, n, k, st);
    return launch_gemv_ksplit<1, BS, 256, 256>(x, w, rs, out, m, n, k, st);
}

hipError_t launch_fp8_gemv_rowscale(const uint16_t *x, const uint8_t *w,
                                    const float *rs, uint16_t *out, uint32_t m,
                                    uint32_t n, uint32_t k, hipStream_t st)
{
    if (gemv_rows(n, m)) {
        launch_gemv_rows<2, 1, false>(x, w, rs, out, m, n, k, st);
    } else {
        const hipError_t e = launch_gemv_narrow<false>(x, w, rs, out, m, n, k, st);
        if (e != hipSuccess)
            return e;
    }
    count_launch();
    return hipGetLastError();
}

// n % 128 == 0 and k % 128 == 0 (checked by the caller).
hipError_t launch_fp8_gemv_blockscale(const uint16_t *x, const uint8_t *w,
                                      const float *grid, uint16_t *out, uint32_t m,
                                      uint32_t n, uint32_t k, hipStream_t st)
{
    if (gemv_rows(n, m)) {
        launch_gemv_rows<2, 1, true>(x, w, grid, out, m, n, k, st);
    } else {
        const hipError_t e = launch_gemv_narrow<true>(x, w, grid, out, m, n, k, st);
        if (e != hipSuccess)
            return e;
    }
    count_launch();
    return hipGetLastError();
}

} // namespace qp
