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
//  * Two work splits, chosen from N alone (see gemv_wide): wide weights give
//    each wave its own rows over all of K, with the activation segment staged
//    once per workgroup in LDS and shared by its four waves; narrow weights
//    split K over the four waves of a workgroup (everything wave-private) and
//    add the partial tiles in a fixed order.  The narrow kernel's launch
//    shape (8 or 16 rows per workgroup, activation rows loaded, segments in
//    flight) may follow M, but no summation order depends on M, so every
//    output row is bit-identical to an M = 1 call on that row.
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
                        (uint16_t)f32_to_bf16(BS ? acc[t][i] : acc[t][i] * sc);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Narrow weights: too few rows to give every CU several workgroups, so the
// four waves of a workgroup share R rows (8 or 16) and split K into
// contiguous quarters.  Everything is wave-private (the weight transpose tile
// and the activation segment live in the wave's own LDS region, so the loop
// has no barrier), D segments are loaded ahead, and the four partial tiles
// are added in a fixed order at the end.
//
// R = 8 halves the work unit so that narrow weights spread evenly over the
// CUs (N = 6144: 768 workgroups, three per CU, against 384 of 16 rows); the
// MFMA's weight rows 8..15 then read an all-zero LDS row.  XP is the number
// of activation row pairs loaded per segment (M <= 2 XP); the rows past them
// likewise read a zero row.  Neither changes any summation order.
//
// Every load is a raw buffer load from a 32-bit offset (n*k < 2^31,
// m*k < 2^31).  Rows past N, bytes past K, activation rows past M and
// segments outside the wave's K range take an offset past the end of the
// buffer, which reads zero without touching memory: no load sits under a
// branch, so the compiler counts the loads in flight exactly and waits only
// for the stage it is about to use.
// ---------------------------------------------------------------------------
template <int R, int XP>
struct GvSegK {
    u32x4 w[R / 4];      // R rows x 256 B, 4 rows per instruction
    u32x4 x[XP];         // 2 XP rows x 256 bf16, 16 B per lane and row pair
    float s[2];          // block scales of the segment's two K blocks (BS)
};

template <int R, int XP, int D, bool BS>
__global__ __launch_bounds__(256) void k_fp8_gemv_ksplit(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ w,
    const float *__restrict__ rs, uint16_t *__restrict__ out,
    uint32_t m, uint32_t n, uint32_t k)
{
    static_assert(R == 8 || R == 16, "8 or 16 rows per workgroup");
    static_assert(XP == 1 || XP == 2 || XP == 4 || XP == 8, "1, 2, 4 or 8 row pairs");
    // per wave: R weight rows + a zero row; 2 XP activation rows + a zero row
    constexpr int WROWS = R < 16 ? R + 1 : 16, XROWS = XP < 8 ? 2 * XP + 1 : 16;
    __shared__ __attribute__((aligned(16))) uint8_t sw[4][WROWS * GV_WPITCH];
    __shared__ __attribute__((aligned(16))) uint16_t sx[4][XROWS * GV_XPITCH];
    __shared__ f32x4 red[3][WAVE];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const uint32_t row0 = blockIdx.x * R;
    const uint32_t nseg = (k + GV_SEG - 1) / GV_SEG;
    const uint32_t per = (nseg + 3) / 4;
    const uint32_t s_beg = min(nseg, per * wave), s_end = min(nseg, s_beg + per);
    const uint32_t kbl = k / 128;

    constexpr uint32_t OOB = 0x80000000u;
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc((void *)w, 0, n * k, 0x00020000);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc((void *)x, 0, 2 * m * k, 0x00020000);
    const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)rs, 0, BS ? 4 * (n / 128) * kbl : 4 * n, 0x00020000);
    const uint32_t sbase = BS ? 4 * (row0 / 128) * kbl : 0;

    // weight instruction j: row 4j + grp, bytes 16 col .. +15 of the segment
    uint32_t wofs[R / 4];
#pragma unroll
    for (int j = 0; j < R / 4; ++j) {
        const uint32_t r = row0 + 4 * j + grp;
        wofs[j] = r < n ? r * k + 16 * col : OOB;
    }
    // activation chunk c = lane + 64 i: row c / 32, elements 8 (c % 32) .. +7
    uint32_t xofs[XP];
#pragma unroll
    for (int i = 0; i < XP; ++i) {
        const int c = lane + 64 * i, r = c >> 5;
        xofs[i] = (uint32_t)r < m ? 2 * ((uint32_t)r * k + 8 * (c & 31)) : OOB;
    }

    auto load = [&](GvSegK<R, XP> &g, uint32_t seg) {
        const bool live = seg < s_end;
        const uint32_t kb = seg * GV_SEG;
        if constexpr (BS) {
            g.s[0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                sr, live ? sbase + 8 * seg : OOB, 0, 0));
            g.s[1] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                sr, live && 2 * seg + 1 < kbl ? sbase + 8 * seg + 4 : OOB, 0, 0));
        }
        const bool wlive = live && kb + 16 * col < k;
#pragma unroll
        for (int j = 0; j < R / 4; ++j)
            g.w[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                wr, wlive ? wofs[j] + kb : OOB, 0, 2));
#pragma unroll
        for (int i = 0; i < XP; ++i) {
            const int c = lane + 64 * i;
            g.x[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                xr, live && kb + 8 * (c & 31) < k ? xofs[i] + 2 * kb : OOB, 0, 0));
        }
    };
    auto stash = [&](const GvSegK<R, XP> &g) {
#pragma unroll
        for (int j = 0; j < R / 4; ++j)
            *reinterpret_cast<u32x4 *>(&sw[wave][(4 * j + grp) * GV_WPITCH + 16 * col]) = g.w[j];
#pragma unroll
        for (int i = 0; i < XP; ++i) {
            const int c = lane + 64 * i;
            *reinterpret_cast<u32x4 *>(&sx[wave][(c >> 5) * GV_XPITCH + 8 * (c & 31)]) = g.x[i];
        }
    };
    // the zero rows (written once; stash never touches them)
    if constexpr (R < 16)
        if (lane < GV_WPITCH / 16)
            *reinterpret_cast<u32x4 *>(&sw[wave][R * GV_WPITCH + 16 * lane]) = (u32x4){0, 0, 0, 0};
    if constexpr (XP < 8)
        if (lane < GV_XPITCH / 8)
            *reinterpret_cast<u32x4 *>(&sx[wave][2 * XP * GV_XPITCH + 8 * lane]) = (u32x4){0, 0, 0, 0};
    // the LDS rows this lane's MFMA operands come from
    const int wrow = R < 16 && col >= R ? R : col;
    const int xrow = XP < 8 && col >= 2 * XP ? 2 * XP : col;

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    // BS: the last block partial not yet folded, and its scale (a zero
    // partial with scale 0 before the first segment)
    f32x4 p_pend = {0.f, 0.f, 0.f, 0.f};
    float s_pend = 0.f;

    // D stages in flight.  The loop is unrolled by D so every stage is a
    // statically named variable: stage d holds segment seg + d, and is
    // reloaded with segment seg + d + D as soon as it has been stashed.
    GvSegK<R, XP> g[D];
#pragma unroll
    for (int d = 0; d < D; ++d)
        load(g[d], s_beg + d);

    for (uint32_t seg0 = s_beg; seg0 < s_end; seg0 += D)
#pragma unroll
    for (int d = 0; d < D; ++d) {
        const uint32_t seg = seg0 + d;
        if (seg >= s_end)
            break;
        stash(g[d]);
        // The second block of a segment may lie past K (K an odd number of
        // 128-blocks); its scale then reads zero and its zero partial adds
        // nothing.
        const float s_lo = g[d].s[0];
        const float s_hi = g[d].s[1];
        load(g[d], seg + D);
        f32x4 p[2];         // partials of the segment's two K blocks (BS)
#pragma unroll
        for (int u = 0; u < GV_SEG / 64; ++u) {
            const uint16_t *xp = &sx[wave][xrow * GV_XPITCH + 64 * u + 16 * grp];
            const u32x4 xa = *reinterpret_cast<const u32x4 *>(xp);
            const u32x4 xb = *reinterpret_cast<const u32x4 *>(xp + 8);
            const u32x4 wv = *reinterpret_cast<const u32x4 *>(
                &sw[wave][wrow * GV_WPITCH + 64 * u + 16 * grp]);
            bf16x8 blo, bhi;
            fp8x16_to_bf16(wv, blo, bhi);
            if constexpr (BS) {
                f32x4 &pb = p[u / 2];
                if (u % 2 == 0)
                    pb = (f32x4){0.f, 0.f, 0.f, 0.f};
                pb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa), blo, pb, 0, 0, 0);
                pb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xb), bhi, pb, 0, 0, 0);
                // Folds trail the MFMAs that produce them by one K step, so
                // the MFMA results are not waited for: the previous
                // segment's second block after this segment's first step,
                // this segment's first block after its third step.  The
                // order of the additions is still block by block along K.
                if (u == 0)
                    fold_block(acc, s_pend, p_pend);
                if (u == 2)
                    fold_block(acc, s_lo, p[0]);
            } else {
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa), blo, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xb), bhi, acc, 0, 0, 0);
            }
        }
        if constexpr (BS) {
            p_pend = p[1];
            s_pend = s_hi;
        }
    }
    if constexpr (BS)
        fold_block(acc, s_pend, p_pend);

    // Fixed-order reduction of the four K-quarter partial tiles.
    if (wave > 0)
        red[wave - 1][lane] = acc;
    __syncthreads();
    if (wave != 0)
        return;
#pragma unroll
    for (int v = 0; v < 3; ++v)
        acc += red[v][lane];
    const uint32_t nn = row0 + col;
    if (col < R && nn < n) {
        const float sc = BS ? 1.0f : rs[nn];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t mm = 4u * grp + i;
            if (mm < m)
                out[(size_t)mm * n + nn] = (uint16_t)f32_to_bf16(BS ? acc[i] : acc[i] * sc);
        }
    }
}

// Rows per workgroup and activation row pairs follow M: at M <= 2 the
// 8-row unit spreads the weight evenly over the CUs; from M = 3 on, the
// activation rows every workgroup loads outweigh the balance, and 16 rows
// halve them (measured on N = 6144 and 17408).  Neither choice changes any
// row's summation order.
template <int D, bool BS>
static void launch_gemv_ksplit(const uint16_t *x, const uint8_t *w, const float *rs,
                               uint16_t *out, uint32_t m, uint32_t n, uint32_t k,
                               hipStream_t st)
{
#define QP_GEMV_KSPLIT(R, XP)                                                             \
    hipLaunchKernelGGL((k_fp8_gemv_ksplit<R, XP, D, BS>), dim3((n + R - 1) / R), dim3(256), \
                       0, st, x, w, rs, out, m, n, k)
    if (m <= 2)
        QP_GEMV_KSPLIT(8, 1);
    else if (m <= 4)
        QP_GEMV_KSPLIT(16, 2);
    else if (m <= 8)
        QP_GEMV_KSPLIT(16, 4);
    else
        QP_GEMV_KSPLIT(16, 8);
#undef QP_GEMV_KSPLIT
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

// Work-split choice: it depends on n only (never on m), which keeps every
// row's summation order, and so its bits, the same for every m.  Wide
// weights (lm_head-class) give every CU several row-split workgroups; narrow
// ones split K inside the workgroup to keep enough waves streaming.
static bool gemv_wide(uint32_t n) { return n >= 65536u; }

// Segments in flight per wave for the K-split kernel: two once the grid has
// several workgroups per CU (measured: N = 17408 gains 4-5% at every M,
// N = 6144 loses 0-3%).  The depth changes no summation order.
template <bool BS>
static void launch_gemv_narrow(const uint16_t *x, const uint8_t *w, const float *rs,
                               uint16_t *out, uint32_t m, uint32_t n, uint32_t k,
                               hipStream_t st)
{
    if (n >= 12288u)
        launch_gemv_ksplit<2, BS>(x, w, rs, out, m, n, k, st);
    else
        launch_gemv_ksplit<1, BS>(x, w, rs, out, m, n, k, st);
}

hipError_t launch_fp8_gemv_rowscale(const uint16_t *x, const uint8_t *w,
                                    const float *rs, uint16_t *out, uint32_t m,
                                    uint32_t n, uint32_t k, hipStream_t st)
{
    if (gemv_wide(n))
        launch_gemv_rows<2, 1, false>(x, w, rs, out, m, n, k, st);
    else
        launch_gemv_narrow<false>(x, w, rs, out, m, n, k, st);
    count_launch();
    return hipGetLastError();
}

// n % 128 == 0 and k % 128 == 0 (checked by the caller).
hipError_t launch_fp8_gemv_blockscale(const uint16_t *x, const uint8_t *w,
                                      const float *grid, uint16_t *out, uint32_t m,
                                      uint32_t n, uint32_t k, hipStream_t st)
{
    if (gemv_wide(n))
        launch_gemv_rows<2, 1, true>(x, w, grid, out, m, n, k, st);
    else
        launch_gemv_narrow<true>(x, w, grid, out, m, n, k, st);
    count_launch();
    return hipGetLastError();
}

} // namespace qp
