// gemv_w4a16.hip -- NVFP4-weight GEMV (W4A16) for decode / verify batches
// (M <= 8) on gfx950 (fp8_gemv_batch.rs names w4a16_gemv_batch8_rt2 as the
// NVFP4-weight twin of the register-tiled row-scaled FP8 GEMV).
//
//   C[i,j] = bf16( scale2 * sum_t x[i,t] * e2m1(w[j,t]) * e4m3(s[j,t/16]) )
//
// x [M,K] BF16; the weight is E2M1 codes packed [N,K/2] (element 2t in the
// low nibble of byte t) with one E4M3 scale per 16 elements [N,K/16] and a
// per-tensor F32 scale2.
//
// Design (MI355X-first):
//  * The contraction runs on v_mfma_f32_4x4x4_16b_bf16: 16 independent
//    4x4x4 blocks per instruction.  Here the 16 blocks are 16 K-slices of the
//    same 4 weight rows and 4 activation rows, so one MFMA covers 64 K
//    elements, and the block results are summed once at the end (a fixed
//    butterfly over lanes).  Lane l supplies column l%4 of block l/4 of the
//    weight operand and row l%4 of block l/4 of the activation operand, and
//    receives column l%4 of block l/4 of the result: all four of its results
//    belong to one weight row.
//  * Dequantisation by folding the scale.  A lane's 32 consecutive elements
//    of one weight row are exactly two 16-element scale blocks.  The E2M1
//    codes go to BF16 exactly with the hardware converter at unit scale;
//    the 4 MFMAs of one block accumulate into a fresh F32 partial, which is
//    added to the running sum with one FMA per result by the block's
//    decoded E4M3 scale.  Per 32 weight elements a lane spends 16
//    conversions, 2 scale decodes and 8 FMAs (the converters' own scale
//    operand applies only the power-of-two part of a scale, and gfx950 has
//    no packed BF16 multiply, so scaling each element would cost twice
//    that).  scale2 multiplies the F32 sum at write-out.
//  * That layout also lets one 64-lane load feed the MFMAs directly: lane l
//    loads 16 bytes (32 elements) of weight row l%4 at byte 16 (l/4) of a
//    256-byte window, so every load instruction covers 4 rows x 256
//    contiguous bytes -- the burst HBM serves best -- and the weights need
//    no LDS transpose.  A lane needs 2 scale bytes per window; the workgroup
//    stages its rows' scale bytes for two windows at a time in LDS.
//  * Activations: for each 512-element window, lane l uses 32 elements of
//    activation row 4g + l%4 (M group g) for every weight row group of the
//    wave.  The four waves of a workgroup stage the window in LDS once
//    (double-buffered, one barrier per window) instead of each fetching it
//    from L2.
//  * Two register stages (four for small narrow grids) are used in turn, so
//    each wave keeps the next two (four) windows in flight.  Every load is a
//    raw buffer load: a lane whose data does not exist (rows >= n or >= m, K
//    past the end, a prefetch past the last window) gets an offset beyond
//    the buffer and reads zero without touching memory, so no load sits
//    under a branch.
//  * Each wave owns 4 or 8 rows (chosen from N alone) over all of K.  No
//    summation order depends on M, so every output row is bit-identical to
//    an M = 1 call on that row.
#include "qp_device.hpp"
#include "qp_launch.hpp"

namespace qp {

constexpr int W4_WIN = 512;                 // K elements per window
constexpr int W4_WB = W4_WIN / 2;           // packed bytes per row per window
constexpr int W4_SB = W4_WIN / 16;          // scale bytes per row per window

typedef __amdgpu_buffer_rsrc_t buf_rsrc;
typedef __attribute__((ext_vector_type(4))) short s16x4;

// Offsets >= W4_OOB lie beyond every buffer (each is < 2^30 bytes, checked
// by the caller); a base offset plus a window offset, either possibly
// W4_OOB, stays below 2^31.
constexpr uint32_t W4_OOB = 1u << 30;
constexpr int W4_NT = 2;                    // cache policy: nontemporal

__device__ __forceinline__ buf_rsrc make_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                             0x00020000);
}

// Four E2M1 codes (bytes SEL, SEL+1 of w; low nibble first) as BF16, exact.
template <int SEL>
__device__ __forceinline__ s16x4 fp4x4_bf16(uint32_t w)
{
    bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL);
    bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL + 1);
    return __builtin_bit_cast(s16x4, (u32x2){__builtin_bit_cast(uint32_t, lo),
                                             __builtin_bit_cast(uint32_t, hi)});
}

// Activation fragments of one window: 32 BF16 of row 4 g + l%4 per group.
template <int MG>
struct W4Act {
    u32x4 x[MG][4];
};

// One window's weights in registers (RG groups of 4 rows).
template <int RG>
struct W4Wts {
    u32x4 w[RG];            // 32 codes of weight row 4 rg + l%4
    uint32_t s[RG];         // its two block scales (low 16 bits)
};

// Per-lane load offsets at window 0 of one wave (rows row0 .. row0 + 4 RG - 1).
//   weights: lane l -> row 4 rg + l%4, bytes 16 (l/4) .. of the 256-byte window
template <int MG, int RG>
struct W4Src {
    buf_rsrc rw, rs, rx;
    uint32_t wo[RG];
    uint32_t kc;            // K index of the lane's chunk within a window

    __device__ __forceinline__ void init(const uint16_t *x, const uint8_t *wp, const uint8_t *ws,
                                         uint32_t row0, uint32_t rpv, uint32_t m, uint32_t n,
                                         uint32_t k, int lane)
    {
        rw = make_rsrc(wp, n * (k / 2));
        rs = make_rsrc(ws, n * (k / 16));
        rx = make_rsrc(x, m * k * 2);
        kc = 32 * (lane / 4);
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            uint32_t q = 4 * rg + lane % 4, r = row0 + q;
            wo[rg] = q < rpv && r < n ? r * (k / 2) + kc / 2 : W4_OOB;
        }
    }
    // The packed codes of window `win`; lanes whose 32-element chunk lies
    // past K (or every lane, when ok is false) read zero.  (Scale bytes are
    // staged in LDS by the workgroup.)
    __device__ __forceinline__ void load_w(W4Wts<RG> &g, uint32_t win, bool ok, uint32_t k) const
    {
        bool in = ok && win * W4_WIN + kc < k;
        uint32_t dw = in ? win * W4_WB : W4_OOB;
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
            g.w[rg] = __builtin_amdgcn_raw_buffer_load_b128(rw, wo[rg] + dw, 0, W4_NT);
    }
};

// One 16-element scale block (half H of the lane's chunk) of row group rg:
// 4 MFMAs into a fresh partial per M group, then acc += scale * partial.
template <int MG, int RG, int H>
__device__ __forceinline__ void w4_block(f32x4 *acc, const W4Wts<RG> &w, const W4Act<MG> &a, int rg)
{
    const float s = __builtin_amdgcn_cvt_f32_fp8((int)w.s[rg], H);
    s16x4 b[4];
    b[0] = fp4x4_bf16<0>(w.w[rg][2 * H]);
    b[1] = fp4x4_bf16<2>(w.w[rg][2 * H]);
    b[2] = fp4x4_bf16<0>(w.w[rg][2 * H + 1]);
    b[3] = fp4x4_bf16<2>(w.w[rg][2 * H + 1]);
    f32x4 p[MG];
#pragma unroll
    for (int g = 0; g < MG; ++g)
        p[g] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = 4 * H + i;        // activation elements 4e .. 4e+3 of the chunk
#pragma unroll
        for (int g = 0; g < MG; ++g) {
            u32x2 xa = (u32x2){a.x[g][e / 2][2 * (e % 2)], a.x[g][e / 2][2 * (e % 2) + 1]};
            p[g] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s16x4, xa), b[i],
                                                          p[g], 0, 0, 0);
        }
    }
#pragma unroll
    for (int g = 0; g < MG; ++g)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            acc[g][q] = __builtin_fmaf(s, p[g][q], acc[g][q]);
}

template <int MG, int RG>
__device__ __forceinline__ void w4_window(f32x4 (*acc)[MG], const W4Wts<RG> &w, const W4Act<MG> &a)
{
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        w4_block<MG, RG, 0>(acc[rg], w, a, rg);
        w4_block<MG, RG, 1>(acc[rg], w, a, rg);
    }
}

// Sum the 16 block results (lanes with equal l%4) with a fixed butterfly;
// lanes 0..3 end up with the totals.
template <int MG, int RG>
__device__ __forceinline__ void w4_block_sum(f32x4 (*acc)[MG])
{
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int g = 0; g < MG; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v = acc[rg][g][i];
                v += __shfl_xor(v, 4, WAVE);
                v += __shfl_xor(v, 8, WAVE);
                v += __shfl_xor(v, 16, WAVE);
                v += __shfl_xor(v, 32, WAVE);
                acc[rg][g][i] = v;
            }
}

// Lanes 0..3: C[4g + i][row0 + 4rg + lane] = bf16(acc * scale2), for the
// wave's rpv live rows.
template <int MG, int RG>
__device__ __forceinline__ void w4_store(f32x4 (*acc)[MG], float scale2, uint16_t *out,
                                         uint32_t row0, uint32_t rpv, uint32_t m, uint32_t n,
                                         int lane)
{
    if (lane >= 4)
        return;
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        uint32_t nn = row0 + 4 * rg + lane;
        if (4 * rg + lane >= (int)rpv || nn >= n)
            continue;
#pragma unroll
        for (int g = 0; g < MG; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t mm = 4 * g + i;
                if (mm < m)
                    out[(size_t)mm * n + nn] = (uint16_t)f32_to_bf16(acc[rg][g][i] * scale2);
            }
    }
}

template <int MG, int RG>
__device__ __forceinline__ void w4_zero(f32x4 (*acc)[MG])
{
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int g = 0; g < MG; ++g)
            acc[rg][g] = (f32x4){0.f, 0.f, 0.f, 0.f};
}

// ---------------------------------------------------------------------------
// Wide weights: each wave owns 4 RG rows over all of K.  The workgroup's four
// waves stage each activation window [4 MG rows x 512] in LDS together
// (thread t loads 16-byte chunks t, t + 256, ...), one barrier per window.
// ---------------------------------------------------------------------------
constexpr int W4_XPITCH = W4_WIN + 8;       // LDS bf16 per activation row
constexpr int W4_GW = 2;                    // windows per scale group
constexpr int W4_GB = W4_GW * W4_SB;        // scale bytes per row per group (64)

// Wide weights, scales: the workgroup loads the scale bytes of all its rows
// for a group of 2 windows (64 bytes per row, 8 bytes per thread) one group
// ahead and keeps them in LDS (double-buffered), instead of each lane
// fetching its own 2 bytes per window.  The one-group kernel is held to five
// waves per SIMD (<= 102 VGPRs); the two-group kernel is left to the
// compiler, whose unconstrained schedule keeps the scale and activation
// loads in flight across the window barrier (measured).
template <int MG, int RG, int ST>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MG == 1 && ST == 2 ? 5 : 1))) void k_w4a16_gemv_rows(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ wp,
    const uint8_t *__restrict__ ws, float scale2, uint16_t *__restrict__ out,
    uint32_t m, uint32_t n, uint32_t k, uint32_t rpv)
{
    // each wave holds ROWS rows, of which the first rpv are live
    static_assert(ST == 2 || ST == 4, "two or four register stages");
    constexpr int ROWS = 4 * RG;
    constexpr int WG_ROWS = 4 * ROWS;
    constexpr int XC = MG;                  // activation chunks per thread and window
    constexpr int SCH = (WG_ROWS * (W4_GB / 8) + 255) / 256;    // scale chunks per thread
    __shared__ __attribute__((aligned(16))) uint16_t sx[2][4 * MG * W4_XPITCH];
    __shared__ __attribute__((aligned(16))) uint8_t ss[2][WG_ROWS * W4_GB];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const uint32_t wg_row0 = blockIdx.x * 4 * rpv;
    const uint32_t row0 = wg_row0 + wave * rpv;
    const uint32_t nwin = (k + W4_WIN - 1) / W4_WIN;
    const uint32_t srow = k / 16;           // scale bytes per row

    W4Src<MG, RG> src;
    src.init(x, wp, ws, row0, rpv, m, n, k, lane);
    // staged activation chunk c = tid + 256 j: row c / 64, elements 8 (c % 64) ..
    buf_rsrc rx = src.rx;
    uint32_t xso[XC], xke[XC];
    int xlo[XC];
#pragma unroll
    for (int j = 0; j < XC; ++j) {
        int c = tid + 256 * j, r = c >> 6;
        xke[j] = 8 * (c & 63);
        xso[j] = (uint32_t)r < m ? (r * k + xke[j]) * 2 : W4_OOB;
        xlo[j] = r * W4_XPITCH + xke[j];
    }
    auto load_xs = [&](u32x4 *v, uint32_t win, bool ok) {
#pragma unroll
        for (int j = 0; j < XC; ++j) {
            uint32_t dx = ok && win * W4_WIN + xke[j] < k ? win * W4_WIN * 2 : W4_OOB;
            v[j] = __builtin_amdgcn_raw_buffer_load_b128(rx, xso[j] + dx, 0, 0);
        }
    };
    // staged scale chunk c = tid + 256 j: LDS row c / 8 (row q = c/8 % ROWS
    // of wave c/8 / ROWS, live if q < rpv), bytes 8 (c % 8) of the row's
    // 64-byte group segment; chunks beyond the rows (or, for a workgroup of
    // one row group, beyond the 128 RG chunks) read zero.
    buf_rsrc rs = src.rs;
    uint32_t sso[SCH], sbo[SCH], gr_of[SCH];
    int slo[SCH];
#pragma unroll
    for (int j = 0; j < SCH; ++j) {
        int c = tid + 256 * j, r = c >> 3;
        sbo[j] = 8 * (c & 7);
        const uint32_t q = r % ROWS;
        gr_of[j] = wg_row0 + (r / ROWS) * rpv + q;
        sso[j] = (c < WG_ROWS * 8 && q < rpv && gr_of[j] < n) ? gr_of[j] * srow + sbo[j] : W4_OOB;
        slo[j] = r * W4_GB + sbo[j];
    }
    // Scale bytes at or beyond k/16 in a row are zeroed in registers (an
    // 8-byte piece can straddle the end of a row's scales when k % 128 != 0);
    // a zero scale times a zero partial adds nothing.
    //
    // The range check of a buffer load zeroes every dword that reaches past
    // the end of the buffer, in-range bytes included.  When k/16 % 4 == 2,
    // the dword holding the matrix's last two scale bytes (the end of the
    // last row) is such a dword, so those two bytes are loaded once on
    // their own and put back when that piece is stashed: in dword fix_d of
    // piece j of group fix_g[j], on the one thread that owns it.
    const uint32_t stot = n * srow;         // scale bytes in the buffer
    const uint32_t last2 = __builtin_amdgcn_raw_buffer_load_b16(rs, stot - 2, 0, 0);
    uint32_t fix_g[SCH];
    const uint32_t fix_d = ((srow - 2) % 8) / 4;
#pragma unroll
    for (int j = 0; j < SCH; ++j) {
        const bool owner = srow % 4 == 2 && sso[j] < W4_OOB && gr_of[j] == n - 1 &&
                           (srow - 2) % W4_GB / 8 * 8 == sbo[j];
        fix_g[j] = owner ? (srow - 2) / W4_GB : ~0u;
    }
    auto load_sg = [&](u32x2 *v, uint32_t grp) {
#pragma unroll
        for (int j = 0; j < SCH; ++j) {
            uint32_t o = grp * W4_GB + sbo[j];
            v[j] = __builtin_amdgcn_raw_buffer_load_b64(rs, sso[j] + (o < srow ? grp * W4_GB : W4_OOB),
                                                        0, 0);
            uint32_t valid = o < srow ? srow - o : 0;      // bytes of this piece inside the row
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                uint32_t keep = valid >= 4 * d + 4 ? 0xFFFFFFFFu
                                : valid > 4 * d    ? 0x0000FFFFu   // valid is even
                                                   : 0u;
                v[j][d] &= keep;
            }
        }
    };
    auto stash_sg = [&](const u32x2 *v, uint32_t grp, int buf) {
#pragma unroll
        for (int j = 0; j < SCH; ++j) {
            u32x2 p = v[j];
            const uint32_t fix = grp == fix_g[j] ? last2 : 0u;
            p[0] |= fix_d == 0 ? fix : 0u;
            p[1] |= fix_d == 1 ? fix : 0u;
            if (tid + 256 * j < WG_ROWS * 8)
                *reinterpret_cast<u32x2 *>(&ss[buf][slo[j]]) = p;
        }
    };
    // a lane's fragments: row 4 g + l%4, elements 32 (l/4) + 8 i ..
    auto read_frags = [&](W4Act<MG> &a, int buf) {
#pragma unroll
        for (int g = 0; g < MG; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a.x[g][i] = *reinterpret_cast<const u32x4 *>(
                    &sx[buf][(4 * g + lane % 4) * W4_XPITCH + 32 * (lane / 4) + 8 * i]);
    };
    // the lane's two scale bytes of window `wig` (0 or 1) of the group in buffer sb
    auto read_scales = [&](W4Wts<RG> &g, int sb, int wig) {
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
            g.s[rg] = *reinterpret_cast<const uint16_t *>(
                &ss[sb][(wave * ROWS + 4 * rg + lane % 4) * W4_GB + wig * W4_SB + 2 * (lane / 4)]);
    };

    f32x4 acc[RG][MG];
    w4_zero<MG, RG>(acc);

    // ST register stages, each holding one window's weights and staged
    // activations; window w lives in stage w % ST and its stage is refilled
    // with window w + ST as soon as it has been used.
    W4Wts<RG> S[ST];
    u32x4 X[ST][XC];
    u32x2 sg[SCH];
    load_sg(sg, 0);
#pragma unroll
    for (int d = 0; d < ST; ++d) {
        src.load_w(S[d], d, (uint32_t)d < nwin, k);
        load_xs(X[d], d, (uint32_t)d < nwin);
    }
    W4Act<MG> frag;

    // One window: stage its activations, prefetch the window ST ahead,
    // synchronise, compute.
    auto step = [&](W4Wts<RG> &W, u32x4 *xs, uint32_t w, int buf, int sb, int wig) {
#pragma unroll
        for (int j = 0; j < XC; ++j)
            *reinterpret_cast<u32x4 *>(&sx[buf][xlo[j]]) = xs[j];
        load_xs(xs, w + ST, w + ST < nwin);
        __syncthreads();
        read_frags(frag, buf);
        read_scales(W, sb, wig);
        w4_window<MG, RG>(acc, W, frag);
        src.load_w(W, w + ST, w + ST < nwin, k);
    };
    // Scale groups are window pairs: group g (windows 2g, 2g + 1) is staged
    // in ss[g % 2] before its first window, and the next group is fetched.
    // ST is even, so a window's activation buffer and its half of the
    // group follow from its stage.
    auto window = [&](int d, uint32_t w) {
        const uint32_t grp = w / 2;
        const int sb = grp & 1;
        if (d % 2 == 0) {
            stash_sg(sg, grp, sb);
            load_sg(sg, grp + 1);
        }
        step(S[d], X[d], w, d & 1, sb, d & 1);
    };
    uint32_t win = 0;
    for (; win + ST <= nwin; win += ST)
#pragma unroll
        for (int d = 0; d < ST; ++d)
            window(d, win + d);
#pragma unroll
    for (int d = 0; d < ST; ++d)    // the last windows, fewer than ST
        if (win + d < nwin)
            window(d, win + d);
    w4_block_sum<MG, RG>(acc);
    w4_store<MG, RG>(acc, scale2, out, row0, rpv, m, n, lane);
}

// Row groups per wave, from n alone (never m): two (8 weight rows) for wide
// weights; one (4 rows, or 3 live rows of 4, below) for narrow ones, so that
// they still spread over all CUs (N = 6144: 384 workgroups of 16 rows).
// Measured at K = 5120 against an earlier K-split kernel for narrow weights
// (four waves sharing 8 rows, each a quarter of K): N = 17408, M = 1 / 2 /
// 8: 17.4 / 18.6 / 36.5 -> 12.5 / 12.9 / 18.8 us; N = 6144: 8.3 / 8.9 / 15.2
// -> 7.4 / 7.5 / 9.2 us.  A second K-split form (rows per workgroup sized to
// the CUs, wave-private activation windows, no barrier, three windows in
// flight) was also slower at every measured shape (N = 17408, M = 1: 16.7
// us; N = 6144, M = 1: 7.9 us), its registers capping residency.
static bool w4_gemv_wide(uint32_t n) { return n >= 65536u; }

// Register stages: four (window loads four ahead) for the one-group kernel
// when the whole grid is resident at its 146 registers, i.e. at most three
// workgroups per CU; two otherwise.  Narrow grids are a few memory round
// trips long, and the deeper prefetch removes some of them: N = 6144, M = 1 /
// 2: 7.7 / 7.8 -> 7.0 / 7.1 us; N = 12288: 9.2 -> 9.0 us.  Where the grid
// needs more rounds (N = 17408: 12.5 -> 14.3 us) or at two activation groups
// (218 registers; N = 6144, M = 8: 8.5 -> 9.5 us) four stages lose.  The
// stage count changes no summation order.
template <int MG, int RG, int ST>
static void launch_w4_st(const uint16_t *x, const uint8_t *wp, const uint8_t *ws, float scale2,
                         uint16_t *out, uint32_t m, uint32_t n, uint32_t k, uint32_t rpv,
                         uint32_t grid, hipStream_t st)
{
    hipLaunchKernelGGL((k_w4a16_gemv_rows<MG, RG, ST>), dim3(grid), dim3(256), 0, st,
                       x, wp, ws, scale2, out, m, n, k, rpv);
}

template <int MG, int RG>
static void launch_w4(const uint16_t *x, const uint8_t *wp, const uint8_t *ws, float scale2,
                      uint16_t *out, uint32_t m, uint32_t n, uint32_t k, uint32_t rpv,
                      hipStream_t st)
{
    const uint32_t grid = (n + 4 * rpv - 1) / (4 * rpv);
    if constexpr (MG == 1 && RG == 1) {
        const uint32_t cus = cu_count();
        if (cus != 0 && grid <= 3 * cus) {
            launch_w4_st<1, 1, 4>(x, wp, ws, scale2, out, m, n, k, rpv, grid, st);
            return;
        }
    }
    launch_w4_st<MG, RG, 2>(x, wp, ws, scale2, out, m, n, k, rpv, grid, st);
}

// Live rows per wave for narrow weights: 4, or 3 when that cuts the rows on
// the busiest CU by at least a quarter (a narrow grid is short, and the CUs
// holding one workgroup more than the others set its time; a wave with 3
// live rows of 4 issues a third more per row, which the cut must repay).
// N = 6144: 384 workgroups of 16 rows put 32 rows on some CUs, 512 of 12
// rows put 24 on every CU (M = 8: 9.2 -> 9.0 us, M = 1, 2 equal).  N =
// 17408 (80 -> 72 rows) measured slower with 3 (M = 1: 12.5 -> 13.3 us).
static uint32_t w4_rows_per_wave(uint32_t n)
{
    const uint32_t cus = cu_count();
    if (cus == 0)
        return 4;
    auto busiest = [&](uint32_t rpv) {
        const uint32_t wgs = (n + 4 * rpv - 1) / (4 * rpv);
        return (wgs + cus - 1) / cus * 4 * rpv;
    };
    return 4 * busiest(3) <= 3 * busiest(4) ? 3 : 4;
}

// 1 <= m <= 8, k % 32 == 0 and every buffer < 2^30 bytes (checked by the
// caller).  M groups of 4 rows: the group count changes no summation order.
hipError_t launch_w4a16_gemv(const uint16_t *x, const uint8_t *wp, const uint8_t *ws,
                             float scale2, uint16_t *out, uint32_t m, uint32_t n,
                             uint32_t k, hipStream_t st)
{
    const bool wide = w4_gemv_wide(n);
    const uint32_t rpv = wide ? 8 : w4_rows_per_wave(n);
    if (m <= 4)
        wide ? launch_w4<1, 2>(x, wp, ws, scale2, out, m, n, k, rpv, st)
             : launch_w4<1, 1>(x, wp, ws, scale2, out, m, n, k, rpv, st);
    else
        wide ? launch_w4<2, 2>(x, wp, ws, scale2, out, m, n, k, rpv, st)
             : launch_w4<2, 1>(x, wp, ws, scale2, out, m, n, k, rpv, st);
    count_launch();
    return hipGetLastError();
}

} // namespace qp
