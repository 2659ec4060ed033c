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

#include <type_traits>

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


// ---------------------------------------------------------------------------
// Large-tile variant for K % 128 == 0 and M, N >= 256: 256 x 256 workgroup
// tiles, each wave a 128 x 128 block of 4 x 4 MFMA tiles (accumulators in
// AGPRs).  K advances in stages of 128 bytes (two MFMA steps).  Operand
// panels (256 rows x 128 bytes = 32 KB of A or of W) are DMA'd into a ring
// of five LDS slots, all 160 KB of the CU: while a stage computes from two
// slots, the other three hold loads in flight 1 to 2 stages ahead, enough
// to cover L2 and HBM latency at the rate the MFMAs consume data (32 bytes
// per clock per CU).  Panel i of the sequence A0, W0, A1, W1, ... lives in
// slot i % 5.
//
// The last tile row / column is shifted back to end at M / N, so every row a
// tile loads exists (no clamping: DMA addresses stay affine in the
// instruction index) and the rows / columns it shares with its neighbour are
// not stored twice.
//
// The MFMAs compute C^T tiles (W fragment as the first operand): lane l then
// holds row l % 32 of C and, in accumulator registers 4q .. 4q+3, four
// consecutive columns 8q + 4*(l/32) .. +3, so the epilogue scales and
// converts four outputs at a time.  Written straight from that layout, each
// store instruction would touch 32 rows (32 cache lines, 16 bytes each);
// instead every wave stages its 128 x 128 BF16 block in a free LDS slot and
// stores it row by row, 4 rows of 256 bytes per instruction.
// The MFMA is issued with zero scale operands, which selects the unscaled
// encoding (identical results to unit E8M0 scales, at lower power).
//
// NT is the number of 32-column W tiles per wave: 4 for the 256 x 256 tile,
// 2 for a 256 x 128 half tile (W panels of 128 rows, 16 KB of their slot).
// One workgroup runs per CU, so time goes by rounds of one tile per CU; a
// grid whose last round is at most half full runs that round's tiles as
// half tiles in a second launch (NT = 2), on twice as many CUs.  Every
// output still takes its whole K sum from one wave in the same order, so
// the results do not depend on the split.  The NT = 4 launch covers the
// first nfull tiles of the banded order (tile_coords), the NT = 2 launch
// the rest, workgroups 2i and 2i + 1 the halves of tile nfull + i.
// ---------------------------------------------------------------------------
template <int NT>
__global__ __launch_bounds__(256, 1) void k_fp8_gemm_rowscale_big(
    const uint8_t *__restrict__ A, const float *__restrict__ as,
    const uint8_t *__restrict__ W, const float *__restrict__ ws,
    uint16_t *__restrict__ out, uint32_t M, uint32_t N, uint32_t K,
    uint32_t mtiles, uint32_t ntiles, uint32_t nfull, uint32_t vec_ok)
{
    static_assert(NT == 4 || NT == 2, "whole or half tiles");
    constexpr int TN = 64 * NT;        // tile columns = W panel rows
    constexpr int WL = 2 * NT;         // DMA loads per wave of a W panel
    // The five slots are separate LDS variables: accesses to distinct
    // variables carry distinct alias scopes, so the compiler can see that
    // reading one slot need not wait for the DMA into another (with one
    // array it would wait for every DMA in flight).
    __shared__ __attribute__((aligned(1024))) uint8_t S0[BIG_ROWS * BIG_KB];
    __shared__ __attribute__((aligned(1024))) uint8_t S1[BIG_ROWS * BIG_KB];
    __shared__ __attribute__((aligned(1024))) uint8_t S2[BIG_ROWS * BIG_KB];
    __shared__ __attribute__((aligned(1024))) uint8_t S3[BIG_ROWS * BIG_KB];
    __shared__ __attribute__((aligned(1024))) uint8_t S4[BIG_ROWS * BIG_KB];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const uint32_t nst = K / BIG_KB;

    uint32_t tm, tn, half = 0;
    if (NT == 4) {
        banded_tile(xcd_remap(blockIdx.x, nfull), mtiles, ntiles, tm, tn);
    } else {
        banded_tile(nfull + blockIdx.x / 2, mtiles, ntiles, tm, tn);
        half = blockIdx.x & 1;
    }
    const uint32_t m0 = tm * 256, n0 = tn * 256 + 128 * half;
    const uint32_t m0e = min(m0, M - 256), n0e = min(n0, N - TN);
    const uint8_t *const a_rows = A + (size_t)(m0e + 64 * wave) * K;
    const uint8_t *const w_rows = W + (size_t)(n0e + (TN / 4) * wave) * K;

    // DMA of one panel of L kilobytes per wave (8 for A and whole-tile W
    // panels, 4 for half-tile W panels): instruction j of wave w fills
    // kilobyte Lw+j = rows 8(Lw+j) + lane/8, a multiple of 32 plus
    // 8j + lane/8; lane's physical chunk lane%8 holds logical chunk
    // (lane%8) ^ swz(row) with swz(row) = ((j & 1) << 2) | (lane >> 4).  The
    // lane part of the source offset therefore takes two values (even / odd
    // j); the rest is uniform.
    uint32_t dvo[2];
#pragma unroll
    for (int e = 0; e < 2; ++e)
        dvo[e] = (uint32_t)(lane >> 3) * K + 16u * ((lane & 7) ^ ((e << 2) | (lane >> 4)));
    // Panel of stage st; stages past the end reload the last one (in bounds,
    // never read) so that every stage issues the same loads.
    auto dma_panel = [&](const uint8_t *rows, uint32_t st, uint8_t *slot, auto nl) {
        constexpr int L = decltype(nl)::value;
        const uint8_t *src = rows + (st < nst ? st : nst - 1) * BIG_KB;
#pragma unroll
        for (int j = 0; j < L; ++j)
            __builtin_amdgcn_global_load_lds(src + (size_t)(8 * j) * K + dvo[j & 1],
                                             (lds_void *)(slot + 1024 * (L * wave + j)), 16, 0, 0);
    };
    const std::integral_constant<int, 8> LA;
    const std::integral_constant<int, WL> LW;

    // LDS fragment reads: A row wm*128 + 32t + lane%32 of a slot (W row
    // wn*32*NT + 32t + lane%32), logical chunk c at physical
    // c ^ (((lane%32) >> 1) & 7).  The lane part of the
    // address depends on c only; t and the wave's half are immediate or
    // uniform offsets.
    const int g = lane >> 5;
    uint32_t lrow[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int lc = (c >> 1) * 4 + 2 * g + (c & 1);         // chunks 2g, 2g+1, 4+2g, 5+2g
        lrow[c] = (lane & 31) * BIG_KB + 16 * (lc ^ (((lane & 31) >> 1) & 7));
    }
    // Lane offsets for the current stage.  They are re-derived once per
    // stage (an empty asm hides their value; it is placed ahead of all of
    // the stage's memory operations, which it orders), so each read costs
    // one add instead of one register per slot and offset held across the
    // whole loop.
    uint32_t lo[4];
    auto launder = [&]() {
#pragma unroll
        for (int c = 0; c < 4; ++c)
            lo[c] = lrow[c];
        asm volatile("" : "+v"(lo[0]), "+v"(lo[1]), "+v"(lo[2]), "+v"(lo[3]));
    };
    struct Frags {
        i32x8 a[4], w[NT];
    };
    auto read_frags = [&](Frags &f, const uint8_t *la, const uint8_t *lw, int ks) {
        const uint32_t o0 = lo[2 * ks], o1 = lo[2 * ks + 1];
        const uint8_t *pa0 = la + wm * 128 * BIG_KB + o0, *pa1 = la + wm * 128 * BIG_KB + o1;
        const uint8_t *pw0 = lw + wn * 32 * NT * BIG_KB + o0, *pw1 = lw + wn * 32 * NT * BIG_KB + o1;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            u32x4 a0 = *reinterpret_cast<const u32x4 *>(pa0 + 32 * BIG_KB * t);
            u32x4 a1 = *reinterpret_cast<const u32x4 *>(pa1 + 32 * BIG_KB * t);
            f.a[t] = (i32x8){(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                             (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
            if (t < NT) {
                u32x4 w0 = *reinterpret_cast<const u32x4 *>(pw0 + 32 * BIG_KB * t);
                u32x4 w1 = *reinterpret_cast<const u32x4 *>(pw1 + 32 * BIG_KB * t);
                f.w[t < NT ? t : 0] = (i32x8){(int)w0[0], (int)w0[1], (int)w0[2], (int)w0[3],
                                              (int)w1[0], (int)w1[1], (int)w1[2], (int)w1[3]};
            }
        }
    };
    // acc[ti][tj]: C^T block of A tile ti (32 rows of C) and W tile tj
    f32x16 acc[4][NT];
    // MFMAs [lo, hi) of the 4 * NT of one K step
    auto mfma_range = [&](const Frags &f, int lo_, int hi_) {
#pragma unroll
        for (int i = 0; i < 4 * NT; ++i)
            if (i >= lo_ && i < hi_)
                acc[i / NT][i % NT] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    f.w[i % NT], f.a[i / NT], acc[i / NT][i % NT], 0, 0, 0, 0, 0, 0);
    };
    auto interleave = [&](int n_mfma, int n_ds, int n_vmem) {
        // n_ds LDS reads, two after each of the first MFMAs (early, so they
        // have returned by the time their fragments are needed), and n_vmem
        // DMA loads, one after each of the first MFMAs: the DMA of a stage
        // is spread over its 16 MFMAs so that the address unit never holds
        // a burst of them (issued two per MFMA the kernel ran 6% slower)
        for (int i = 0; i < n_mfma; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (2 * i < n_ds)
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            const int nv = (i + 1) * n_vmem / n_mfma - i * n_vmem / n_mfma;   // 0, 1 or 2
            if (nv >= 1)
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            if (nv >= 2)
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
    };
    // Wait until at most n of this wave's loads are in flight and its LDS
    // reads have returned, then for every wave.  Hard scheduling fences
    // keep the MFMAs on their side of it.
    auto sync_stage = [&](auto n) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(decltype(n)::value));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    // Stage st, X = (st, K step 0) already in registers, A(st) and W(st) in
    // slots ca and cw, A(st+1) and W(st+1) due in na and nw:
    //   4 NT MFMAs on X + LDS reads of Y = (st, K step 1)
    //   sync: A(st+1) and W(st+1) have landed (only A(st+2) may still be
    //         in flight: 8 loads per wave), and every wave has finished
    //         reading ca and cw
    //   DMA of W(st+2) into ca and A(st+3) into cw
    //   4 NT MFMAs on Y + LDS reads of X = (st+1, K step 0), issued two
    //      per MFMA from the first so that they have returned before the
    //      next stage needs them, and the 8 + WL DMA loads spread evenly
    //      (one per MFMA for whole tiles)
    // The slots are passed as the LDS variables themselves so that every
    // access names its slot statically.
    Frags X, Y;
    auto stage = [&](uint32_t st, uint8_t *ca, uint8_t *cw, const uint8_t *na,
                     const uint8_t *nw) {
        launder();
        read_frags(Y, ca, cw, 1);
        mfma_range(X, 0, 4 * NT);
        interleave(4 * NT, 8 + 2 * NT, 0);
        sync_stage(std::integral_constant<int, 8>());
        dma_panel(w_rows, st + 2, ca, LW);
        dma_panel(a_rows, st + 3, cw, LA);
        read_frags(X, na, nw, 0);
        mfma_range(Y, 0, 4 * NT);
        interleave(4 * NT, 8 + 2 * NT, 8 + WL);
        __builtin_amdgcn_sched_barrier(0);
    };

#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.0f;
    dma_panel(a_rows, 0, S0, LA);
    dma_panel(w_rows, 0, S1, LW);
    dma_panel(a_rows, 1, S2, LA);
    dma_panel(w_rows, 1, S3, LW);
    dma_panel(a_rows, 2, S4, LA);
    // A0 and W0 landed: A1, W1 and A2 may be in flight
    sync_stage(std::integral_constant<int, 16 + WL>());
    launder();
    read_frags(X, S0, S1, 0);
    uint32_t st = 0;
    for (; st + 5 <= nst; st += 5) {
        stage(st + 0, S0, S1, S2, S3);
        stage(st + 1, S2, S3, S4, S0);
        stage(st + 2, S4, S0, S1, S2);
        stage(st + 3, S1, S2, S3, S4);
        stage(st + 4, S3, S4, S0, S1);
    }
    if (st < nst)
        stage(st + 0, S0, S1, S2, S3);
    if (st + 1 < nst)
        stage(st + 1, S2, S3, S4, S0);
    if (st + 2 < nst)
        stage(st + 2, S4, S0, S1, S2);
    if (st + 3 < nst)
        stage(st + 3, S1, S2, S3, S4);
    // the loads past the end must land before the workgroup's LDS is freed
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));

    // Epilogue: C[i][j] = bf16(acc * (as[i] * ws[j])).  Lane rows
    // i = ib + 32*ti, columns j = jb + 32*tj + 8*q + c (c = 0..3); a shifted
    // tile stores only rows >= m0 and columns >= n0.  With N % 8 == 0 the
    // shift n0 - n0e is a multiple of 8, so every 8-column unit lies wholly
    // on one side of n0 and shifted tiles take the staged path too.
    const uint32_t ib = m0e + wm * 128 + (lane & 31);
    const uint32_t jb = n0e + wn * 32 * NT + 4 * (lane >> 5);
    if (vec_ok) {
        float sa[4];
        f32x4 sw[NT][4];
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
            sa[ti] = as[ib + 32 * ti];
#pragma unroll
        for (int tj = 0; tj < NT; ++tj)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                sw[tj][q] = *reinterpret_cast<const f32x4 *>(ws + jb + 32 * tj + 8 * q);
        // Stage the wave's 128 x 32NT block in slot `wave` (every wave has
        // finished reading the slots and its DMA has landed), RB = 64NT
        // bytes per row.  8-byte unit u of row r sits at u ^ x(r), with
        // x(r) = r % 32 for 256-byte rows and (r % 32) / 2 for 128-byte
        // rows: the 32 lanes of a half-wave (rows r % 32 = 0..31, one unit
        // each) then write 32 different 8-byte places of the 256-byte bank
        // row, all 64 banks.
        constexpr int RB = 64 * NT, XS = NT == 4 ? 0 : 1;
        __syncthreads();
        uint8_t *const ep = wave == 0 ? S0 : wave == 1 ? S1 : wave == 2 ? S2 : S3;
        const int r5 = lane & 31, hh = lane >> 5;
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
#pragma unroll
            for (int tj = 0; tj < NT; ++tj)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x16 &c = acc[ti][tj];
                    u32x2 pk;
                    pk[0] = pk_bf16(c[4 * q + 0] * (sa[ti] * sw[tj][q][0]),
                                    c[4 * q + 1] * (sa[ti] * sw[tj][q][1]));
                    pk[1] = pk_bf16(c[4 * q + 2] * (sa[ti] * sw[tj][q][2]),
                                    c[4 * q + 3] * (sa[ti] * sw[tj][q][3]));
                    *reinterpret_cast<u32x2 *>(ep + (r5 + 32 * ti) * RB + 8 * ((8 * tj + 2 * q + hh) ^ (r5 >> XS))) = pk;
                }
        }
        // Read back the PU = RB / 16 physical 16-byte units p of 64 / PU
        // rows per instruction: unit p holds logical unit p ^ (x(r) / 2),
        // its two 8-byte halves swapped where x(r) is odd.  Other lanes of
        // the wave wrote them; a wave's LDS operations execute in order, and
        // the wavefront-scope fence (no instruction) keeps the compiler from
        // treating the reads as independent of those writes.
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        constexpr int PU = RB / 16, RPI = 64 / PU;
        const int p = lane & (PU - 1);
        const uint32_t rb = m0e + wm * 128, cb = n0e + wn * 32 * NT;
        uint16_t *const obase = out + (size_t)rb * N + cb;
        // Two copies of the loop: the per-store row / column test of a
        // shifted tile cost 1.5% when every tile ran it.
        auto store_block = [&](auto guarded) {
#pragma unroll 4
            for (int it = 0; it < 128 / RPI; ++it) {
                const int r = RPI * it + lane / PU;
                u32x4 v = *reinterpret_cast<const u32x4 *>(ep + r * RB + 16 * p);
                const int x = (r & 31) >> XS;
                if (x & 1)
                    v = (u32x4){v[2], v[3], v[0], v[1]};
                const int lc = p ^ (x >> 1);
                if (!decltype(guarded)::value || (rb + r >= m0 && cb + 8 * lc >= n0))
                    *reinterpret_cast<u32x4 *>(obase + (size_t)r * N + 8 * lc) = v;
            }
        };
        if (m0e == m0 && n0e == n0)
            store_block(std::false_type());
        else
            store_block(std::true_type());
    } else {
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
            const uint32_t gi = ib + 32 * ti;
            const float sai = as[gi];
#pragma unroll
            for (int tj = 0; tj < NT; ++tj)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const uint32_t gj = jb + 32 * tj + 8 * (r >> 2) + (r & 3);
                    if (gi >= m0 && gj >= n0)
                        out[(size_t)gi * N + gj] =
                            (uint16_t)f32_to_bf16(acc[ti][tj][r] * (sai * ws[gj]));
                }
        }
    }
}

hipError_t launch_fp8_gemm_rowscale(const uint8_t *a, const float *as,
                                    const uint8_t *w, const float *ws,
                                    uint16_t *out, uint32_t m, uint32_t n,
                                    uint32_t k, hipStream_t st)
{
    if (k % BIG_KB == 0 && m >= 256 && n >= 256) {
        const uint32_t mt = (m + 255) / 256, nt = (n + 255) / 256, tiles = mt * nt;
        // 16-byte output stores and column-scale loads need N % 8 == 0 and
        // aligned base pointers; otherwise every tile takes the element-wise
        // epilogue.
        const uint32_t vec_ok = n % 8 == 0 && reinterpret_cast<uintptr_t>(out) % 16 == 0 &&
                                reinterpret_cast<uintptr_t>(ws) % 16 == 0;
        // One tile per CU at a time: a last round at most half full runs as
        // twice as many half tiles (with the CU count unknown, no split).
        const uint32_t cus = cu_count(), tail = cus ? tiles % cus : 0;
        const uint32_t nfull = tail != 0 && 2 * tail <= cus ? tiles - tail : tiles;
        if (nfull) {
            hipLaunchKernelGGL(k_fp8_gemm_rowscale_big<4>, dim3(nfull), dim3(256), 0, st,
                               a, as, w, ws, out, m, n, k, mt, nt, nfull, vec_ok);
            count_launch();
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess)
                return e;
        }
        if (nfull < tiles) {
            hipLaunchKernelGGL(k_fp8_gemm_rowscale_big<2>, dim3(2 * (tiles - nfull)), dim3(256),
                               0, st, a, as, w, ws, out, m, n, k, mt, nt, nfull, vec_ok);
            count_launch();
        }
        return hipGetLastError();
    } else {
        uint32_t mt = (m + F8_BM - 1) / F8_BM, nt = (n + F8_BN - 1) / F8_BN;
        hipLaunchKernelGGL(k_fp8_gemm_rowscale, dim3(mt * nt), dim3(256), 0, st,
                           a, as, w, ws, out, m, n, k, mt, nt);
    }
    count_launch();
    return hipGetLastError();
}

} // namespace qp
