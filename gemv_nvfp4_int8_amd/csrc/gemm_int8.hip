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
//
// The fold is the kernel's bound: with no packed FP32 math it costs the
// vector ALU 4 cycles per wave instruction, against 32 cycles for the int8
// MFMA of a whole 32x32x32 block.  It therefore keeps the VALU work per
// output and block at two instructions (the scale product moves to the
// matrix core) and keeps the VALU fed: inside a wave each fold waits for its
// MFMAs, so four waves share every SIMD (eight 64x32 waves per 128x128 tile,
// two tiles per CU) and fill each other's waits.  That fits in 128 VGPRs
// because operand stages arrive by LDS-DMA, which holds no registers.
#include "gemm_common.hpp"
#include "qp_launch.hpp"

namespace qp {

constexpr int I8_BM = 128, I8_BN = 128, I8_BK = 128;   // BK in bytes = elements
constexpr int I8_KB = I8_BK / 32;                       // K blocks per stage
constexpr int I8_SLOT = I8_BM * I8_BK;                  // one operand stage, 16 KB

// Eight waves per 128x128 tile, each 64 rows x 32 columns (two 32x32 int32
// tiles).  Four waves per SIMD hide each other's MFMA and LDS latencies,
// which the fold cannot hide inside one wave in 128 VGPRs.
template <bool PARTIALS>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void k_int8_gemm(
    const int8_t *__restrict__ A, const int8_t *__restrict__ W,
    const float *__restrict__ as, const float *__restrict__ ws,
    uint16_t *__restrict__ out, int32_t *__restrict__ part,
    uint32_t M, uint32_t N, uint32_t K, uint32_t mtiles, uint32_t ntiles)
{
    // Four separately named slots: every access below names its slot
    // statically, so the compiler sees that the DMA into the next stage's
    // slots cannot alias the reads of the current ones and does not wait
    // for it.
    __shared__ __attribute__((aligned(1024))) uint8_t sA0[I8_SLOT], sA1[I8_SLOT];
    __shared__ __attribute__((aligned(1024))) uint8_t sW0[I8_SLOT], sW1[I8_SLOT];
    // scales stored row-major: a row's four K blocks are one 16-byte read
    __shared__ __attribute__((aligned(16))) float sAs[2][I8_BM][I8_KB];
    __shared__ __attribute__((aligned(16))) float sWs[2][I8_BN][I8_KB];

    uint32_t tm, tn;
    tile_coords(mtiles, ntiles, tm, tn);
    const uint32_t m0 = tm * I8_BM, n0 = tn * I8_BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave & 1, wn = wave >> 1;      // 64-row half, 32-column quarter
    const uint32_t nb = K / 32;
    const uint32_t nst = (K + I8_BK - 1) / I8_BK;

    // Buffer resources: every load below takes a 32-bit offset and is
    // range-checked, so no load can fault.  Rows past M or N are not clamped:
    // whatever they load feeds only accumulators that are never stored.
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void *)A, 0, M * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void *)W, 0, N * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t ras_r = __builtin_amdgcn_make_buffer_rsrc((void *)as, 0, M * nb * 4, 0x00020000);
    const __amdgpu_buffer_rsrc_t rws_r = __builtin_amdgcn_make_buffer_rsrc((void *)ws, 0, N * nb * 4, 0x00020000);
    constexpr uint32_t OOB = 0x80000000u;

    // Operand stages go global -> LDS by 16-byte buffer loads to LDS.  A
    // 16 KB slot holds 128 rows of 128 bytes, unpadded, the 16-byte chunks
    // XOR-swizzled as in swz(); instruction j of wave w fills kilobyte 2w+j =
    // rows 16w + 8j + lane/8, lane i landing in physical chunk i%8, which
    // holds logical chunk (i%8) ^ swz(row) = (i%8) ^ ((4j + i/16) % 8).  The
    // lane part of the source offset takes two values (j even / odd), the
    // rest is uniform.  A chunk past the end of K (only in the last stage
    // when K % 128 != 0) holds whatever lies there: its K block has zero
    // scales, so it adds exactly zero.
    uint32_t dlane[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
        dlane[j] = (uint32_t)(lane >> 3) * K + 16u * ((lane & 7) ^ ((4 * j + (lane >> 4)) & 7));
    const uint32_t wrow = 16u * __builtin_amdgcn_readfirstlane(wave);
    auto dma = [&](__amdgpu_buffer_rsrc_t rsrc, uint32_t row0, uint32_t k0, uint8_t *slot) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc, (lds_void *)(slot + 1024 * (2 * (wrow / 16) + j)), 16,
                dlane[j] + (row0 + wrow + 8 * j) * K + k0, 0, 0, 0);
    };

    // scales: thread t loads K block t%4 of the stage for row t/4 of each
    // operand; a block past the end of K reads zero
    const uint32_t srow = threadIdx.x / I8_KB, sb = threadIdx.x % I8_KB;
    const uint32_t soff_a = 4 * ((m0 + srow) * nb + sb), soff_w = 4 * ((n0 + srow) * nb + sb);
    float ras, rws;
    // the scale loads go first, so that nothing waits on the DMA behind them
    auto load_stage = [&](uint32_t kst, uint8_t *la, uint8_t *lw) {
        if constexpr (!PARTIALS) {      // the partials export has no scales
            const bool live = kst * I8_KB + sb < nb;
            ras = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                ras_r, live ? soff_a + 16 * kst : OOB, 0, 0));
            rws = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                rws_r, live ? soff_w + 16 * kst : OOB, 0, 0));
        }
        dma(ra, m0, kst * I8_BK, la);
        dma(rw, n0, kst * I8_BK, lw);
    };
    auto store_scales = [&](int buf) {
        if constexpr (!PARTIALS) {
            sAs[buf][srow][sb] = ras;
            sWs[buf][srow][sb] = rws;
        }
    };
    // wait for this wave's DMA and LDS accesses, then for every wave's
    auto sync_stage = [&]() {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
        __syncthreads();
    };

    f32x16 acc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            acc[i][r] = 0.0f;

    load_stage(0, sA0, sW0);
    store_scales(0);
    sync_stage();

    // Fragment reads: tile row 32t + lane%32 of the wave's rows, logical
    // chunk 2kb + lane/32 (the lane's 16 bytes of K block kb), i.e. physical
    // chunk (lane/32 ^ s) ^ 2kb with s = ((lane%32) >> 1) % 8.  Block kb's
    // offset is the block-0 offset XOR 32kb (the slot base is 1 KB aligned).
    const int lr = lane & 31;
    const uint32_t fofs = lr * I8_BK + 16 * ((lane >> 5) ^ ((lr >> 1) & 7));
    const uint32_t fa_ofs = wm * 64 * I8_BK + fofs, fw_ofs = wn * 32 * I8_BK + fofs;
    const i32x16 zero = {};

    auto stage = [&](uint32_t st, int buf, const uint8_t *ca, const uint8_t *cw, uint8_t *na,
                     uint8_t *nw) {
        // the stage's scales, read before the next stage's DMA is issued
        // (lane l: a_scale of row 64wm + l, w_scale of column 32wn + l%32)
        f32x4 asv, wsv;
        if constexpr (!PARTIALS) {
            asv = *reinterpret_cast<const f32x4 *>(&sAs[buf][wm * 64 + lane][0]);
            wsv = *reinterpret_cast<const f32x4 *>(&sWs[buf][wn * 32 + (lane & 31)][0]);
        }
        if (st + 1 < nst)
            load_stage(st + 1, na, nw);

        // K blocks two at a time (a full unroll runs out of registers):
        // block kb = 2*kp + h takes scale component h, and the upper two
        // components move down after each pair
#pragma unroll 1
        for (int kp = 0; kp < I8_KB / 2; ++kp) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int kb = 2 * kp + h;
                const uint32_t ao = fa_ofs ^ (32u * kb), wo = fw_ofs ^ (32u * kb);
                i32x4 fa[2];
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    fa[t] = *reinterpret_cast<const i32x4 *>(&ca[ao + 32 * t * I8_BK]);
                const i32x4 fw = *reinterpret_cast<const i32x4 *>(&cw[wo]);
                if constexpr (PARTIALS) {
                    uint32_t gb = st * I8_KB + kb;
                    const uint32_t gj = n0 + wn * 32 + (lane & 31);
#pragma unroll
                    for (int ti = 0; ti < 2; ++ti) {
                        i32x16 p = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[ti], fw, zero, 0, 0, 0);
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            uint32_t gi = m0 + wm * 64 + 32 * ti + mfma32_row(r, lane);
                            if (gb < nb && gi < M && gj < N)
                                part[((size_t)gi * N + gj) * nb + gb] = p[r];
                        }
                    }
                } else {
                    // scale-and-add: acc += float(P) * (a_scale[row] * w_scale[col]).
                    // The scale products of the wave's two 32x32 tiles are two
                    // outer products, which one v_mfma_f32_32x32x1_2b_f32 forms
                    // (block 0: row tile 0, block 1: row tile 1) in the register
                    // layout of the int32 tiles, each product rounded as a plain
                    // f32 multiply rounds it.  That leaves two VALU operations
                    // per output and K block (convert, FMA).
                    const f32x32 sc = __builtin_amdgcn_mfma_f32_32x32x1f32(asv[h], wsv[h], f32x32{}, 0, 0, 0);
                    const i32x16 p0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[0], fw, zero, 0, 0, 0);
                    const i32x16 p1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[1], fw, zero, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        acc[0][r] = __builtin_fmaf((float)p0[r], sc[r], acc[0][r]);
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        acc[1][r] = __builtin_fmaf((float)p1[r], sc[16 + r], acc[1][r]);
                }
            }
            if constexpr (!PARTIALS) {
                asv = asv.zwzw;
                wsv = wsv.zwzw;
            }
        }

        if (st + 1 < nst)
            store_scales(buf ^ 1);
        sync_stage();
    };
    for (uint32_t st = 0; st < nst; st += 2) {
        stage(st, 0, sA0, sW0, sA1, sW1);
        if (st + 1 < nst)
            stage(st + 1, 1, sA1, sW1, sA0, sW0);
    }

    if constexpr (!PARTIALS) {
        const uint32_t gj = n0 + wn * 32 + (lane & 31);
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                uint32_t gi = m0 + wm * 64 + 32 * ti + mfma32_row(r, lane);
                if (gi < M && gj < N)
                    out[(size_t)gi * N + gj] = (uint16_t)f32_to_bf16(acc[ti][r]);
            }
    }
}

// ---------------------------------------------------------------------------
// The same GEMM with its operands on the FP16 matrix core (the operand-route
// ablation; int8_gemm_blockscaled itself runs the int8-MFMA kernel above).
//
// An int8 value is exact in FP16, and every partial sum of a block's 32
// products is an integer of magnitude below 2^24, so two
// v_mfma_f32_32x32x16_f16 (K = 16 each, F32 accumulation, the second
// continuing the first) return P_b exactly, already in F32.  The fold is
// then one FMA per output and block instead of a convert and an FMA, at the
// price of twice the int8 kernel's matrix-core cycles per block.  The
// outputs are bit-identical to the int8-MFMA kernel's: the same P_b, the
// same scale products, the same FMAs in the same K order.
//
// Operands are converted once per workgroup and stage: each thread loads
// its share of the stage's int8 rows from global memory into registers two
// stages ahead, and converts them into FP16 tiles in LDS (x + 1152 built by
// byte permutes under the FP16 exponent of 1024, then 1152 taken off with a
// packed FP16 add).  Each 256 x 128 output tile has eight waves of 64 x 64
// (2 x 2 MFMA tiles of 32 x 32), so a fragment read from LDS feeds two MFMAs.
//
// Measured on the 2048 x 17408 x 5120 prefill it is the slower route (633
// against 479 us): FP16 fragments are twice the bytes of int8 ones, so at
// full MFMA rate the fragment reads alone fill the LDS's 128 bytes per clock,
// and with the conversion writes on top the matrix core stays about a third
// busy; with two waves per SIMD the MFMA -> fold dependency is not hidden
// either (SQ counters: MFMA and VALU co-issue on 9% of cycles).
// ---------------------------------------------------------------------------
constexpr int F_BM = 256, F_BN = 128, F_BK = 64;       // F_BK: K elements per stage (2 blocks)
constexpr int F_KMULT = 2 * F_BK;                      // K multiple the kernel needs (even stage count)
constexpr int F_ROWB = 2 * F_BK;                       // bytes of one FP16 row of a stage

// Two FP16 values of signed bytes 2h and 2h+1 of d (h = 0, 1), exactly.
template <int H>
__device__ __forceinline__ uint32_t i8x2_to_f16x2(uint32_t dx)
{
    // dx = d ^ 0x80808080 (bytes biased by 128); under the FP16 exponent of
    // 1024 a byte u is the value 1024 + u = 1152 + x
    const uint32_t biased = __builtin_amdgcn_perm(0x64646464u, dx, H ? 0x04030402u : 0x04010400u);
    const f16x2 v = __builtin_bit_cast(f16x2, biased) - (f16x2){(_Float16)1152.0f, (_Float16)1152.0f};
    return __builtin_bit_cast(uint32_t, v);
}

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void k_int8_gemm_f16(
    const int8_t *__restrict__ A, const int8_t *__restrict__ W,
    const float *__restrict__ as, const float *__restrict__ ws,
    uint16_t *__restrict__ out, uint32_t M, uint32_t N, uint32_t K,
    uint32_t mtiles, uint32_t ntiles)
{
    // FP16 stage tiles, rows of 128 bytes, 16-byte chunks XOR-swizzled as in
    // swz() (chunk c of row r at physical chunk c ^ ((r / 2) % 8)): the 64
    // banks span two rows, and the sixteen lanes a 16-byte LDS access serves
    // together read sixteen consecutive rows at one logical chunk, which the
    // swizzle spreads over all 64 banks.
    __shared__ __attribute__((aligned(1024))) uint8_t sA0[F_BM * F_ROWB], sA1[F_BM * F_ROWB];
    __shared__ __attribute__((aligned(1024))) uint8_t sW0[F_BN * F_ROWB], sW1[F_BN * F_ROWB];
    // block scales of a stage, [block][row]: A rows 0..255, then W rows
    // (256 + n); each thread writes its own slot (the last 128 are unused)
    __shared__ __attribute__((aligned(16))) float sS0[2][512], sS1[2][512];

    uint32_t tm, tn;
    tile_coords(mtiles, ntiles, tm, tn);
    const uint32_t m0 = tm * F_BM, n0 = tn * F_BN;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave & 3, wn = wave >> 2;      // 64-row quarter, 64-column half
    const uint32_t nb = K / 32;
    const uint32_t nst = K / F_BK;

    constexpr uint32_t OOB = 0x80000000u;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void *)A, 0, M * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void *)W, 0, N * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t ras_r = __builtin_amdgcn_make_buffer_rsrc((void *)as, 0, M * nb * 4, 0x00020000);
    const __amdgpu_buffer_rsrc_t rws_r = __builtin_amdgcn_make_buffer_rsrc((void *)ws, 0, N * nb * 4, 0x00020000);

    // Thread t loads, per stage, 16 bytes (one 16-element quarter of the
    // stage's 64 K elements) of A rows t/4 and 128 + t/4 and of W row t/4,
    // and the two block scales of A row t/2 (t < 256... see below) or W row.
    const int lr = t >> 2, lq = t & 3;
    const uint32_t ga0 = m0 + lr, ga1 = m0 + 128 + lr, gw = n0 + lr;
    const uint32_t oa0 = ga0 < M ? ga0 * K + 16 * lq : OOB;
    const uint32_t oa1 = ga1 < M ? ga1 * K + 16 * lq : OOB;
    const uint32_t ow = gw < N ? gw * K + 16 * lq : OOB;
    // scales: thread t < 256 takes A row t, 256 <= t < 384 W row t - 256;
    // both blocks of the stage in one 8-byte load
    const uint32_t wave_u = __builtin_amdgcn_readfirstlane(wave);   // waves 0-3: A, 4-5: W
    const bool sa_thr = wave_u < F_BM / 64, sw_thr = !sa_thr && wave_u < (F_BM + F_BN) / 64;
    const uint32_t srow = sa_thr ? m0 + t : n0 + (t - F_BM);
    const bool s_live = sa_thr ? srow < M : (sw_thr && srow < N);
    const uint32_t soff = s_live ? 4 * srow * nb : OOB;

    struct Stage {
        u32x4 a0, a1, w;
        float sc0, sc1;
    };
    // Loads never sit under a branch, so the compiler waits only for the
    // stage it uses.  The two prefetches past the last stage read the next
    // row's bytes (or zeros past the end of the buffer); they are converted
    // into the spare LDS buffer, which nothing reads afterwards.
    auto load = [&](Stage &g, uint32_t st) {
        const uint32_t k0 = st * F_BK;
        g.a0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, oa0 + k0, 0, 0));
        g.a1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, oa1 + k0, 0, 0));
        g.w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, ow + k0, 0, 0));
        // two 4-byte loads (merged into one 8-byte load by the compiler): on
        // this toolchain, elements taken from the 8-byte buffer-load builtin's
        // result both read its first dword
        const __amdgpu_buffer_rsrc_t rs = sa_thr ? ras_r : rws_r;
        g.sc0 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, soff + 8 * st, 0, 0));
        g.sc1 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, soff + 8 * st + 4, 0, 0));
    };
    // 16 int8 -> 16 FP16 = logical chunks 2q, 2q+1 of FP16 row r
    auto put = [&](uint8_t *tile, int r, u32x4 v) {
        u32x4 lo, hi;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t d0 = v[2 * i] ^ 0x80808080u, d1 = v[2 * i + 1] ^ 0x80808080u;
            const u32x4 c = {i8x2_to_f16x2<0>(d0), i8x2_to_f16x2<1>(d0),
                             i8x2_to_f16x2<0>(d1), i8x2_to_f16x2<1>(d1)};
            if (i == 0)
                lo = c;
            else
                hi = c;
        }
        *reinterpret_cast<u32x4 *>(tile + r * F_ROWB + 16 * swz(r, 2 * lq)) = lo;
        *reinterpret_cast<u32x4 *>(tile + r * F_ROWB + 16 * swz(r, 2 * lq + 1)) = hi;
    };
    auto convert = [&](const Stage &g, uint8_t *ta, uint8_t *tw, float (*ss)[512]) {
        put(ta, lr, g.a0);
        put(ta, 128 + lr, g.a1);
        put(tw, lr, g.w);
        ss[0][t] = g.sc0;
        ss[1][t] = g.sc1;
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.0f;

    // fragment rows of this lane: tile row 32 i + lane % 32 of the wave's rows
    const int fr = lane & 31, fh = lane >> 5;
    auto frag = [&](const uint8_t *tile, int row, int kh) -> f16x8 {
        // K half kh (16 elements) of the stage: lane reads logical chunk 2 kh + fh
        return *reinterpret_cast<const f16x8 *>(tile + row * F_ROWB + 16 * swz(row, 2 * kh + fh));
    };

    // One stage: both K blocks of the current tiles, with the next stage's
    // conversion split between them so its vector-ALU work sits among the
    // MFMAs (measured: 671 -> 633 us against converting after both blocks).
    auto compute = [&](const uint8_t *ta, const uint8_t *tw, const float (*ss)[512],
                       const Stage &gn, uint8_t *na, uint8_t *nw, float (*nss)[512]) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            if (b == 0) {
                put(na, lr, gn.a0);
            } else {
                put(na, 128 + lr, gn.a1);
                put(nw, lr, gn.w);
                nss[0][t] = gn.sc0;
                nss[1][t] = gn.sc1;
            }
            // lane's scales of block b: A rows 64 wm + lane (the rows of both
            // 32-row tiles), W columns 64 wn + 32 j + lane % 32
            const float asv = ss[b][64 * wm + lane];
            f16x8 fa[2][2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    fa[i][h] = frag(ta, 64 * wm + 32 * i + fr, 2 * b + h);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float wsv = ss[b][F_BM + 64 * wn + 32 * j + fr];
                f16x8 fw[2];
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    fw[h] = frag(tw, 64 * wn + 32 * j + fr, 2 * b + h);
                // scale products a_s[row] * w_s[col] of the two row tiles of
                // column tile j, in the layout of the 32 x 32 results
                const f32x32 sc = __builtin_amdgcn_mfma_f32_32x32x1f32(asv, wsv, f32x32{}, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    f32x16 p = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i][0], fw[0], f32x16{}, 0, 0, 0);
                    p = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i][1], fw[1], p, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        acc[i][j][r] = __builtin_fmaf(p[r], sc[16 * i + r], acc[i][j][r]);
                }
            }
        }
    };

    // The scheduling barriers keep the prologue's loads in stage order, as
    // the loop issues them, so that the waits the compiler derives at the
    // loop head cover only the stage about to be converted.
    Stage g0, g1;
    load(g0, 0);
    __builtin_amdgcn_sched_barrier(0);
    load(g1, 1);
    __builtin_amdgcn_sched_barrier(0);
    convert(g0, sA0, sW0, sS0);
    __builtin_amdgcn_sched_barrier(0);
    load(g0, 2);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();

    // Stage s is in LDS buffer s % 2; the registers hold stage s + 1 (landed
    // or in flight) and stage s + 2 (in flight).  The stage count is even,
    // and nothing here branches: past the last stage the loads read zeros
    // and the conversion fills the spare buffer, which nothing reads.
    auto step = [&](uint32_t s, const uint8_t *ca, const uint8_t *cw, const float (*css)[512],
                    Stage &gn, uint8_t *na, uint8_t *nw, float (*nss)[512]) {
        compute(ca, cw, css, gn, na, nw, nss);
        load(gn, s + 3);
        __syncthreads();
    };
    for (uint32_t s = 0; s < nst; s += 2) {
        step(s, sA0, sW0, sS0, g1, sA1, sW1, sS1);
        step(s + 1, sA1, sW1, sS1, g0, sA0, sW0, sS0);
    }

    const uint32_t col0 = n0 + 64 * wn + fr;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t gj = col0 + 32 * j;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const uint32_t gi = m0 + 64 * wm + 32 * i + mfma32_row(r, lane);
                if (gi < M && gj < N)
                    out[(size_t)gi * N + gj] = (uint16_t)f32_to_bf16(acc[i][j][r]);
            }
        }
}

hipError_t launch_int8_gemm(const int8_t *a, const int8_t *w, const float *as,
                            const float *ws, uint16_t *out, int32_t *partials,
                            uint32_t m, uint32_t n, uint32_t k, hipStream_t st)
{
    uint32_t mt = (m + I8_BM - 1) / I8_BM, nt = (n + I8_BN - 1) / I8_BN;
    dim3 grid(mt * nt), block(512);
    if (partials)
        hipLaunchKernelGGL(k_int8_gemm<true>, grid, block, 0, st, a, w, as, ws,
                           out, partials, m, n, k, mt, nt);
    else
        hipLaunchKernelGGL(k_int8_gemm<false>, grid, block, 0, st, a, w, as, ws,
                           out, partials, m, n, k, mt, nt);
    count_launch();
    return hipGetLastError();
}

hipError_t launch_int8_gemm_f16ops(const int8_t *a, const int8_t *w, const float *as,
                                   const float *ws, uint16_t *out, uint32_t m, uint32_t n,
                                   uint32_t k, hipStream_t st)
{
    const uint32_t mt = (m + F_BM - 1) / F_BM, nt = (n + F_BN - 1) / F_BN;
    hipLaunchKernelGGL(k_int8_gemm_f16, dim3(mt * nt), dim3(512), 0, st, a, w, as, ws, out,
                       m, n, k, mt, nt);
    count_launch();
    return hipGetLastError();
}

} // namespace qp
