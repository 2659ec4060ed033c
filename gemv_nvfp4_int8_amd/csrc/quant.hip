// quant.hip -- streaming quantizers and weight requantizers for gfx950.
//
// All of them are HBM-bound: every byte is read once with 16-byte vector
// loads, codes are written with 8- or 16-byte non-temporal stores (about 3-6%
// faster than plain stores here: the outputs are not read back by the same
// kernel), and absmax reductions
// stay in registers (per-block kernels) or use wave shuffles plus one LDS
// exchange per workgroup (per-row kernels).
#include <type_traits>

#include "qp_device.hpp"
#include "qp_launch.hpp"

namespace qp {

// ---------------------------------------------------------------------------
// Access pattern of the elementwise kernels: a thread owns one 16-byte input
// chunk per round, and the 64 lanes of a wave own 64 consecutive chunks, so
// every load and store instruction covers one contiguous window (HBM serves
// that about 1.5x faster than lanes walking their own 64-byte strips).  The
// few lanes that share a scaling block combine their absmax with shuffles.
// Each workgroup runs QR rounds of 256 chunks with all loads issued first
// (QR per kernel as measured best on MI355X at the benchmark sizes: 1 for
// the small activation requant, 2 for the others).
// ---------------------------------------------------------------------------

// ---------------------------------------------------------------------------
// BF16 -> int8, one F32 scale per 32 (gemm_dense_int8.rs,
// int8_gemm_faith2_prefill, activation launch).  A 32-block is 4 chunks of
// 8 elements, held by 4 adjacent lanes.  Flattened indexing is valid because
// k % 32 == 0: a block never straddles a row, and block id = chunk id / 4 in
// the [m, k/32] scale grid.
// ---------------------------------------------------------------------------
template <int QR>
__global__ __launch_bounds__(256) void k_requant_a_bf16_int8(
    const uint16_t *__restrict__ a, int8_t *__restrict__ q,
    float *__restrict__ s, uint32_t nchunks)
{
    const uint32_t base = blockIdx.x * (256u * QR) + threadIdx.x;
    u32x4 raw[QR];
#pragma unroll
    for (int u = 0; u < QR; ++u) {
        const uint32_t c = base + 256u * u;
        raw[u] = (u32x4){0, 0, 0, 0};
        if (c < nchunks)
            raw[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(a + (size_t)c * 8));
    }
#pragma unroll
    for (int u = 0; u < QR; ++u) {
        const uint32_t c = base + 256u * u;     // nchunks % 4 == 0: a block's lanes agree
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = bf16_lo(raw[u][i]);
            x[2 * i + 1] = bf16_hi(raw[u][i]);
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            amax = __builtin_fmaxf(amax, __builtin_fabsf(x[i]));
        amax = __builtin_fmaxf(amax, __shfl_xor(amax, 1, WAVE));
        amax = __builtin_fmaxf(amax, __shfl_xor(amax, 2, WAVE));
        const float sc = div_by_const<127>(amax);
        u32x2 out = {0, 0};
        if (sc != 0.0f) {
            ScaleDiv d(sc);
            float t[8];
            div_all<8>(d, x, t);
            out[0] = pack_i8x4(&t[0]);
            out[1] = pack_i8x4(&t[4]);
        }
        if (c < nchunks) {
            __builtin_nontemporal_store(out, reinterpret_cast<u32x2 *>(q + (size_t)c * 8));
            if ((c & 3u) == 0u)
                s[c >> 2] = sc;
        }
    }
}

hipError_t launch_requant_a_bf16_int8(const uint16_t *a, int8_t *q, float *s,
                                      uint32_t m, uint32_t k, hipStream_t st)
{
    uint32_t nchunks = (uint32_t)((uint64_t)m * k / 8);
    constexpr int QR = 1;
    uint32_t grid = (nchunks + 256 * QR - 1) / (256 * QR);
    hipLaunchKernelGGL(k_requant_a_bf16_int8<QR>, dim3(grid), dim3(256), 0, st,
                       a, q, s, nchunks);
    count_launch();
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// NVFP4 -> int8 weight requant (gemm_dense_int8.rs, requant_w_nvfp4_int8).
// A 32-block (16 packed bytes + 2 E4M3 sub-block scales in, 32 int8 + 1 F32
// out) is held by two adjacent lanes, one 16-element sub-block each: 8
// packed bytes and one scale byte in, 16 int8 out.  v = fl(fl(e2m1*e4m3) *
// scale2) (the first product exact), then absmax / 127 and RNE(v/s).
// ---------------------------------------------------------------------------
template <int QR>
__global__ __launch_bounds__(256) void k_requant_w_nvfp4_int8(
    const uint8_t *__restrict__ packed, const uint8_t *__restrict__ sc16,
    float scale2, int8_t *__restrict__ q, float *__restrict__ s,
    uint32_t nhalves)
{
    const uint32_t base = blockIdx.x * (256u * QR) + threadIdx.x;
    u32x2 p[QR];
    uint32_t scb[QR];
#pragma unroll
    for (int u = 0; u < QR; ++u) {
        const uint32_t h = base + 256u * u;
        p[u] = (u32x2){0, 0};
        scb[u] = 0;
        if (h < nhalves) {
            p[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(packed + (size_t)h * 8));
            scb[u] = sc16[h];
        }
    }
#pragma unroll
    for (int u = 0; u < QR; ++u) {
        const uint32_t h = base + 256u * u;     // nhalves is even: a block's lanes agree
        // e2m1 * e4m3 is exact in FP16 (at most 6 significant bits, magnitudes
        // 2^-10 .. 2688), so it is formed two at a time in packed FP16; the
        // one rounded step, times scale2, is a mixed-precision FMA.
        const _Float16 dh = (_Float16)dec_e4m3(scb[u]);
        const f16x2 dd2 = (f16x2){dh, dh};
        float v[16];
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const f16x2 e[4] = {e2m1_pair_f16<0>(p[u][w]) * dd2, e2m1_pair_f16<1>(p[u][w]) * dd2,
                                e2m1_pair_f16<2>(p[u][w]) * dd2, e2m1_pair_f16<3>(p[u][w]) * dd2};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[8 * w + 2 * j] = (float)e[j][0] * scale2;
                v[8 * w + 2 * j + 1] = (float)e[j][1] * scale2;
            }
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
        amax = __builtin_fmaxf(amax, __shfl_xor(amax, 1, WAVE));
        const float sc = div_by_const<127>(amax);
        u32x4 o = {0, 0, 0, 0};
        if (sc != 0.0f) {
            ScaleDiv d(sc);
            div_all<16>(d, v, v);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                o[j] = pack_i8x4(&v[4 * j]);
        }
        if (h < nhalves) {
            __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(q + (size_t)h * 16));
            if ((h & 1u) == 0u)
                s[h >> 1] = sc;
        }
    }
}

hipError_t launch_requant_w_nvfp4_int8(const uint8_t *packed, const uint8_t *sc16,
                                       float scale2, int8_t *q, float *s,
                                       uint32_t n, uint32_t k, hipStream_t st)
{
    uint32_t nhalves = (uint32_t)((uint64_t)n * (k / 16));
    constexpr int QR = 2;
    hipLaunchKernelGGL(k_requant_w_nvfp4_int8<QR>, dim3((nhalves + 256 * QR - 1) / (256 * QR)),
                       dim3(256), 0, st, packed, sc16, scale2, q, s, nhalves);
    count_launch();
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// BF16 -> NVFP4 (gemm_fp4.rs, quantize_bf16_to_nvfp4).  A 16-element block
// is held by two adjacent lanes, 8 elements (one 16-byte chunk) each, and
// each lane writes its 8 codes as one dword.  sb = E4M3(fl(amax /
// fl(6*scale2))), d = fl(e4m3(sb)*scale2), code = E2M1(fl(x/d)), or +0
// everywhere when d == 0.  The block scales of four blocks (8 lanes) are
// gathered into one dword store.
//
// The divisions are the kernel's arithmetic bound, so none is repeated per
// block: fl(amax / fl(6*scale2)) is one correction step with that divisor's
// reciprocal (one IEEE division per thread), and the decoded scale d takes
// only 127 values per call, whose reciprocals a workgroup computes once into
// LDS.  With a normal block scale that did not saturate, every |x/d| stays
// below 6 * (1 + 2^-4) < 8, inside the E2M1 converter's checked range, so
// the clamp to +-6 is skipped when a whole wave is in that case.
// ---------------------------------------------------------------------------
template <int QR>
__global__ __launch_bounds__(256) void k_quantize_bf16_nvfp4(
    const uint16_t *__restrict__ x, uint8_t *__restrict__ packed,
    uint8_t *__restrict__ sc16, float scale2, uint32_t nchunks)
{
    // RN(1/d) for d = fl(e4m3(c)*scale2), c = 0..126; 0 marks a d outside
    // the range where the correction step is valid (ScaleDiv::fast).
    __shared__ float rtab[128];
    if (threadIdx.x < 128) {
        const float d = dec_e4m3(threadIdx.x & 0x7Fu) * scale2;
        rtab[threadIdx.x] = (d >= 0x1p-100f && d <= 0x1p100f) ? div_rn(1.0f, d) : 0.0f;
    }
    const uint32_t base = blockIdx.x * (256u * QR) + threadIdx.x;
    const int lane = threadIdx.x & 63;
    u32x4 raw[QR];
#pragma unroll
    for (int u = 0; u < QR; ++u) {
        const uint32_t c = base + 256u * u;
        raw[u] = (u32x4){0, 0, 0, 0};
        if (c < nchunks)
            raw[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(x + (size_t)c * 8));
    }
    const float six_s2 = 6.0f * scale2;
    const bool six_ok = six_s2 >= 0x1p-60f && six_s2 <= 0x1p60f;
    const float r6 = six_ok ? div_rn(1.0f, six_s2) : 0.0f;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < QR; ++u) {
        const uint32_t c = base + 256u * u;     // nchunks % 4 == 0: a block's lanes agree
        float v[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16_lo(raw[u][i]);
            v[2 * i + 1] = bf16_hi(raw[u][i]);
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
        amax = __builtin_fmaxf(amax, __shfl_xor(amax, 1, WAVE));
        float t;
        if (__all(six_ok && (amax == 0.0f || (amax >= 0x1p-60f && amax <= 0x1p60f))))
            t = div_corr(amax, six_s2, r6);
        else
            t = div_rn(amax, six_s2);
        // E4M3 of t >= 0 (saturated at 448) by the converter
        const uint32_t sb = enc_e4m3_scale(t);
        const float d = dec_e4m3(sb) * scale2;
        uint32_t codes = 0;
        if (d != 0.0f) {
            const ScaleDiv dv(d, rtab[sb]);
            float q[8];
            div_all<8>(dv, v, q);
            codes = __all(sb >= 0x08u && t < 448.0f) ? cvt_e2m1x8_nosat(q) : cvt_e2m1x8(q);
        }
        // scales of the blocks of lanes 8g .. 8g+7 (every other lane) -> lane 8g
        const uint32_t w4 = sb | (__shfl_down(sb, 2, WAVE) << 8) |
                            (__shfl_down(sb, 4, WAVE) << 16) | (__shfl_down(sb, 6, WAVE) << 24);
        if (c < nchunks) {
            __builtin_nontemporal_store(codes, reinterpret_cast<uint32_t *>(packed + (size_t)c * 4));
            if ((lane & 7) == 0) {
                // c % 8 == 0, so block c/2 starts a 4-byte-aligned word
                if (c + 8 <= nchunks)
                    *reinterpret_cast<uint32_t *>(sc16 + (c >> 1)) = w4;
                else
                    *reinterpret_cast<uint16_t *>(sc16 + (c >> 1)) = (uint16_t)w4;  // 2 blocks left
            }
        }
    }
}

hipError_t launch_quantize_bf16_nvfp4(const uint16_t *x, uint8_t *packed,
                                      uint8_t *sc16, float scale2, uint32_t rows,
                                      uint32_t k, hipStream_t st)
{
    uint32_t nchunks = (uint32_t)((uint64_t)rows * k / 8);
    constexpr int QR = 2;
    hipLaunchKernelGGL(k_quantize_bf16_nvfp4<QR>, dim3((nchunks + 256 * QR - 1) / (256 * QR)),
                       dim3(256), 0, st, x, packed, sc16, scale2, nchunks);
    count_launch();
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-row kernels.  A row of up to 64*CPL 16-byte chunks is one wave's (four
// rows per workgroup): the chunks stay in registers between the absmax pass
// and the encode pass, so every input byte is read once; lane l takes
// chunks l, l + 64, ..., so every load and store instruction covers one
// contiguous window; the row absmax is a wave reduction alone (no LDS, no
// barrier); and the scale, one per row, is wave-uniform, so its division
// path is chosen once.  Longer rows take a workgroup per row and two passes
// over global memory.
//
// The row scale s = fl(amax/448) bounds every quotient: |x/s| <= amax/s <=
// 448 * (1 + 2^-23), so its RNE binary32 value is at most 448 plus one ulp,
// below 464, where the E4M3 converter rounds to 448 by itself: no clamp.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float block_max_256(float v, float *red)
{
    v = wave_max(v);
    int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0)
        red[wave] = v;
    __syncthreads();
    return __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]),
                           __builtin_fmaxf(red[2], red[3]));
}

// E4M3 codes of v[0..7] / d.s in two dwords (quotients below 464 in
// magnitude), by the path FAST (the caller branches once per scale).
template <bool FAST>
__device__ __forceinline__ u32x2 enc8_e4m3_path(const float *v, const ScaleDiv &d)
{
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        t[i] = FAST ? d.quick(v[i]) : div_rn(v[i], d.s);
    return (u32x2){cvt_e4m3x4_nosat(t[0], t[1], t[2], t[3]),
                   cvt_e4m3x4_nosat(t[4], t[5], t[6], t[7])};
}

// Row-wise FP8 quantizer (dispatch_proj_rowwise.rs, quant_rowwise_fp8):
// s = fl(amax/448), code = E4M3(fl(x/s)), or scale 0 and +0 codes.
template <int CPL>
__global__ __launch_bounds__(256) void k_quant_rowwise_fp8_wave(
    const uint16_t *__restrict__ x, uint8_t *__restrict__ q,
    float *__restrict__ s, uint32_t rows, uint32_t k)
{
    const uint32_t row = blockIdx.x * 4u + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows)
        return;                          // the whole wave
    const uint16_t *xr = x + (size_t)row * k;
    uint8_t *qr = q + (size_t)row * k;
    const uint32_t nch = k / 8;
    u32x4 raw[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const uint32_t c = lane + 64u * j;
        raw[j] = (u32x4){0, 0, 0, 0};
        if (c < nch)
            raw[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(xr + (size_t)c * 8));
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < CPL; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            amax = __builtin_fmaxf(amax, __builtin_fmaxf(__builtin_fabsf(bf16_lo(raw[j][i])),
                                                         __builtin_fabsf(bf16_hi(raw[j][i]))));
    amax = wave_max(amax);
    const float sc = div_by_const<448>(amax);
    const ScaleDiv dv(sc);
    auto encode = [&](auto fast_tag) {
        constexpr bool FAST = decltype(fast_tag)::value;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const uint32_t c = lane + 64u * j;
            if (c < nch) {
                float v[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[2 * i] = bf16_lo(raw[j][i]);
                    v[2 * i + 1] = bf16_hi(raw[j][i]);
                }
                __builtin_nontemporal_store(
                    sc != 0.0f ? enc8_e4m3_path<FAST>(v, dv) : (u32x2){0, 0},
                    reinterpret_cast<u32x2 *>(qr + (size_t)c * 8));
            }
        }
    };
    if (dv.fast)
        encode(std::true_type{});
    else
        encode(std::false_type{});
    if (lane == 0)
        s[row] = sc;
}

// Rows longer than a wave's registers hold: a workgroup per row, CPT chunks
// per thread in registers (one pass over global memory).
template <int CPT>
__global__ __launch_bounds__(256) void k_quant_rowwise_fp8_wg(
    const uint16_t *__restrict__ x, uint8_t *__restrict__ q,
    float *__restrict__ s, uint32_t k)
{
    __shared__ float red[4];
    const uint32_t row = blockIdx.x;
    const uint16_t *xr = x + (size_t)row * k;
    uint8_t *qr = q + (size_t)row * k;
    const uint32_t nch = k / 8;
    u32x4 raw[CPT];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const uint32_t c = threadIdx.x + 256u * j;
        raw[j] = (u32x4){0, 0, 0, 0};
        if (c < nch)
            raw[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(xr + (size_t)c * 8));
#pragma unroll
        for (int i = 0; i < 4; ++i)
            amax = __builtin_fmaxf(amax, __builtin_fmaxf(__builtin_fabsf(bf16_lo(raw[j][i])),
                                                         __builtin_fabsf(bf16_hi(raw[j][i]))));
    }
    amax = block_max_256(amax, red);
    const float sc = div_by_const<448>(amax);
    const ScaleDiv dv(sc);
    auto encode = [&](auto fast_tag) {
        constexpr bool FAST = decltype(fast_tag)::value;
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const uint32_t c = threadIdx.x + 256u * j;
            if (c < nch) {
                float v[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[2 * i] = bf16_lo(raw[j][i]);
                    v[2 * i + 1] = bf16_hi(raw[j][i]);
                }
                __builtin_nontemporal_store(
                    sc != 0.0f ? enc8_e4m3_path<FAST>(v, dv) : (u32x2){0, 0},
                    reinterpret_cast<u32x2 *>(qr + (size_t)c * 8));
            }
        }
    };
    if (dv.fast)
        encode(std::true_type{});
    else
        encode(std::false_type{});
    if (threadIdx.x == 0)
        s[row] = sc;
}

// Long rows: the same arithmetic, a workgroup per row, in two passes over
// global memory.
__global__ __launch_bounds__(256) void k_quant_rowwise_fp8_long(
    const uint16_t *__restrict__ x, uint8_t *__restrict__ q,
    float *__restrict__ s, uint32_t k)
{
    __shared__ float red[4];
    const uint32_t row = blockIdx.x;
    const uint16_t *xr = x + (size_t)row * k;
    const uint32_t nch = k / 8;
    float amax = 0.0f;
    for (uint32_t c = threadIdx.x; c < nch; c += 256) {
        u32x4 r = *reinterpret_cast<const u32x4 *>(xr + (size_t)c * 8);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            amax = __builtin_fmaxf(amax, __builtin_fmaxf(__builtin_fabsf(bf16_lo(r[i])),
                                                         __builtin_fabsf(bf16_hi(r[i]))));
    }
    amax = block_max_256(amax, red);
    const float sc = div_by_const<448>(amax);
    const ScaleDiv dv(sc);
    for (uint32_t c = threadIdx.x; c < nch; c += 256) {
        u32x4 r = *reinterpret_cast<const u32x4 *>(xr + (size_t)c * 8);
        float v[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16_lo(r[i]);
            v[2 * i + 1] = bf16_hi(r[i]);
        }
        u32x2 o = {0, 0};
        if (sc != 0.0f)
            o = dv.fast ? enc8_e4m3_path<true>(v, dv) : enc8_e4m3_path<false>(v, dv);
        __builtin_nontemporal_store(o, reinterpret_cast<u32x2 *>(q + (size_t)row * k + (size_t)c * 8));
    }
    if (threadIdx.x == 0)
        s[row] = sc;
}

hipError_t launch_quant_rowwise_fp8(const uint16_t *x, uint8_t *q, float *s,
                                    uint32_t rows, uint32_t k, hipStream_t st)
{
    const uint32_t nch = k / 8;
    const dim3 gw((rows + 3) / 4), b(256);
#define QP_ROW_WAVE(C)                                                                        \
    else if (nch <= 64u * C) hipLaunchKernelGGL(k_quant_rowwise_fp8_wave<C>, gw, b, 0, st, x, q, \
                                                 s, rows, k);
    if (false) {
    }
    QP_ROW_WAVE(1) QP_ROW_WAVE(2) QP_ROW_WAVE(4) QP_ROW_WAVE(6) QP_ROW_WAVE(8)
    QP_ROW_WAVE(10) QP_ROW_WAVE(12) QP_ROW_WAVE(16)
    else if (nch <= 256u * 8)
        hipLaunchKernelGGL(k_quant_rowwise_fp8_wg<8>, dim3(rows), b, 0, st, x, q, s, k);
    else
        hipLaunchKernelGGL(k_quant_rowwise_fp8_long, dim3(rows), b, 0, st, x, q, s, k);
#undef QP_ROW_WAVE
    count_launch();
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Block-scaled FP8 -> row-wise FP8 (dispatch_proj_rowwise.rs,
// requant_weight_rowwise_fp8_cached), fused into one pass: the BF16
// intermediate y = bf16(fl(e4m3(w)*S)) is formed in registers, never stored.
// The row absmax is taken over the F32 products before their BF16 rounding:
// rounding is monotonic and sign-symmetric, so max|bf16(p)| = bf16(max|p|).
// ---------------------------------------------------------------------------

// Eight F32 products e4m3(code)*scale of the codes in dword pair (w0, w1)
// (two codes per converter call, exactly), then their BF16 pairs.
__device__ __forceinline__ void blockfp8_products(uint32_t w0, uint32_t w1, float scale,
                                                  float *p)
{
    const f32x2 e0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, false);
    const f32x2 e1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, true);
    const f32x2 e2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, false);
    const f32x2 e3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, true);
    p[0] = e0[0] * scale; p[1] = e0[1] * scale;
    p[2] = e1[0] * scale; p[3] = e1[1] * scale;
    p[4] = e2[0] * scale; p[5] = e2[1] * scale;
    p[6] = e3[0] * scale; p[7] = e3[1] * scale;
}

// RNE of a binary32 to BF16 and back (the BF16 intermediate of one value).
__device__ __forceinline__ float bf16_round(float v)
{
    return bf16_lo(pk_bf16(v, 0.0f));
}

// Long rows: a workgroup per row, two passes over global memory.
__global__ __launch_bounds__(256) void k_requant_blockfp8_rowwise_long(
    const uint8_t *__restrict__ w, const float *__restrict__ grid,
    uint8_t *__restrict__ q, float *__restrict__ s, uint32_t k)
{
    __shared__ float red[4];
    const uint32_t row = blockIdx.x;
    const uint8_t *wr = w + (size_t)row * k;
    const float *gr = grid + (size_t)(row / 128) * (k / 128);
    const uint32_t nch = k / 16;
    float amax = 0.0f;
    for (uint32_t c = threadIdx.x; c < nch; c += 256) {
        const u32x4 raw = *reinterpret_cast<const u32x4 *>(wr + (size_t)c * 16);
        const float bs = gr[(c * 16) / 128];
        float p[16];
        blockfp8_products(raw[0], raw[1], bs, &p[0]);
        blockfp8_products(raw[2], raw[3], bs, &p[8]);
#pragma unroll
        for (int i = 0; i < 16; ++i)
            amax = __builtin_fmaxf(amax, __builtin_fabsf(p[i]));
    }
    amax = bf16_round(block_max_256(amax, red));
    const float sc = div_by_const<448>(amax);
    const ScaleDiv dv(sc);
    for (uint32_t c = threadIdx.x; c < nch; c += 256) {
        const u32x4 raw = *reinterpret_cast<const u32x4 *>(wr + (size_t)c * 16);
        const float bs = gr[(c * 16) / 128];
        float y[16];
        blockfp8_products(raw[0], raw[1], bs, &y[0]);
        blockfp8_products(raw[2], raw[3], bs, &y[8]);
#pragma unroll
        for (int i = 0; i < 16; ++i)
            y[i] = bf16_round(y[i]);
        u32x4 o = {0, 0, 0, 0};
        if (sc != 0.0f) {
            const u32x2 lo = dv.fast ? enc8_e4m3_path<true>(&y[0], dv) : enc8_e4m3_path<false>(&y[0], dv);
            const u32x2 hi = dv.fast ? enc8_e4m3_path<true>(&y[8], dv) : enc8_e4m3_path<false>(&y[8], dv);
            o = (u32x4){lo[0], lo[1], hi[0], hi[1]};
        }
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(q + (size_t)row * k + (size_t)c * 16));
    }
    if (threadIdx.x == 0)
        s[row] = sc;
}

// Rows of up to 64*CPL 16-code chunks: one wave per row, the BF16
// intermediate kept packed (two values per register) between the passes.
template <int CPL>
__global__ __launch_bounds__(256) void k_requant_blockfp8_rowwise_wave(
    const uint8_t *__restrict__ w, const float *__restrict__ grid,
    uint8_t *__restrict__ q, float *__restrict__ s, uint32_t n, uint32_t k)
{
    const uint32_t row = blockIdx.x * 4u + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= n)
        return;                          // the whole wave
    const uint8_t *wr = w + (size_t)row * k;
    const float *gr = grid + (size_t)(row / 128) * (k / 128);
    const uint32_t nch = k / 16;
    u32x4 raw[CPL];
    float bs[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const uint32_t c = lane + 64u * j;
        raw[j] = (u32x4){0, 0, 0, 0};
        bs[j] = 0.0f;
        if (c < nch) {
            raw[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(wr + (size_t)c * 16));
            bs[j] = gr[(c * 16) / 128];
        }
    }
    uint32_t yb[CPL][8];                 // BF16 pairs of the intermediate
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        float p[16];
        blockfp8_products(raw[j][0], raw[j][1], bs[j], &p[0]);
        blockfp8_products(raw[j][2], raw[j][3], bs[j], &p[8]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            yb[j][i] = pk_bf16(p[2 * i], p[2 * i + 1]);
            amax = __builtin_fmaxf(amax, __builtin_fmaxf(__builtin_fabsf(p[2 * i]),
                                                         __builtin_fabsf(p[2 * i + 1])));
        }
    }
    amax = bf16_round(wave_max(amax));
    const float sc = div_by_const<448>(amax);
    const ScaleDiv dv(sc);
    // The scale is one per row (wave-uniform): pick the division path once.
    auto encode = [&](auto fast_tag) {
        constexpr bool FAST = decltype(fast_tag)::value;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const uint32_t c = lane + 64u * j;
            if (c < nch) {
                float v[16];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    v[2 * i] = bf16_lo(yb[j][i]);
                    v[2 * i + 1] = bf16_hi(yb[j][i]);
                }
                u32x4 o = {0, 0, 0, 0};
                if (sc != 0.0f) {
                    const u32x2 lo = enc8_e4m3_path<FAST>(&v[0], dv);
                    const u32x2 hi = enc8_e4m3_path<FAST>(&v[8], dv);
                    o = (u32x4){lo[0], lo[1], hi[0], hi[1]};
                }
                __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(q + (size_t)row * k + (size_t)c * 16));
            }
        }
    };
    if (dv.fast)
        encode(std::true_type{});
    else
        encode(std::false_type{});
    if (lane == 0)
        s[row] = sc;
}

hipError_t launch_requant_blockfp8_rowwise(const uint8_t *w, const float *grid,
                                           uint8_t *q, float *s, uint32_t n,
                                           uint32_t k, hipStream_t st)
{
    const uint32_t nch = k / 16;
    const dim3 gw((n + 3) / 4), b(256);
#define QP_BF8_WAVE(C)                                                                            \
    else if (nch <= 64u * C) hipLaunchKernelGGL(k_requant_blockfp8_rowwise_wave<C>, gw, b, 0, st, \
                                                 w, grid, q, s, n, k);
    if (false) {
    }
    QP_BF8_WAVE(2) QP_BF8_WAVE(4) QP_BF8_WAVE(5) QP_BF8_WAVE(6) QP_BF8_WAVE(8) QP_BF8_WAVE(12)
    QP_BF8_WAVE(16)
    else
        hipLaunchKernelGGL(k_requant_blockfp8_rowwise_long, dim3(n), b, 0, st, w, grid, q, s, k);
#undef QP_BF8_WAVE
    count_launch();
    return hipGetLastError();
}

} // namespace qp
