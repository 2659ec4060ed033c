// quant.hip -- streaming quantizers and weight requantizers for gfx950.
//
// All of them are HBM-bound: every byte is read once with 16-byte vector
// loads, codes are written with 8- or 16-byte stores, and absmax reductions
// stay in registers (per-block kernels) or use wave shuffles plus one LDS
// exchange per workgroup (per-row kernels).
#include "qp_device.hpp"
#include "qp_launch.hpp"

namespace qp {

// ---------------------------------------------------------------------------
// BF16 -> int8, one F32 scale per 32 (gemm_dense_int8.rs,
// int8_gemm_faith2_prefill, activation launch).  Two lanes per 32-block,
// 16 elements per lane; the pair exchanges its partial absmax with one
// shuffle.  Flattened indexing is valid because k % 32 == 0: a block never
// straddles a row, and block id = chunk id / 2 in the [m, k/32] scale grid.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_requant_a_bf16_int8(
    const uint16_t *__restrict__ a, int8_t *__restrict__ q,
    float *__restrict__ s, uint32_t nchunks)
{
    uint32_t c = blockIdx.x * 256u + threadIdx.x;
    bool valid = c < nchunks;            // nchunks is even: pairs agree
    u32x4 v0 = {0, 0, 0, 0}, v1 = {0, 0, 0, 0};
    if (valid) {
        const u32x4 *p = reinterpret_cast<const u32x4 *>(a + (size_t)c * 16);
        v0 = __builtin_nontemporal_load(p);
        v1 = __builtin_nontemporal_load(p + 1);
    }
    float x[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = bf16_lo(v0[i]);
        x[2 * i + 1] = bf16_hi(v0[i]);
        x[8 + 2 * i] = bf16_lo(v1[i]);
        x[8 + 2 * i + 1] = bf16_hi(v1[i]);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        amax = __builtin_fmaxf(amax, __builtin_fabsf(x[i]));
    amax = __builtin_fmaxf(amax, __shfl_xor(amax, 1, WAVE));
    float sc = div_rn(amax, 127.0f);
    u32x4 out = {0, 0, 0, 0};
    if (sc != 0.0f) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            uint32_t b = (uint32_t)enc_i8(div_rn(x[i], sc)) & 0xFFu;
            out[i / 4] |= b << (8 * (i % 4));
        }
    }
    if (valid) {
        *reinterpret_cast<u32x4 *>(q + (size_t)c * 16) = out;
        if ((c & 1u) == 0u)
            s[c >> 1] = sc;
    }
}

hipError_t launch_requant_a_bf16_int8(const uint16_t *a, int8_t *q, float *s,
                                      uint32_t m, uint32_t k, hipStream_t st)
{
    uint32_t nchunks = (uint32_t)((uint64_t)m * k / 16);
    uint32_t grid = (nchunks + 255) / 256;
    hipLaunchKernelGGL(k_requant_a_bf16_int8, dim3(grid), dim3(256), 0, st,
                       a, q, s, nchunks);
    count_launch();
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// NVFP4 -> int8 weight requant (gemm_dense_int8.rs, requant_w_nvfp4_int8).
// One lane per 32-block: 16 packed bytes + 2 E4M3 sub-block scales in, 32
// int8 + 1 F32 out.  v = fl(fl(e2m1*e4m3)*scale2) (the first product exact),
// then absmax / 127 and RNE(v/s).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_requant_w_nvfp4_int8(
    const uint8_t *__restrict__ packed, const uint8_t *__restrict__ sc16,
    float scale2, int8_t *__restrict__ q, float *__restrict__ s,
    uint32_t nblocks)
{
    uint32_t b = blockIdx.x * 256u + threadIdx.x;
    if (b >= nblocks)
        return;
    u32x4 p = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4 *>(packed + (size_t)b * 16));
    uint32_t scw = *reinterpret_cast<const uint16_t *>(sc16 + (size_t)b * 2);
    float d0 = dec_e4m3(scw & 0xFFu), d1 = dec_e4m3(scw >> 8);
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        uint32_t byte = (p[i / 8] >> (8 * ((i / 2) % 4))) & 0xFFu;
        uint32_t code = (i % 2 == 0) ? (byte & 15u) : (byte >> 4);
        float prod = dec_e2m1(code) * (i < 16 ? d0 : d1);   // exact
        v[i] = prod * scale2;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i)
        amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
    float sc = div_rn(amax, 127.0f);
    u32x4 o0 = {0, 0, 0, 0}, o1 = {0, 0, 0, 0};
    if (sc != 0.0f) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            o0[i / 4] |= ((uint32_t)enc_i8(div_rn(v[i], sc)) & 0xFFu) << (8 * (i % 4));
            o1[i / 4] |= ((uint32_t)enc_i8(div_rn(v[16 + i], sc)) & 0xFFu) << (8 * (i % 4));
        }
    }
    u32x4 *qo = reinterpret_cast<u32x4 *>(q + (size_t)b * 32);
    qo[0] = o0;
    qo[1] = o1;
    s[b] = sc;
}

hipError_t launch_requant_w_nvfp4_int8(const uint8_t *packed, const uint8_t *sc16,
                                       float scale2, int8_t *q, float *s,
                                       uint32_t n, uint32_t k, hipStream_t st)
{
    uint32_t nblocks = (uint32_t)((uint64_t)n * (k / 32));
    hipLaunchKernelGGL(k_requant_w_nvfp4_int8, dim3((nblocks + 255) / 256),
                       dim3(256), 0, st, packed, sc16, scale2, q, s, nblocks);
    count_launch();
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// BF16 -> NVFP4 (gemm_fp4.rs, quantize_bf16_to_nvfp4).  One lane per 32
// elements = two 16-element blocks: 64 bytes in, 16 packed bytes and two
// E4M3 scales out.  sb = E4M3(fl(amax/fl(6*scale2))), d = fl(e4m3(sb)*scale2),
// code = E2M1(fl(x/d)), or +0 everywhere when d == 0.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_quantize_bf16_nvfp4(
    const uint16_t *__restrict__ x, uint8_t *__restrict__ packed,
    uint8_t *__restrict__ sc16, float scale2, uint32_t nchunks)
{
    uint32_t c = blockIdx.x * 256u + threadIdx.x;
    if (c >= nchunks)
        return;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(x + (size_t)c * 32);
    u32x4 raw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        raw[i] = __builtin_nontemporal_load(src + i);
    const float six_s2 = 6.0f * scale2;
    u32x4 out = {0, 0, 0, 0};
    uint32_t scales = 0;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t wd = raw[2 * blk + i / 4][i % 4];
            v[2 * i] = bf16_lo(wd);
            v[2 * i + 1] = bf16_hi(wd);
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
        uint32_t sb = enc_e4m3(div_rn(amax, six_s2));
        float d = dec_e4m3(sb) * scale2;
        scales |= sb << (8 * blk);
        if (d != 0.0f) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                uint32_t code = enc_e2m1(div_rn(v[i], d));
                out[2 * blk + i / 8] |= code << (4 * (i % 8));
            }
        }
    }
    *reinterpret_cast<u32x4 *>(packed + (size_t)c * 16) = out;
    *reinterpret_cast<uint16_t *>(sc16 + (size_t)c * 2) = (uint16_t)scales;
}

hipError_t launch_quantize_bf16_nvfp4(const uint16_t *x, uint8_t *packed,
                                      uint8_t *sc16, float scale2, uint32_t rows,
                                      uint32_t k, hipStream_t st)
{
    uint32_t nchunks = (uint32_t)((uint64_t)rows * k / 32);
    hipLaunchKernelGGL(k_quantize_bf16_nvfp4, dim3((nchunks + 255) / 256),
                       dim3(256), 0, st, x, packed, sc16, scale2, nchunks);
    count_launch();
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-row kernels: one 256-thread workgroup per row.
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

// Encode 8 f32 values (already divided-by-scale inputs are formed here) to
// E4M3 bytes packed in two dwords.
__device__ __forceinline__ u32x2 enc8_e4m3(const float *v, float sc)
{
    u32x2 o = {0, 0};
    if (sc != 0.0f) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            o[i / 4] |= enc_e4m3(div_rn(v[i], sc)) << (8 * (i % 4));
    }
    return o;
}

// Row-wise FP8 quantizer (dispatch_proj_rowwise.rs, quant_rowwise_fp8).
// CPT 16-byte chunks (8 BF16 each) per thread stay in registers between the
// absmax pass and the encode pass, so each input byte is read once.
template <int CPT>
__global__ __launch_bounds__(256) void k_quant_rowwise_fp8(
    const uint16_t *__restrict__ x, uint8_t *__restrict__ q,
    float *__restrict__ s, uint32_t k)
{
    __shared__ float red[4];
    const uint32_t row = blockIdx.x;
    const uint16_t *xr = x + (size_t)row * k;
    const uint32_t nch = k / 8;
    u32x4 raw[CPT];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        uint32_t c = threadIdx.x + 256u * j;
        raw[j] = (u32x4){0, 0, 0, 0};
        if (c < nch)
            raw[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(xr + (size_t)c * 8));
#pragma unroll
        for (int i = 0; i < 4; ++i)
            amax = __builtin_fmaxf(amax, __builtin_fmaxf(__builtin_fabsf(bf16_lo(raw[j][i])),
                                                         __builtin_fabsf(bf16_hi(raw[j][i]))));
    }
    amax = block_max_256(amax, red);
    const float sc = div_rn(amax, 448.0f);
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        uint32_t c = threadIdx.x + 256u * j;
        if (c < nch) {
            float v[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = bf16_lo(raw[j][i]);
                v[2 * i + 1] = bf16_hi(raw[j][i]);
            }
            *reinterpret_cast<u32x2 *>(q + (size_t)row * k + (size_t)c * 8) = enc8_e4m3(v, sc);
        }
    }
    if (threadIdx.x == 0)
        s[row] = sc;
}

// Long rows: the same arithmetic in two passes over global memory.
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
    const float sc = div_rn(amax, 448.0f);
    for (uint32_t c = threadIdx.x; c < nch; c += 256) {
        u32x4 r = *reinterpret_cast<const u32x4 *>(xr + (size_t)c * 8);
        float v[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16_lo(r[i]);
            v[2 * i + 1] = bf16_hi(r[i]);
        }
        *reinterpret_cast<u32x2 *>(q + (size_t)row * k + (size_t)c * 8) = enc8_e4m3(v, sc);
    }
    if (threadIdx.x == 0)
        s[row] = sc;
}

hipError_t launch_quant_rowwise_fp8(const uint16_t *x, uint8_t *q, float *s,
                                    uint32_t rows, uint32_t k, hipStream_t st)
{
    uint32_t nch = k / 8;
    dim3 g(rows), b(256);
    if (nch <= 256)
        hipLaunchKernelGGL(k_quant_rowwise_fp8<1>, g, b, 0, st, x, q, s, k);
    else if (nch <= 512)
        hipLaunchKernelGGL(k_quant_rowwise_fp8<2>, g, b, 0, st, x, q, s, k);
    else if (nch <= 768)
        hipLaunchKernelGGL(k_quant_rowwise_fp8<3>, g, b, 0, st, x, q, s, k);
    else if (nch <= 1024)
        hipLaunchKernelGGL(k_quant_rowwise_fp8<4>, g, b, 0, st, x, q, s, k);
    else if (nch <= 2048)
        hipLaunchKernelGGL(k_quant_rowwise_fp8<8>, g, b, 0, st, x, q, s, k);
    else
        hipLaunchKernelGGL(k_quant_rowwise_fp8_long, g, b, 0, st, x, q, s, k);
    count_launch();
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Block-scaled FP8 -> row-wise FP8 (dispatch_proj_rowwise.rs,
// requant_weight_rowwise_fp8_cached), fused into one pass: the BF16
// intermediate y = bf16(fl(e4m3(w)*S)) is formed in registers, never stored.
// CPT 16-byte chunks (16 codes each, inside one 128-column block) per thread.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void blockfp8_to_bf16_vals(u32x4 raw, float scale, float *y)
{
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float p = dec_e4m3((raw[i / 4] >> (8 * (i % 4))) & 0xFFu) * scale;
        y[i] = __uint_as_float(f32_to_bf16(p) << 16);
    }
}

template <int CPT>
__global__ __launch_bounds__(256) void k_requant_blockfp8_rowwise(
    const uint8_t *__restrict__ w, const float *__restrict__ grid,
    uint8_t *__restrict__ q, float *__restrict__ s, uint32_t k)
{
    __shared__ float red[4];
    const uint32_t row = blockIdx.x;
    const uint8_t *wr = w + (size_t)row * k;
    const float *gr = grid + (size_t)(row / 128) * (k / 128);
    const uint32_t nch = k / 16;
    float y[CPT][16];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        uint32_t c = threadIdx.x + 256u * j;
        u32x4 raw = {0, 0, 0, 0};
        float scale = 0.0f;
        if (c < nch) {
            raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(wr + (size_t)c * 16));
            scale = gr[(c * 16) / 128];
        }
        blockfp8_to_bf16_vals(raw, scale, y[j]);
#pragma unroll
        for (int i = 0; i < 16; ++i)
            amax = __builtin_fmaxf(amax, __builtin_fabsf(y[j][i]));
    }
    amax = block_max_256(amax, red);
    const float sc = div_rn(amax, 448.0f);
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        uint32_t c = threadIdx.x + 256u * j;
        if (c < nch) {
            u32x2 lo = enc8_e4m3(&y[j][0], sc), hi = enc8_e4m3(&y[j][8], sc);
            u32x4 o = {lo[0], lo[1], hi[0], hi[1]};
            *reinterpret_cast<u32x4 *>(q + (size_t)row * k + (size_t)c * 16) = o;
        }
    }
    if (threadIdx.x == 0)
        s[row] = sc;
}

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
    float y[16];
    for (uint32_t c = threadIdx.x; c < nch; c += 256) {
        u32x4 raw = *reinterpret_cast<const u32x4 *>(wr + (size_t)c * 16);
        blockfp8_to_bf16_vals(raw, gr[(c * 16) / 128], y);
#pragma unroll
        for (int i = 0; i < 16; ++i)
            amax = __builtin_fmaxf(amax, __builtin_fabsf(y[i]));
    }
    amax = block_max_256(amax, red);
    const float sc = div_rn(amax, 448.0f);
    for (uint32_t c = threadIdx.x; c < nch; c += 256) {
        u32x4 raw = *reinterpret_cast<const u32x4 *>(wr + (size_t)c * 16);
        blockfp8_to_bf16_vals(raw, gr[(c * 16) / 128], y);
        u32x2 lo = enc8_e4m3(&y[0], sc), hi = enc8_e4m3(&y[8], sc);
        u32x4 o = {lo[0], lo[1], hi[0], hi[1]};
        *reinterpret_cast<u32x4 *>(q + (size_t)row * k + (size_t)c * 16) = o;
    }
    if (threadIdx.x == 0)
        s[row] = sc;
}

hipError_t launch_requant_blockfp8_rowwise(const uint8_t *w, const float *grid,
                                           uint8_t *q, float *s, uint32_t n,
                                           uint32_t k, hipStream_t st)
{
    uint32_t nch = k / 16;
    dim3 g(n), b(256);
    if (nch <= 256)
        hipLaunchKernelGGL(k_requant_blockfp8_rowwise<1>, g, b, 0, st, w, grid, q, s, k);
    else if (nch <= 512)
        hipLaunchKernelGGL(k_requant_blockfp8_rowwise<2>, g, b, 0, st, w, grid, q, s, k);
    else if (nch <= 1024)
        hipLaunchKernelGGL(k_requant_blockfp8_rowwise<4>, g, b, 0, st, w, grid, q, s, k);
    else
        hipLaunchKernelGGL(k_requant_blockfp8_rowwise_long, g, b, 0, st, w, grid, q, s, k);
    count_launch();
    return hipGetLastError();
}

} // namespace qp
