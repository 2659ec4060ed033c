/*
 * qproj.h -- C ABI of the quantized dense projection library (libqproj.so),
 * hand-written HIP for AMD Instinct MI355X (gfx950).
 *
 * The operations are the ones described on five documentation pages about an
 * LLM inference engine's quantized projections; each declaration below cites
 * the page (by its source file name) and the item on it.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer to dense, row-major memory whose
 *    last dimension (K) is contiguous.  BF16 is passed as uint16_t bit
 *    patterns; E4M3 (OCP E4M3FN) and packed E2M1 as uint8_t; packed E2M1
 *    holds element 2j in the low nibble of byte j and 2j+1 in the high one.
 *  - The caller owns every buffer, including scratch; the library allocates
 *    nothing, keeps no state beyond a launch counter, and never synchronises
 *    the host.  Work is enqueued on `stream` (a hipStream_t passed as void*;
 *    NULL = the default stream) and is ordered with the caller's other work
 *    on that stream.
 *  - Pointers must be 16-byte aligned.  Outputs must not alias inputs.
 *    Inputs holding NaN or Inf give unspecified (but in-bounds) results.
 *  - Each tensor must have fewer than 2^31 elements.
 *  - All arguments are checked on the host before any HIP call; a failed
 *    check returns a negative QP_ERR_* code and enqueues nothing.
 *
 * Rounding rules (the pages leave them open; this library fixes them):
 * absmax scaling (int8: amax/127; row-wise FP8: amax/448; NVFP4 sub-block:
 * E4M3(amax/(6*scale2))), one IEEE binary32 division of the element by the
 * stored scale, round-to-nearest-even onto the code grid, saturation at
 * +-127 / +-448 / +-6, the sign of a value rounding to zero kept (E4M3 0x80,
 * E2M1 0x8), and a block whose scale is 0 encoded as scale 0 with +0 codes.
 */
#ifndef QPROJ_H
#define QPROJ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define QP_OK 0
#define QP_ERR_NULL (-1)   /* a required pointer is NULL                   */
#define QP_ERR_SHAPE (-2)  /* a size is 0, too large, or breaks a multiple */
#define QP_ERR_RANGE (-3)  /* GEMV M outside its range (1..16, or 1..8)     */
#define QP_ERR_FORMAT (-4) /* unsupported weight format tag                 */
#define QP_ERR_HIP (-5)    /* the HIP runtime rejected a launch             */
#define QP_ERR_ALIGN (-6)  /* a pointer is not 16-byte aligned              */
#define QP_ERR_ALLOC (-7)  /* a derived-weight cache could not allocate     */
#define QP_ERR_SCRATCH (-8) /* the problem exceeds a fixed scratch array     */

/* Weight format tags of an FP8 weight (dispatch_proj_rowwise.rs tests:
 * Fp8PerRow, Fp8BlockScaled, Fp8SingleScale, Bf16, Nvfp4). */
enum qp_weight_format {
    QP_FP8_PER_ROW = 0,      /* E4M3 [N,K] + F32 [N]                        */
    QP_FP8_BLOCK128 = 1,     /* E4M3 [N,K] + F32 grid [N/128, K/128]        */
    QP_FP8_SINGLE_SCALE = 2, /* not accepted by the row-wise requant        */
    QP_BF16 = 3,             /* not accepted by the row-wise requant        */
    QP_NVFP4 = 4             /* not accepted by the row-wise requant        */
};

/* ------------------------------------------------------------------------
 * Weight requant, NVFP4 -> int8 with one F32 scale per 32
 * (gemm_dense_int8.rs, requant_w_nvfp4_int8).
 *   w_packed [n, k/2]  packed E2M1 codes
 *   w_e4m3   [n, k/16] E4M3 scale of each 16-element sub-block
 *   scale2             per-tensor F32 multiplier
 *   w_i8     [n, k]    out: int8 codes in -127..127
 *   w_scale  [n, k/32] out: F32 scale per 32-element block
 * Each value is dequantised as fl(e2m1 * e4m3 * scale2) (the first product is
 * exact), two sub-blocks are re-blocked into one 32-block, and the block is
 * quantised with s = amax/127, q = RNE(x/s).  Requires k % 32 == 0.
 * Each weight is derived once, either eagerly by the caller or by the
 * derived-weight cache below on its first request.
 * ---------------------------------------------------------------------- */
int requant_w_nvfp4_int8(const uint8_t *w_packed, const uint8_t *w_e4m3,
                         float scale2, int8_t *w_i8, float *w_scale,
                         uint32_t n, uint32_t k, void *stream);

/* ------------------------------------------------------------------------
 * Activation requant, BF16 -> int8 with one F32 scale per 32
 * (gemm_dense_int8.rs, int8_gemm_faith2_prefill, first launch).
 *   a       [m, k]    BF16
 *   a_i8    [m, k]    out: int8 codes
 *   a_scale [m, k/32] out: F32 scale per block, amax/127
 * Requires k % 32 == 0.
 * ---------------------------------------------------------------------- */
int requant_a_bf16_int8(const uint16_t *a, int8_t *a_i8, float *a_scale,
                        uint32_t m, uint32_t k, void *stream);

/* ------------------------------------------------------------------------
 * int8 x int8 block-scaled GEMM (gemm_dense_int8.rs, int8_gemm_faith2_prefill,
 * second launch):
 *   C[i,j] = bf16( sum_b a_scale[i,b] * w_scale[j,b] * P_b[i,j] ),
 *   P_b[i,j] = sum_{t in block b} a_i8[i,t] * w_i8[j,t]   (exact int32).
 *   a_i8 [m,k], w_i8 [n,k] (both K-contiguous), a_scale [m,k/32],
 *   w_scale [n,k/32], out [m,n] BF16.  Requires k % 32 == 0.
 * Each P_b is formed exactly on int8 MFMA; the scale-and-add runs in F32.
 * ---------------------------------------------------------------------- */
int int8_gemm_blockscaled(const int8_t *a_i8, const int8_t *w_i8,
                          const float *a_scale, const float *w_scale,
                          uint16_t *out, uint32_t m, uint32_t n, uint32_t k,
                          void *stream);

/* The two launches of the W4A8 prefill call in one: BF16 activations are
 * requantised into caller-owned scratch (a_i8_scratch >= m*k bytes,
 * a_scale_scratch >= m*(k/32) floats) and the GEMM above consumes them
 * (gemm_dense_int8.rs, int8_gemm_faith2_prefill). */
int int8_w4a8_prefill(const uint16_t *a_bf16, const int8_t *w_i8,
                      const float *w_scale, int8_t *a_i8_scratch,
                      float *a_scale_scratch, uint16_t *out,
                      uint32_t m, uint32_t n, uint32_t k, void *stream);

/* Ablation export: int8_gemm_blockscaled with the int8 operands converted
 * to FP16 in LDS and P_b formed on FP16 MFMA (exact: int8 values and block
 * partial sums are integers FP16 and F32 hold exactly), the fold one FMA per
 * output and block.  Same arguments and bit-identical output; requires
 * k % 128 == 0.  Measured slower than the int8-MFMA kernel on the prefill
 * shape, it is kept to time the two operand routes side by side
 * (gemm_dense_int8.rs, int8_gemm_faith2_prefill: int8 x int8 with per-32
 * block scales). */
int int8_gemm_blockscaled_f16ops(const int8_t *a_i8, const int8_t *w_i8,
                                 const float *a_scale, const float *w_scale,
                                 uint16_t *out, uint32_t m, uint32_t n, uint32_t k,
                                 void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * call as int8_w4a8_prefill, same kernels and bit-identical output, with the
 * activation scratch held in a fixed device array inside the library
 * (QP_NOALLOC_SCRATCH_BYTES per GPU, kept until the process ends) instead of
 * caller buffers.  It allocates nothing.  The scratch needs
 * align256(m*k) + 4*m*(k/32) bytes; a larger problem returns QP_ERR_SCRATCH
 * and enqueues nothing.  All calls on one GPU share that GPU's array, so
 * calls that overlap on one GPU (other streams, other threads) race: the
 * caller must order them.  The first call on each device looks the array's
 * address up once (hipGetSymbolAddress). */
#define QP_NOALLOC_SCRATCH_BYTES (24u << 20)
int int8_w4a8_prefill_noalloc(const uint16_t *a_bf16, const int8_t *w_i8,
                              const float *w_scale, uint16_t *out,
                              uint32_t m, uint32_t n, uint32_t k, void *stream);
/* QP_NOALLOC_SCRATCH_BYTES, as built into the library. */
uint64_t qproj_noalloc_scratch_bytes(void);

/* Test export: the exact int32 partial sum of every 32-K block,
 * p [m, n, k/32] (p[(i*n + j)*(k/32) + b] = P_b[i,j]), computed by the same
 * MFMA tile code as int8_gemm_blockscaled.  Requires k % 32 == 0. */
int int8_gemm_block_partials(const int8_t *a_i8, const int8_t *w_i8,
                             int32_t *p, uint32_t m, uint32_t n, uint32_t k,
                             void *stream);

/* Test export: the device encoders of the quantizer kernels applied to n
 * arbitrary binary32 values y (n % 8 == 0, n <= 2^30), one code per output
 * byte (E2M1 codes in the low nibble, int8 codes as two's-complement bytes).
 * Domains: E4M3_NOSAT |y| < 464; E2M1_NOSAT |y| <= 8; INT8 |y| < 127.5;
 * E4M3 and E2M1 (saturating first) any finite y; E4M3_SCALE finite y >= 0
 * (the NVFP4 block-scale encoder).  Outside its domain an encoder's output
 * is unspecified.  Rounding: to nearest, ties to the even code; a value
 * that rounds to zero keeps its sign. */
enum qp_encoder {
    QP_ENC_E4M3_NOSAT = 0, QP_ENC_E2M1_NOSAT = 1, QP_ENC_INT8 = 2,
    QP_ENC_E4M3 = 3, QP_ENC_E2M1 = 4, QP_ENC_E4M3_SCALE = 5
};
int qproj_encode_test(int kind, const float *y, uint8_t *out, uint32_t n, void *stream);

/* ------------------------------------------------------------------------
 * BF16 -> NVFP4 quantizer (gemm_fp4.rs, quantize_bf16_to_nvfp4).
 *   x       [rows, k]    BF16
 *   packed  [rows, k/2]  out: packed E2M1
 *   scale   [rows, k/16] out: E4M3 per 16-element block
 *   scale2               per-tensor F32 (the pages launch it with 1.0 for
 *                        activations)
 * sb = E4M3(fl(amax / fl(6*scale2))), d = fl(e4m3(sb)*scale2),
 * code = E2M1(fl(x/d)) (all +0 when d == 0).  Requires k % 32 == 0.
 * ---------------------------------------------------------------------- */
int quantize_bf16_nvfp4(const uint16_t *x, uint8_t *packed, uint8_t *scale,
                        float scale2, uint32_t rows, uint32_t k, void *stream);

/* ------------------------------------------------------------------------
 * NVFP4 x NVFP4 GEMM (gemm_fp4.rs, w4a4_gemm / w4a4_gemm_mfast):
 *   C[i,j] = bf16( scale_a2 * scale_w2 *
 *                  sum_b e4m3(a_scale[i,b]) * e4m3(w_scale[j,b]) * P_b ),
 *   P_b = sum_{t in 16-block b} e2m1(a[i,t]) * e2m1(w[j,t]).
 *   a_packed [m,k/2], a_scale [m,k/16], w_packed [n,k/2], w_scale [n,k/16],
 *   out [m,n] BF16.  Requires k % 32 == 0.  All five pointers 16-byte
 *   aligned, the scale grids included (unlike quantize_bf16_nvfp4's scale
 *   output, which needs only 2 bytes); else QP_ERR_ALIGN.
 * Each block's E4M3 scale is folded into its E2M1 operands (the product is
 * exact in FP16), so the contraction runs on FP16 MFMA with F32
 * accumulation and the per-block scaling costs no extra pass.
 * Enqueues one kernel, or two when the last round of large tiles is thin
 * enough to run as half tiles; the output bits are the same either way.
 * ---------------------------------------------------------------------- */
int w4a4_gemm(const uint8_t *a_packed, const uint8_t *a_scale,
              const uint8_t *w_packed, const uint8_t *w_scale, uint16_t *out,
              float scale_a2, float scale_w2, uint32_t m, uint32_t n,
              uint32_t k, void *stream);

/* w4a4_gemm with a chosen workgroup -> output-tile order, for the tile-order
 * ablation of gemm_fp4.rs (w4a4_gemm with an N-fast grid against
 * w4a4_gemm_mfast, whose M-fast grid lets neighbouring workgroups reuse one
 * weight panel):
 *   QP_TILES_BANDED  bands of 8 M-tiles walked M-fast, each XCD given a
 *                    contiguous range of workgroups (what w4a4_gemm uses);
 *   QP_TILES_MFAST   workgroup id = m-tile + (m-tiles) * n-tile;
 *   QP_TILES_NFAST   workgroup id = n-tile + (n-tiles) * m-tile.
 * Every order computes each output element identically (same bits).
 * Any other value: QP_ERR_FORMAT. */
#define QP_TILES_BANDED 0
#define QP_TILES_MFAST 1
#define QP_TILES_NFAST 2
int w4a4_gemm_tiles(const uint8_t *a_packed, const uint8_t *a_scale,
                    const uint8_t *w_packed, const uint8_t *w_scale, uint16_t *out,
                    float scale_a2, float scale_w2, uint32_t m, uint32_t n,
                    uint32_t k, int tile_order, void *stream);

/* ------------------------------------------------------------------------
 * Block-scaled FP8 -> row-wise FP8 weight requant
 * (dispatch_proj_rowwise.rs, rowwise_pair_passthrough and
 *  requant_weight_rowwise_fp8_cached).
 *   fmt == QP_FP8_PER_ROW: the weight already is the row-wise pair; sets
 *       *w_res = w, *scale_res = scale and returns QP_OK with no launch and
 *       no write to w_out / scale_out (w_out / scale_out may be NULL; n and k
 *       are not checked).
 *   fmt == QP_FP8_BLOCK128: w [n,k] E4M3 with an F32 grid scale
 *       [n/128, k/128]; per row y = bf16(fl(e4m3(w)*S[i/128][t/128])), then
 *       s = amax(y)/448, code = E4M3(fl(y/s)) into w_out [n,k] and
 *       scale_out [n]; sets *w_res = w_out, *scale_res = scale_out.  The BF16
 *       intermediate never touches memory (one fused pass).  Requires
 *       n % 128 == 0 and k % 128 == 0.
 *   any other tag: QP_ERR_FORMAT.
 * w_res / scale_res may be NULL when the caller does not want them.
 * ---------------------------------------------------------------------- */
int requant_w_blockfp8_rowwise(int fmt, const uint8_t *w, const float *scale,
                               uint8_t *w_out, float *scale_out,
                               const uint8_t **w_res, const float **scale_res,
                               uint32_t n, uint32_t k, void *stream);

/* ------------------------------------------------------------------------
 * Row-wise FP8 quantizer (dispatch_proj_rowwise.rs, quant_rowwise_fp8; the
 * same arithmetic as quantize_fns.rs, quantize_to_fp8).
 *   x [rows,k] BF16 -> q [rows,k] E4M3, scale [rows] F32 = amax/448.
 * Requires k % 16 == 0.
 * ---------------------------------------------------------------------- */
int quant_rowwise_fp8(const uint16_t *x, uint8_t *q, float *scale,
                      uint32_t rows, uint32_t k, void *stream);

/* ------------------------------------------------------------------------
 * Row-wise FP8 GEMM (the contraction at the end of dispatch_proj_rowwise.rs,
 * cublas_fp8_rowwise_proj):
 *   C[i,j] = bf16( a_scale[i] * w_scale[j] * sum_t e4m3(a[i,t]) * e4m3(w[j,t]) ).
 *   a [m,k] E4M3, a_scale [m] F32, w [n,k] E4M3, w_scale [n] F32,
 *   out [m,n] BF16.  Requires k % 16 == 0.  Any m is served (no padding).
 * Enqueues one kernel, or two when the last round of large tiles is thin
 * enough to run as half tiles; the output bits are the same either way.
 * ---------------------------------------------------------------------- */
int fp8_gemm_rowscale(const uint8_t *a, const float *a_scale, const uint8_t *w,
                      const float *w_scale, uint16_t *out, uint32_t m,
                      uint32_t n, uint32_t k, void *stream);

/* The whole row-wise projection (dispatch_proj_rowwise.rs,
 * cublas_fp8_rowwise_proj): the weight goes through
 * requant_w_blockfp8_rowwise (passthrough when fmt == QP_FP8_PER_ROW, else
 * requantised into w_rowwise / w_rowwise_scale, which may be NULL for the
 * passthrough), the BF16 activations are quantised per row into caller-owned
 * scratch (act_q >= m*k bytes, act_scale >= m floats), then
 * fp8_gemm_rowscale writes out [m,n].  Requires k % 128 == 0 for block
 * weights, k % 16 == 0 otherwise. */
int fp8_rowwise_proj(int fmt, const uint8_t *w, const float *w_scale,
                     uint8_t *w_rowwise, float *w_rowwise_scale,
                     const uint16_t *act, uint8_t *act_q, float *act_scale,
                     uint16_t *out, uint32_t m, uint32_t n, uint32_t k,
                     void *stream);

/* ------------------------------------------------------------------------
 * Row-scaled FP8 GEMV for decode / verify batches
 * (fp8_gemv_batch.rs, fp8_gemv_rowscale_batch8_rt2 / _batch16_rt2,
 *  dense_gemv_fp8w_batch2):
 *   C[i,j] = bf16( row_scale[j] * sum_t x[i,t] * e4m3(w[j,t]) ),
 *   x [m,k] BF16, w [n,k] E4M3, row_scale [n] F32, out [m,n] BF16.
 * 1 <= m <= 16 (else QP_ERR_RANGE); k % 16 == 0, n*k and m*n < 2^31 and
 * 2*m*k < 2^31 (else QP_ERR_SHAPE).  The weight is streamed from memory
 * once for all m rows, and every output row is bit-identical to the m == 1
 * call on that row.  A row's K summation order depends on k alone, so an
 * output is also bit-identical across calls with different n (a weight's
 * first rows called as a weight of their own).
 * ---------------------------------------------------------------------- */
int fp8_gemv_rowscale(const uint16_t *x, const uint8_t *w,
                      const float *row_scale, uint16_t *out, uint32_t m,
                      uint32_t n, uint32_t k, void *stream);

/* ------------------------------------------------------------------------
 * fp8_gemv_blockscale -- block-scaled FP8-weight GEMV for decode and verify
 * batches (fp8_gemv_batch.rs, w8a16_gemv_batch4 / w8a16_gemv_batch2, the
 * batched siblings of w8a16_gemv, which take the raw 2D block-scaled FP8
 * weight):
 *   C[i,j] = bf16( sum_t x[i,t] * e4m3(w[j,t]) * block_scale[j/128][t/128] ),
 *   x [m,k] BF16, w [n,k] E4M3, block_scale [n/128, k/128] F32 row-major,
 *   out [m,n] BF16; all device memory owned by the caller, out written.
 * 1 <= m <= 16 (else QP_ERR_RANGE; the pages' batched kernels stop at 4);
 * n % 128 == 0, k % 128 == 0, n*k and m*n < 2^31 and 2*m*k < 2^31 (else
 * QP_ERR_SHAPE).  Each 128-element K
 * block is summed in F32 and added to the running F32 sum with one FMA by
 * its scale; the BF16 rounding happens once at the end.  The weight is
 * streamed once for all m rows, and every output row is bit-identical to the
 * m == 1 call on that row, and across calls with different n.
 * ---------------------------------------------------------------------- */
int fp8_gemv_blockscale(const uint16_t *x, const uint8_t *w,
                        const float *block_scale, uint16_t *out, uint32_t m,
                        uint32_t n, uint32_t k, void *stream);

/* ------------------------------------------------------------------------
 * w4a16_gemv -- NVFP4-weight GEMV for decode and verify batches
 * (fp8_gemv_batch.rs names w4a16_gemv_batch8_rt2 as the NVFP4 twin of the
 * row-scaled FP8 GEMV):
 *   C[i,j] = bf16( scale2 * sum_t x[i,t] * e2m1(w[j,t]) * e4m3(s[j,t/16]) ),
 *   x        [m, k]    BF16
 *   w_packed [n, k/2]  E2M1 codes, element 2t in the low nibble of byte t
 *   w_e4m3   [n, k/16] E4M3 scale of each 16-element block
 *   scale2             per-tensor F32 multiplier (value = e2m1*e4m3*scale2,
 *                      the layout quantize_bf16_nvfp4 writes)
 *   out      [m, n]    BF16, written
 * All device memory owned by the caller.  1 <= m <= 8, the pages' batch
 * (else QP_ERR_RANGE); k % 32 == 0 and 2*m*k < 2^30 (else QP_ERR_SHAPE).
 * Each dequantised weight e2m1*e4m3 is exact in BF16; the products with x
 * are exact and summed in F32; scale2 multiplies the F32 sum at write-out
 * and BF16 rounding happens once.  The weight is streamed once for all m rows,
 * and every output row is bit-identical to the m == 1 call on that row.
 * ---------------------------------------------------------------------- */
int w4a16_gemv(const uint16_t *x, const uint8_t *w_packed, const uint8_t *w_e4m3,
               float scale2, uint16_t *out, uint32_t m, uint32_t n, uint32_t k,
               void *stream);

/* ------------------------------------------------------------------------
 * Derived-weight cache (dispatch_proj_rowwise.rs,
 * requant_weight_rowwise_fp8_cached and its DerivedWeights cache, keyed by
 * the weight pointer; gemm_dense_int8.rs, requant_w_nvfp4_int8, whose int8
 * copy is made once per weight).
 *
 * A cache maps (derivation, source weight address) to a requantised copy
 * that the cache allocates with hipMalloc on the first request (a miss),
 * fills with the stateless entry point's kernel on the caller's stream, and
 * keeps until qproj_cache_evict or qproj_cache_destroy.  Later requests (hits)
 * return the same device pointers, enqueue no kernel, and make the caller's
 * stream wait for the derivation (an event recorded after it), so a derived
 * weight may be used from any stream.  Nothing here synchronises the host.
 * A request whose sizes (or NVFP4 scale2) differ from the entry's returns
 * QP_ERR_SHAPE: the address then holds another weight, so evict it first.
 * A miss is not safe under stream capture (it allocates); hits are.  All
 * functions are thread-safe; a miss holds the cache's lock, so concurrent
 * requests for one weight derive it once.  Errors: QP_ERR_NULL, QP_ERR_ALIGN,
 * QP_ERR_SHAPE, QP_ERR_FORMAT as for the stateless entry points;
 * QP_ERR_ALLOC when hipMalloc fails (nothing is inserted).
 * ---------------------------------------------------------------------- */
typedef struct qp_cache qp_cache;

int qproj_cache_create(qp_cache **cache);
/* Frees every derived buffer; no kernel that reads one may still be pending. */
int qproj_cache_destroy(qp_cache *cache);
/* Drops every derivation of the weight at `weight` (no-op if there is none);
 * no kernel that reads one may still be pending. */
int qproj_cache_evict(qp_cache *cache, const void *weight);
int qproj_cache_stats(qp_cache *cache, uint64_t *entries, uint64_t *bytes);

/* requant_w_blockfp8_rowwise through the cache, keyed by w.  QP_FP8_PER_ROW
 * returns (w, scale) itself with no work, no allocation and no entry (the
 * pages' passthrough); QP_FP8_BLOCK128 returns the cached row-wise copy
 * (E4M3 [n,k] + F32 [n], owned by the cache). */
int requant_w_blockfp8_rowwise_cached(qp_cache *cache, int fmt, const uint8_t *w,
                                      const float *scale, uint32_t n, uint32_t k,
                                      const uint8_t **w_rowwise,
                                      const float **w_rowwise_scale, void *stream);
/* requant_w_nvfp4_int8 through the cache, keyed by w_packed: the int8 copy
 * [n,k] and its F32 per-32 scales [n,k/32], owned by the cache. */
int requant_w_nvfp4_int8_cached(qp_cache *cache, const uint8_t *w_packed,
                                const uint8_t *w_e4m3, float scale2, uint32_t n,
                                uint32_t k, const int8_t **w_i8,
                                const float **w_scale, void *stream);
/* fp8_rowwise_proj with the weight requantised through the cache (the pages'
 * cublas_fp8_rowwise_proj): no weight scratch argument. */
int fp8_rowwise_proj_cached(qp_cache *cache, int fmt, const uint8_t *w,
                            const float *w_scale, const uint16_t *act,
                            uint8_t *act_q, float *act_scale, uint16_t *out,
                            uint32_t m, uint32_t n, uint32_t k, void *stream);
/* int8_w4a8_prefill from an NVFP4 weight, requantised to int8 through the
 * cache on first use. */
int int8_w4a8_prefill_cached(qp_cache *cache, const uint16_t *a_bf16,
                             const uint8_t *w_packed, const uint8_t *w_e4m3,
                             float scale2, int8_t *a_i8_scratch,
                             float *a_scale_scratch, uint16_t *out, uint32_t m,
                             uint32_t n, uint32_t k, void *stream);

/* ------------------------------------------------------------------------
 * Library information.
 * ---------------------------------------------------------------------- */
/* Number of kernel launches this process has enqueued through the library
 * (a passthrough adds none). */
uint64_t qproj_launch_count(void);
/* Static description of a return code. */
const char *qproj_status_string(int status);
/* ABI version of this header. */
int qproj_abi_version(void);
#define QPROJ_ABI_VERSION 1

#ifdef __cplusplus
}
#endif

#endif /* QPROJ_H */
