// qp_device.hpp -- device-side codecs and small helpers shared by the
// gfx950 kernels of libqproj.  Written for CDNA4 wave64 only.
//
// Formats (the documentation pages name them "E2M1" and "E4M3"; the bit
// layouts are the OCP ones): E4M3FN with bias 7, max 448, S.1111.111 = NaN;
// E2M1 with magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}.  Rounding onto any grid
// is to nearest with ties to the even code, saturating at the largest
// finite magnitude, keeping the sign of a value that rounds to zero.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qp {

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(32))) float f32x32;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(16))) int i32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;

constexpr int WAVE = 64;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// f32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ------------------------------------------------------------------ E4M3
// Encode a finite f32 to E4M3FN: RNE, |y| >= 448 saturates to 0x7E.
// Normal range: integer round-to-nearest-even on the f32 bit pattern (keep
// 3 mantissa bits), then re-bias the exponent 127 -> 7.  Below 2^-6 the grid
// is uniform with step 2^-9, so RNE of y*2^9 is the code itself.
__device__ __forceinline__ uint32_t enc_e4m3(float y)
{
    uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
    float a = __builtin_fabsf(y);
    uint32_t code;
    if (a >= 448.0f) {
        code = 0x7Eu;
    } else if (a < 0.015625f) {
        code = (uint32_t)__builtin_rintf(a * 512.0f);
    } else {
        uint32_t ua = __float_as_uint(a);
        code = ((ua + 0x7FFFFu + ((ua >> 20) & 1u)) >> 20) - (120u << 3);
    }
    return code | sign;
}

// Decode E4M3FN (finite codes) to f32, exactly, with the gfx950 converter.
__device__ __forceinline__ float dec_e4m3(uint32_t byte)
{
    return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
}

// ------------------------------------------------------------------ E2M1
// Encode a finite f32 to E2M1: the code index is the number of decision
// thresholds |y| has passed.  Thresholds sit at the midpoints 0.25, 0.75,
// 1.25, 1.75, 2.5, 3.5, 5; a value exactly on one goes to the even code,
// hence ">" where the lower neighbour is even and ">=" where the upper one is.
__device__ __forceinline__ uint32_t enc_e2m1(float y)
{
    uint32_t sign = (__float_as_uint(y) >> 28) & 8u;
    float a = __builtin_fabsf(y);
    uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) +
                 (uint32_t)(a > 1.25f) + (uint32_t)(a >= 1.75f) +
                 (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                 (uint32_t)(a > 5.0f);
    return c | sign;
}

// E2M1 value of code c (0..15).
__device__ __forceinline__ float dec_e2m1(uint32_t c)
{
    // Table packed in two 32-bit words: twice the magnitude, 4 bits each.
    // 2*{0, .5, 1, 1.5, 2, 3, 4, 6} = {0, 1, 2, 3, 4, 6, 8, 12}.
    uint32_t twice = (0xC8643210u >> ((c & 7u) * 4u)) & 15u;
    float v = (float)twice * 0.5f;
    return (c & 8u) ? -v : v;
}

// ------------------------------------------------------------------ int8
__device__ __forceinline__ int enc_i8(float y)
{
    float r = __builtin_rintf(y);
    r = __builtin_fminf(__builtin_fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

// IEEE binary32 division, correctly rounded (the library is built with
// correctly rounded f32 division).
__device__ __forceinline__ float div_rn(float x, float y) { return x / y; }

// One correction step of a quotient by a known reciprocal (Markstein): with
// r = RN(1/s) and q0 = RN(x*r) (within an ulp of x/s), the remainder
// x - q0*s is exact in one FMA, and RN(q0 + rem*r) is RN(x/s), barring
// underflow and overflow in the intermediate steps.  The remainder is formed
// negated, t = q0*s - x, and enters the second FMA with its sign flipped:
// that is the same value whenever it is nonzero, while an exactly zero
// remainder becomes -0, so q0 + (-0)*r keeps q0's sign and x = -0 gives
// -0 (the plain form would turn it into +0).
__device__ __forceinline__ float div_corr(float x, float s, float r)
{
    const float q0 = x * r;
    const float t = __builtin_fmaf(q0, s, -x);
    return __builtin_fmaf(-t, r, q0);
}

// fl(a / 127) and fl(a / 448) through div_corr with the constant's correctly
// rounded reciprocal.  Valid for a == 0 and for a in [2^-100, 2^126], where no
// step under- or overflows; there the result depends on a's significand
// alone (scaling a by a power of two scales every step exactly), and it was
// checked against the IEEE quotient for every binary32 significand.
constexpr float RCP_127 = 0x1.020408p-7f;   // RN(1/127)
constexpr float RCP_448 = 0x1.24924ap-9f;   // RN(1/448)
__device__ __forceinline__ bool const_div_ok(float a)
{
    return a == 0.0f || (a >= 0x1p-100f && a <= 0x1p126f);
}

// a / 127 (or 448) correctly rounded, for one value per lane: the reciprocal
// form when every active lane of the wave allows it, else the division
// instruction sequence.
template <int B>
__device__ __forceinline__ float div_by_const(float a)
{
    constexpr float R = B == 127 ? RCP_127 : RCP_448;
    static_assert(B == 127 || B == 448, "constant divisors: 127, 448");
    if (__all(const_div_ok(a)))
        return div_corr(a, (float)B, R);
    return div_rn(a, (float)B);
}

// Correctly rounded x / s for many x and one s, in three operations per x:
// r = RN(1/s) (one IEEE division per scale), then div_corr.  Scales outside
// [2^-100, 2^100] take the division instruction sequence instead.
struct ScaleDiv {
    float s, r;
    bool fast;
    __device__ __forceinline__ explicit ScaleDiv(float s_) : s(s_)
    {
        fast = s_ >= 0x1p-100f && s_ <= 0x1p100f;
        r = fast ? div_rn(1.0f, s_) : 0.0f;
    }
    // From a reciprocal known to be RN(1/s_) (a table entry).
    __device__ __forceinline__ ScaleDiv(float s_, float r_) : s(s_), r(r_)
    {
        fast = s_ >= 0x1p-100f && s_ <= 0x1p100f;
    }
    __device__ __forceinline__ float quick(float x) const { return div_corr(x, s, r); }
    __device__ __forceinline__ float operator()(float x) const
    {
        return fast ? quick(x) : div_rn(x, s);
    }
};

// t[i] = x[i] / d.s for N values, each correctly rounded.  One wave vote picks
// the branch-free quotient for every value when every active lane's scale
// allows it (the common case); otherwise each value takes operator(), whose
// per-value branches would otherwise be paid by every call.
template <int N>
__device__ __forceinline__ void div_all(const ScaleDiv &d, const float *x, float *t)
{
    if (__all(d.fast)) {
#pragma unroll
        for (int i = 0; i < N; ++i)
            t[i] = d.quick(x[i]);
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i)
            t[i] = d(x[i]);
    }
}

// Hardware converters.  Through the quantizer kernels they are checked bit
// for bit against grid-search reference encoders on every BF16 input of
// their domain at unit scale (every grid point, midpoint and neighbour, both
// signs), and directly, through the encoder test export, on every binary32
// value within 64 ulps of each rounding boundary and on a strided sample of
// the rest of the domain.  E4M3 for |y| < 464 (from 464 on the converter
// returns the NaN code, so callers whose values may reach it clamp them to
// +-448 first, which RNE maps to 448 anyway), E2M1 for |y| <= 8, int8 for
// |y| <= 127.5.
__device__ __forceinline__ uint32_t cvt_e4m3x2(float a, float b)
{
    a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
    b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// BF16 bits of (a, b), a in the low half, by the packed converter (round to
// nearest even; the same bits as f32_to_bf16 for every finite input).
__device__ __forceinline__ uint32_t pk_bf16(float a, float b)
{
    bf16x2 v = (bf16x2){(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// Four E4M3 codes of (a, b, c, d) in one dword, a in the low byte, for
// values known to satisfy |y| < 464 (no clamp).
__device__ __forceinline__ uint32_t cvt_e4m3x4_nosat(float a, float b, float c, float d)
{
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// The same for any finite values: saturated to +-448 first.
__device__ __forceinline__ uint32_t cvt_e4m3x4(float a, float b, float c, float d)
{
    return cvt_e4m3x4_nosat(__builtin_amdgcn_fmed3f(a, -448.0f, 448.0f),
                            __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f),
                            __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f),
                            __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f));
}

// E4M3 code of a block scale t >= 0 (finite), saturated at 448.
__device__ __forceinline__ uint32_t enc_e4m3_scale(float t)
{
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_fminf(t, 448.0f), 0.0f, 0,
                                                     false) & 0xFFu;
}

// Eight E2M1 codes of v[0..7] in one dword, v[0] in the low nibble, for
// values known to satisfy |y| <= 8 (no clamp).
__device__ __forceinline__ uint32_t cvt_e2m1x8_nosat(const float *c)
{
    uint32_t o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, c[0], c[1], 1.0f, 0);
    o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, c[2], c[3], 1.0f, 1);
    o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, c[4], c[5], 1.0f, 2);
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, c[6], c[7], 1.0f, 3);
}

// The same for any finite values: saturated to +-6 first.
__device__ __forceinline__ uint32_t cvt_e2m1x8(const float *v)
{
    float c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        c[i] = __builtin_amdgcn_fmed3f(v[i], -6.0f, 6.0f);
    return cvt_e2m1x8_nosat(c);
}

// Four int8 codes RNE(v[i]) for |v| < 127.5, v[0] in the low byte.  Adding
// 1.5 * 2^23 rounds v to an integer (the sum lies in [2^23, 2^24), where the
// binary32 spacing is 1, so the addition's own round-to-nearest-even is the
// integer rounding) and leaves that integer, two's complement, in the low
// byte of the sum's bit pattern; v_perm gathers the four low bytes.
__device__ __forceinline__ uint32_t pack_i8x4(const float *v)
{
    const uint32_t b0 = __float_as_uint(v[0] + 12582912.0f);
    const uint32_t b1 = __float_as_uint(v[1] + 12582912.0f);
    const uint32_t b2 = __float_as_uint(v[2] + 12582912.0f);
    const uint32_t b3 = __float_as_uint(v[3] + 12582912.0f);
    const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);   // b0.0, b1.0, 0, 0
    const uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x04000c0cu);   // 0, 0, b2.0, b3.0
    return lo | hi;
}

// The two E2M1 values of byte SEL of w (low nibble first), exactly.
template <int SEL>
__device__ __forceinline__ f32x2 e2m1_pair(uint32_t w)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

// The two E2M1 values of byte SEL of w (low nibble first) in FP16, exactly.
template <int SEL>
__device__ __forceinline__ f16x2 e2m1_pair_f16(uint32_t w)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}

// ------------------------------------------------------- wave reductions
__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v = __builtin_fmaxf(v, __shfl_xor(v, off, WAVE));
    return v;
}

// XCD-aware remap of a linear workgroup id.  Workgroups are dispatched
// round-robin over the 8 XCDs (each with its own L2); this makes the ids an
// XCD runs contiguous, so neighbouring tiles that share an operand panel run
// behind the same L2.  Returns a permutation of [0, total).
__device__ __forceinline__ uint32_t xcd_remap(uint32_t id, uint32_t total)
{
    constexpr uint32_t NX = 8;
    uint32_t per = total / NX;           // full rounds
    uint32_t full = per * NX;
    if (id >= full)
        return id;                       // the ragged tail keeps its order
    return (id % NX) * per + id / NX;
}

} // namespace qp
