// kvd_fp8_common.h -- device helpers of the fp8-cache kernels: widening
// OCP FP8 E4M3 codes to bf16 matrix-core operands with gfx950's scaled
// conversion, and the quantization of new rows (the append kernel, and the
// partial kernels' fused append).
#pragma once

#include "kvd_lds_common.h"

namespace kvd {
namespace fp8 {

using mfma::u32x2_t;
using mfma::u32x4_t;

// Range of the stored row exponents.  Every code * 2^e in it is zero or a
// finite normal bf16 number -- the smallest subnormal code, 2^-9, times
// 2^-117 is 2^-126, bf16's smallest normal value, and the largest, 448, times
// 2^119 is 1.75 * 2^127 -- so widened operands and scaled weights hold the
// dequantized cache exactly.  The append clamps to it; an exponent stored
// outside it is read as the nearest bound.
constexpr int EXP_MIN = -117;
constexpr int EXP_MAX = 119;

// 2^e as an fp32 whose exponent field is e + 127, for e clamped to
// [EXP_MIN, EXP_MAX]; the scaled conversions read only that field.
__device__ __forceinline__ float pow2_scale(int e) {
    e = max(EXP_MIN, min(EXP_MAX, e));
    return __builtin_bit_cast(float, (uint32_t)(e + 127) << 23);
}

// Two E4M3 codes (bytes 2h, 2h+1 of w) times 2^e(scale) as a bf16 pair.
template <bool HI>
__device__ __forceinline__ uint32_t widen2(uint32_t w, float scale) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, scale, HI));
}

// Eight codes (two dwords) -> a bf16x8 matrix-core operand.
__device__ __forceinline__ u32x4_t widen8(u32x2_t x, float scale) {
    u32x4_t o;
    o[0] = widen2<false>(x[0], scale);
    o[1] = widen2<true>(x[0], scale);
    o[2] = widen2<false>(x[1], scale);
    o[3] = widen2<true>(x[1], scale);
    return o;
}

// Nearest OCP E4M3 code of y (finite, |y| <= 448), ties to the even code;
// the sign bit is y's.  Codes 0..8 below 2^-6 are the subnormals (and 2^-6
// itself), spaced 2^-9; above, 3 mantissa bits are kept by rounding the
// fp32 mantissa half to even.
__device__ inline uint32_t e4m3_encode(float y) {
    const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
    const float a = fabsf(y);
    uint32_t code;
    if (a < 0.015625f) {
        code = (uint32_t)__builtin_rintf(a * 512.0f);  // exact scaling; round half to even
    } else {
        const uint32_t ab = __float_as_uint(a);
        int E = (int)(ab >> 23) - 127;  // -6 .. 8
        uint32_t q = (ab >> 20) & 7u;
        const uint32_t rem = ab & 0xFFFFFu;
        if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ++q;
        if (q == 8u) {
            q = 0;
            ++E;
        }
        code = ((uint32_t)(E + 7) << 3) | q;
    }
    return sign | code;
}

// Smallest e with amax <= 448 * 2^e, clamped to [EXP_MIN, EXP_MAX]; 0 for
// amax 0.  With amax = m * 2^k, m in [1, 2): e = k - 8, plus 1 when m > 1.75.
__device__ inline int e4m3_row_exponent(float amax) {
    if (!(amax > 0.f)) return 0;
    const uint32_t b = __float_as_uint(amax);
    const int E = (int)(b >> 23);
    if (E == 0) return EXP_MIN;  // subnormal amax: far below the clamp
    const int e = E - 127 - 8 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
    return max(EXP_MIN, min(EXP_MAX, e));
}

// Quantizing append of one row, by the 64 lanes of a wave: the row's largest
// magnitude gives its exponent e (a wave reduction), every value becomes the
// code of x * 2^-e (exact scaling; saturated at +-448 when e was clamped at
// EXP_MAX, and rounded to 0 below half the smallest code when it was
// clamped at EXP_MIN); lane l handles values l*D/64 .. (l+1)*D/64 - 1 of
// the bf16 row src, the codes go to dst and e to *xdst.
template <int D>
__device__ inline void quantize_row(const uint16_t* src, uint8_t* dst, int8_t* xdst, int lane) {
    constexpr int PER = D / 64;
    float y[PER];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        y[i] = __uint_as_float((uint32_t)src[lane * PER + i] << 16);
        amax = fmaxf(amax, fabsf(y[i]));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    const int e = e4m3_row_exponent(amax);
#pragma unroll
    for (int i = 0; i < PER; ++i)
        dst[lane * PER + i] = (uint8_t)e4m3_encode(fminf(fmaxf(ldexpf(y[i], -e), -448.f), 448.f));
    if (lane == 0) *xdst = (int8_t)e;
}

}  // namespace fp8
}  // namespace kvd
