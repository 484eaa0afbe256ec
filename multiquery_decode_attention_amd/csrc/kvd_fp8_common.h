// kvd_fp8_common.h -- device helpers of the fp8-cache partial kernels:
// widening OCP FP8 E4M3 codes to bf16 matrix-core operands with gfx950's
// scaled conversion.
#pragma once

#include "kvd_lds_common.h"

namespace kvd {
namespace fp8 {

using mfma::u32x2_t;
using mfma::u32x4_t;

// 2^e as an fp32 whose exponent field is e + 127 (e in [-127, 127]); the
// scaled conversions read only that field.
__device__ __forceinline__ float pow2_scale(int e) {
    e = max(-127, min(127, e));
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

}  // namespace fp8
}  // namespace kvd
