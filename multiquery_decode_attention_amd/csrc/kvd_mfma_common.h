// kvd_mfma_common.h -- device helpers shared by the matrix-core kernels.
#pragma once

#include "kvd_internal.h"

namespace kvd {
namespace mfma {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4_t mfma16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const uint32_t l = __builtin_bit_cast(uint16_t, (__bf16)lo);
    const uint32_t h = __builtin_bit_cast(uint16_t, (__bf16)hi);
    return l | (h << 16);
}

// Token (row of the tile) held in k-slot j of lane group gq.  Slots 0-3 are
// rows 4gq..4gq+3 of the first 16-token half, slots 4-7 the same rows of the
// second half: this is where the score MFMA leaves them.
__device__ __forceinline__ int slot_token(int gq, int j) { return (j < 4 ? 0 : 12) + 4 * gq + j; }

// Columns owned by lane c in the value product: for D >= 128 the 8-column
// pieces c, c+16, ...; for D == 64 the 4 columns 4c..4c+3.
template <int D>
__device__ __forceinline__ int owned_col(int c, int e) {
    if constexpr (D >= 128) {
        return 8 * (c + 16 * (e / 8)) + (e % 8);
    } else {
        return 4 * c + e;
    }
}

// Row i (of the lane's four accumulator rows) of a value product, times
// inv, rounded to bf16 (nearest even) and stored: one 16-byte store per 8
// owned columns for D >= 128, one 8-byte store of the 4 owned columns for
// D == 64.  The partials are read once, by the combine that follows at
// once; ordinary stores leave them in the memory-side cache for it
// (non-temporal ones made the long-context combine 0.5 us slower).
template <int D>
__device__ __forceinline__ void store_partial_row(uint16_t* orow, const f32x4_t (&acc)[D / 16], int i, int c,
                                                  float inv) {
    if constexpr (D >= 128) {
#pragma unroll
        for (int e = 0; e < D / 16; e += 8) {
            const u32x4_t o = {pack_bf16x2(acc[e][i] * inv, acc[e + 1][i] * inv),
                               pack_bf16x2(acc[e + 2][i] * inv, acc[e + 3][i] * inv),
                               pack_bf16x2(acc[e + 4][i] * inv, acc[e + 5][i] * inv),
                               pack_bf16x2(acc[e + 6][i] * inv, acc[e + 7][i] * inv)};
            *reinterpret_cast<u32x4_t*>(orow + owned_col<D>(c, e)) = o;
        }
    } else {
        const u32x2_t o = {pack_bf16x2(acc[0][i] * inv, acc[1][i] * inv),
                           pack_bf16x2(acc[2][i] * inv, acc[3][i] * inv)};
        *reinterpret_cast<u32x2_t*>(orow + owned_col<D>(c, 0)) = o;
    }
}

// B operand of the value product for output column block e: the 8 tokens'
// bf16 values of that column, two per dword, gathered with byte permutes
// from v[j][w] (token slot j, dword w of the lane's owned columns).
template <int VW>
__device__ __forceinline__ u32x4_t v_operand(const uint32_t (&v)[8][VW], int e) {
    const int w = e / 2;
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
    u32x4_t o;
    o[0] = __builtin_amdgcn_perm(v[1][w], v[0][w], sel);
    o[1] = __builtin_amdgcn_perm(v[3][w], v[2][w], sel);
    o[2] = __builtin_amdgcn_perm(v[5][w], v[4][w], sel);
    o[3] = __builtin_amdgcn_perm(v[7][w], v[6][w], sel);
    return o;
}

}  // namespace mfma
}  // namespace kvd
