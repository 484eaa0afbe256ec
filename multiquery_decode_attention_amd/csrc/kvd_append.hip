// kvd_append.hip -- the generate-side KV-cache update.
//
// For every sequence b with room, copy the new tokens' keys and values of
// each KV head into slots lengths[b], lengths[b] + 1, ... of the cache, then
// advance lengths[b] (one new token in a decode step; several to verify
// drafted tokens, "All About Transformer Inference", appendix on
// speculative sampling).
// ("All About Transformer Inference", section "Transformer inference basics":
// generation writes the new token's key/value projections back into the
// cache; section "Implementation: JetStream": generate appends the
// single-token KV cache to the decode state.)
//
// One workgroup per sequence; 16-byte vector copies.  The copy is bit-exact:
// k_new/v_new already have the cache dtype.  With a paged cache the slot's
// row is found through the block table.
#include "kvd_fp8_common.h"

namespace kvd {
namespace {

__global__ __launch_bounds__(256) void append_kernel(const uint4* __restrict__ k_new,
                                                     const uint4* __restrict__ v_new,
                                                     uint4* __restrict__ k_cache,
                                                     uint4* __restrict__ v_cache,
                                                     KvLayout kv, int32_t* __restrict__ lengths,
                                                     int* __restrict__ err, int* __restrict__ n_new,
                                                     int Hkv, int vec_per_row, int T_cap, int T_q) {
    const int b = blockIdx.x;
    const int n = lengths[b];
    if (n < 0 || n > T_cap - T_q) {
        // Uniform across the block: nobody writes, lengths stays as is.  A
        // length outside [0, T_cap] is a bad length; one without room for
        // the new rows, a full cache.
        if (threadIdx.x == 0) {
            atomicOr(err, n < 0 || n > T_cap ? ERRBIT_LENGTH : ERRBIT_CAPACITY);
            if (n_new) n_new[b] = 0;
        }
        return;
    }
    const int total = Hkv * T_q * vec_per_row;  // source rows [Hkv, T_q] of this sequence
    const uint4* ks = k_new + (size_t)b * total;
    const uint4* vs = v_new + (size_t)b * total;
    for (int i = threadIdx.x; i < total; i += blockDim.x) {
        const int r = i / vec_per_row;  // g * T_q + token
        const int w = i - r * vec_per_row;
        const int g = r / T_q, t = n + (r - g * T_q);
        const size_t row = kv.block_table
                               ? kv_row_paged(kv, kv_page(kv, b, t >> kv.page_shift, err), g, Hkv, t)
                               : kv_row_contiguous(b, g, Hkv, T_cap, t);
        const size_t dst = row * vec_per_row + w;
        k_cache[dst] = ks[i];
        v_cache[dst] = vs[i];
    }
    // Every thread has read lengths[b] above; only then is it advanced.
    __syncthreads();
    if (threadIdx.x == 0) {
        lengths[b] = n + T_q;
        if (n_new) n_new[b] = T_q;
    }
}

// --- fp8 cache: quantizing append ------------------------------------------

// One workgroup of APPEND_FP8_WAVES waves per sequence; wave w quantizes
// new rows w, w+16, ... (row r = g * T_q + i, token i of KV head g): the
// row's largest magnitude gives its exponent e (a wave reduction), every
// value becomes the code of x * 2^-e (exact scaling).  Sixteen waves, not
// four: a sequence holds Hkv * T_q rows of K and of V (320 each for 40 KV
// heads and 8 new tokens), and with four waves the MHA step's append took
// about 110 us (37 us with sixteen).
constexpr int APPEND_FP8_WAVES = 16;
template <int D>
__global__ __launch_bounds__(64 * APPEND_FP8_WAVES) void append_fp8_kernel(const uint16_t* __restrict__ k_new,
                                                         const uint16_t* __restrict__ v_new,
                                                         uint8_t* __restrict__ k_cache,
                                                         uint8_t* __restrict__ v_cache,
                                                         int8_t* __restrict__ k_exp,
                                                         int8_t* __restrict__ v_exp,
                                                         KvLayout kvl, int32_t* __restrict__ lengths,
                                                         int* __restrict__ err, int* __restrict__ n_new,
                                                         int Hkv, int T_cap, int T_q) {
    const int b = blockIdx.x;
    const int n = lengths[b];
    if (n < 0 || n > T_cap - T_q) {
        // uniform across the block: nobody writes, lengths stays as is (a
        // bad length, or a full cache, as in append_kernel)
        if (threadIdx.x == 0) {
            atomicOr(err, n < 0 || n > T_cap ? ERRBIT_LENGTH : ERRBIT_CAPACITY);
            if (n_new) n_new[b] = 0;
        }
        return;
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // source row r = g * T_q + i goes to slot n + i of KV head g
    for (int r = wave; r < Hkv * T_q; r += APPEND_FP8_WAVES) {
        const int g = r / T_q, t = n + (r - g * T_q);
        const size_t src = ((size_t)b * Hkv * T_q + r) * D;
        // the exponent of a row sits at the row's index in the exponent
        // array; paged: a bad block-table entry writes page 0 and is flagged
        const size_t row = kvl.block_table ? kv_row_paged(kvl, kv_page(kvl, b, t >> kvl.page_shift, err), g, Hkv, t)
                                           : kv_row_contiguous(b, g, Hkv, T_cap, t);
#pragma unroll
        for (int kv = 0; kv < 2; ++kv)
            fp8::quantize_row<D>((kv ? v_new : k_new) + src, (kv ? v_cache : k_cache) + row * D,
                                 (kv ? v_exp : k_exp) + row, lane);
    }
    // Every thread has read lengths[b] above; only then is it advanced.
    __syncthreads();
    if (threadIdx.x == 0) {
        lengths[b] = n + T_q;
        if (n_new) n_new[b] = T_q;
    }
}

}  // namespace

hipError_t launch_append_fp8(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                             int8_t* k_exp, int8_t* v_exp, const KvLayout& kv, int32_t* lengths, int* err,
                             int* n_new, int B, int Hkv, int D, int T_cap, int T_q, const Launch& on) {
    auto go = [&](auto kernel) {
        KVD_LAUNCH(kernel, dim3(B), dim3(64 * APPEND_FP8_WAVES), 0, on, static_cast<const uint16_t*>(k_new),
                           static_cast<const uint16_t*>(v_new), static_cast<uint8_t*>(k_cache),
                           static_cast<uint8_t*>(v_cache), k_exp, v_exp, kv, lengths, err, n_new, Hkv, T_cap, T_q);
    };
    switch (D) {
        case 64: go(append_fp8_kernel<64>); break;
        case 128: go(append_fp8_kernel<128>); break;
        case 256: go(append_fp8_kernel<256>); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                         const KvLayout& kv, int32_t* lengths, int* err, int* n_new, int B, int Hkv,
                         int D, int T_cap, int T_q, int elem_bytes, const Launch& on) {
    const int vec_per_row = D * elem_bytes / 16;
    KVD_LAUNCH(append_kernel, dim3(B), dim3(256), 0, on,
                       static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new),
                       static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), kv, lengths,
                       err, n_new, Hkv, vec_per_row, T_cap, T_q);
    return hipGetLastError();
}

}  // namespace kvd
