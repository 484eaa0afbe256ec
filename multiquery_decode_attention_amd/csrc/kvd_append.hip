// kvd_append.hip -- the generate-side KV-cache update.
//
// For every sequence b below capacity, copy the new token's key and value of
// each KV head into slot lengths[b] of the cache, then advance lengths[b].
// ("All About Transformer Inference", section "Transformer inference basics":
// generation writes the new token's key/value projections back into the
// cache; section "Implementation: JetStream": generate appends the
// single-token KV cache to the decode state.)
//
// One workgroup per sequence; 16-byte vector copies.  The copy is bit-exact:
// k_new/v_new already have the cache dtype.  With a paged cache the slot's
// row is found through the block table.
#include "kvd_internal.h"

namespace kvd {
namespace {

__global__ __launch_bounds__(256) void append_kernel(const uint4* __restrict__ k_new,
                                                     const uint4* __restrict__ v_new,
                                                     uint4* __restrict__ k_cache,
                                                     uint4* __restrict__ v_cache,
                                                     KvLayout kv, int32_t* __restrict__ lengths,
                                                     int* __restrict__ err, int Hkv,
                                                     int vec_per_row, int T_cap) {
    const int b = blockIdx.x;
    const int n = lengths[b];
    if (n < 0 || n >= T_cap) {
        // Uniform across the block: nobody writes, lengths stays as is.
        if (threadIdx.x == 0) atomicOr(err, n < 0 ? ERRBIT_LENGTH : ERRBIT_CAPACITY);
        return;
    }
    const int page = kv.block_table ? kv_page(kv, b, n >> kv.page_shift, err) : 0;
    const int total = Hkv * vec_per_row;
    const uint4* ks = k_new + (size_t)b * total;
    const uint4* vs = v_new + (size_t)b * total;
    for (int i = threadIdx.x; i < total; i += blockDim.x) {
        const int g = i / vec_per_row;
        const int w = i - g * vec_per_row;
        const size_t row = kv.block_table ? kv_row_paged(kv, page, g, Hkv, n)
                                          : kv_row_contiguous(b, g, Hkv, T_cap, n);
        const size_t dst = row * vec_per_row + w;
        k_cache[dst] = ks[i];
        v_cache[dst] = vs[i];
    }
    // Every thread has read lengths[b] above; only then is it advanced.
    __syncthreads();
    if (threadIdx.x == 0) lengths[b] = n + 1;
}

}  // namespace

hipError_t launch_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                         const KvLayout& kv, int32_t* lengths, int* err, int B, int Hkv, int D,
                         int T_cap, int elem_bytes, hipStream_t stream) {
    const int vec_per_row = D * elem_bytes / 16;
    hipLaunchKernelGGL(append_kernel, dim3(B), dim3(256), 0, stream,
                       static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new),
                       static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), kv, lengths,
                       err, Hkv, vec_per_row, T_cap);
    return hipGetLastError();
}

}  // namespace kvd
