// kvd_combine.hip -- merge the split-KV partials of each (sequence, head).
//
// Split j of a sequence covers its share of the valid prefix (the partial
// kernel's token tiles j, j+S, ...) and left its softmax-normalised output
// O_j and its base-2 log-sum-exp L_j = m_j + log2(l_j).  The full attention is the softmax over
// all tokens, which factorises over the splits:
//     out = sum_j 2^(L_j - L) O_j / sum_j 2^(L_j - L),   L = max_j L_j.
// Only min(S, ceil(len/tile)) splits hold data; a sequence with no tokens
// gets a zero row.  This is the accumulation across sequence shards "like Flash
// Attention" of "All About Transformer Inference", section "Sharding the KV
// cache", carried out inside one GPU.
//
// One wave per (head, sequence); each lane owns 4 consecutive columns.
#include "kvd_internal.h"

namespace kvd {
namespace {

__device__ inline float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ inline float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ inline void store4(float* out, size_t i, float4 v) {
    *reinterpret_cast<float4*>(out + i) = v;
}
__device__ inline void store4(uint16_t* out, size_t i, float4 v) {
    // Round to nearest even (the hardware conversion) and store 8 bytes.
    const uint32_t a = __builtin_bit_cast(uint16_t, (__bf16)v.x);
    const uint32_t b = __builtin_bit_cast(uint16_t, (__bf16)v.y);
    const uint32_t c = __builtin_bit_cast(uint16_t, (__bf16)v.z);
    const uint32_t d = __builtin_bit_cast(uint16_t, (__bf16)v.w);
    *reinterpret_cast<uint2*>(out + i) = make_uint2(a | (b << 16), c | (d << 16));
}

template <typename T>
__global__ __launch_bounds__(64) void combine_kernel(CombineArgs a) {
    const int h = blockIdx.x, b = blockIdx.y;
    const int lane = threadIdx.x;
    const int len = a.len_att[b];
    if (a.fused_append && h == 0 && lane == 0) {
        // the only reader and writer of lengths[b] in this launch
        const int l0 = a.lengths[b];
        if (l0 >= 0 && l0 < a.T_cap) a.lengths[b] = l0 + 1;
    }
    const int nsplit = splits_with_data(len, a.tile, a.S);
    T* orow = static_cast<T*>(a.out);
    const size_t obase = ((size_t)b * a.Hq + h) * a.D;
    const int nvec = a.D / 4;

    if (nsplit == 0) {
        for (int v = lane; v < nvec; v += 64) store4(orow, obase + 4 * v, make_float4(0.f, 0.f, 0.f, 0.f));
        return;
    }
    const size_t prow = ((size_t)b * a.Hq + h) * a.S;
    const float* lse = a.lse_part + prow;
    // Global maximum and normaliser over all splits (lane j holds split j of
    // each block of 64).
    float L = -INFINITY;
    for (int j = lane; j < nsplit; j += 64) L = fmaxf(L, lse[j]);
    L = wave_max(L);
    float z = 0.f;
    for (int j = lane; j < nsplit; j += 64) z += exp2f(lse[j] - L);
    z = wave_sum(z);
    const float inv_z = 1.f / z;

    const float* op = a.o_part + prow * a.D;
    // Wave-uniform loop (the weight shuffles below need every lane active);
    // lanes past the row's last column vector only skip their loads/stores.
    for (int v0 = 0; v0 < nvec; v0 += 64) {
        const int v = v0 + lane;
        const bool col_ok = v < nvec;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int j0 = 0; j0 < nsplit; j0 += 64) {
            const int jn = min(64, nsplit - j0);
            const float wl = lane < jn ? exp2f(lse[j0 + lane] - L) : 0.f;
            // eight independent partial loads in flight per lane
            for (int u0 = 0; u0 < jn; u0 += 8) {
                float4 o[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int j = j0 + u0 + u;
                    o[u] = (col_ok && u0 + u < jn)
                               ? *reinterpret_cast<const float4*>(op + (size_t)j * a.D + 4 * v)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const float w = __shfl(wl, (u0 + u) & 63);
                    acc.x = fmaf(w, o[u].x, acc.x);
                    acc.y = fmaf(w, o[u].y, acc.y);
                    acc.z = fmaf(w, o[u].z, acc.z);
                    acc.w = fmaf(w, o[u].w, acc.w);
                }
            }
        }
        acc.x *= inv_z;
        acc.y *= inv_z;
        acc.z *= inv_z;
        acc.w *= inv_z;
        if (col_ok) store4(orow, obase + 4 * v, acc);
    }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, bool bf16, hipStream_t stream) {
    dim3 grid(a.Hq, a.B), block(64);
    if (bf16) hipLaunchKernelGGL(combine_kernel<uint16_t>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(combine_kernel<float>, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace kvd
