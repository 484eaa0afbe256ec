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

// One workgroup per (head, sequence) of D/4 * G threads, G = min(1024/D,
// splits) rounded so the workgroup is whole waves.  Thread t owns column
// vector t % (D/4) (four columns) and split group t / (D/4): group k sums
// splits k, k+G, ... so G loads per column are in flight at once; the G
// partial sums meet in LDS.
// Partials are read exactly once: non-temporal loads.
__device__ inline float4 load4_once(const float* p) {
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    return make_float4(v[0], v[1], v[2], v[3]);
}

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
    const int h = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63;
    const int len = a.len_att[b];
    if (a.fused_append && h == 0 && tid == 0) {
        // the only reader and writer of lengths[b] in this launch
        const int l0 = a.lengths[b];
        if (l0 >= 0 && l0 < a.T_cap) a.lengths[b] = l0 + 1;
    }
    const int nsplit = splits_with_data(len, a.tile, a.S);
    T* orow = static_cast<T*>(a.out);
    const size_t obase = ((size_t)b * a.Hq + h) * a.D;
    const int nvec = a.D / 4;          // column vectors per row (16, 32 or 64)
    const int G = a.groups;            // split groups
    const int v = tid % nvec, sg = tid / nvec;

    if (nsplit == 0) {
        if (sg == 0) store4(orow, obase + 4 * v, make_float4(0.f, 0.f, 0.f, 0.f));
        return;
    }
    const size_t prow = ((size_t)b * a.Hq + h) * a.S;
    const float* lse = a.lse_part + prow;
    // every wave finds the maximum and normaliser over all splits itself
    float L = -INFINITY;
    for (int j = lane; j < nsplit; j += 64) L = fmaxf(L, lse[j]);
    L = wave_max(L);
    float z = 0.f;
    for (int j = lane; j < nsplit; j += 64) z += exp2f(lse[j] - L);
    z = wave_sum(z);

    const float* op = a.o_part + prow * a.D + 4 * v;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    int j = sg;
    for (; j + 3 * G < nsplit; j += 4 * G) {
        float4 o[4];
        float w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            o[u] = load4_once(op + (size_t)(j + u * G) * a.D);
            w[u] = lse[j + u * G];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float wu = exp2f(w[u] - L);
            acc.x = fmaf(wu, o[u].x, acc.x);
            acc.y = fmaf(wu, o[u].y, acc.y);
            acc.z = fmaf(wu, o[u].z, acc.z);
            acc.w = fmaf(wu, o[u].w, acc.w);
        }
    }
    for (; j < nsplit; j += G) {
        const float4 o = load4_once(op + (size_t)j * a.D);
        const float wu = exp2f(lse[j] - L);
        acc.x = fmaf(wu, o.x, acc.x);
        acc.y = fmaf(wu, o.y, acc.y);
        acc.z = fmaf(wu, o.z, acc.z);
        acc.w = fmaf(wu, o.w, acc.w);
    }

    __shared__ float4 part[256];
    if (G > 1) {
        part[tid] = acc;
        __syncthreads();
    }
    if (sg == 0) {
        for (int k = 1; k < G; ++k) {
            const float4 p = part[k * nvec + v];
            acc.x += p.x;
            acc.y += p.y;
            acc.z += p.z;
            acc.w += p.w;
        }
        const float inv_z = 1.f / z;
        acc.x *= inv_z;
        acc.y *= inv_z;
        acc.z *= inv_z;
        acc.w *= inv_z;
        store4(orow, obase + 4 * v, acc);
    }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, bool bf16, hipStream_t stream) {
    dim3 grid(a.Hq, a.B), block(a.D / 4 * a.groups);
    if (bf16) hipLaunchKernelGGL(combine_kernel<uint16_t>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(combine_kernel<float>, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace kvd
