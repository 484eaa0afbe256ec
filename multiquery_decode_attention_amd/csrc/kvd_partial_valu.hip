// kvd_partial_valu.hip -- vector-ALU split-KV partial pass (any dtype).
//
// One wave per (split, query head, sequence).  Lane t of the wave scores
// token t0+t of a 64-token tile against the query held in LDS, the wave keeps
// the running maximum and sum of the split's softmax with cross-lane
// reductions, and every lane accumulates the probability-weighted values for
// D/64 of the head's columns.  The split's result is stored normalised,
// together with its base-2 log-sum-exp, for the combine pass.
//
// This is the fp32-cache path (the tiny multiquery workload) and an
// independent cross-check of the MFMA kernel in bf16; it makes no attempt
// at bandwidth efficiency (each head re-reads its KV head's slab).
//
// Sources: scores, softmax over the sequence and weighted sum of values as in
// the grouped contraction of "All About Transformer Inference", section
// "Sharding the KV cache"; accumulating across sequence splits the way Flash
// Attention does, same section; base-2 softmax, "Efficiently Scaling
// Transformer Inference", section 3.5.
#include "kvd_internal.h"

namespace kvd {
namespace {

__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

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

template <typename T, int D>
__global__ __launch_bounds__(64) void partial_valu_kernel(PartialArgs a) {
    constexpr int DPL = D / 64;  // value columns per lane
    // unit = (sequence b, query head h), head fastest
    const BlockCoord bc = block_coord(a.B * a.Hq);
    const int s = bc.split;
    const int h = bc.unit % a.Hq;
    const int b = bc.unit / a.Hq;
    const int lane = threadIdx.x;
    const int len = sequence_length(a.lengths, a.err, a.len_att, b, a.T_cap, false,
                                    s == 0 && h == 0 && lane == 0).len;
    const int n_seq_tiles = (len + VALU_TILE - 1) / VALU_TILE;
    if (s >= n_seq_tiles) return;  // no tile of this sequence for this split
    const int g = h / a.M;  // query head h reads KV head floor(h / M)

    __shared__ float qs[D];
    const T* qrow = static_cast<const T*>(a.q) + ((size_t)b * a.Hq + h) * D;
    for (int d = lane; d < D; d += 64) qs[d] = to_f32(qrow[d]);
    __syncthreads();

    const size_t slab = ((size_t)b * a.Hkv + g) * (size_t)a.T_cap * D;
    const T* kb = static_cast<const T*>(a.k_cache) + slab;
    const T* vb = static_cast<const T*>(a.v_cache) + slab;

    float acc[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) acc[k] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    for (int tile = s; tile < n_seq_tiles; tile += a.S) {
        const int t0 = tile * VALU_TILE;
        const int t = t0 + lane;
        float x = -INFINITY;
        if (t < len) {
            const T* kr = kb + (size_t)t * D;
            float dot = 0.f;
#pragma unroll 8
            for (int d = 0; d < D; ++d) dot = fmaf(qs[d], to_f32(kr[d]), dot);
            x = dot * a.scale_log2e;
        }
        const float m_new = fmaxf(m_run, wave_max(x));
        const float alpha = exp2f(m_run - m_new);
        const float p = exp2f(x - m_new);
        l_run = l_run * alpha + wave_sum(p);
        m_run = m_new;
#pragma unroll
        for (int k = 0; k < DPL; ++k) acc[k] *= alpha;
        const int nt = min(VALU_TILE, len - t0);
        for (int j = 0; j < nt; ++j) {
            const float pj = __shfl(p, j);
            const T* vr = vb + (size_t)(t0 + j) * D;
#pragma unroll
            for (int k = 0; k < DPL; ++k) acc[k] = fmaf(pj, to_f32(vr[lane + 64 * k]), acc[k]);
        }
    }

    const size_t row = ((size_t)b * a.Hq + h) * a.S + s;
    const float inv = 1.f / l_run;
#pragma unroll
    for (int k = 0; k < DPL; ++k) a.o_part[row * D + lane + 64 * k] = acc[k] * inv;
    if (lane == 0) a.lse_part[row] = m_run + log2f(l_run);
}

template <typename T>
hipError_t launch_typed(const PartialArgs& a, hipStream_t stream) {
    dim3 grid((unsigned)a.S * a.B * a.Hq), block(64);
    switch (a.D) {
        case 64: hipLaunchKernelGGL((partial_valu_kernel<T, 64>), grid, block, 0, stream, a); break;
        case 128: hipLaunchKernelGGL((partial_valu_kernel<T, 128>), grid, block, 0, stream, a); break;
        case 256: hipLaunchKernelGGL((partial_valu_kernel<T, 256>), grid, block, 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_partial_valu(const PartialArgs& a, bool bf16, hipStream_t stream) {
    return bf16 ? launch_typed<uint16_t>(a, stream) : launch_typed<float>(a, stream);
}

}  // namespace kvd
