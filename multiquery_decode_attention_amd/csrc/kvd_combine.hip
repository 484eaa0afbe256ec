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

// Workgroups of 256 threads; a (sequence, head) row takes D/4 * G of them
// (G a power of two), so a workgroup merges 256 / (D/4 * G) rows.  Within
// its row, thread t owns column vector v = t % (D/4) (four columns) and
// split group k = t / (D/4), which takes splits k, k+G, k+2G, ...: all of
// its partial vectors and their log-sum-exps are requested at once, up to
// UNROLL of them, so one memory round trip covers the row whenever
// splits <= UNROLL * G.  Each thread merges its splits against its own
// maximum; the G groups then meet in LDS, rescaled to the row's maximum:
//     out = sum_k 2^(m_k - m) A_k / sum_k 2^(m_k - m) Z_k,
// with A_k = sum_j 2^(L_j - m_k) O_j and Z_k = sum_j 2^(L_j - m_k) over the
// splits j of group k.  Partials are read exactly once: non-temporal loads.
constexpr int THREADS = 256;
constexpr int UNROLL = 16;

__device__ inline float4 load4_once(const float* p) {
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    return make_float4(v[0], v[1], v[2], v[3]);
}

template <typename T>
__global__ __launch_bounds__(THREADS) void combine_kernel(CombineArgs a) {
    const int tid = threadIdx.x;
    const int nvec = a.D / 4;          // column vectors per row (16, 32 or 64)
    const int G = a.groups;            // split groups per row
    const int row_threads = nvec * G;
    const int rt = tid % row_threads;  // thread within its row
    const int v = rt % nvec, sg = rt / nvec;
    const int row = blockIdx.x * (THREADS / row_threads) + tid / row_threads;
    const bool live = row < a.B * a.Hq;  // the last workgroup may hold fewer rows
    const int b = live ? row / a.Hq : 0, h = row % a.Hq;
    const int len = a.len_att[b];
    if (live && a.fused_append && h == 0 && rt == 0) {
        // the only reader and writer of lengths[b] in this launch
        const int l0 = a.lengths[b];
        if (l0 >= 0 && l0 < a.T_cap) a.lengths[b] = l0 + 1;
    }
    const int nsplit = live ? splits_with_data(len, a.tile, a.S) : 0;
    const size_t prow = ((size_t)b * a.Hq + h) * a.S;
    const float* lse = a.lse_part + prow;
    const float* op = a.o_part + prow * a.D + 4 * v;

    float m = -INFINITY, z = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j0 = sg; j0 < nsplit; j0 += UNROLL * G) {
        float4 o[UNROLL];
        float w[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int j = j0 + u * G;
            w[u] = -INFINITY;
            o[u] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (j < nsplit) {
                w[u] = lse[j];
                o[u] = load4_once(op + (size_t)j * a.D);
            }
        }
        float mc = m;
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) mc = fmaxf(mc, w[u]);
        // a split can be empty for an early query of a several-token step
        // (log-sum-exp -inf); all of this thread's may be
        const float r = mc == -INFINITY ? 1.f : exp2f(m - mc);
        z *= r;
        acc.x *= r;
        acc.y *= r;
        acc.z *= r;
        acc.w *= r;
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const float wu = w[u] == -INFINITY ? 0.f : exp2f(w[u] - mc);
            z += wu;
            acc.x = fmaf(wu, o[u].x, acc.x);
            acc.y = fmaf(wu, o[u].y, acc.y);
            acc.z = fmaf(wu, o[u].z, acc.z);
            acc.w = fmaf(wu, o[u].w, acc.w);
        }
        m = mc;
    }

    __shared__ float4 part[THREADS];
    __shared__ float2 mz[THREADS];
    if (G > 1) {
        part[tid] = acc;
        mz[tid] = make_float2(m, z);
        __syncthreads();
    }
    if (!live || sg != 0) return;
    T* orow = static_cast<T*>(a.out);
    const size_t obase = ((size_t)b * a.Hq + h) * a.D;
    if (nsplit == 0) {
        // a sequence with no tokens: zero row
        store4(orow, obase + 4 * v, make_float4(0.f, 0.f, 0.f, 0.f));
        return;
    }
    // group 0 holds split 0, which holds token 0 for every row: its maximum
    // is finite
    const int base = tid - rt;  // first thread of this row
    float mt = m;
    for (int k = 1; k < G; ++k) mt = fmaxf(mt, mz[base + k * nvec + v].x);
    const float r0 = exp2f(m - mt);
    float zt = z * r0;
    acc.x *= r0;
    acc.y *= r0;
    acc.z *= r0;
    acc.w *= r0;
    for (int k = 1; k < G; ++k) {
        const float2 q = mz[base + k * nvec + v];
        const float rk = exp2f(q.x - mt);  // 0 for a group with no splits
        const float4 p = part[base + k * nvec + v];
        zt += rk * q.y;
        acc.x = fmaf(rk, p.x, acc.x);
        acc.y = fmaf(rk, p.y, acc.y);
        acc.z = fmaf(rk, p.z, acc.z);
        acc.w = fmaf(rk, p.w, acc.w);
    }
    const float inv_z = 1.f / zt;
    acc.x *= inv_z;
    acc.y *= inv_z;
    acc.z *= inv_z;
    acc.w *= inv_z;
    store4(orow, obase + 4 * v, acc);
}

}  // namespace

hipError_t launch_combine(const CombineArgs& args, bool bf16, hipStream_t stream) {
    // split groups per row: enough that UNROLL loads per thread cover the
    // splits in one round, and a row no wider than a workgroup
    CombineArgs a = args;
    const int nvec = a.D / 4;
    int G = 1;
    while (G * UNROLL < a.S && nvec * G * 2 <= THREADS) G *= 2;
    a.groups = G;
    const int rows = a.B * a.Hq;
    const int per_block = THREADS / (nvec * G);
    dim3 grid((rows + per_block - 1) / per_block), block(THREADS);
    if (bf16) hipLaunchKernelGGL(combine_kernel<uint16_t>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(combine_kernel<float>, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace kvd
