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
// split group k = t / (D/4), which takes splits k, k+G, k+2G, ...: U of its
// partial vectors and their log-sum-exps are requested at once (U * G >= S
// whenever a row fits a workgroup), so one memory round trip covers the row.
// The requests depend on nothing loaded: indices are clamped to the
// workspace's splits, and which of them hold data this launch (those below
// splits_with_data of the attended length) is decided only when the values
// are used, by selects -- a conditional load would make the compiler wait
// for each load before the next.  Each thread merges its splits against its
// own maximum; the G groups then meet in LDS, rescaled to the row's maximum:
//     out = sum_k 2^(m_k - m) A_k / sum_k 2^(m_k - m) Z_k,
// with A_k = sum_j 2^(L_j - m_k) O_j and Z_k = sum_j 2^(L_j - m_k) over the
// splits j of group k.  Partials are read exactly once: non-temporal loads.
constexpr int THREADS = 256;
constexpr int MAX_UNROLL = 16;

// Four consecutive partial columns; the partials have the output's
// precision (fp32, or bf16 widened exactly).
__device__ inline float4 load4_once(const float* p) {
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ inline float4 load4_once(const uint16_t* p) {
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
    return make_float4(__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xffff0000u),
                       __uint_as_float(v[1] << 16), __uint_as_float(v[1] & 0xffff0000u));
}

// Sequences by this step's attended length, longest first (ties by
// index), for the next partial pass: a bitonic sort of (length, ~index)
// keys in LDS, N = the next power of two >= B <= COMBINE_SORT_MAX (padding
// keys are 0 and sort last).  Only the dispatch order of the next pass
// depends on it.
__device__ void sort_by_length(const CombineArgs& a, unsigned long long* keys) {
    const int n = a.B;
    bool differs = false;
    const int l_first = a.len_att[0];
    for (int i = threadIdx.x; i < n; i += THREADS) differs |= a.len_att[i] != l_first;
    if (!__syncthreads_or(differs)) {
        if (threadIdx.x == 0) a.order[n] = 0;  // equal lengths: any order serves
        return;
    }
    int N = 1;
    while (N < n) N <<= 1;
    for (int i = threadIdx.x; i < N; i += THREADS) {
        const int len = i < n ? a.len_att[i] : 0;
        keys[i] = i < n ? ((unsigned long long)(unsigned)(len > 0 ? len : 0) << 32) | (unsigned)~i : 0ull;
    }
    __syncthreads();
    for (int k = 2; k <= N; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = threadIdx.x; i < N; i += THREADS) {
                const int l = i ^ j;
                if (l > i) {
                    const unsigned long long x = keys[i], y = keys[l];
                    // runs with (i & k) == 0 descend, the others ascend
                    if ((i & k) == 0 ? x < y : x > y) {
                        keys[i] = y;
                        keys[l] = x;
                    }
                }
            }
            __syncthreads();
        }
    }
    for (int i = threadIdx.x; i < n; i += THREADS) a.order[i] = (int)~(unsigned)keys[i];
    if (threadIdx.x == 0) a.order[n] = 1;  // valid from the next launch on
}

constexpr int SMEM_BYTES = THREADS * (16 + 8) > COMBINE_SORT_MAX * 8 ? THREADS * (16 + 8) : COMBINE_SORT_MAX * 8;

template <typename T, int U>
__global__ __launch_bounds__(THREADS) void combine_kernel(CombineArgs a) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM_BYTES];
    // the extra workgroup is the first, so its sort runs beside the merges
    // instead of after them
    if (a.order != nullptr && blockIdx.x == 0) {
        sort_by_length(a, reinterpret_cast<unsigned long long*>(smem));
        return;
    }
    const int blk = (int)blockIdx.x - (a.order != nullptr ? 1 : 0);
    const int tid = threadIdx.x;
    const int nvec = a.D / 4;          // column vectors per row (16, 32 or 64)
    const int G = a.groups;            // split groups per row
    const int row_threads = nvec * G;
    const int rt = tid % row_threads;  // thread within its row
    const int v = rt % nvec, sg = rt / nvec;
    const int row = blk * (THREADS / row_threads) + tid / row_threads;
    const bool live = row < a.B * a.Hq;  // the last workgroup may hold fewer rows
    const int b = live ? row / a.Hq : 0, h = row % a.Hq;
    const size_t prow = ((size_t)b * a.Hq + h) * a.S;
    const float* lse = a.lse_part + prow;
    const T* op = static_cast<const T*>(a.o_part) + prow * a.D + 4 * v;

    float m = -INFINITY, z = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    int nsplit = 0;
    for (int j0 = sg; j0 < a.S; j0 += U * G) {
        float4 o[U];
        float w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int jc = min(j0 + u * G, a.S - 1);
            w[u] = lse[jc];
            o[u] = load4_once(op + (size_t)jc * a.D);
        }
        // the attended length is requested after the partials (the compiler
        // would otherwise hoist it, and wait for it, ahead of them)
        asm volatile("" ::: "memory");
        nsplit = live ? splits_with_data(a.len_att[b], a.tile, a.S) : 0;
        float mc = m;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // a split can be empty for an early query of a several-token
            // step (log-sum-exp -inf); splits past nsplit hold stale data
            const bool ok = j0 + u * G < nsplit && w[u] != -INFINITY;
            w[u] = ok ? w[u] : -INFINITY;
            o[u] = ok ? o[u] : make_float4(0.f, 0.f, 0.f, 0.f);
            mc = fmaxf(mc, w[u]);
        }
        // all of this thread's splits may be empty
        const float r = mc == -INFINITY ? 1.f : exp2f(m - mc);
        z *= r;
        acc.x *= r;
        acc.y *= r;
        acc.z *= r;
        acc.w *= r;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float wu = w[u] == -INFINITY ? 0.f : exp2f(w[u] - mc);
            z += wu;
            acc.x = fmaf(wu, o[u].x, acc.x);
            acc.y = fmaf(wu, o[u].y, acc.y);
            acc.z = fmaf(wu, o[u].z, acc.z);
            acc.w = fmaf(wu, o[u].w, acc.w);
        }
        m = mc;
    }
    if (live && a.fused_append && h == 0 && rt == 0) {
        // the only reader and writer of lengths[b] in this launch
        const int l0 = a.lengths[b];
        if (l0 >= 0 && l0 < a.T_cap) a.lengths[b] = l0 + 1;
    }

    float4* part = reinterpret_cast<float4*>(smem);
    float2* mz = reinterpret_cast<float2*>(smem + THREADS * sizeof(float4));
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

template <typename T>
hipError_t launch_t(const CombineArgs& a, int U, dim3 grid, const Launch& on) {
    switch (U) {
        case 1: KVD_LAUNCH((combine_kernel<T, 1>), grid, dim3(THREADS), 0, on, a); break;
        case 2: KVD_LAUNCH((combine_kernel<T, 2>), grid, dim3(THREADS), 0, on, a); break;
        case 4: KVD_LAUNCH((combine_kernel<T, 4>), grid, dim3(THREADS), 0, on, a); break;
        case 8: KVD_LAUNCH((combine_kernel<T, 8>), grid, dim3(THREADS), 0, on, a); break;
        default: KVD_LAUNCH((combine_kernel<T, MAX_UNROLL>), grid, dim3(THREADS), 0, on, a); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const CombineArgs& args, bool bf16, const Launch& on) {
    // split groups per row: enough that MAX_UNROLL loads per thread cover
    // the splits in one round, and a row no wider than a workgroup; then
    // the smallest power-of-two unroll that covers them
    CombineArgs a = args;
    if (a.B > COMBINE_SORT_MAX) a.order = nullptr;  // no order: the next pass keeps the batch's
    const int nvec = a.D / 4;
    int G = 1;
    while (G * MAX_UNROLL < a.S && nvec * G * 2 <= THREADS) G *= 2;
    a.groups = G;
    int U = 1;
    while (U < MAX_UNROLL && U * G < a.S) U *= 2;
    const int rows = a.B * a.Hq;
    const int per_block = THREADS / (nvec * G);
    dim3 grid((rows + per_block - 1) / per_block + (a.order != nullptr ? 1 : 0));
    return bf16 ? launch_t<uint16_t>(a, U, grid, on) : launch_t<float>(a, U, grid, on);
}

}  // namespace kvd
