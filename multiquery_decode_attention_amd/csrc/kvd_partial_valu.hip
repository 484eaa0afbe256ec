// kvd_partial_valu.hip -- vector-ALU split-KV partial pass (any dtype).
//
// One workgroup of four waves per (split, query head, sequence); wave w takes
// the split's tiles w, w+4, ... (of its own tiles s, s+S, ...).  Lane t of a
// wave scores token t0+t of a 64-token tile against the query held in LDS,
// the wave keeps the running maximum and sum of its share of the softmax
// with cross-lane reductions, and every lane accumulates the
// probability-weighted values for D/64 of the head's columns.  The four
// waves' states then merge in LDS by the same log-sum-exp rescaling as the
// combine, and the split's result is stored normalised, with its base-2
// log-sum-exp, for the combine pass -- or, in a one-split pass, as the
// output row itself.  Four waves take four tiles at once: a short sequence
// costs one tile's latency rather than one per tile.
//
// With k_new/v_new set (one decode step) the append is folded in: the new
// token's row is read from k_new/v_new and copied to its cache slot here.
// A paged cache is read through its block table, one page lookup per token.
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
template <typename T>
__device__ inline T from_f32(float x);
template <>
__device__ inline float from_f32<float>(float x) { return x; }
template <>
__device__ inline uint16_t from_f32<uint16_t>(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

// Element i of a 16-byte piece held as four 32-bit words.
template <typename T>
__device__ inline float element(const uint32_t (&w)[4], int i);
template <>
__device__ inline float element<float>(const uint32_t (&w)[4], int i) { return __uint_as_float(w[i]); }
template <>
__device__ inline float element<uint16_t>(const uint32_t (&w)[4], int i) {
    const uint32_t x = w[i / 2];
    return __uint_as_float(i % 2 ? (x & 0xffff0000u) : (x << 16));
}

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

template <typename T, int D, bool PAGED>
__global__ __launch_bounds__(64 * VALU_WAVES) void partial_valu_kernel(PartialArgs a) {
    constexpr int DPL = D / 64;  // value columns per lane
    // unit = (sequence b, query head h), head fastest
    const BlockCoord bc = block_coord(a.B * a.Hq);
    const int s = bc.split;
    const int h = bc.unit % a.Hq;
    const int b = bc.unit / a.Hq;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const SeqLen sl = sequence_length(a.lengths, a.err, a.len_att, b, a.T_cap, a.k_new != nullptr,
                                      s == 0 && h == 0 && threadIdx.x == 0);
    const int len = sl.len;
    const int n_seq_tiles = (len + VALU_TILE - 1) / VALU_TILE;
    if (s >= n_seq_tiles) {
        // no tile of this sequence for this split; a single-split pass
        // writes the zero row of a sequence with no tokens
        if (a.out != nullptr && n_seq_tiles == 0) {
            T* orow = static_cast<T*>(a.out) + ((size_t)b * a.Hq + h) * D;
            for (int d = threadIdx.x; d < D; d += 64 * VALU_WAVES) orow[d] = from_f32<T>(0.f);
        }
        return;
    }
    const int g = h / a.M;  // query row h reads KV head floor(h / M)
    const int row_len = row_limit(len, h, a.T_q, a.n_new, b);  // tokens this row attends

    __shared__ float qs[D];
    const T* qrow = static_cast<const T*>(a.q) + ((size_t)b * a.Hq + h) * D;
    for (int d = threadIdx.x; d < D; d += 64 * VALU_WAVES) qs[d] = to_f32(qrow[d]);
    __syncthreads();

    // Rows are counted from kb/vb: the (b, g) slab of a contiguous cache, or
    // the start of the page pool (rows < 2^31, checked at creation).
    const size_t slab = PAGED ? 0 : kv_row_contiguous(b, g, a.Hkv, a.T_cap, 0) * D;
    const T* kb = static_cast<const T*>(a.k_cache) + slab;
    const T* vb = static_cast<const T*>(a.v_cache) + slab;
    auto row_of = [&](int t) -> int {
        if constexpr (PAGED)
            return (int)kv_row_paged(a.kv, kv_page(a.kv, b, t >> a.kv.page_shift, a.err), g, a.Hkv, t);
        else
            return t;
    };

    // Fused append: the new token (slot sl.slot, the sequence's last) is
    // read from k_new/v_new, and wave 0 of the group's first head in the
    // split owning its tile writes it to the cache slot, which nothing else
    // in this launch reads.
    const T* knew = nullptr;
    const T* vnew = nullptr;
    const int slot = sl.appended ? sl.slot : -1;
    if (sl.appended) {
        const size_t nrow = ((size_t)b * a.Hkv + g) * D;
        knew = static_cast<const T*>(a.k_new) + nrow;
        vnew = static_cast<const T*>(a.v_new) + nrow;
        if (wave == 0 && h % a.M == 0 && s == (slot / VALU_TILE) % a.S) {
            const size_t row = (size_t)row_of(slot);
            T* kw = const_cast<T*>(kb) + row * D;
            T* vw = const_cast<T*>(vb) + row * D;
            for (int d = lane; d < D; d += 64) {
                kw[d] = knew[d];
                vw[d] = vnew[d];
            }
        }
    }

    float acc[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) acc[k] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    for (int tile = s + wave * a.S; tile < n_seq_tiles; tile += VALU_WAVES * a.S) {
        const int t0 = tile * VALU_TILE;
        const int t = t0 + lane;
        // the row of this lane's token (of the sequence's last token past
        // the end); the value loop reads other lanes' rows by shuffle
        const int row = row_of(min(t, len - 1));
        float x = -INFINITY;
        if (t < row_len) {
            // the lane's key row in 16-byte pieces, all requested before use
            const T* kr = t == slot ? knew : kb + (size_t)row * D;
            constexpr int PIECE = 16 / sizeof(T);
            float dot = 0.f;
#pragma unroll 8
            for (int d0 = 0; d0 < D; d0 += PIECE) {
                const uint4 kv = *reinterpret_cast<const uint4*>(kr + d0);
                const uint32_t w4[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
                for (int i = 0; i < PIECE; ++i) dot = fmaf(qs[d0 + i], element<T>(w4, i), dot);
            }
            x = dot * a.scale_log2e;
        }
        const float m_new = fmaxf(m_run, wave_max(x));
        // nothing seen yet in this split (only with several new tokens)
        const bool none = m_new == -INFINITY;
        const float alpha = none ? 1.f : exp2f(m_run - m_new);
        const float p = none ? 0.f : exp2f(x - m_new);
        l_run = l_run * alpha + wave_sum(p);
        m_run = m_new;
#pragma unroll
        for (int k = 0; k < DPL; ++k) acc[k] *= alpha;
        const int nt = min(VALU_TILE, len - t0);
        // Value rows in blocks of 16, all loads of a block in flight at
        // once.  Rows past the sequence's end re-read its last row: their
        // weights p are exactly 0 (scores of -inf).
        for (int jb = 0; jb < nt; jb += 16) {
            float vv[16][DPL];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int j = min(jb + u, nt - 1);
                const int tv = t0 + j;
                const int rv = PAGED ? __shfl(row, j) : tv;
                const T* vr = tv == slot ? vnew : vb + (size_t)rv * D;
#pragma unroll
                for (int k = 0; k < DPL; ++k) vv[u][k] = to_f32(vr[lane + 64 * k]);
            }
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const float pj = __shfl(p, jb + u);
#pragma unroll
                for (int k = 0; k < DPL; ++k) acc[k] = fmaf(pj, vv[u][k], acc[k]);
            }
        }
    }

    // The four waves' states meet in LDS: rescaled to the largest reference
    // m, the sums and accumulators add (a wave with no token weighs 0).
    __shared__ float ml[VALU_WAVES][2];
    __shared__ float accs[VALU_WAVES][D];
    if (lane == 0) {
        ml[wave][0] = m_run;
        ml[wave][1] = l_run;
    }
#pragma unroll
    for (int k = 0; k < DPL; ++k) accs[wave][lane + 64 * k] = acc[k];
    __syncthreads();
    if (wave != 0) return;
    float m_all = ml[0][0];
#pragma unroll
    for (int w = 1; w < VALU_WAVES; ++w) m_all = fmaxf(m_all, ml[w][0]);
    l_run = 0.f;
#pragma unroll
    for (int k = 0; k < DPL; ++k) acc[k] = 0.f;
#pragma unroll
    for (int w = 0; w < VALU_WAVES; ++w) {
        const float f = ml[w][0] == -INFINITY ? 0.f : exp2f(ml[w][0] - m_all);
        l_run = fmaf(f, ml[w][1], l_run);
#pragma unroll
        for (int k = 0; k < DPL; ++k) acc[k] = fmaf(f, accs[w][lane + 64 * k], acc[k]);
    }
    m_run = m_all;
    const size_t row = ((size_t)b * a.Hq + h) * a.S + s;
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    // partials in the output's precision (bf16 rounded to nearest even for
    // a bf16 cache); a single-split pass writes the output row itself
    T* orow = a.out != nullptr ? static_cast<T*>(a.out) + ((size_t)b * a.Hq + h) * D
                               : static_cast<T*>(a.o_part) + row * D;
#pragma unroll
    for (int k = 0; k < DPL; ++k) orow[lane + 64 * k] = from_f32<T>(acc[k] * inv);
    if (a.out == nullptr) {
        if (lane == 0) a.lse_part[row] = l_run > 0.f ? m_run + log2f(l_run) : -INFINITY;
    } else if (sl.appended && a.lengths_adv != nullptr && lane == 0) {
        // the sequence's Hq workgroups have all read its length once the
        // last of them arrives
        advance_when_last(a.seq_ctr + b, a.Hq, a.lengths_adv, b, sl.slot + 1);
    }
}

template <typename T, bool PAGED>
hipError_t launch_typed(const PartialArgs& a, const Launch& on) {
    dim3 grid((unsigned)a.S * a.B * a.Hq), block(64 * VALU_WAVES);
    switch (a.D) {
        case 64: KVD_LAUNCH((partial_valu_kernel<T, 64, PAGED>), grid, block, 0, on, a); break;
        case 128: KVD_LAUNCH((partial_valu_kernel<T, 128, PAGED>), grid, block, 0, on, a); break;
        case 256: KVD_LAUNCH((partial_valu_kernel<T, 256, PAGED>), grid, block, 0, on, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_partial_valu(const PartialArgs& a, bool bf16, const Launch& on) {
    if (a.kv.block_table)
        return bf16 ? launch_typed<uint16_t, true>(a, on) : launch_typed<float, true>(a, on);
    return bf16 ? launch_typed<uint16_t, false>(a, on) : launch_typed<float, false>(a, on);
}

}  // namespace kvd
