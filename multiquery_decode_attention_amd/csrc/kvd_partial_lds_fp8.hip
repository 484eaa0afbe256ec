// kvd_partial_lds_fp8.hip -- split-KV partial pass over an fp8 KV cache.
//
// The cache holds OCP FP8 E4M3 codes (one byte per value) and, per
// (sequence, KV head, token), a power-of-two exponent e: the stored value is
// code * 2^e.  Queries, the appended rows and the output are bf16.  The
// kernel has the structure of the bf16 LDS kernel -- one workgroup of four
// waves per (split, sequence, KV head), a ring of NS stages filled by direct
// global->LDS loads, matrix-core score and value products, a lazily raised
// softmax reference -- with half the bytes per tile:
//   - K codes are widened to bf16 as they are read from LDS for the score
//     product, with gfx950's scaled conversion, whose scale operand carries
//     the row's 2^e (it uses the scale's exponent only, and every E4M3 value
//     times a power of two within range is exact in bf16);
//   - V codes are widened with scale 1, and each token's 2^e multiplies its
//     softmax weight before the weights are packed for the value product
//     (the normaliser sums the unscaled weights).
// A stage holds 32 K rows and 32 V rows of codes (K chunks XOR-swizzled by
// row as in the bf16 kernel) and a 1 KB block whose first 64 bytes are the
// tile's 32 K and 32 V exponents, loaded by one more 16-byte direct load per
// wave.  Rows past the sequence's end re-read its last valid row (their
// weights are zero, and finite codes keep the products finite).
//
// Sources: quantized KV caches save memory bandwidth ("All About Transformer
// Inference", section on tricks for generation throughput); quantized
// storage with bf16 arithmetic for the products ("Efficiently Scaling
// Transformer Inference", section 3.6); the attention itself as in the bf16
// kernel ("All About Transformer Inference", section "Sharding the KV
// cache"; "Efficiently Scaling Transformer Inference", sections 3.3, 3.5).
#include "kvd_fp8_common.h"

namespace kvd {
namespace {

using namespace mfma;
using namespace lds;
using namespace fp8;

template <int D, int NS, bool PAGED>
__global__ __launch_bounds__(256) void partial_lds_fp8_kernel(PartialArgs a, int head_groups) {
    constexpr int CH = D / 16;                   // 16-byte chunks per row of codes
    constexpr int SWZ = CH - 1;                  // K chunk swizzle mask
    constexpr int KS = D / 32;                   // k-steps of the score product
    constexpr int NE = D / 16;                   // output column blocks per lane
    constexpr int REGION = MFMA_TILE * D;        // bytes of K (or V) codes per stage
    constexpr int EXPS = 1024;                   // exponent block per stage
    constexpr int STAGE = 2 * REGION + EXPS;
    constexpr int PERWD = 2 * REGION / (4 * 64 * 16);  // code loads per wave per stage (D/64)
    constexpr int PERW = PERWD + 1;                     // + the exponent load
    const float TAU = a.tau;  // reference headroom (base-2 exponent)
    static_assert(PERWD >= 1 && REGION == 2 * PERWD * 64 * 16, "waves 0-1 load K, waves 2-3 load V");
    static_assert(NS >= 2 && NS - 2 <= 6 && (NS - 2) * PERW < 64, "ring depth");
    __shared__ __attribute__((aligned(16))) unsigned char lds[NS * STAGE];

    // units dealt to the XCDs and run longest first, as in the bf16 kernel
    const LdsCoord lc = lds_coord(a.S, head_groups, a.Hkv, a.B);
    if (!lc.live) return;  // padding, before any barrier
    const SeqAt sa = seq_at(lc.p, a.B, a.order, a.lengths);
    const int s = lc.split, hg = lc.hg, g = lc.g, b = sa.b;
    const int len = sequence_length_of(sa.len0, a.err, a.len_att, b, a.T_cap, false,
                                       s == 0 && g == 0 && hg == 0 && threadIdx.x == 0).len;
    const int n_seq_tiles = (len + MFMA_TILE - 1) / MFMA_TILE;
    if (s >= n_seq_tiles) return;  // whole workgroup, before any barrier
    const int t_end = len;
    const int n_tiles = (n_seq_tiles - s + a.S - 1) / a.S;
    const int tstride = a.S * MFMA_TILE;
    const int t_first = s * MFMA_TILE;

    const int wave = wave_index();
    const int lane = threadIdx.x & 63;
    const int c = lane & 15, gq = lane >> 4;
    const int mg = min(a.M - hg * 64, 64);
    // heads fill the waves' 16-row blocks in turn: each wave with heads
    // widens every tile, so fewer such waves do less of it (48 heads: three
    // widening waves instead of four)
    const int hpw = mg < 16 ? mg : 16;
    const int hw0 = hg * 64 + wave * hpw;
    const int nh = max(0, min(hpw, mg - wave * hpw));
    const bool head_ok = c < nh;
    // Tokens this lane's query row attends (fewer for the earlier queries of
    // a several-token step); tiles past the smallest limit are masked per row.
    const int lim = row_limit(len, hg * 64 + min(wave * hpw + (head_ok ? c : max(nh - 1, 0)), mg - 1), a.T_q,
                              a.n_new, b);
    const int mask_from = a.T_q == 1 ? len : len - a.T_q + 1;

    // Rows are counted from kb/vb (codes) and ke/ve (exponents, one byte
    // per row): the (b, g) slab of a contiguous cache, or the page pools.
    const size_t slab = PAGED ? 0 : kv_row_contiguous(b, g, a.Hkv, a.T_cap, 0);
    const char* kb = static_cast<const char*>(a.k_cache) + slab * D;
    const char* vb = static_cast<const char*>(a.v_cache) + slab * D;
    const char* ke = reinterpret_cast<const char*>(a.k_exp) + slab;
    const char* ve = reinterpret_cast<const char*>(a.v_exp) + slab;
    // Paged: every wave issues the stages in order and fetches the page of
    // its next tile while issuing the current one (block table through the
    // constant address space, as in the bf16 kernel).
    typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
    const const_i32_ptr bt_row = PAGED ? (const_i32_ptr)(a.kv.block_table + (size_t)b * a.kv.max_pages) : nullptr;
    int next_entry = 0;
    if constexpr (PAGED) next_entry = bt_row[t_first >> a.kv.page_shift];
    auto tile_row = [&](int st, int t0) -> size_t {
        if constexpr (!PAGED) {
            return (size_t)t0;
        } else {
            int page = next_entry;
            if (st + 1 < n_tiles) next_entry = bt_row[(t0 + tstride) >> a.kv.page_shift];
            if ((unsigned)page >= (unsigned)a.kv.num_pages) {
                if (threadIdx.x % 64 == 0) atomicOr(a.err, ERRBIT_PAGE);
                page = 0;
            }
            return kv_row_paged(a.kv, page, g, a.Hkv, t0);
        }
    };

    // Queries (bf16), as in the bf16 kernel: lanes past the wave's last head
    // load a copy of its last row.
    u32x4_t qop[KS];
    {
        // (a wave with no heads reads the group's last row: every row read
        // lies inside the group)
        const int hq = hg * 64 + min(wave * hpw + (head_ok ? c : max(nh - 1, 0)), mg - 1);
        const uint16_t* qrow =
            static_cast<const uint16_t*>(a.q) + ((size_t)b * a.Hq + (size_t)g * a.M + hq) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qop[ks] = *reinterpret_cast<const u32x4_t*>(qrow + 32 * ks + 8 * gq);
    }

    // Code loads of one stage: chunks j0 .. j0+63, j0 = (wave*PERWD + n)*64;
    // waves 0-1 the K rows (swizzled), waves 2-3 the V rows.
    const bool v_wave = wave >= 2;
    uint32_t doff[PERWD];
#pragma unroll
    for (int n = 0; n < PERWD; ++n) {
        const int j0 = (wave * PERWD + n) * 64;
        const int j = (v_wave ? j0 - MFMA_TILE * CH : j0) + lane;
        const int t = j / CH;
        const int p = v_wave ? j % CH : (j % CH) ^ (t & SWZ);
        doff[n] = (uint32_t)((t * CH + p) * 16);
    }
    // Exponent load: lane l fetches 16 bytes -- K exponents of tokens
    // 16(l&1) .. +15 for (l&3) < 2, else V exponents -- into byte 16 l of the
    // block; the first 64 bytes are K[0..31], V[0..31].  Every wave issues
    // it (same bytes, same place), so all waves count PERW loads per stage.
    const int xl = lane & 3;
    auto issue = [&](int st) {
        unsigned char* stage = lds + (st % NS) * STAGE;
        const char* tbase = v_wave ? vb : kb;
        if (st >= n_tiles) {
#pragma unroll
            for (int n = 0; n < PERWD; ++n) {
                const int j0 = (wave * PERWD + n) * 64;
                __builtin_amdgcn_global_load_lds((const void*)tbase, (lds_void_t*)(stage + j0 * 16), 16, 0, 0);
            }
            __builtin_amdgcn_global_load_lds((const void*)ke, (lds_void_t*)(stage + 2 * REGION), 16, 0, 0);
            return;
        }
        const int t0 = t_first + st * tstride;
        const size_t r0 = tile_row(st, t0);
        const char* base = tbase + r0 * D;
        if (t0 + MFMA_TILE <= t_end) {
#pragma unroll
            for (int n = 0; n < PERWD; ++n) {
                const int j0 = (wave * PERWD + n) * 64;
                __builtin_amdgcn_global_load_lds((const void*)(base + doff[n]),
                                                 (lds_void_t*)(stage + j0 * 16), 16, 0, 2);
            }
        } else {
#pragma unroll
            for (int n = 0; n < PERWD; ++n) {
                const int j0 = (wave * PERWD + n) * 64;
                const int t = (int)(doff[n] / D);
                const int row = min(t, t_end - 1 - t0);
                __builtin_amdgcn_global_load_lds((const void*)(base + (int)doff[n] + (row - t) * D),
                                                 (lds_void_t*)(stage + j0 * 16), 16, 0, 2);
            }
        }
        const char* xsrc = (xl < 2 ? ke : ve) + r0 + 16 * (xl & 1);
        __builtin_amdgcn_global_load_lds((const void*)xsrc, (lds_void_t*)(stage + 2 * REGION), 16, 0, 0);
    };

    // LDS read offsets of the score operand: k-step ks, rows c and 16+c,
    // bytes 32ks + 8gq .. +7 (half of a swizzled chunk).
    uint32_t koff[2][KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const int t = 16 * sb + c;
            const int p = 2 * ks + (gq >> 1);
            koff[sb][ks] = (uint32_t)((t * CH + (p ^ (t & SWZ))) * 16 + 8 * (gq & 1));
        }
    }

    f32x4_t acc[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_ref = a.m_init, l_run = 0.f;  // -inf, or the unified maximum

#pragma unroll
    for (int i = 0; i < NS - 1; ++i) issue(i);

    if (nh == 0) {
        for (int it = 0; it < n_tiles; ++it) {
            wait_stage<PERW, NS - 2>(min(n_tiles - 1, it + NS - 2) - it);
            if (it + NS - 1 < n_tiles) issue(it + NS - 1);
        }
        return;
    }

    for (int it = 0; it < n_tiles; ++it) {
        wait_stage<PERW, NS - 2>(min(n_tiles - 1, it + NS - 2) - it);
        if (it + NS - 1 < n_tiles) issue(it + NS - 1);
        const unsigned char* Kl = lds + (it % NS) * STAGE;
        const unsigned char* Vl = Kl + REGION;
        const signed char* X = reinterpret_cast<const signed char*>(Kl + 2 * REGION);
        const int t0 = t_first + it * tstride;

        // scores: K rows c and 16+c widened with their own 2^e
        const float sk0 = pow2_scale(X[c]), sk1 = pow2_scale(X[16 + c]);
        f32x4_t sc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x2_t k0 = *reinterpret_cast<const u32x2_t*>(Kl + koff[0][ks]);
            const u32x2_t k1 = *reinterpret_cast<const u32x2_t*>(Kl + koff[1][ks]);
            sc[0] = mfma16x16x32(widen8(k0, sk0), qop[ks], sc[0]);
            sc[1] = mfma16x16x32(widen8(k1, sk1), qop[ks], sc[1]);
        }
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = j < 4 ? sc[0][j] : sc[1][j - 4];  // unscaled q.k
        if (t0 + MFMA_TILE > mask_from) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (t0 + slot_token(gq, j) >= lim) x[j] = -INFINITY;
        }
        float mx = x[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) mx = fmaxf(mx, x[j]);
        // (the scale is positive: the row maximum of q.k times the scale is
        // that of the scaled logits)
        mx = max_over_row_groups(mx) * a.scale_log2e;
        // raise the reference past the headroom; on the first tile also drop a
        // unified maximum that lies far above every score
        const bool low = it == 0 && mx < m_ref - TAU;
        if (wave_any(mx > m_ref + TAU || low)) {
            const float m_new = mx > m_ref + TAU || low ? mx : m_ref;
            // (a row with no token yet keeps m_ref = m_new = -inf: factor 1)
            // (nothing is accumulated before the first tile: factor 1)
            const float alpha = it == 0 || m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
            l_run *= alpha;
            m_ref = m_new;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float ai = __shfl(alpha, 4 * gq + i);
#pragma unroll
                for (int e = 0; e < NE; ++e) acc[e][i] *= ai;
            }
        }

        // weights: the normaliser sums them as they are; the value product
        // takes them times their token's 2^e
        const uint32_t xv0 = *reinterpret_cast<const uint32_t*>(X + 32 + 4 * gq);
        const uint32_t xv1 = *reinterpret_cast<const uint32_t*>(X + 48 + 4 * gq);
        // a row with no token yet keeps m_ref = -inf; its scores are -inf
        // too and must weigh 0, not NaN
        const float m_sub = m_ref == -INFINITY ? 0.f : m_ref;
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            p[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[j], a.scale_log2e, -m_sub));
            l_run += p[j];
            const uint32_t w = j < 4 ? xv0 : xv1;
            p[j] *= pow2_scale((int)(signed char)(w >> (8 * (j & 3))));
        }
        u32x4_t pop;
        pop[0] = pack_bf16x2(p[0], p[1]);
        pop[1] = pack_bf16x2(p[2], p[3]);
        pop[2] = pack_bf16x2(p[4], p[5]);
        pop[3] = pack_bf16x2(p[6], p[7]);
        if constexpr (D >= 128) {
#pragma unroll
            for (int i = 0; i < D / 128; ++i) {
                uint32_t v[8][4];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const u32x2_t xw = *reinterpret_cast<const u32x2_t*>(Vl + slot_token(gq, j) * D + 128 * i + 8 * c);
                    const u32x4_t w = widen8(xw, 1.0f);
                    v[j][0] = w[0];
                    v[j][1] = w[1];
                    v[j][2] = w[2];
                    v[j][3] = w[3];
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[8 * i + e] = mfma16x16x32(pop, v_operand(v, e), acc[8 * i + e]);
            }
        } else {
            uint32_t v[8][2];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t xw = *reinterpret_cast<const uint32_t*>(Vl + slot_token(gq, j) * D + 4 * c);
                v[j][0] = widen2<false>(xw, 1.0f);
                v[j][1] = widen2<true>(xw, 1.0f);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = mfma16x16x32(pop, v_operand(v, e), acc[e]);
        }
    }

    float l = l_run;
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const size_t row0 = ((size_t)b * a.Hq + (size_t)g * a.M + hw0) * a.S + s;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * gq + i;
        const float li = __shfl(l, r);
        if (r < nh) {
            const float inv = li > 0.f ? 1.f / li : 0.f;  // a row with no token in this split: 0
            store_partial_row<D>(static_cast<uint16_t*>(a.o_part) + (row0 + (size_t)r * a.S) * D, acc, i, c, inv);
        }
    }
    if (gq == 0 && head_ok)
        a.lse_part[row0 + (size_t)c * a.S] = l > 0.f ? m_ref + __builtin_log2f(l) : -INFINITY;
}

template <int D>
hipError_t launch_d(const PartialArgs& a, const Launch& on) {
    const int groups = (a.M + 63) / 64;
    const dim3 grid(lds_grid_blocks(a.S, groups, a.Hkv, a.B));
    if (a.kv.block_table)
        KVD_LAUNCH((partial_lds_fp8_kernel<D, lds_fp8_stages(D), true>), grid, dim3(256), 0, on, a,
                           groups);
    else
        KVD_LAUNCH((partial_lds_fp8_kernel<D, lds_fp8_stages(D), false>), grid, dim3(256), 0, on, a,
                           groups);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_partial_lds_fp8(const PartialArgs& a, const Launch& on) {
    switch (a.D) {
        case 64: return launch_d<64>(a, on);
        case 128: return launch_d<128>(a, on);
        case 256: return launch_d<256>(a, on);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kvd
