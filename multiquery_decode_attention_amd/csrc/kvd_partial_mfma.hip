// kvd_partial_mfma.hip -- bf16 split-KV partial pass on the matrix cores.
//
// Work unit: (split s, KV head g, sequence b) -> one workgroup of NW waves
// per group of up to four 16-head blocks (ceil(M/16) blocks in all).  Wave hb
// owns query heads hb*16 .. hb*16+15 of the group (zero queries past M).  All waves of the group
// walk the same tokens of the split, 32 per iteration, so every K/V tile is
// fetched from HBM once per group and reused by all M query heads.
//
// Per 32-token tile and wave, with v_mfma_f32_16x16x32_bf16 (fp32 accumulate):
//   scores   S^T[tok, head] = K[tok, :] . Q[head, :]      2 x D/32 MFMAs
//            A = K rows straight from global memory (16 B per lane),
//            B = the wave's queries, held in registers for the whole split.
//   softmax  each lane holds 8 scores of one head; the running maximum and
//            sum use two cross-lane steps (xor 16, xor 32); exponentials are
//            base 2 with scale*log2(e) folded into one multiplier.
//   values   O[head, col] += P[head, tok] V[tok, col]     D/16 MFMAs
//            The score tile's register layout is exactly the A operand of
//            this product (rows = heads, 8 tokens per lane), so P never
//            leaves registers.  Each lane loads, for its 8 tokens, the D/16
//            contiguous value columns it owns and transposes them to the
//            B-operand layout with byte permutes.
// Loads for tile i+1 are issued as soon as tile i has consumed the
// registers they overwrite (K after the score MFMAs, V after the value
// MFMAs), so about one tile per wave is always in flight.
//
// The contraction index of each MFMA is only ever paired between A and B of
// the same lane group, so the token order inside a tile and the column
// order inside a lane are free choices; they are chosen for contiguous
// 16-byte loads and stores.
//
// Sources: the grouped contraction and the cross-shard Flash-style
// accumulation, "All About Transformer Inference", section "Sharding the KV
// cache"; multiquery K/V shared by all query heads, "Efficiently Scaling
// Transformer Inference", section 3.3; base-2 softmax, same page, section 3.5;
// reading only each sequence's valid prefix, "All About Transformer
// Inference", ragged-reads paragraph.
#include "kvd_mfma_common.h"

namespace kvd {
namespace {

using namespace mfma;

// Registers of one 32-token tile.
template <int D>
struct TileRegs {
    static constexpr int KS = D / 32;  // k-steps of the score product
    static constexpr int VW = D / 32;  // dwords of value columns per token per lane
    u32x4_t k[2][KS];
    uint32_t v[8][VW];
};

template <int D, bool FULL>
__device__ inline void load_k(TileRegs<D>& r, const uint16_t* __restrict__ kb, int t0, int t_end,
                              int c, int gq) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
        const int row = t0 + 16 * sb + c;
        const uint16_t* p = kb + (size_t)row * D + 8 * gq;
        const bool ok = FULL || row < t_end;
#pragma unroll
        for (int ks = 0; ks < TileRegs<D>::KS; ++ks) {
            r.k[sb][ks] = ok ? *reinterpret_cast<const u32x4_t*>(p + 32 * ks) : u32x4_t{0, 0, 0, 0};
        }
    }
}

template <int D, bool FULL>
__device__ inline void load_v(TileRegs<D>& r, const uint16_t* __restrict__ vb, int t0, int t_end,
                              int c, int gq) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int row = t0 + slot_token(gq, j);
        const bool ok = FULL || row < t_end;
        const uint16_t* p = vb + (size_t)row * D;
        if constexpr (D >= 128) {
#pragma unroll
            for (int i = 0; i < D / 128; ++i) {
                const u32x4_t x =
                    ok ? *reinterpret_cast<const u32x4_t*>(p + 8 * (c + 16 * i)) : u32x4_t{0, 0, 0, 0};
                r.v[j][4 * i + 0] = x[0];
                r.v[j][4 * i + 1] = x[1];
                r.v[j][4 * i + 2] = x[2];
                r.v[j][4 * i + 3] = x[3];
            }
        } else {
            const u32x2_t x = ok ? *reinterpret_cast<const u32x2_t*>(p + 4 * c) : u32x2_t{0, 0};
            r.v[j][0] = x[0];
            r.v[j][1] = x[1];
        }
    }
}

template <int D>
__device__ inline void load_tile(TileRegs<D>& r, const uint16_t* kb, const uint16_t* vb, int t0,
                                 int t_end, int c, int gq, bool k_part) {
    const bool full = t0 + MFMA_TILE <= t_end;
    if (k_part) {
        if (full) load_k<D, true>(r, kb, t0, t_end, c, gq);
        else load_k<D, false>(r, kb, t0, t_end, c, gq);
    } else {
        if (full) load_v<D, true>(r, vb, t0, t_end, c, gq);
        else load_v<D, false>(r, vb, t0, t_end, c, gq);
    }
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void partial_mfma_kernel(PartialArgs a, int hb_groups) {
    constexpr int KS = D / 32;
    constexpr int NE = D / 16;  // value columns per lane = output blocks
    // unit = (sequence b, KV head g, head-block group), group fastest
    const BlockCoord bc = block_coord(a.B * a.Hkv * hb_groups);
    const int s = bc.split;
    const int hbg = bc.unit % hb_groups;
    const int g = (bc.unit / hb_groups) % a.Hkv;
    const int b = bc.unit / (hb_groups * a.Hkv);
    const int hb = hbg * NW + (int)(threadIdx.x >> 6);
    if (hb * MFMA_HEADS >= a.M) return;  // whole wave past the group's last head
    const int len = sequence_length(a.lengths, a.err, a.len_att, b, a.T_cap, false,
                                    s == 0 && g == 0 && hbg == 0 && threadIdx.x == 0).len;
    const int n_seq_tiles = (len + MFMA_TILE - 1) / MFMA_TILE;
    if (s >= n_seq_tiles) return;  // no tile of this sequence for this split
    const int t_end = len;
    const int tstride = a.S * MFMA_TILE;  // this split owns tiles s, s+S, ...

    const int lane = threadIdx.x & 63;
    const int c = lane & 15;   // row/column index inside the 16x16 tile
    const int gq = lane >> 4;  // k-group of the lane
    const int head = hb * MFMA_HEADS + c;  // head (within the group) of B columns / A rows
    const bool head_ok = head < a.M;

    // Queries: B operand of the score product, k-slots 32ks + 8gq .. +7.
    // Lanes past the group's last head load a copy of its last row (their
    // output rows are never stored) so that no load needs a mask.
    u32x4_t qop[KS];
    {
        const int hq = head_ok ? head : a.M - 1;
        const uint16_t* qrow =
            static_cast<const uint16_t*>(a.q) + ((size_t)b * a.Hq + (size_t)g * a.M + hq) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qop[ks] = *reinterpret_cast<const u32x4_t*>(qrow + 32 * ks + 8 * gq);
    }

    const size_t slab = ((size_t)b * a.Hkv + g) * (size_t)a.T_cap * D;
    const uint16_t* kb = static_cast<const uint16_t*>(a.k_cache) + slab;
    const uint16_t* vb = static_cast<const uint16_t*>(a.v_cache) + slab;

    f32x4_t acc[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;  // running max (base 2) of head `head`
    float l_run = 0.f;        // this lane's share of the running sum

    TileRegs<D> r;
    load_tile<D>(r, kb, vb, s * MFMA_TILE, t_end, c, gq, true);
    load_tile<D>(r, kb, vb, s * MFMA_TILE, t_end, c, gq, false);

    for (int t0 = s * MFMA_TILE; t0 < t_end; t0 += tstride) {
        const int tn = t0 + tstride;
        f32x4_t sc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            sc[0] = mfma16x16x32(r.k[0][ks], qop[ks], sc[0]);
            sc[1] = mfma16x16x32(r.k[1][ks], qop[ks], sc[1]);
        }
        if (tn < t_end) load_tile<D>(r, kb, vb, tn, t_end, c, gq, true);

        // Online softmax over this tile for head `head`.
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int tok = t0 + slot_token(gq, j);
            const float v = (j < 4 ? sc[0][j] : sc[1][j - 4]) * a.scale_log2e;
            x[j] = tok < t_end ? v : -INFINITY;
        }
        float mx = x[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) mx = fmaxf(mx, x[j]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        float p[8], ps = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            p[j] = __builtin_amdgcn_exp2f(x[j] - m_new);
            ps += p[j];
        }
        l_run = l_run * alpha + ps;
        m_run = m_new;

        // Output rows are heads 4gq..4gq+3: fetch their rescale factors.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float ai = __shfl(alpha, 4 * gq + i);
#pragma unroll
            for (int e = 0; e < NE; ++e) acc[e][i] *= ai;
        }

        u32x4_t pop;
        pop[0] = pack_bf16x2(p[0], p[1]);
        pop[1] = pack_bf16x2(p[2], p[3]);
        pop[2] = pack_bf16x2(p[4], p[5]);
        pop[3] = pack_bf16x2(p[6], p[7]);
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[e] = mfma16x16x32(pop, v_operand(r.v, e), acc[e]);
        if (tn < t_end) load_tile<D>(r, kb, vb, tn, t_end, c, gq, false);
    }

    // Finish: total sum per head, normalise, store the split's partial.
    float l = l_run;
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const size_t row0 = ((size_t)b * a.Hq + (size_t)g * a.M) * a.S + s;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int hi = hb * MFMA_HEADS + 4 * gq + i;
        const float li = __shfl(l, 4 * gq + i);
        if (hi < a.M) {
            const float inv = 1.f / li;
            store_partial_row<D>(static_cast<uint16_t*>(a.o_part) + (row0 + (size_t)hi * a.S) * D, acc, i, c, inv);
        }
    }
    if (gq == 0 && head_ok) a.lse_part[row0 + (size_t)head * a.S] = m_run + __builtin_log2f(l);
}

template <int D>
hipError_t launch_d(const PartialArgs& a, const Launch& on) {
    const int hbs = mfma_head_blocks(a.M);
    const int nw = hbs < 4 ? hbs : 4;
    const int groups = (hbs + nw - 1) / nw;
    dim3 grid((unsigned)a.S * a.B * a.Hkv * groups);
    switch (nw) {
        case 1: KVD_LAUNCH((partial_mfma_kernel<D, 1>), grid, dim3(64), 0, on, a, groups); break;
        case 2: KVD_LAUNCH((partial_mfma_kernel<D, 2>), grid, dim3(128), 0, on, a, groups); break;
        case 3: KVD_LAUNCH((partial_mfma_kernel<D, 3>), grid, dim3(192), 0, on, a, groups); break;
        default: KVD_LAUNCH((partial_mfma_kernel<D, 4>), grid, dim3(256), 0, on, a, groups); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_partial_mfma(const PartialArgs& a, const Launch& on) {
    switch (a.D) {
        case 64: return launch_d<64>(a, on);
        case 128: return launch_d<128>(a, on);
        case 256: return launch_d<256>(a, on);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kvd
