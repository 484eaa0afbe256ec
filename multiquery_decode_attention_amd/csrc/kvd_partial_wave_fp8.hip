// kvd_partial_wave_fp8.hip -- split-KV partial pass over an fp8 KV cache in
// which each wave streams its own tiles for every query row of its group.
//
// Work unit: (split s, sequence b, KV head g[, group hg of up to 16*RB query
// rows]) -> one workgroup of four waves.  The split's 32-token tiles are
// dealt to the waves in turn (wave w takes the split's tiles w, w+4, ...),
// and a wave runs each of its tiles for all of the group's rows: RB blocks
// of 16 rows share every K and V operand it widens and reads from LDS.  In
// the shared-tile fp8 kernel (kvd_partial_lds_fp8.hip) every wave widens and
// reads every tile for its own quarter of the rows, four times per tile in
// all, which makes grouped heads compute-bound; here each tile is widened
// and read once.
//
// Each wave owns a ring of NSW stages in LDS, filled by its own direct
// global->LDS loads (K codes XOR-swizzled by row, V codes as stored, and a
// 1 KB block whose first 64 bytes are the tile's 32 K and 32 V exponents),
// and waits only for its own loads: the loop has no workgroup barrier.
// Widening and the products follow the shared-tile kernel: K is widened with
// its rows' 2^e as the conversion scale, V with scale 1, and each token's
// 2^e multiplies its softmax weight (the normaliser sums the unscaled
// weights).  The softmax reference is raised lazily, past TAU of headroom.
//
// At the end the four waves' states -- reference m, partial sums l and the
// accumulators, per row -- meet in LDS in two rounds (waves 2, 3 into 0, 1,
// then 1 into 0), merged by the same exact rescaling as the log-sum-exp
// combine, and wave 0 writes the split's partial.
//
// In a decode step the kernel also appends the new token: the workgroups
// owning its tile quantize its rows into the cache slot first (below).
//
// Sources: quantized KV caches save memory bandwidth ("All About Transformer
// Inference", section on tricks for generation throughput); bf16 arithmetic
// on quantized storage ("Efficiently Scaling Transformer Inference", section
// 3.6); multiquery K/V read once for all query heads of a group (same page,
// section 3.3); accumulation across sequence shards ("All About Transformer
// Inference", section "Sharding the KV cache").
#include "kvd_fp8_common.h"

namespace kvd {
namespace {

using namespace mfma;
using namespace lds;
using namespace fp8;

template <int D, int RB, int NSW, bool GROUPED, bool PAGED>
__global__ __launch_bounds__(256) void partial_wave_fp8_kernel(PartialArgs a, int head_groups) {
    constexpr int CH = D / 16;                 // 16-byte chunks per row of codes
    constexpr int SWZ = CH - 1;                // K chunk swizzle mask
    constexpr int KS = D / 32;                 // k-steps of the score product
    constexpr int NE = D / 16;                 // output column blocks per lane
    constexpr int REGION = MFMA_TILE * D;      // bytes of K (or V) codes per tile
    constexpr int EXPS = 1024;                 // exponent block per stage
    constexpr int STAGE = 2 * REGION + EXPS;
    constexpr int PERC = REGION / (64 * 16);   // loads of K (and of V) codes per stage
    constexpr int PERW = 2 * PERC + 1;         // + the exponent load
    constexpr int ROWS = 16 * RB;              // query rows per workgroup
    constexpr int MERGE = RB * (NE * 64 * 16 + 64 * 8);  // one wave's state in LDS
    static_assert(D >= 128, "value operands of 16-byte code chunks");
    static_assert(NSW >= 2 && NSW - 1 <= 4 && NSW * PERW < 64, "ring depth");
    static_assert(2 * MERGE <= 4 * NSW * STAGE, "merge buffers fit in the rings");
    __shared__ __attribute__((aligned(16))) unsigned char lds[4 * NSW * STAGE];
    const float TAU = a.tau;

    // unit = (sequence b, KV head g[, row group hg]), dealt to the XCDs and
    // run longest first as in the bf16 LDS kernel; the row groups of one
    // (split, unit) run one after another on one XCD, so their loads of the
    // same tiles meet in that XCD's L2
    const LdsCoord lc = lds_coord(a.S, head_groups, a.Hkv, a.B);
    if (!lc.live) return;  // padding, before any barrier
    const SeqAt sa = seq_at(lc.p, a.B, a.order, a.lengths);
    const int s = lc.split, hg = lc.hg, g = lc.g, b = sa.b;
    const SeqLen sl = sequence_length_of(sa.len0, a.err, a.len_att, b, a.T_cap, a.k_new != nullptr,
                                         s == 0 && g == 0 && hg == 0 && threadIdx.x == 0);
    const int len = sl.len;
    const int n_seq_tiles = (len + MFMA_TILE - 1) / MFMA_TILE;
    if (s >= n_seq_tiles) return;  // whole workgroup, before any barrier
    const int t_end = len;
    const int n_tiles = (n_seq_tiles - s + a.S - 1) / a.S;  // tiles of this split
    const int tstride = a.S * MFMA_TILE;
    const int t_first = s * MFMA_TILE;

    const int wave = wave_index();
    const int lane = threadIdx.x & 63;
    const int c = lane & 15, gq = lane >> 4;

    // Fused append (one new token; k_new/v_new set): the split owning the
    // token's tile quantizes its K and V rows into the cache slot before any
    // load of that tile -- waves 0 and 1 write them, and the barrier (a
    // workgroup-scope release and acquire) makes the stores visible to every
    // wave's loads.  Every head group of that split writes the same bytes; no
    // other workgroup reads the slot in this launch.
    if (sl.appended && s == (sl.slot / MFMA_TILE) % a.S) {
        if (wave < 2) {
            size_t row;
            if constexpr (PAGED)
                row = kv_row_paged(a.kv, kv_page(a.kv, b, sl.slot >> a.kv.page_shift, a.err), g, a.Hkv, sl.slot);
            else
                row = kv_row_contiguous(b, g, a.Hkv, a.T_cap, sl.slot);
            const uint16_t* src = static_cast<const uint16_t*>(wave ? a.v_new : a.k_new) + ((size_t)b * a.Hkv + g) * D;
            uint8_t* cache = static_cast<uint8_t*>(const_cast<void*>(wave ? a.v_cache : a.k_cache));
            int8_t* exps = const_cast<int8_t*>(wave ? a.v_exp : a.k_exp);
            quantize_row<D>(src, cache + row * D, exps + row, lane);
        }
        __syncthreads();
    }
    const int n_my = n_tiles > wave ? (n_tiles - wave + 3) / 4 : 0;  // this wave's tiles
    const int mg = min(a.M - hg * ROWS, ROWS);                        // rows of the group
    // Tokens the lane's query row of each block attends: all `len`, except
    // in a step with several new tokens, where the earlier ones see fewer;
    // tiles reaching past the smallest such limit are masked per row.
    int lim[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) lim[rb] = row_limit(len, hg * ROWS + min(rb * 16 + c, mg - 1), a.T_q, a.n_new, b);
    const int mask_from = a.T_q == 1 ? len : len - a.T_q + 1;

    // Rows below are counted from kb/vb (codes) and ke/ve (exponents, one
    // byte per row): the (b, g) slab of a contiguous cache, or the start of
    // the page pools.
    const size_t slab = PAGED ? 0 : kv_row_contiguous(b, g, a.Hkv, a.T_cap, 0);
    const char* kb = static_cast<const char*>(a.k_cache) + slab * D;
    const char* vb = static_cast<const char*>(a.v_cache) + slab * D;
    const char* ke = reinterpret_cast<const char*>(a.k_exp) + slab;
    const char* ve = reinterpret_cast<const char*>(a.v_exp) + slab;
    // Paged: the wave issues its tiles in order, so the page of its next
    // tile is fetched while the current one is issued; the block table is
    // read through the constant address space (scalar loads, tracked apart
    // from the direct loads in flight), and an entry is range-checked when
    // used (outside the pool: page 0, flagged).
    typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
    const const_i32_ptr bt_row = PAGED ? (const_i32_ptr)(a.kv.block_table + (size_t)b * a.kv.max_pages) : nullptr;
    auto tile_t0 = [&](int k) { return t_first + (wave + 4 * k) * tstride; };
    int next_entry = 0;
    if constexpr (PAGED) {
        if (n_my > 0) next_entry = bt_row[tile_t0(0) >> a.kv.page_shift];
    }
    // first row of the wave's tile k (its 32 rows are consecutive: pages
    // hold whole tiles); called for k = 0, 1, ... in order
    auto tile_row = [&](int k, int t0) -> size_t {
        if constexpr (!PAGED) {
            return (size_t)t0;
        } else {
            int page = next_entry;
            if (k + 1 < n_my) next_entry = bt_row[tile_t0(k + 1) >> a.kv.page_shift];
            if ((unsigned)page >= (unsigned)a.kv.num_pages) {
                if (threadIdx.x % 64 == 0) atomicOr(a.err, ERRBIT_PAGE);
                page = 0;
            }
            return kv_row_paged(a.kv, page, g, a.Hkv, t0);
        }
    };

    // Queries of every row block: B operands of the score product.  Lanes
    // past the group's last row load a copy of it (never stored).
    u32x4_t qop[RB][KS];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int r = min(rb * 16 + c, mg - 1);
        const uint16_t* qrow =
            static_cast<const uint16_t*>(a.q) + ((size_t)b * a.Hq + (size_t)g * a.M + hg * ROWS + r) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qop[rb][ks] = *reinterpret_cast<const u32x4_t*>(qrow + 32 * ks + 8 * gq);
    }

    // Stage layout: K codes (chunk position q of row t holds chunk
    // q ^ (t & SWZ)), V codes, exponents.  Load n of the K (V) codes puts
    // lane l's 16 bytes at chunk n*64 + l.
    unsigned char* const ring = lds + wave * (NSW * STAGE);
    uint32_t koffg[PERC];
#pragma unroll
    for (int n = 0; n < PERC; ++n) {
        const int j = n * 64 + lane;
        const int t = j / CH;
        koffg[n] = (uint32_t)((t * CH + ((j % CH) ^ (t & SWZ))) * 16);
    }
    // Non-temporal K/V loads (each byte is read once), except where several
    // row groups read the same tiles through L2.
    constexpr int KV_POLICY = GROUPED ? 0 : 2;
    const int xl = lane & 3;
    auto issue = [&](int k) {
        unsigned char* stage = ring + (k % NSW) * STAGE;
        if (k >= n_my) {
            // past the wave's last tile: the same count of loads, all of one
            // cached chunk (never read), keeps the waits' arithmetic fixed
#pragma unroll
            for (int n = 0; n < 2 * PERC; ++n)
                __builtin_amdgcn_global_load_lds((const void*)kb, (lds_void_t*)(stage + n * 1024), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const void*)ke, (lds_void_t*)(stage + 2 * REGION), 16, 0, 0);
            return;
        }
        const int t0 = tile_t0(k);
        const size_t r0 = tile_row(k, t0);
        const char* kt = kb + r0 * D;
        const char* vt = vb + r0 * D;
        if (t0 + MFMA_TILE <= t_end) {
#pragma unroll
            for (int n = 0; n < PERC; ++n)
                __builtin_amdgcn_global_load_lds((const void*)(kt + koffg[n]), (lds_void_t*)(stage + n * 1024), 16, 0,
                                                 KV_POLICY);
#pragma unroll
            for (int n = 0; n < PERC; ++n)
                __builtin_amdgcn_global_load_lds((const void*)(vt + n * 1024 + lane * 16),
                                                 (lds_void_t*)(stage + REGION + n * 1024), 16, 0, KV_POLICY);
        } else {
            // the sequence's last tile: rows past its end re-read its last
            // valid row (zero weight; finite codes keep the products finite)
            const int last = t_end - 1 - t0;
#pragma unroll
            for (int n = 0; n < PERC; ++n) {
                const int t = (int)koffg[n] / D;
                __builtin_amdgcn_global_load_lds((const void*)(kt + (int)koffg[n] + (min(t, last) - t) * D),
                                                 (lds_void_t*)(stage + n * 1024), 16, 0, KV_POLICY);
            }
#pragma unroll
            for (int n = 0; n < PERC; ++n) {
                const int j = n * 64 + lane;
                const int t = j / CH;
                __builtin_amdgcn_global_load_lds((const void*)(vt + j * 16 + (min(t, last) - t) * D),
                                                 (lds_void_t*)(stage + REGION + n * 1024), 16, 0, KV_POLICY);
            }
        }
        // lane l: K exponents of tokens 16(l&1).. for (l&3) < 2, else V
        // exponents, at byte 16 l: bytes 0-31 K, 32-63 V (T_cap, and a page,
        // is a multiple of the tile, so all 32 lie inside the cache row)
        __builtin_amdgcn_global_load_lds((const void*)((xl < 2 ? ke : ve) + r0 + 16 * (xl & 1)),
                                         (lds_void_t*)(stage + 2 * REGION), 16, 0, 0);
    };

    // LDS read offsets of the score operand: k-step ks, rows c and 16+c,
    // codes 32ks + 8gq .. +7 (half of a swizzled chunk).
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

    f32x4_t acc[RB][NE];
    float m_ref[RB], l_run[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[rb][e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        m_ref[rb] = a.m_init;  // -inf, or the unified maximum
        l_run[rb] = 0.f;
    }

    // The fast loop below never rescales the accumulators, so they can stay
    // in the matrix cores' accumulation registers: when a row block's
    // reference has to move, the loop stops before that tile's weights, the
    // block below rescales, and the loop resumes at the same tile (its
    // scores are recomputed; this happens on a wave's first tile and rarely
    // after).  A stage is refilled at the end of the iteration that read it.
#pragma unroll
    for (int i = 0; i < NSW; ++i) issue(i);

    int it = 0;
    while (it < n_my) {
        float mxs[RB];
        bool moved = false;
        for (; it < n_my; ++it) {
            // loads issued after stage `it`: its stages it+1 .. min(it+NSW-1, n_my-1)
            wait_own_stage<PERW, NSW - 1>(min(n_my - 1, it + NSW - 1) - it);
            const unsigned char* Kl = ring + (it % NSW) * STAGE;
            const unsigned char* Vl = Kl + REGION;
            const signed char* X = reinterpret_cast<const signed char*>(Kl + 2 * REGION);
            const int t0 = tile_t0(it);

            // scores of every row block: K rows c and 16+c widened once,
            // with their own 2^e
            const float sk0 = pow2_scale(X[c]), sk1 = pow2_scale(X[16 + c]);
            f32x4_t sc[RB][2];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) sc[rb][0] = sc[rb][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const u32x4_t k0 = widen8(*reinterpret_cast<const u32x2_t*>(Kl + koff[0][ks]), sk0);
                const u32x4_t k1 = widen8(*reinterpret_cast<const u32x2_t*>(Kl + koff[1][ks]), sk1);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    sc[rb][0] = mfma16x16x32(k0, qop[rb][ks], sc[rb][0]);
                    sc[rb][1] = mfma16x16x32(k1, qop[rb][ks], sc[rb][1]);
                }
            }
            float x[RB][8];
            bool move = false;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
                for (int j = 0; j < 8; ++j) x[rb][j] = j < 4 ? sc[rb][0][j] : sc[rb][1][j - 4];  // unscaled q.k
                if (t0 + MFMA_TILE > mask_from) {
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        if (t0 + slot_token(gq, j) >= lim[rb]) x[rb][j] = -INFINITY;
                }
                float mx = x[rb][0];
#pragma unroll
                for (int j = 1; j < 8; ++j) mx = fmaxf(mx, x[rb][j]);
                // (the scale is positive: the row maximum of q.k times the
                // scale is that of the scaled logits)
                mx = max_over_row_groups(mx) * a.scale_log2e;
                mxs[rb] = mx;
                // past the headroom; on the wave's first tile also a unified
                // maximum far above every score
                move = move || mx > m_ref[rb] + TAU || (it == 0 && mx < m_ref[rb] - TAU);
            }
            if (wave_any(move)) {
                moved = true;
                break;
            }

            // 2^e of the V rows of this lane's 8 token slots
            const uint32_t xv0 = *reinterpret_cast<const uint32_t*>(X + 32 + 4 * gq);
            const uint32_t xv1 = *reinterpret_cast<const uint32_t*>(X + 48 + 4 * gq);
            u32x4_t pop[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                // a row with no token yet keeps m_ref = -inf and weighs 0
                const float m_sub = m_ref[rb] == -INFINITY ? 0.f : m_ref[rb];
                float p[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    p[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[rb][j], a.scale_log2e, -m_sub));
                    l_run[rb] += p[j];
                    p[j] *= pow2_scale((int)(signed char)((j < 4 ? xv0 : xv1) >> (8 * (j & 3))));
                }
                pop[rb][0] = pack_bf16x2(p[0], p[1]);
                pop[rb][1] = pack_bf16x2(p[2], p[3]);
                pop[rb][2] = pack_bf16x2(p[4], p[5]);
                pop[rb][3] = pack_bf16x2(p[6], p[7]);
            }

            // values: each 8-column piece of the 8 token slots is widened
            // once and serves every row block
#pragma unroll
            for (int i = 0; i < D / 128; ++i) {
                uint32_t v[8][4];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const u32x4_t w = widen8(
                        *reinterpret_cast<const u32x2_t*>(Vl + slot_token(gq, j) * D + 128 * i + 8 * c), 1.0f);
                    v[j][0] = w[0];
                    v[j][1] = w[1];
                    v[j][2] = w[2];
                    v[j][3] = w[3];
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const u32x4_t vop = v_operand(v, e);
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb)
                        acc[rb][8 * i + e] = mfma16x16x32(pop[rb], vop, acc[rb][8 * i + e]);
                }
            }
            // this slot's LDS reads have returned: refill it
            if (it + NSW < n_my) {
                wait_vm<63>();  // lgkmcnt(0); vmcnt untouched
                issue(it + NSW);
            }
        }
        if (!moved) break;
        // Move the references of tile `it` and rescale what was accumulated
        // with the old ones; the loop then resumes at the same tile.
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const float mx = mxs[rb];
            const bool low = it == 0 && mx < m_ref[rb] - TAU;
            if (wave_any(mx > m_ref[rb] + TAU || low)) {
                const float m_new = mx > m_ref[rb] + TAU || low ? mx : m_ref[rb];
                // (nothing is accumulated before the first tile; a row with
                // no token yet keeps m_ref = m_new = -inf: factor 1)
                const float alpha =
                    it == 0 || m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_ref[rb] - m_new);
                l_run[rb] *= alpha;
                m_ref[rb] = m_new;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float ai = __shfl(alpha, 4 * gq + i);
#pragma unroll
                    for (int e = 0; e < NE; ++e) acc[rb][e][i] *= ai;
                }
            }
        }
    }

    // Merge.  Every direct load of this wave has landed (dummies included)
    // before the rings are reused for the states.
    wait_vm<0>();
    __syncthreads();
    // State of a wave: accumulators in its own lane layout, then (m, l) per
    // row block and lane.  A row that saw no token in this wave's tiles (no
    // tiles at all, or an early query of a several-token step: its first
    // tile already lies past the row's limit) offers m = -inf, weight 0 --
    // its reference may still hold a unified maximum far above the others.
    bool has[RB];  // the row saw a token (in this wave, or in a state it took)
    {
        const int t_mine = n_my > 0 ? tile_t0(0) : INT32_MAX;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) has[rb] = t_mine < lim[rb];
    }
    auto m_offered = [&](int rb) { return has[rb] ? m_ref[rb] : -INFINITY; };
    auto put = [&](unsigned char* buf) {
        f32x4_t* A = reinterpret_cast<f32x4_t*>(buf);
        float2* ML = reinterpret_cast<float2*>(buf + RB * NE * 64 * 16);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
            for (int e = 0; e < NE; ++e) A[(rb * NE + e) * 64 + lane] = acc[rb][e];
            ML[rb * 64 + lane] = make_float2(m_offered(rb), l_run[rb]);
        }
    };
    auto take = [&](const unsigned char* buf) {
        const f32x4_t* A = reinterpret_cast<const f32x4_t*>(buf);
        const float2* ML = reinterpret_cast<const float2*>(buf + RB * NE * 64 * 16);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const float2 o = ML[rb * 64 + lane];
            const float m_self = m_offered(rb);
            const float m_new = fmaxf(m_self, o.x);
            // both -inf: neither holds a token of this row (factors 1, 0)
            const float f_self = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_self - m_new);
            const float f_other = m_new == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(o.x - m_new);
            l_run[rb] = l_run[rb] * f_self + o.y * f_other;
            m_ref[rb] = m_new;
            has[rb] = has[rb] || o.x != -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float fs = __shfl(f_self, 4 * gq + i), fo = __shfl(f_other, 4 * gq + i);
#pragma unroll
                for (int e = 0; e < NE; ++e) acc[rb][e][i] = acc[rb][e][i] * fs + A[(rb * NE + e) * 64 + lane][i] * fo;
            }
        }
    };
    if (wave >= 2) put(lds + (wave - 2) * MERGE);
    __syncthreads();
    if (wave < 2) take(lds + wave * MERGE);
    __syncthreads();
    if (wave == 1) put(lds);
    __syncthreads();
    if (wave != 0) return;
    take(lds);

    // wave 0 now holds the split's state; normalise and store (a row with
    // no token in the split: partial 0, log-sum-exp -inf)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int r0 = rb * 16;  // first row of the block in the group
        if (r0 >= mg) break;
        float l = l_run[rb];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        const size_t row0 = ((size_t)b * a.Hq + (size_t)g * a.M + hg * ROWS + r0) * a.S + s;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * gq + i;
            const float li = __shfl(l, r);
            if (r0 + r < mg) {
                const float inv = li > 0.f ? 1.f / li : 0.f;
                store_partial_row<D>(static_cast<uint16_t*>(a.o_part) + (row0 + (size_t)r * a.S) * D, acc[rb], i, c,
                                     inv);
            }
        }
        if (gq == 0 && r0 + c < mg)
            a.lse_part[row0 + (size_t)c * a.S] = l > 0.f ? m_ref[rb] + __builtin_log2f(l) : -INFINITY;
    }
}

template <int D, int RB, int NSW>
hipError_t launch_rb(const PartialArgs& a, const Launch& on) {
    const int groups = (a.M + 16 * RB - 1) / (16 * RB);
    const dim3 grid(lds_grid_blocks(a.S, groups, a.Hkv, a.B)), block(256);
    const bool paged = a.kv.block_table != nullptr;
    if (groups == 1) {
        if (paged)
            KVD_LAUNCH((partial_wave_fp8_kernel<D, RB, NSW, false, true>), grid, block, 0, on, a, 1);
        else
            KVD_LAUNCH((partial_wave_fp8_kernel<D, RB, NSW, false, false>), grid, block, 0, on, a, 1);
    } else {
        if (paged)
            KVD_LAUNCH((partial_wave_fp8_kernel<D, RB, NSW, true, true>), grid, block, 0, on, a, groups);
        else
            KVD_LAUNCH((partial_wave_fp8_kernel<D, RB, NSW, true, false>), grid, block, 0, on, a,
                               groups);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_partial_wave_fp8(const PartialArgs& a, const Launch& on) {
    if (a.D == 256) return launch_rb<256, 1, wave_fp8_stages(256)>(a, on);
    if (a.D == 128) {
        constexpr int NSW = wave_fp8_stages(128);
        switch (wave_fp8_row_blocks(128, a.M)) {
            case 1: return launch_rb<128, 1, NSW>(a, on);
            case 2: return launch_rb<128, 2, NSW>(a, on);
            default: return launch_rb<128, 3, NSW>(a, on);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace kvd
