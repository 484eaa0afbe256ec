// kvd_partial_lds.hip -- bf16 split-KV partial pass with LDS-shared K/V tiles.
//
// Work unit: (split s, KV head g, sequence b[, block of 64 query heads]) ->
// one workgroup of 4 waves.  The group's M query heads fill the waves' 16-row
// matrix-core blocks in turn (16 heads per wave; a group of at most 16 lives
// in wave 0); every wave with heads runs the same score / online-softmax /
// value products as the register kernel on them, but all read one shared
// copy of each 32-token K/V tile from LDS, so a tile crosses HBM and the
// cache hierarchy once for all M heads.  A wave without heads only loads its
// share of every stage: spreading a small group over all four waves made
// each wave read every tile from LDS for two or three heads (ragged GQA
// with 8 heads per KV head: 366 us packed into one wave against 383 us
// spread).
//
// Tiles arrive through a ring of NS LDS stages filled by gfx950's direct
// global->LDS 16-byte loads (no registers held while in flight): stage i+NS-1
// is requested while stage i is computed, so up to NS-1 tiles per workgroup
// are in flight.  Each wave issues D/32 loads per stage; before a stage is
// read every wave waits for its own loads of that stage (vmcnt) and the
// workgroup meets at a barrier, which also retires the stage read in the
// previous iteration before it is refilled.
//
// LDS layout of a stage: K rows then V rows, 32 rows of D bf16 each, in
// 16-byte chunks.  Chunk p of K row t sits at position p ^ (t & SWZ) of the
// row (SWZ = 15, or 7 for d = 64), so the score operand reads (16 lanes = 16
// rows, one chunk each) touch 16 different bank groups while every aligned
// group of 16 chunks -- the 256 bytes a quarter-wave loads -- stays within
// its own two cache lines; V rows are read a row at a time (16 lanes = 16
// consecutive chunks of one row) and are stored as they are.  Rows past
// the split's end are loaded as copies of its last valid row and masked out
// of the softmax.
//
// A paged cache (pages of >= 32 tokens, so a tile never straddles two) is
// read through its block table: one page lookup per tile, from block-table
// entries each wave holds in a register.
//
// Softmax bookkeeping per head keeps a reference maximum m and the sum l of
// 2^(x - m).  A tile whose scores stay below m + 8 (base 2) leaves m alone:
// its weights are at most 2^8, far inside fp32 and bf16 range, and since the
// sum uses the same m the normalised result is unchanged.  Only when some
// head of the wave exceeds m + 8 are m, l and that wave's accumulators
// rescaled, which after the first tiles almost never happens.
//
// Unified maximum (kvdecode_set_unified_max): every split starts from the
// caller's bound phi instead of its own first scores and keeps it unless a
// score exceeds it by more than 2^64 -- weights and sums stay far inside
// fp32 -- so with a good bound no split ever rescales; a bound far above
// every score of a split's first tile is replaced by that tile's maximum
// (nothing has been accumulated yet), so small weights never underflow.
// FlashDecoding++'s asynchronous softmax with a unified maximum ("FlashDecoding++"
// blog summary) is the idea; the splits' log-sum-exps stay exact, so the
// combine is unchanged.
//
// Sources: as for the register kernel -- the grouped contraction and the
// cross-shard Flash-style accumulation ("All About Transformer Inference",
// section "Sharding the KV cache"); multiquery K/V shared by all query heads
// and the aim of loading the cache as few times as possible ("Efficiently
// Scaling Transformer Inference", section 3.3); base-2 softmax (same page,
// section 3.5).  FlashDecoding++'s double-buffered shared-memory loads (the
// blog summary of that paper) are the prior art for the staging.
#include "kvd_lds_common.h"

namespace kvd {
namespace {

using namespace mfma;
using namespace lds;

template <int D, int NS, int VL, bool PAGED, bool GROUPED>
__global__ __launch_bounds__(256) void partial_lds_kernel(PartialArgs a, int head_groups) {
    constexpr int CH = D / 8;                        // 16-byte chunks per row
    constexpr int SWZ = (CH < 16 ? CH : 16) - 1;     // K chunk swizzle mask
    constexpr int KS = D / 32;                       // k-steps of the score product
    constexpr int NE = D / 16;                       // output column blocks per lane
    constexpr int REGION = MFMA_TILE * D * 2;        // bytes of K (or V) per stage
    constexpr int STAGE = 2 * REGION;
    constexpr int PERW = STAGE / (4 * 64 * 16);      // loads per wave per stage (= D/32)
    const float TAU = a.tau;                         // reference headroom (base-2 exponent)
    static_assert(NS >= 2 && NS - 2 <= 6 && (NS - 2) * PERW < 64, "ring depth");
    static_assert(2 * MFMA_TILE * CH == 4 * PERW * 64 && MFMA_TILE * CH == 2 * PERW * 64,
                  "waves 0-1 load K, waves 2-3 load V");
    __shared__ __attribute__((aligned(16))) unsigned char lds[NS * STAGE];

    // unit = (sequence b, KV head g[, head group hg]).  More than 64 query
    // rows per KV head take several workgroups (head groups), and each
    // streams the same K/V tiles: dispatched one after another on one XCD,
    // they walk the same tiles at about the same pace, and the loads of all
    // but the first meet that XCD's L2.
    const LdsCoord lc = lds_coord(a.S, head_groups, a.Hkv, a.B);
    if (!lc.live) return;  // padding, before any barrier
    const SeqAt sa = seq_at(lc.p, a.B, a.order, a.lengths);
    const int s = lc.split, hg = lc.hg, g = lc.g, b = sa.b;
    const SeqLen sl = sequence_length_of(sa.len0, a.err, a.len_att, b, a.T_cap, a.k_new != nullptr,
                                         s == 0 && g == 0 && hg == 0 && threadIdx.x == 0);
    const int len = sl.len;
    const int n_seq_tiles = (len + MFMA_TILE - 1) / MFMA_TILE;
    if (s >= n_seq_tiles) {
        // whole workgroup, before any barrier; a single-split pass writes
        // the zero rows of a sequence with no tokens
        if (a.out != nullptr && n_seq_tiles == 0) {
            const size_t r0 = (size_t)b * a.Hq + (size_t)g * a.M + (size_t)hg * 64;
            const int rows = min(a.M - hg * 64, 64);
            for (int p = threadIdx.x; p < rows * (D / 8); p += 256)
                *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(a.out) + (r0 + p / (D / 8)) * D + (p % (D / 8)) * 8) =
                    u32x4_t{0u, 0u, 0u, 0u};
        }
        return;
    }
    const int t_end = len;
    // this split owns the sequence's tiles s, s+S, s+2S, ...
    const int n_tiles = (n_seq_tiles - s + a.S - 1) / a.S;
    const int tstride = a.S * MFMA_TILE;
    const int t_first = s * MFMA_TILE;

    const int wave = wave_index();
    const int lane = threadIdx.x & 63;
    const int c = lane & 15, gq = lane >> 4;
    const int mg = min(a.M - hg * 64, 64);   // heads of this workgroup
    const int hpw = mg < 16 ? mg : 16;        // heads per wave
    const int hw0 = hg * 64 + wave * hpw;     // first head (within the KV group) of this wave
    const int nh = max(0, min(hpw, mg - wave * hpw));
    const bool head_ok = c < nh;
    // Tokens this lane's query row attends: all `len` of them, except in a
    // step with several new tokens, where the earlier ones see fewer; tiles
    // reaching past the smallest such limit are masked per row.
    const int lim = row_limit(len, hg * 64 + min(wave * hpw + (head_ok ? c : max(nh - 1, 0)), mg - 1),
                              a.T_q, a.n_new, b);
    const int mask_from = a.T_q == 1 ? len : len - a.T_q + 1;

    // Rows below are counted from kb/vb: the (b, g) slab of a contiguous
    // cache, or the start of the page pool.
    const size_t slab = PAGED ? 0 : kv_row_contiguous(b, g, a.Hkv, a.T_cap, 0) * D;
    const char* kb = reinterpret_cast<const char*>(static_cast<const uint16_t*>(a.k_cache) + slab);
    const char* vb = reinterpret_cast<const char*>(static_cast<const uint16_t*>(a.v_cache) + slab);

    // Row of the first token t0 of the split's tile `tile`.  Paged: each
    // wave visits its tiles in order (tile, tile + 1, ...), so the page of
    // its next tile is fetched while the current one is issued.  The block
    // table is read through the constant address space: the kernel never
    // writes it, and a wave-uniform address then becomes a scalar load,
    // whose completion the compiler tracks apart from the K/V loads in
    // flight (a vector load here made it wait for all of them).
    typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
    const const_i32_ptr bt_row = PAGED ? (const_i32_ptr)(a.kv.block_table + (size_t)b * a.kv.max_pages) : nullptr;
    auto table_entry = [&](int tile) { return bt_row[(t_first + tile * tstride) >> a.kv.page_shift]; };
    int next_entry = 0;  // raw entry of the wave's next tile, checked when used
    if constexpr (PAGED) next_entry = table_entry(0);
    auto tile_row = [&](int tile, int t0) -> size_t {
        if constexpr (!PAGED) {
            return (size_t)t0;
        } else {
            int page = next_entry;
            if (tile + 1 < n_tiles) next_entry = table_entry(tile + 1);
            if ((unsigned)page >= (unsigned)a.kv.num_pages) {
                if (threadIdx.x % 64 == 0) atomicOr(a.err, ERRBIT_PAGE);
                page = 0;
            }
            return kv_row_paged(a.kv, page, g, a.Hkv, t0);
        }
    };

    // Fused append.  The new token is the sequence's last, so only the split
    // owning its tile reads that slot in this launch, and it takes the row
    // straight from k_new/v_new (below); the cache slot itself is written
    // here with ordinary stores that nothing in this launch waits for.
    const char* knew = nullptr;
    const char* vnew = nullptr;
    if (sl.appended) {
        const size_t nrow = ((size_t)b * a.Hkv + g) * D * 2;
        knew = static_cast<const char*>(a.k_new) + nrow;
        vnew = static_cast<const char*>(a.v_new) + nrow;
        if (hg == 0 && s == (sl.slot / MFMA_TILE) % a.S && threadIdx.x < 2 * CH) {
            const bool v_half = threadIdx.x >= CH;
            const int ch = v_half ? threadIdx.x - CH : threadIdx.x;
            const u32x4_t x = *reinterpret_cast<const u32x4_t*>((v_half ? vnew : knew) + ch * 16);
            size_t row = (size_t)sl.slot;
            if constexpr (PAGED)
                row = kv_row_paged(a.kv, kv_page(a.kv, b, sl.slot >> a.kv.page_shift, a.err), g, a.Hkv, sl.slot);
            char* dst = const_cast<char*>(v_half ? vb : kb) + row * D * 2 + ch * 16;
            *reinterpret_cast<u32x4_t*>(dst) = x;
        }
    }
    // tiles ending at or before this token need no redirection
    const int t_fast_end = sl.appended ? sl.slot : t_end;

    // Queries of this wave's heads: B operand of the score product.  Lanes
    // past the wave's last head load a copy of its last row instead of a
    // masked load: a row of P only feeds the same row of the output, which
    // is never stored for those lanes, and unmasked loads let all of them
    // be in flight at once.
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

    // Loads of one stage: this wave's PERW loads cover LDS chunks
    // j0 .. j0+63 with j0 = (wave*PERW + n)*64; lane -> (row t, chunk p).
    // Byte offsets inside a tile are loop invariant.
    uint32_t doff[PERW];
#pragma unroll
    for (int n = 0; n < PERW; ++n) {
        const int j0 = (wave * PERW + n) * 64;
        const bool is_v = j0 >= MFMA_TILE * CH;
        const int j = (is_v ? j0 - MFMA_TILE * CH : j0) + lane;
        const int t = j / CH;
        const int p = is_v ? j % CH : (j % CH) ^ (t & SWZ);  // K: position q holds chunk q ^ (t & SWZ)
        doff[n] = (uint32_t)((t * CH + p) * 16);
    }
    // Stage st of the ring holds K of the split's tile st and V of its tile
    // st - VL.  Waves 0-1 load the K half of every stage and waves 2-3 the V
    // half.  A half whose tile does not exist (V of the first VL stages, K of
    // the last VL) points every lane at one 16-byte chunk: the load count per
    // stage stays fixed for the vmcnt bookkeeping, and one cached line costs
    // no HBM traffic.
    const bool v_wave = wave >= 2;
    // Cache policy of the K/V loads: non-temporal.  Every cache byte is read
    // once per launch, and streaming it past the caches measured up to 14%
    // faster out of HBM than ordinary loads (the dummy loads above stay
    // cacheable: they are meant to hit).
    // Head groups sharing tiles through L2 load them cacheable instead.
    constexpr int KV_POLICY = GROUPED ? 0 : 2;
    auto issue = [&](int st) {
        unsigned char* stage = lds + (st % NS) * STAGE;
        const int tile = v_wave ? st - VL : st;
        const char* tbase = v_wave ? vb : kb;
        if (tile < 0 || tile >= n_tiles) {
#pragma unroll
            for (int n = 0; n < PERW; ++n) {
                const int j0 = (wave * PERW + n) * 64;
                __builtin_amdgcn_global_load_lds((const void*)tbase, (lds_void_t*)(stage + j0 * 16), 16, 0, 0);
            }
            return;
        }
        const int t0 = t_first + tile * tstride;
        const char* base = tbase + tile_row(tile, t0) * (D * 2);
        if (t0 + MFMA_TILE <= t_fast_end) {
#pragma unroll
            for (int n = 0; n < PERW; ++n) {
                const int j0 = (wave * PERW + n) * 64;
                // (the source must reach the builtin as const void*: with a
                // char pointer the host pass drops the kernel's launch stub)
                __builtin_amdgcn_global_load_lds((const void*)(base + doff[n]),
                                                 (lds_void_t*)(stage + j0 * 16), 16, 0, KV_POLICY);
            }
        } else {
            // the sequence's last tile: rows past the end re-read the last
            // valid row, and the appended token's row comes from k_new/v_new
#pragma unroll
            for (int n = 0; n < PERW; ++n) {
                const int j0 = (wave * PERW + n) * 64;
                const int t = (int)(doff[n] / (D * 2));
                const int row = min(t, t_end - 1 - t0);
                const char* src = base + (int)doff[n] + (row - t) * (D * 2);
                if (sl.appended && t0 + row == sl.slot)
                    src = (v_wave ? vnew : knew) + ((int)doff[n] - t * (D * 2));
                __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(stage + j0 * 16), 16, 0, KV_POLICY);
            }
        }
    };

    // Per-lane LDS read offsets: K operand of k-step ks (rows c and 16+c),
    // and V row 0 of this lane's chunk (rows advance by whole rows).
    uint32_t koff[2][KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const int t = 16 * sb + c;
            koff[sb][ks] = (uint32_t)((t * CH + ((4 * ks + gq) ^ (t & SWZ))) * 16);
        }
    }

    f32x4_t acc[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_ref = a.m_init, l_run = 0.f;  // -inf, or the unified maximum

    // Probabilities of one tile's scores against the current reference,
    // times that tile's V from LDS, into the accumulators; 128 columns (one
    // 16-byte chunk per lane) at a time.
    auto value_product = [&](const float (&xs)[8], const unsigned char* Vl) {
        // a row with no token yet in this split keeps m_ref = -inf; its
        // scores are -inf too and must weigh 0, not NaN
        const float m_sub = m_ref == -INFINITY ? 0.f : m_ref;
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            p[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(xs[j], a.scale_log2e, -m_sub));
            l_run += p[j];
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
                    const int t = slot_token(gq, j);
                    const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(Vl + (t * CH + c + 16 * i) * 16);
                    v[j][0] = xv[0];
                    v[j][1] = xv[1];
                    v[j][2] = xv[2];
                    v[j][3] = xv[3];
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[8 * i + e] = mfma16x16x32(pop, v_operand(v, e), acc[8 * i + e]);
            }
        } else {
            uint32_t v[8][2];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const u32x2_t xv = *reinterpret_cast<const u32x2_t*>(Vl + slot_token(gq, j) * CH * 16 + c * 8);
                v[j][0] = xv[0];
                v[j][1] = xv[1];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = mfma16x16x32(pop, v_operand(v, e), acc[e]);
        }
    };

    // The prologue always requests NS-1 stages (stages past the last are
    // the one-chunk dummies), so the number of loads issued after the
    // queries is a compile-time constant for the compiler's own wait on them.
    const int n_stages = n_tiles + VL;
#pragma unroll
    for (int i = 0; i < NS - 1; ++i) issue(i);

    if (nh == 0) {
        // a wave with no heads of its own still loads its share of every stage
        for (int it = 0; it < n_stages; ++it) {
            wait_stage<PERW, NS - 2>(min(n_stages - 1, it + NS - 2) - it);
            if (it + NS - 1 < n_stages) issue(it + NS - 1);
        }
        return;
    }

    // scores of the last VL tiles, waiting for their V (oldest first)
    float xh[VL > 0 ? VL : 1][8];
    for (int it = 0; it < n_stages; ++it) {
        // loads issued after stage `it`: stages it+1 .. min(it+NS-2, n_stages-1)
        wait_stage<PERW, NS - 2>(min(n_stages - 1, it + NS - 2) - it);
        if (it + NS - 1 < n_stages) issue(it + NS - 1);

        const unsigned char* Kl = lds + (it % NS) * STAGE;
        const unsigned char* Vl = Kl + REGION;

        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = -INFINITY;
        if (it < n_tiles) {
            const int t0 = t_first + it * tstride;
            f32x4_t sc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const u32x4_t k0 = *reinterpret_cast<const u32x4_t*>(Kl + koff[0][ks]);
                const u32x4_t k1 = *reinterpret_cast<const u32x4_t*>(Kl + koff[1][ks]);
                sc[0] = mfma16x16x32(k0, qop[ks], sc[0]);
                sc[1] = mfma16x16x32(k1, qop[ks], sc[1]);
            }
            // x: the unscaled products q.k (the scale is positive, so the
            // row maximum of x times the scale is that of the scaled logits)
#pragma unroll
            for (int j = 0; j < 8; ++j) x[j] = j < 4 ? sc[0][j] : sc[1][j - 4];
            if (t0 + MFMA_TILE > mask_from) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (t0 + slot_token(gq, j) >= lim) x[j] = -INFINITY;
            }
            float mx = x[0];
#pragma unroll
            for (int j = 1; j < 8; ++j) mx = fmaxf(mx, x[j]);
            mx = max_over_row_groups(mx) * a.scale_log2e;
            // raise the reference past the headroom; on the first tile also drop a
            // unified maximum that lies far above every score
            const bool low = it == 0 && mx < m_ref - TAU;
            if (wave_any(mx > m_ref + TAU || low)) {
                // raise the reference of the heads that outgrew it and rescale
                // what was accumulated with the old one (pending tiles are
                // converted later, with whatever reference holds then)
                const float m_new = mx > m_ref + TAU || low ? mx : m_ref;
                // (nothing is accumulated before the first tile's value
                // product, and a row with no token yet keeps m_ref = m_new =
                // -inf: factor 1 in both cases)
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
        }
        if constexpr (VL > 0) {
            float xp[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) xp[j] = xh[0][j];
#pragma unroll
            for (int k = 0; k + 1 < VL; ++k)
#pragma unroll
                for (int j = 0; j < 8; ++j) xh[k][j] = xh[k + 1][j];
#pragma unroll
            for (int j = 0; j < 8; ++j) xh[VL - 1][j] = x[j];
            if (it >= VL) value_product(xp, Vl);
        } else {
            value_product(x, Vl);
        }
    }

    float l = l_run;
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const size_t qrow0 = (size_t)b * a.Hq + (size_t)g * a.M + hw0;  // query row of the wave's first head
    const size_t row0 = qrow0 * a.S + s;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * gq + i;
        const float li = __shfl(l, r);
        if (r < nh) {
            const float inv = li > 0.f ? 1.f / li : 0.f;  // a row with no token in this split: 0
            // (a single-split pass stores the output rows the same way)
            uint16_t* dst = a.out != nullptr ? static_cast<uint16_t*>(a.out) + (qrow0 + r) * D
                                             : static_cast<uint16_t*>(a.o_part) + (row0 + (size_t)r * a.S) * D;
            store_partial_row<D>(dst, acc, i, c, inv);
        }
    }
    if (a.out == nullptr) {
        if (gq == 0 && head_ok)
            a.lse_part[row0 + (size_t)c * a.S] = l > 0.f ? m_ref + __builtin_log2f(l) : -INFINITY;
    } else if (sl.appended && a.lengths_adv != nullptr && threadIdx.x == 0) {
        // Wave 0 always holds heads, so it gets here; every wave of this
        // workgroup read the length before the ring's first barrier.
        advance_when_last(a.seq_ctr + b, a.Hkv * head_groups, a.lengths_adv, b, sl.slot + 1);
    }
}

template <int D, int NS, int VL>
hipError_t launch_d(const PartialArgs& a, const Launch& on) {
    const int groups = (a.M + 63) / 64;
    const dim3 grid(lds_grid_blocks(a.S, groups, a.Hkv, a.B)), block(256);
    if (groups == 1) {
        if (a.kv.block_table)
            KVD_LAUNCH((partial_lds_kernel<D, NS, VL, true, false>), grid, block, 0, on, a, 1);
        else
            KVD_LAUNCH((partial_lds_kernel<D, NS, VL, false, false>), grid, block, 0, on, a, 1);
    } else {
        if (a.kv.block_table)
            KVD_LAUNCH((partial_lds_kernel<D, NS, VL, true, true>), grid, block, 0, on, a, groups);
        else
            KVD_LAUNCH((partial_lds_kernel<D, NS, VL, false, true>), grid, block, 0, on, a, groups);
    }
    return hipGetLastError();
}

template <int D, int WHICH>
hipError_t launch_cfg(const PartialArgs& a, const Launch& on) {
    constexpr LdsConfig c = lds_config(D, WHICH);
    return launch_d<D, c.stages, c.v_lag>(a, on);
}

}  // namespace

hipError_t launch_partial_lds(const PartialArgs& a, const Launch& on) {
    switch (a.D) {
        case 64: return launch_cfg<64, LDS_SHORT>(a, on);
        case 128: return launch_cfg<128, LDS_SHORT>(a, on);
        case 256:
            return a.lds_config == LDS_LONG ? launch_cfg<256, LDS_LONG>(a, on)
                                            : launch_cfg<256, LDS_SHORT>(a, on);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kvd
