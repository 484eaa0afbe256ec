// kvd_partial_xchg.hip -- split-KV partial pass over an fp8 KV cache for
// large query groups (many query heads per KV head, as in multiquery
// attention), in which the four waves of a workgroup split every tile and
// exchange the softmax weights through LDS.
//
// Work unit: (split s, sequence b, KV head g[, group hg of up to 16*R query
// rows]) -> one workgroup of four waves, over 64-token tiles.  In the other
// fp8 kernels a code is widened to bf16 by every wave that reads it: each
// wave takes whole tiles for all rows (kvd_partial_wave_fp8.hip, whose
// registers hold 16 rows at d = 256), or every tile for its own rows
// (kvd_partial_lds_fp8.hip, where 48 rows mean three widenings of each
// code).  Here every code is widened exactly once:
//   - scores: wave w takes tokens 16w .. 16w+15 of the tile for every row
//     block of the group, widening its 16 K rows once;
//   - weights: it turns those scores into softmax weights, times each
//     token's V exponent as in the other fp8 kernels (the normaliser sums
//     the unscaled weights), and writes them, bf16, to LDS with its per-row
//     maxima;
//   - values: after one workgroup barrier every wave reads the weights of
//     all 64 tokens and accumulates output columns w*D/4 .. (w+1)*D/4 - 1 of
//     every row, widening only those columns of the V rows.
// Every wave holds the same softmax reference per row: after the barrier
// all read the same tile maxima and apply the same lazy rule (raise past
// TAU of headroom).  Weights are first computed under the current
// reference; only when a reference moves (on the first tile, and rarely
// after) are they recomputed and rewritten, and the waves meet at a second
// barrier before the value product.
//
// LDS holds NS slots (two; xchg_slots) of K codes, V codes and exponents,
// two buffers of weights and two of row maxima (tile it uses slot it % NS
// and buffers it & 1).
// Each wave fills its own 16 rows of a slot with direct global->LDS loads:
// K rows with their 16-byte chunks XOR-swizzled by row (the score operand
// reads 16 rows at once), V rows swizzled by 8-token group (the value
// operand reads four such groups at once), and the rows' exponents.  Only
// the wave itself reads its K rows and exponents, so it refills them a tile
// ahead as soon as the tile before is done; V rows are read by every wave
// and are refilled after the barrier.  Weight rows are swizzled by row pair
// for the same reason.  At d = 256 with 48 rows this is 81408 bytes, two
// workgroups per CU.
//
// In a decode step the kernel also appends the new token: the workgroups
// owning its tile quantize its rows into the cache slot first (below).
//
// Sources: quantized KV caches save memory bandwidth ("All About Transformer
// Inference", section on tricks for generation throughput); bf16 arithmetic
// on quantized storage ("Efficiently Scaling Transformer Inference", section
// 3.6); multiquery K/V read once for all query heads (same page, section
// 3.3); accumulation across sequence shards ("All About Transformer
// Inference", section "Sharding the KV cache").
#include "kvd_fp8_common.h"

namespace kvd {
namespace {

using namespace mfma;
using namespace lds;
using namespace fp8;

// s_waitcnt lgkmcnt(0), then s_barrier: LDS writes of every wave visible.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int D, int R, int NS, bool GROUPED, bool PAGED>
__global__ __launch_bounds__(256, 2) void partial_xchg_fp8_kernel(PartialArgs a, int head_groups) {
    constexpr int TT = XCHG_TILE;          // tokens per tile
    constexpr int ROWB = D;                // bytes per cache row (one code per value)
    constexpr int CH = ROWB / 16;          // 16-byte chunks per row
    constexpr int SWZ = CH - 1;            // K chunk swizzle mask
    constexpr int VKEY = CH / 4;           // V chunk swizzle step per 8-token group
    constexpr int KS = D / 32;             // k-steps of the score product
    constexpr int DQ = D / 4;              // value columns per wave
    constexpr int NC = DQ / 16;            // output column blocks per wave = codes per lane and token
    constexpr int ROWS = 16 * R;           // query rows per workgroup
    constexpr int NKV = 16 * ROWB / 1024;  // 1 KB loads of a wave's 16 K (or V) rows
    constexpr int REGION = TT * ROWB;      // bytes of K (or V) rows per slot
    constexpr int XBYTES = 4 * 256;        // exponents per slot: 256 bytes per wave
    constexpr int SLOT = 2 * REGION + XBYTES;
    constexpr int PST = 2 * TT;            // bytes per row of weights
    constexpr int PBUF = ROWS * PST;
    constexpr int MBUF = ROWS * 4 * 4;     // per row, the maxima of the four waves
    constexpr int P_AT = NS * SLOT, M_AT = P_AT + 2 * PBUF;
    constexpr int KX = NKV + 1;            // loads of a wave's K rows and exponents per tile
    constexpr int PERT = NKV + KX;            // loads of a wave per tile
    static_assert(NC == 2 || NC == 4, "d = 128 or 256");
    static_assert(NS >= 2 && (NS - 1) * PERT < 64, "vmcnt range");
    __shared__ __attribute__((aligned(16))) unsigned char lds[M_AT + 2 * MBUF];
    const float TAU = a.tau;

    // units dealt to the XCDs and run longest first, as in the other
    // LDS-staged kernels; the row groups of one (split, unit) run one after
    // another on one XCD, so their loads of the same tiles meet in its L2
    const LdsCoord lc = lds_coord(a.S, head_groups, a.Hkv, a.B);
    if (!lc.live) return;  // padding, before any barrier
    const SeqAt sa = seq_at(lc.p, a.B, a.order, a.lengths);
    const int s = lc.split, hg = lc.hg, g = lc.g, b = sa.b;
    const SeqLen sl = sequence_length_of(sa.len0, a.err, a.len_att, b, a.T_cap, a.k_new != nullptr,
                                         s == 0 && g == 0 && hg == 0 && threadIdx.x == 0);
    const int len = sl.len;
    const int n_seq_tiles = (len + TT - 1) / TT;
    if (s >= n_seq_tiles) return;  // whole workgroup, before any barrier
    const int n_tiles = (n_seq_tiles - s + a.S - 1) / a.S;  // tiles of this split
    const int tstride = a.S * TT;
    const int t_first = s * TT;
    const int last_block = (len - 1) & ~15;  // first token of the sequence's last 16-token block

    const int wave = wave_index();
    const int lane = threadIdx.x & 63;
    const int c = lane & 15, gq = lane >> 4;

    // Fused append (one new token; k_new/v_new set): the split owning the
    // token's tile quantizes its K and V rows into the cache slot before any
    // load of that tile -- waves 0 and 1 write them, and the barrier (a
    // workgroup-scope release and acquire) makes the stores visible to every
    // wave's loads.  Every head group of that split writes the same bytes; no
    // other workgroup reads the slot in this launch.
    if (sl.appended && s == (sl.slot / TT) % a.S) {
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

    const int mg = min(a.M - hg * ROWS, ROWS);  // rows of the group
    // Tokens the lane's query row of each block attends: all `len`, except
    // in a step with several new tokens, where the earlier ones see fewer;
    // tiles reaching past the smallest such limit are masked per row.
    int lim[R];
#pragma unroll
    for (int rb = 0; rb < R; ++rb) lim[rb] = row_limit(len, hg * ROWS + min(16 * rb + c, mg - 1), a.T_q, a.n_new, b);
    const int mask_from = a.T_q == 1 ? len : len - a.T_q + 1;

    // Rows are counted from kb/vb (codes) and ke/ve (exponents, one byte per
    // row): the (b, g) slab of a contiguous cache, or the page pools.
    const size_t slab = PAGED ? 0 : kv_row_contiguous(b, g, a.Hkv, a.T_cap, 0);
    const char* kb = static_cast<const char*>(a.k_cache) + slab * ROWB;
    const char* vb = static_cast<const char*>(a.v_cache) + slab * ROWB;
    const char* ke = reinterpret_cast<const char*>(a.k_exp) + slab;
    const char* ve = reinterpret_cast<const char*>(a.v_exp) + slab;
    // This wave's 16-token block of tile k starts at block_t(k); a block
    // wholly past the sequence's end re-reads its last block (zero weights),
    // and rows past the end re-read the last row, so every code read is a
    // written one.  Paged: 16 consecutive tokens lie in one page (pages hold
    // a power of two >= 32 tokens); the wave fetches the page of its next
    // block while issuing the current one, through the constant address
    // space as in the other kernels, and range-checks it when used (outside
    // the pool: page 0, flagged).
    auto block_t = [&](int k) { return min(t_first + k * tstride + 16 * wave, last_block); };
    typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
    const const_i32_ptr bt_row = PAGED ? (const_i32_ptr)(a.kv.block_table + (size_t)b * a.kv.max_pages) : nullptr;
    int next_entry = 0;
    if constexpr (PAGED) next_entry = bt_row[block_t(0) >> a.kv.page_shift];
    auto block_row = [&](int k, int tb) -> size_t {  // called for k = 0, 1, ... in order
        if constexpr (!PAGED) {
            return (size_t)tb;
        } else {
            int page = next_entry;
            if (k + 1 < n_tiles) next_entry = bt_row[block_t(k + 1) >> a.kv.page_shift];
            if ((unsigned)page >= (unsigned)a.kv.num_pages) {
                if (lane == 0) atomicOr(a.err, ERRBIT_PAGE);
                page = 0;
            }
            return kv_row_paged(a.kv, page, g, a.Hkv, tb);
        }
    };

    // Queries of every row block: B operands of the score product.  Lanes
    // past the group's last row load a copy of it (never stored).
    u32x4_t qop[R][KS];
#pragma unroll
    for (int rb = 0; rb < R; ++rb) {
        const int r = min(16 * rb + c, mg - 1);
        const uint16_t* qrow =
            static_cast<const uint16_t*>(a.q) + ((size_t)b * a.Hq + (size_t)g * a.M + hg * ROWS + r) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qop[rb][ks] = *reinterpret_cast<const u32x4_t*>(qrow + 32 * ks + 8 * gq);
    }

    // Direct loads of the wave's 16 rows: load n puts lane l's 16 bytes at
    // chunk n*64 + l of the wave's rows, i.e. row t = (n*64 + l) / CH,
    // position p = (n*64 + l) % CH, which holds the row's chunk p ^ (t & SWZ)
    // for K and p ^ vkey for V (vkey: the row's 8-token group within the
    // tile, times VKEY).
    uint32_t kgo[NKV], vgo[NKV];
    int lrow[NKV];
#pragma unroll
    for (int n = 0; n < NKV; ++n) {
        const int j = n * 64 + lane;
        const int t = j / CH, p = j % CH;
        const int vkey = (((16 * wave + t) >> 3) & 3) * VKEY;
        lrow[n] = t;
        kgo[n] = (uint32_t)(t * ROWB + 16 * (p ^ (t & SWZ)));
        vgo[n] = (uint32_t)(t * ROWB + 16 * (p ^ vkey));
    }
    // Non-temporal K/V loads (each byte is read once), except where several
    // row groups read the same tiles through L2.
    constexpr int KV_POLICY = GROUPED ? 0 : 2;
    size_t v_row = 0;  // first row of the block whose V rows are issued next
    int v_last = 15;   // its last row inside the sequence
    // K rows and exponents of tile k (slot k % NS); remembers the block for
    // issue_v(k).  Past the split's last tile: the same count of loads, all
    // of one cached chunk (never read), keeps the waits' arithmetic fixed.
    auto issue_kx = [&](int k) {
        unsigned char* slot = lds + (k % NS) * SLOT;
        unsigned char* kd = slot + 16 * wave * ROWB;
        unsigned char* xd = slot + 2 * REGION + 256 * wave;
        if (k >= n_tiles) {
#pragma unroll
            for (int n = 0; n < NKV; ++n)
                __builtin_amdgcn_global_load_lds((const void*)kb, (lds_void_t*)(kd + n * 1024), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const void*)ke, (lds_void_t*)xd, 4, 0, 0);
            return;
        }
        const int tb = block_t(k);
        const size_t r0 = block_row(k, tb);
        const int last = min(15, len - 1 - tb);
        v_row = r0;
        v_last = last;
        const char* kt = kb + r0 * ROWB;
        if (last == 15) {  // (uniform) a whole block: a scalar base and fixed lane offsets
#pragma unroll
            for (int n = 0; n < NKV; ++n)
                __builtin_amdgcn_global_load_lds((const void*)(kt + kgo[n]), (lds_void_t*)(kd + n * 1024), 16, 0,
                                                 KV_POLICY);
        } else {
#pragma unroll
            for (int n = 0; n < NKV; ++n)
                __builtin_amdgcn_global_load_lds((const void*)(kt + kgo[n] + (min(lrow[n], last) - lrow[n]) * ROWB),
                                                 (lds_void_t*)(kd + n * 1024), 16, 0, KV_POLICY);
        }
        // lane l, q = l & 7: K exponents of rows 4q .. 4q+3 for q < 4, else V
        // exponents of rows 4(q-4) ..; lanes 8-63 repeat them.  Bytes 0-15
        // are K, 16-31 V; those of rows past the sequence's end are never
        // used (the 16 rows lie inside the cache row or page).
        const int q = lane & 7;
        __builtin_amdgcn_global_load_lds((const void*)((q < 4 ? ke : ve) + r0 + 4 * (q & 3)), (lds_void_t*)xd, 4, 0,
                                         0);
    };
    auto issue_v = [&](int k) {
        unsigned char* vd = lds + (k % NS) * SLOT + REGION + 16 * wave * ROWB;
        if (k >= n_tiles) {
#pragma unroll
            for (int n = 0; n < NKV; ++n)
                __builtin_amdgcn_global_load_lds((const void*)kb, (lds_void_t*)(vd + n * 1024), 16, 0, 0);
            return;
        }
        const char* vt = vb + v_row * ROWB;
        if (v_last == 15) {
#pragma unroll
            for (int n = 0; n < NKV; ++n)
                __builtin_amdgcn_global_load_lds((const void*)(vt + vgo[n]), (lds_void_t*)(vd + n * 1024), 16, 0,
                                                 KV_POLICY);
        } else {
#pragma unroll
            for (int n = 0; n < NKV; ++n)
                __builtin_amdgcn_global_load_lds((const void*)(vt + vgo[n] + (min(lrow[n], v_last) - lrow[n]) * ROWB),
                                                 (lds_void_t*)(vd + n * 1024), 16, 0, KV_POLICY);
        }
    };

    // LDS read offsets.  Score operand: K row 16*wave + c, values 32ks + 8gq
    // .. +7 (half of a swizzled chunk of codes).
    // Value operand: V rows 8gq + j (+32 for the second half of the tile),
    // columns vcol .. vcol+NC-1.
    uint32_t koff[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int p = 2 * ks + (gq >> 1);
        koff[ks] = (uint32_t)(16 * wave * ROWB + (c * CH + (p ^ (c & SWZ))) * 16 + 8 * (gq & 1));
    }
    const int vcol = wave * DQ + NC * c;
    const int vbyte = vcol;
    const uint32_t voff = (uint32_t)(REGION + 8 * gq * ROWB + (((vbyte >> 4) ^ (gq * VKEY)) << 4) + (vbyte & 15));

    f32x4_t acc[R][NC];
    float m_ref[R], l_run[R];
#pragma unroll
    for (int rb = 0; rb < R; ++rb) {
#pragma unroll
        for (int e = 0; e < NC; ++e) acc[rb][e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        m_ref[rb] = a.m_init;  // -inf, or the unified maximum
        l_run[rb] = 0.f;
    }

#pragma unroll
    for (int k = 0; k < NS - 1; ++k) {
        issue_kx(k);
        issue_v(k);
    }
    for (int it = 0; it < n_tiles; ++it) {
        const unsigned char* slot = lds + (it % NS) * SLOT;
        unsigned char* Pb = lds + P_AT + (it & 1) * PBUF;
        float* Mb = reinterpret_cast<float*>(lds + M_AT + (it & 1) * MBUF);
        const signed char* X = reinterpret_cast<const signed char*>(slot + 2 * REGION + 256 * wave);
        // K rows and exponents of tile it+NS-1 into the slot tile it-1 used
        // (its reads by this wave have returned)
        issue_kx(it + NS - 1);
        // this wave's K rows and exponents of tile it have landed; in flight
        // may remain its V rows, then the loads of tiles it+1 .. it+NS-2 and
        // the K rows and exponents of tile it+NS-1
        wait_vm<(NS - 1) * PERT>();

        // scores of the wave's 16 tokens for every row block: each K row
        // read and widened once, with its own 2^e (a row past the
        // sequence's end holds the last row's codes and takes its 2^e too)
        const float sk = pow2_scale(X[min(c, len - 1 - block_t(it))]);
        f32x4_t sc[R];
#pragma unroll
        for (int rb = 0; rb < R; ++rb) sc[rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4_t kop = widen8(*reinterpret_cast<const u32x2_t*>(slot + koff[ks]), sk);
#pragma unroll
            for (int rb = 0; rb < R; ++rb) sc[rb] = mfma16x16x32(kop, qop[rb][ks], sc[rb]);
        }
        // lane (c, gq) holds row 16rb + c, tokens tw .. tw+3; x are the
        // unscaled products q.k (the scale is positive, so the row maximum
        // of x times the scale is the maximum of the scaled logits)
        const int t0 = t_first + it * tstride;
        const int tw = t0 + 16 * wave + 4 * gq;
        const float sl = a.scale_log2e;
        float x[R][4], mx[R];
#pragma unroll
        for (int rb = 0; rb < R; ++rb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) x[rb][i] = sc[rb][i];
            if (t0 + TT > mask_from) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (tw + i >= lim[rb]) x[rb][i] = -INFINITY;
            }
            mx[rb] = max_over_row_groups(fmaxf(fmaxf(x[rb][0], x[rb][1]), fmaxf(x[rb][2], x[rb][3]))) * sl;
        }
        // Weights under the current references into this tile's buffer:
        // 2^(x * scale - m) summed as they are, times the token's 2^e for the
        // value product.  A row with no token yet keeps m_ref = -inf and
        // weighs 0.
        const uint32_t xv = *reinterpret_cast<const uint32_t*>(X + 16 + 4 * gq);
        float lt[R];
        // weight row r holds its 16-byte chunk h at position h ^ ((r >> 1) & 7):
        // lane (c, gq) writes tokens 16*wave + 4gq .. +3 (half a chunk)
        const int pkey = (c >> 1) & 7;
        const int pw_off = (((2 * wave + (gq >> 1)) ^ pkey) << 4) + 8 * (gq & 1);
        auto put_weights = [&]() {
#pragma unroll
            for (int rb = 0; rb < R; ++rb) {
                const float m_sub = m_ref[rb] == -INFINITY ? 0.f : m_ref[rb];
                float p[4];
                float sum = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[rb][i], sl, -m_sub));
                    sum += p[i];
                    p[i] *= pow2_scale((int)(signed char)(xv >> (8 * i)));
                }
                lt[rb] = sum;
                const u32x2_t w = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
                *reinterpret_cast<u32x2_t*>(Pb + (16 * rb + c) * PST + pw_off) = w;
            }
        };
        put_weights();
        if (gq == 0) {
#pragma unroll
            for (int rb = 0; rb < R; ++rb) Mb[(16 * rb + c) * 4 + wave] = mx[rb];
        }
        // this wave's V rows of tile it have landed (later tiles' loads may
        // still be in flight); after the barrier every wave's V rows,
        // weights and maxima of tile it are visible, and every wave is past
        // its value product of tile it-1, whose V slot is refilled
        wait_vm_barrier<(NS - 2) * PERT + KX>();
        issue_v(it + NS - 1);

        // tile maxima per row, the same in every wave
        float tm[R];
        bool move = false;
#pragma unroll
        for (int rb = 0; rb < R; ++rb) {
            const f32x4_t v = *reinterpret_cast<const f32x4_t*>(Mb + (16 * rb + c) * 4);
            tm[rb] = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
            // past the headroom; on the first tile also a unified maximum
            // far above every score
            move = move || tm[rb] > m_ref[rb] + TAU || (it == 0 && tm[rb] < m_ref[rb] - TAU);
        }
        if (wave_any(move)) {
            // every wave takes this branch (same maxima, same references)
#pragma unroll
            for (int rb = 0; rb < R; ++rb) {
                const bool low = it == 0 && tm[rb] < m_ref[rb] - TAU;
                if (wave_any(tm[rb] > m_ref[rb] + TAU || low)) {
                    const float m_new = tm[rb] > m_ref[rb] + TAU || low ? tm[rb] : m_ref[rb];
                    // (nothing is accumulated before the first tile; a row
                    // with no token yet keeps m_ref = m_new = -inf: factor 1)
                    const float alpha =
                        it == 0 || m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_ref[rb] - m_new);
                    l_run[rb] *= alpha;
                    m_ref[rb] = m_new;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float ai = __shfl(alpha, 4 * gq + i);
#pragma unroll
                        for (int e = 0; e < NC; ++e) acc[rb][e][i] *= ai;
                    }
                }
            }
            put_weights();
            lds_barrier();
        }
#pragma unroll
        for (int rb = 0; rb < R; ++rb) l_run[rb] += lt[rb];

        // values: the 64 tokens' weights of every row times this wave's
        // columns of the V rows, each value read (and widened) once for all
        // row blocks.  A lane holds NC values (its columns) of each of tokens
        // 8gq + j; byte permutes pair tokens 2m and 2m+1 column by column
        // before widening, so each widened dword is dword m of one column
        // block's operand.
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            u32x4_t vop[NC];
            uint32_t w[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const unsigned char* vp = slot + voff + (32 * h + j) * ROWB;
                w[j] = NC == 4 ? *reinterpret_cast<const uint32_t*>(vp) : (uint32_t)*reinterpret_cast<const uint16_t*>(vp);
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const uint32_t c01 = __builtin_amdgcn_perm(w[2 * m + 1], w[2 * m], 0x05010400u);
                vop[0][m] = widen2<false>(c01, 1.0f);
                vop[1][m] = widen2<true>(c01, 1.0f);
                if constexpr (NC == 4) {
                    const uint32_t c23 = __builtin_amdgcn_perm(w[2 * m + 1], w[2 * m], 0x07030602u);
                    vop[2][m] = widen2<false>(c23, 1.0f);
                    vop[3][m] = widen2<true>(c23, 1.0f);
                }
            }
            u32x4_t pop[R];
#pragma unroll
            for (int rb = 0; rb < R; ++rb)
                pop[rb] = *reinterpret_cast<const u32x4_t*>(Pb + (16 * rb + c) * PST + (((4 * h + gq) ^ pkey) << 4));
#pragma unroll
            for (int e = 0; e < NC; ++e) {
#pragma unroll
                for (int rb = 0; rb < R; ++rb) acc[rb][e] = mfma16x16x32(pop[rb], vop[e], acc[rb][e]);
            }
        }
    }

    // The loads past the last tile (never read) have landed.  Sums of the
    // four waves per row meet in the maxima buffer no wave reads any more.
    wait_vm<0>();
    float* Lb = reinterpret_cast<float*>(lds + M_AT + (n_tiles & 1) * MBUF);
#pragma unroll
    for (int rb = 0; rb < R; ++rb) {
        float l = l_run[rb];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        if (gq == 0) Lb[(16 * rb + c) * 4 + wave] = l;
    }
    __syncthreads();
    // normalise and store this wave's columns (a row with no token in the
    // split: partial 0, log-sum-exp -inf)
    const size_t row0 = ((size_t)b * a.Hq + (size_t)g * a.M + hg * ROWS) * a.S + s;
#pragma unroll
    for (int rb = 0; rb < R; ++rb) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(Lb + (16 * rb + c) * 4);
        const float l = (v[0] + v[1]) + (v[2] + v[3]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * rb + 4 * gq + i;
            const float li = __shfl(l, 4 * gq + i);
            if (r < mg) {
                const float inv = li > 0.f ? 1.f / li : 0.f;
                uint16_t* o = static_cast<uint16_t*>(a.o_part) + (row0 + (size_t)r * a.S) * D + vcol;
                if constexpr (NC == 4) {
                    const u32x2_t w = {pack_bf16x2(acc[rb][0][i] * inv, acc[rb][1][i] * inv),
                                       pack_bf16x2(acc[rb][2][i] * inv, acc[rb][3][i] * inv)};
                    *reinterpret_cast<u32x2_t*>(o) = w;
                } else {
                    *reinterpret_cast<uint32_t*>(o) = pack_bf16x2(acc[rb][0][i] * inv, acc[rb][1][i] * inv);
                }
            }
        }
        if (wave == 0 && gq == 0 && 16 * rb + c < mg)
            a.lse_part[row0 + (size_t)(16 * rb + c) * a.S] = l > 0.f ? m_ref[rb] + __builtin_log2f(l) : -INFINITY;
    }
}

template <int D, int R, int NS, bool GROUPED, bool PAGED>
void launch_one(const PartialArgs& a, int groups, const Launch& on) {
    const dim3 grid(lds_grid_blocks(a.S, groups, a.Hkv, a.B)), block(256);
    KVD_LAUNCH((partial_xchg_fp8_kernel<D, R, NS, GROUPED, PAGED>), grid, block, 0, on, a, groups);
}

template <int D, int R>
hipError_t launch_r(const PartialArgs& a, int groups, const Launch& on) {
    constexpr int NS = xchg_slots(D);
    const bool paged = a.kv.block_table != nullptr;
    if (groups == 1) {
        if (paged)
            launch_one<D, R, NS, false, true>(a, 1, on);
        else
            launch_one<D, R, NS, false, false>(a, 1, on);
    } else {
        if (paged)
            launch_one<D, R, NS, true, true>(a, groups, on);
        else
            launch_one<D, R, NS, true, false>(a, groups, on);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_partial_xchg(const PartialArgs& a, const Launch& on) {
    const XchgShape x = xchg_shape(a.D, a.M);
    if (a.D == 256) {
        switch (x.row_blocks) {
            case 1: return launch_r<256, 1>(a, x.groups, on);
            case 2: return launch_r<256, 2>(a, x.groups, on);
            default: return launch_r<256, 3>(a, x.groups, on);
        }
    }
    if (a.D == 128) {
        switch (x.row_blocks) {
            case 1: return launch_r<128, 1>(a, x.groups, on);
            case 2: return launch_r<128, 2>(a, x.groups, on);
            case 3: return launch_r<128, 3>(a, x.groups, on);
            default: return launch_r<128, 4>(a, x.groups, on);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace kvd
