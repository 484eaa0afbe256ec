// kvd_internal.h -- launchers and shared constants of the decode-attention
// library (internal; the public ABI is include/kvdecode.h).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvd {

// Sticky device error bits, OR-ed into the handle's flag word.
constexpr int ERRBIT_CAPACITY = 1;  // an append found no room in a cache (its length in [0, T_cap])
constexpr int ERRBIT_LENGTH = 2;    // a kernel saw lengths[b] outside [0, T_cap]
constexpr int ERRBIT_PAGE = 4;      // a block-table entry in use was outside [0, num_pages)

// Where the cache rows live.  Contiguous (block_table == nullptr): token t of
// (sequence b, KV head g) is row (b * Hkv + g) * T_cap + t of k_cache/v_cache.
// Paged: the caches are a pool of pages [num_pages, Hkv, page, d] and token t
// is row (block_table[b * max_pages + t / page] * Hkv + g) * page + t % page,
// page = 2^page_shift >= 32 tokens, so a 32-token tile (and each 16-token
// block of the fp8 exchange kernel's 64-token tiles) never straddles pages.
struct KvLayout {
    const int32_t* block_table;
    int page_shift;
    int max_pages;
    int num_pages;
};

// Page of block j of sequence b; an entry outside the pool is replaced by
// page 0 (a valid address) and flagged.
__device__ __forceinline__ int kv_page(const KvLayout& L, int b, int j, int* err) {
    int p = L.block_table[(size_t)b * L.max_pages + j];
    if ((unsigned)p >= (unsigned)L.num_pages) {
        atomicOr(err, ERRBIT_PAGE);
        p = 0;
    }
    return p;
}

// Row of token t of (b, g): contiguous, or paged given the token's page.
__device__ __forceinline__ size_t kv_row_contiguous(int b, int g, int Hkv, int T_cap, int t) {
    return ((size_t)b * Hkv + g) * (size_t)T_cap + t;
}
__device__ __forceinline__ size_t kv_row_paged(const KvLayout& L, int page, int g, int Hkv, int t) {
    return (((size_t)page * Hkv + g) << L.page_shift) + (t & ((1 << L.page_shift) - 1));
}

// Tokens per inner iteration of each partial-pass kernel.
constexpr int MFMA_TILE = 32;
constexpr int VALU_TILE = 64;
// Waves per workgroup of the vector-ALU kernel; each takes every
// VALU_WAVES-th tile of the workgroup's split.
constexpr int VALU_WAVES = 4;

// Query heads per MFMA head block (rows of the 16x16 output tile).
constexpr int MFMA_HEADS = 16;

// log2(e): softmax is evaluated as 2^(x*log2(e) - m) with the score scale
// folded into one fp32 multiplier.
constexpr float LOG2E = 1.4426950408889634f;

struct PartialArgs {
    const void* q;          // [B, Hq, D]
    const void* k_cache;    // [B, Hkv, T_cap, D]
    const void* v_cache;    // [B, Hkv, T_cap, D]
    const int32_t* lengths; // [B]
    // [B, Hq, S, D] normalised partial outputs, in the output's precision:
    // bf16 (rounded to nearest even) when the output is bf16, else fp32
    void* o_part;
    float* lse_part;        // [B, Hq, S]    base-2 log-sum-exp of each split
    int* err;               // sticky error word
    int* len_att;           // [B] attended length of each sequence, for the combine
    // Fused append (null otherwise): the new token's K/V, [B, Hkv, D].  Slot
    // lengths[b] of the cache receives them and the pass attends
    // lengths[b] + 1 tokens; lengths itself is advanced by the combine (or,
    // in a one-split pass, by the pass: see lengths_adv below).
    const void* k_new;
    const void* v_new;
    KvLayout kv;            // contiguous or paged cache rows
    // fp8 cache only: power-of-two exponent of each key / value row,
    // [B, Hkv, T_cap] int8 (the row's values are code * 2^e).
    const int8_t* k_exp;
    const int8_t* v_exp;
    int B, Hq, Hkv, M, D, T_cap;
    int S;                  // splits per (sequence, KV head): split s owns the
                            // kernel's token tiles s, s+S, s+2S, ...
    float scale_log2e;      // scale * log2(e)
    int lds_config;         // LDS kernel: LDS_SHORT or LDS_LONG (see below)
    // Several new tokens per sequence: T_q query rows per head (q and the
    // partials hold Hq = heads * T_q rows, M = group heads * T_q, row
    // r = head * T_q + i), and n_new[b] rows appended by this step (null for
    // a one-token step).  Query i attends over the first
    // len - n_new[b] + min(i + 1, n_new[b]) tokens.
    int T_q;
    const int* n_new;
    // Softmax reference of the LDS kernels (base 2): the starting reference
    // (-inf, or a unified maximum given by the caller) and the headroom past
    // which it is raised (8; 64 with a unified maximum).
    float m_init;
    float tau;
    // LDS kernel: sequences in dispatch order, longest first, as the last
    // combine left them ([B] then a flag word, set once the order is valid;
    // see CombineArgs::order).  A hint only: any permutation gives the same
    // results.
    const int* order;
    // Single-split plans (LDS and VALU kernels; null: a combine follows):
    // the pass writes the output rows [B, Hq, D] itself, in the output's
    // precision, and no combine runs.  After a fused append the last
    // workgroup of a sequence to finish advances lengths_adv[b], counted on
    // seq_ctr[b] (zero between launches: the last arriver resets it).
    void* out;
    int32_t* lengths_adv;
    int* seq_ctr;
};

// Single-split plans: each of a sequence's per_seq workgroups calls this
// once (one lane), after its own read of lengths[b] has been used; the last
// to arrive sets lengths[b] = new_len.  Every read of the length in the
// launch precedes that arrival's counter update, so none sees the new
// value.
__device__ __forceinline__ void advance_when_last(int* ctr, int per_seq, int32_t* lengths, int b, int new_len) {
    if (per_seq == 1 || atomicAdd(ctr, 1) == per_seq - 1) {
        if (per_seq > 1) atomicExch(ctr, 0);
        lengths[b] = new_len;
    }
}

struct CombineArgs {
    int groups;             // split groups per row (set by the launcher)
    const void* o_part;     // bf16 when the output is bf16, else fp32
    const float* lse_part;
    const int* len_att;     // [B] attended lengths written by the partial pass
    int32_t* lengths;       // advanced here after a fused append (else untouched)
    int fused_append;
    void* out;              // [B, Hq, D]
    int B, Hq, D, T_cap;
    int tile;               // tokens per tile of the partial kernel that ran
    int S;
    // [B] + flag: one extra workgroup of the combine sorts the sequences by
    // this step's attended length, longest first, for the next partial pass
    // (which then starts the longest workgroups first).  Equal lengths clear
    // the flag (no order: the next pass keeps the batch's); so does a batch
    // above COMBINE_SORT_MAX sequences, never sorted.
    int* order;
};
constexpr int COMBINE_SORT_MAX = 2048;

// Token tiles of a sequence are dealt round-robin to its S splits: split s
// owns tiles s, s+S, s+2S, ...  At any moment the S workgroups of a
// sequence stream one contiguous window of its cache (good DRAM page
// locality, like a single sequential read), every split gets an equal share
// of full tiles, and only the split holding the sequence's last tile sees a
// partial one.  A sequence of n tokens has min(S, ceil(n / tile)) non-empty
// splits.
// Length bookkeeping shared by the partial kernels: reads lengths[b],
// reports out-of-range lengths and (for a fused append) a full cache, and
// returns the number of tokens to attend.  `appended` tells whether the
// fused append takes slot lengths[b].  The first block of the sequence also
// records the attended length for the combine.
struct SeqLen {
    int len;       // tokens attended
    int slot;      // slot of the appended token (when appended)
    bool appended;
};
__device__ __forceinline__ SeqLen sequence_length_of(int l0, int* err, int* len_att, int b, int T_cap, bool fused,
                                                     bool lead) {
    SeqLen r;
    r.slot = l0;
    r.appended = false;
    if (l0 < 0 || l0 > T_cap) {
        if (lead) atomicOr(err, ERRBIT_LENGTH);
        r.len = l0 < 0 ? 0 : T_cap;
    } else if (fused) {
        r.appended = l0 < T_cap;
        if (!r.appended && lead) atomicOr(err, ERRBIT_CAPACITY);
        r.len = r.appended ? l0 + 1 : l0;
    } else {
        r.len = l0;
    }
    if (lead) len_att[b] = r.len;
    return r;
}
__device__ __forceinline__ SeqLen sequence_length(const int32_t* lengths, int* err, int* len_att,
                                                  int b, int T_cap, bool fused, bool lead) {
    return sequence_length_of(lengths[b], err, len_att, b, T_cap, fused, lead);
}

// Tokens query row r attends to (see PartialArgs::T_q).
__device__ __forceinline__ int row_limit(int len, int r, int T_q, const int* n_new, int b) {
    if (T_q == 1 || n_new == nullptr) return len;
    const int a = n_new[b];
    const int i = r % T_q;
    return len - a + (i + 1 < a ? i + 1 : a);
}

__device__ __forceinline__ int splits_with_data(int len, int tile, int S) {
    const int nt = (len + tile - 1) / tile;
    return nt < S ? nt : S;
}

// Grids of the VALU and register-direct MFMA kernels are one-dimensional
// and split-major: block L = split * units + unit.  Consecutive blocks are
// dealt round-robin to the eight XCDs, so consecutive units of the same
// split land on different XCDs; with ragged lengths the always-active low
// splits are spread evenly and dispatched first, and the mostly-empty high
// splits come last.  (The LDS-staged kernels use lds_coord below.)
struct BlockCoord {
    int split, unit;
};
__device__ __forceinline__ BlockCoord block_coord(int units) {
    const int L = (int)blockIdx.x;
    BlockCoord c;
    c.split = L / units;
    c.unit = L - c.split * units;
    return c;
}

// The LDS-staged kernels' grids (bf16, and the three fp8 kernels) deal work
// units to the eight XCDs in turn (block L runs on XCD L mod 8) and, on each
// XCD, run them unit after unit, longest first: the k-th block of XCD x is
// head group k mod G of split (k / G) mod S of unit slot k / (G * S), i.e.
// unit = slot * 8 + x, with units numbered in dispatch order (sequence
// order[p] at position p once the combine has sorted the lengths).  Every
// split of a unit stays on one XCD, as in the split-major grid (which
// measured 8% faster at long context than splits spread over the XCDs), its
// head groups are dispatched one after another (their loads of the same
// tiles meet in that XCD's L2), and the longest workgroups start first
// (ragged GQA: 333 us against 366 us).  Blocks of padding slots past the
// last unit exit at once.
struct LdsCoord {
    int split, hg, p, g;  // p: dispatch position of the sequence
    bool live;
};
__device__ __forceinline__ LdsCoord lds_coord(int S, int groups, int Hkv, int B) {
    const int L = (int)blockIdx.x;
    const int k = L >> 3;
    LdsCoord c;
    c.hg = k % groups;
    const int k2 = k / groups;
    c.split = k2 % S;
    const int unit = (k2 / S) * 8 + (L & 7);
    c.live = unit < B * Hkv;
    c.g = unit % Hkv;
    c.p = c.live ? unit / Hkv : 0;
    return c;
}
// Sequence at dispatch position p and its length word: order[p] when the
// order is valid (its length then loads after it), else p, whose length is
// requested together with the order words, so a batch the combine left
// unsorted pays no extra memory round trip.
struct SeqAt {
    int b, len0;
};
__device__ __forceinline__ SeqAt seq_at(int p, int B, const int* order, const int32_t* lengths) {
    const int flag = order != nullptr ? order[B] : 0;
    const int o = order != nullptr ? order[p] : p;
    const int len_p = lengths[p];
    SeqAt r;
    if (flag == 1) {
        r.b = o < 0 ? 0 : (o >= B ? B - 1 : o);  // memory-safe whatever the hint holds
        r.len0 = lengths[r.b];
    } else {
        r.b = p;
        r.len0 = len_p;
    }
    return r;
}
// blocks of the LDS kernel's grid: units padded to whole rounds of the XCDs
inline unsigned lds_grid_blocks(int S, int groups, int Hkv, int B) {
    return (unsigned)(((long long)B * Hkv + 7) / 8 * 8 * S * groups);
}

// Where a launcher puts its kernel: the stream and, optionally, events that
// the dispatch itself stamps with the kernel's start and end times (HIP's
// extended launch).  A timed launch then adds no command to the stream, and
// the events bracket the kernel alone, as a kernel trace does.
struct Launch {
    hipStream_t stream;
    hipEvent_t start, stop;
    Launch(hipStream_t s, hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr) : stream(s), start(t0), stop(t1) {}
};
#define KVD_LAUNCH(kernel, grid, block, shmem, on, ...)                                                        \
    do {                                                                                                     \
        if ((on).start || (on).stop)                                                                         \
            hipExtLaunchKernelGGL(kernel, grid, block, shmem, (on).stream, (on).start, (on).stop, 0u, __VA_ARGS__); \
        else                                                                                                 \
            hipLaunchKernelGGL(kernel, grid, block, shmem, (on).stream, __VA_ARGS__);                        \
    } while (0)

// Each launcher returns the hipError_t of its launch.
// Append T_q >= 1 new rows per (sequence, KV head) at slots lengths[b] ..
// lengths[b] + T_q - 1 (k_new/v_new [B, Hkv, T_q, D]); a sequence they do
// not fit is left unchanged and flagged.  n_new (may be null) receives the
// rows appended per sequence.
hipError_t launch_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                         const KvLayout& kv, int32_t* lengths, int* err, int* n_new, int B, int Hkv,
                         int D, int T_cap, int T_q, int elem_bytes, const Launch& on);
hipError_t launch_partial_valu(const PartialArgs& a, bool bf16, const Launch& on);
hipError_t launch_partial_mfma(const PartialArgs& a, const Launch& on);
hipError_t launch_partial_lds(const PartialArgs& a, const Launch& on);

// Configurations of the LDS-staged kernel: ring depth (stages of K and V of
// 32 tokens, 128*D bytes each) and how many of the split's tiles the V loads
// trail the K loads.  LDS_SHORT is the one for d = 64 and 128 and for d = 256
// when each split streams few tiles: one workgroup per CU at d = 256, whose
// deeper ring keeps the per-workgroup fixed costs (pipeline fill, queries,
// output) few.  LDS_LONG (d = 256 only) fits two workgroups per CU, which
// hide each other's compute and barrier waits on long splits.
enum { LDS_SHORT = 0, LDS_LONG = 1 };
struct LdsConfig {
    int stages, v_lag;
};
constexpr LdsConfig lds_config(int D, int which) {
    return D == 64 ? LdsConfig{6, 0}
         : D == 128 ? LdsConfig{3, 0}
         : which == LDS_LONG ? LdsConfig{2, 1} : LdsConfig{3, 0};
}
// The planner takes LDS_LONG at d = 256 when every split then holds at least
// this many tiles of a full cache.
constexpr int LDS_LONG_MIN_TILES = 24;
constexpr int LDS_BYTES_PER_CU = 160 * 1024;
// Workgroups of the LDS-staged kernel resident per CU: the ring must fit the
// CU's 160 KB of LDS.
inline int lds_groups_per_cu(int D, int which) {
    const int g = LDS_BYTES_PER_CU / (lds_config(D, which).stages * 128 * D);
    return g < 1 ? 1 : (g > 8 ? 8 : g);
}
hipError_t launch_combine(const CombineArgs& a, bool bf16, const Launch& on);

// fp8 (OCP E4M3 codes with a power-of-two exponent per row) cache.
// Ring depth of the fp8 LDS kernel; a stage holds K and V codes of 32
// tokens (64*D bytes) and their exponents (a 1 KB block).
constexpr int lds_fp8_stages(int D) { return D == 64 ? 6 : 4; }
inline int lds_fp8_groups_per_cu(int D) {
    const int g = LDS_BYTES_PER_CU / (lds_fp8_stages(D) * (64 * D + 1024));
    return g < 1 ? 1 : (g > 8 ? 8 : g);
}
hipError_t launch_partial_lds_fp8(const PartialArgs& a, const Launch& on);

// fp8 cache, kernel in which each wave streams its own tiles for all rows of
// a group (kvd_partial_wave_fp8.hip): 16-row blocks per group (each wave
// holds the whole group's accumulators and queries in its 256 registers: one
// block at d = 256, three at d = 128) and ring stages per wave (a stage is
// one tile's K and V codes plus a 1 KB exponent block).
constexpr int wave_fp8_max_row_blocks(int D) { return D == 256 ? 1 : 3; }
inline int wave_fp8_row_blocks(int D, int M) {
    const int b = (M + 15) / 16;
    return b < wave_fp8_max_row_blocks(D) ? b : wave_fp8_max_row_blocks(D);
}
// Two stages per wave: at d = 256 four waves' rings take 136 KB of the CU's
// 160 KB; at d = 128 (72 KB) two workgroups fit per CU.
constexpr int wave_fp8_stages(int) { return 2; }
inline int wave_fp8_groups_per_cu(int D) {
    const int g = LDS_BYTES_PER_CU / (4 * wave_fp8_stages(D) * (64 * D + 1024));
    return g < 1 ? 1 : (g > 8 ? 8 : g);
}
hipError_t launch_partial_wave_fp8(const PartialArgs& a, const Launch& on);
// fp8 kernel for large query groups in which the four waves split every
// 64-token tile by tokens for the scores and by value columns for the
// output, exchanging the weights through LDS (kvd_partial_xchg.hip).  A
// workgroup holds up to xchg_max_row_blocks(D) blocks of 16 query rows
// (queries and accumulators in registers: three at d = 256, four at
// d = 128); larger groups take several workgroups of equal row blocks.
constexpr int XCHG_TILE = 64;
constexpr int xchg_max_row_blocks(int D) { return D == 256 ? 3 : 4; }
struct XchgShape {
    int row_blocks, groups;
};
inline XchgShape xchg_shape(int D, int rows) {
    const int blocks = (rows + 15) / 16;
    const int mx = xchg_max_row_blocks(D);
    const int groups = (blocks + mx - 1) / mx;
    return XchgShape{(blocks + groups - 1) / groups, groups};
}
// Ring slots (one 64-token tile's K and V codes and exponents, each).  Two
// slots keep two workgroups per CU at d = 256; four slots with one
// workgroup per CU measured slower (long context 80 against 67 us).
constexpr int xchg_slots(int) { return 2; }
// LDS of one workgroup: the slots, two weight buffers (16 * R rows of 64
// bf16) and two buffers of row maxima (16 * R rows of 4 floats).
constexpr int xchg_lds_bytes(int D, int row_blocks) {
    return xchg_slots(D) * (2 * XCHG_TILE * D + 1024) + 2 * 16 * row_blocks * (2 * XCHG_TILE + 16);
}
// Workgroups per CU: at most two (the kernel keeps to 256 registers per
// lane), fewer where the LDS of two would exceed the CU's 160 KB.
inline int xchg_groups_per_cu(int D, int rows) {
    const int g = LDS_BYTES_PER_CU / xchg_lds_bytes(D, xchg_shape(D, rows).row_blocks);
    return g < 1 ? 1 : (g > 2 ? 2 : g);
}
hipError_t launch_partial_xchg(const PartialArgs& a, const Launch& on);
// Quantize T_q >= 1 new bf16 K/V rows per (sequence, KV head)
// (k_new/v_new [B, Hkv, T_q, D]) into slots lengths[b] .. lengths[b] + T_q - 1
// (contiguous or paged, the exponent at the row's index) and advance
// lengths; a sequence they do not fit is left unchanged and flagged.  n_new
// (may be null) receives the rows appended per sequence.
hipError_t launch_append_fp8(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                             int8_t* k_exp, int8_t* v_exp, const KvLayout& kv, int32_t* lengths, int* err,
                             int* n_new, int B, int Hkv, int D, int T_cap, int T_q, const Launch& on);


// Waves per work unit of the MFMA partial pass for group size M.
inline int mfma_head_blocks(int M) { return (M + MFMA_HEADS - 1) / MFMA_HEADS; }

}  // namespace kvd
