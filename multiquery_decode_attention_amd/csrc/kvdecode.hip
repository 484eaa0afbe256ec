// kvdecode.hip -- host side of the C ABI declared in include/kvdecode.h:
// handle lifetime, argument validation, split planning, workspace and
// kernel launches.  No torch types cross this boundary.
#include "../../include/kvdecode.h"

#include <math.h>
#include <stdlib.h>

#include <mutex>
#include <new>
#include <unordered_set>
#include <vector>

#include "kvd_internal.h"

struct kvdecode_s {
    kvdecode_desc_t d;          // for a paged cache: the pools, and capacity = max_pages * page_size
    kvd::KvLayout kv{nullptr, 0, 0, 0};
    // fp8 cache (d.dtype == KVD_FP8_E4M3): per-row power-of-two exponents
    int8_t* k_exp = nullptr;
    int8_t* v_exp = nullptr;
    int M = 1;
    int elem = 4;
    int variant_req = KVD_VARIANT_AUTO;
    int forced_splits = 0;
    // Plans of steps with 1..KVD_MAX_NEW_TOKENS new tokens, made on first use
    // (cleared when the variant or the forced split count changes).
    struct CachedPlan {
        bool valid;
        int variant, tile, splits, chunk, lds_config;
    } plans[KVD_MAX_NEW_TOKENS + 1] = {};
    bool unified = false;     // unified softmax maximum (LDS kernels)
    float unified_max = 0.f;  // in units of scale * q.k

    // Device resources (allocated on first use, on the then-current device).
    int device = -1;
    int* err = nullptr;
    int noalloc_device = -1;   // device of this handle's allocation-free steps (scratch error word)
    void* o_part = nullptr;    // partials: bf16 for bf16 outputs, else fp32
    float* lse_part = nullptr;
    int ws_splits = 0;

    // Event timing.
    int timing_cap = 0;
    int timing_what = 0;                // KVD_TIME_* bits
    // Events stamped by the timed launches themselves: per timed attend the
    // partial pass's start and end, then the combine's; per timed append
    // the append kernel's.  comb_timed: whether attend i timed a combine
    // (a one-split pass launches none).
    std::vector<hipEvent_t> ev_attend;  // 4 per timed attend
    std::vector<hipEvent_t> ev_append;  // 2 per timed append
    std::vector<char> comb_timed;
    int n_attend = 0, n_append = 0;
};

namespace {

std::mutex g_mu;
std::unordered_set<kvdecode_s*>& live() {
    static std::unordered_set<kvdecode_s*> s;
    return s;
}

bool is_live(kvdecode_s* h) {
    std::lock_guard<std::mutex> lk(g_mu);
    return h && live().count(h);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Plan {
    int variant;
    int tile;    // tokens per tile of the chosen partial kernel
    int splits;  // S: split s owns tiles s, s+S, ... of each sequence
    int chunk;   // most tokens any split holds for a full cache
    int lds_config;  // kvd::LDS_SHORT or kvd::LDS_LONG (LDS kernel)
};

bool is_fp8(const kvdecode_s* h) { return h->d.dtype == KVD_FP8_E4M3; }

// T_q: query rows per head of the step.
int resolve_variant(const kvdecode_s* h, int T_q = 1) {
    if (h->variant_req != KVD_VARIANT_AUTO) return h->variant_req;
    // fp8 at d >= 128: the wave kernel when one workgroup holds all query
    // rows of a KV head (MHA and small GQA groups: no barrier in its loop),
    // else the exchange kernel (each code widened once however many rows
    // share it); d = 64: the shared-tile kernel
    if (is_fp8(h)) {
        if (h->d.head_dim < 128) return KVD_VARIANT_LDS;
        return h->M * T_q <= 16 * kvd::wave_fp8_max_row_blocks(h->d.head_dim) ? KVD_VARIANT_WAVE
                                                                              : KVD_VARIANT_XCHG;
    }
    return h->d.dtype == KVD_BF16 ? KVD_VARIANT_LDS : KVD_VARIANT_VALU;
}

// Split planner.  The grid is splits x (sequences, KV heads [, head groups]);
// lengths live on the device, so the plan is made for full caches and splits
// with no tile of a sequence exit at once.  For every candidate split count
// S the cost model charges each round of resident workgroups
//   (bytes of the busiest split + a fixed fill cost) * max(sat, workgroups in the round)
// plus the partial traffic (written by the partial pass, read by the
// combine), charged at 4 bytes per value although bf16 outputs keep bf16
// partials: the fill constant was tuned with this charge.  Full rounds hold
// `slots` workgroups (all that fit on the GPU at once); the last round may
// hold fewer.  `sat` is how many resident workgroups of the kernel already
// stream the cache at the full HBM rate: a round with fewer is bound by the
// workgroups' own streaming rate (it costs as much as `sat` of them), one
// with more by HBM (it costs its bytes).  Among plans within 2% of the
// cheapest whose workgroups take more than one round, the one with most
// splits wins: there shorter splits balance ragged lengths and the last
// round better.  A plan whose workgroups all fit at once gains nothing from
// shorter splits, and the cheapest stands.  At d = 256 the LDS kernel has a second configuration
// with two workgroups per CU; it is planned first and taken when its splits
// stay long (kvd::LDS_LONG_MIN_TILES tiles of a full cache).
constexpr int CUS = 256;

struct Shape {
    long long units;      // workgroups per split
    long long slots;      // workgroups resident on the whole GPU
    long long sat;        // resident workgroups that saturate HBM (<= slots)
    int waves = 1;        // tiles of a split a workgroup streams at once
};

Shape shape_for(const kvdecode_s* h, int variant, int lds_which, int T_q) {
    const long long bkv = (long long)h->d.batch * h->d.num_kv_heads;
    const int rows = h->M * T_q;  // query rows per KV head
    const int D = h->d.head_dim;
    Shape sh;
    if (variant == KVD_VARIANT_WAVE) {
        const int rows_per_group = 16 * kvd::wave_fp8_max_row_blocks(D);
        sh.units = bkv * ((rows + rows_per_group - 1) / rows_per_group);
        sh.slots = (long long)CUS * kvd::wave_fp8_groups_per_cu(D);
    } else if (variant == KVD_VARIANT_XCHG) {
        sh.units = bkv * kvd::xchg_shape(D, rows).groups;
        sh.slots = (long long)CUS * kvd::xchg_groups_per_cu(D, rows);
    } else if (variant == KVD_VARIANT_LDS) {
        sh.units = bkv * ((rows + 63) / 64);
        sh.slots = (long long)CUS * (is_fp8(h) ? kvd::lds_fp8_groups_per_cu(D) : kvd::lds_groups_per_cu(D, lds_which));
    } else if (variant == KVD_VARIANT_MFMA) {
        const int hb = kvd::mfma_head_blocks(h->M);
        const int nw = hb < 4 ? hb : 4;
        sh.units = bkv * ((hb + nw - 1) / nw);
        const int waves_per_cu = D == 256 ? 4 : (D == 128 ? 8 : 16);
        sh.slots = (long long)CUS * (waves_per_cu / nw > 0 ? waves_per_cu / nw : 1);
    } else {
        // vector-ALU kernel: one workgroup of VALU_WAVES waves per query row
        sh.units = bkv * rows;
        sh.slots = (long long)CUS * 16 / kvd::VALU_WAVES;
        sh.waves = kvd::VALU_WAVES;
    }
    // Measured saturation point: the bf16 LDS kernel with two workgroups
    // per CU at d = 256 streams a long-context step as fast with 384
    // workgroups (1.5 per CU) as with 512.  Elsewhere every slot is taken
    // to be needed: the fp8 exchange kernel, for one, ran the same
    // long-context step 7 us slower on 256 workgroups than on 512.
    sh.sat = sh.slots;
    if (variant == KVD_VARIANT_LDS && !is_fp8(h) && D == 256 && lds_which == kvd::LDS_LONG) sh.sat = sh.slots * 3 / 4;
    return sh;
}

// Cost-model choice of the split count (at most s_max) for one kernel
// shape.  Only the smallest S of each busiest-split size ceil(n_tiles / S)
// is a candidate (a larger S with the same busiest split costs more), and
// those are enumerated directly: O(sqrt(n_tiles)) of them, twice (the
// cheapest cost, then the most splits of several rounds within 2% of it),
// with no heap memory.
long long plan_splits(const kvdecode_s* h, const Shape& sh, int tile, long long n_tiles, int T_q,
                      long long s_max) {
    const double tok_bytes = 2.0 * h->d.head_dim * h->elem + (is_fp8(h) ? 2 : 0);  // K+V of one token
    const double fill = 32.0 * 1024;                              // pipeline fill per split
    const double part_bytes = (double)h->M * T_q * (h->d.head_dim + 1) * 4 * 2;
    // the vector-ALU kernel's waves take a split's tiles VALU_WAVES at a time
    const int waves = sh.waves;
    auto cost_of = [&](long long s, long long per) {
        const long long w = sh.units * s;  // workgroups of the launch
        const long long full = w / sh.slots, rest = w - full * sh.slots;
        const double split_cost = (double)((per + waves - 1) / waves) * tile * tok_bytes + fill;
        return split_cost * ((double)full * sh.slots + (rest > 0 ? (double)(rest > sh.sat ? rest : sh.sat) : 0.0)) +
               (double)w * part_bytes;
    };
    // visit(s, cost) for every candidate, in increasing s
    auto each_candidate = [&](auto&& visit) {
        for (long long s = 1; s <= n_tiles && s <= s_max;) {
            const long long per = (n_tiles + s - 1) / s;  // tiles of the busiest split
            visit(s, cost_of(s, per));
            if (per == 1) break;
            s = (n_tiles + per - 2) / (per - 1);  // smallest S whose busiest split is smaller
        }
    };
    double best = 0;
    long long pick = 1;
    each_candidate([&](long long s, double cost) {
        if (best == 0 || cost < best) {
            best = cost;
            pick = s;
        }
    });
    each_candidate([&](long long s, double cost) {
        if (cost <= best * 1.02 && s > pick && sh.units * s > sh.slots) pick = s;
    });
    return pick;
}

// Grid of the partial-pass launch of a plan: workgroups per split and
// threads per workgroup, as the variant's launcher sizes them.  A launch's
// grid counts work-items in 32 bits per dimension, so blocks * threads must
// stay below 2^32.
struct GridShape {
    long long blocks_per_split;
    int threads;
};
GridShape partial_grid(const kvdecode_s* h, int variant, int T_q) {
    const long long bkv = (long long)h->d.batch * h->d.num_kv_heads;
    const long long padded = (bkv + 7) / 8 * 8;  // lds_grid_blocks: units padded to whole XCD rounds
    const int rows = h->M * T_q;
    const int D = h->d.head_dim;
    GridShape g{0, 256};
    if (variant == KVD_VARIANT_WAVE) {
        const int rb = kvd::wave_fp8_row_blocks(D, rows);
        g.blocks_per_split = padded * ((rows + 16 * rb - 1) / (16 * rb));
    } else if (variant == KVD_VARIANT_XCHG) {
        g.blocks_per_split = padded * kvd::xchg_shape(D, rows).groups;
    } else if (variant == KVD_VARIANT_LDS) {
        g.blocks_per_split = padded * ((rows + 63) / 64);
    } else if (variant == KVD_VARIANT_MFMA) {
        const int hb = kvd::mfma_head_blocks(h->M);
        const int nw = hb < 4 ? hb : 4;
        g.blocks_per_split = bkv * ((hb + nw - 1) / nw);
        g.threads = 64 * nw;
    } else {
        g.blocks_per_split = (long long)h->d.batch * h->d.num_q_heads * T_q;
        g.threads = 64 * kvd::VALU_WAVES;
    }
    return g;
}
constexpr long long GRID_ITEMS_MAX = 0xFFFFFFFFll;
// Most splits whose partial-pass grid fits (0: not even one).
long long max_splits_for_grid(const kvdecode_s* h, int variant, int T_q) {
    const GridShape g = partial_grid(h, variant, T_q);
    return GRID_ITEMS_MAX / ((long long)g.threads * g.blocks_per_split);
}

// T_q: query rows per head (new tokens per sequence in this step).
Plan compute_plan(const kvdecode_s* h, int T_q);
Plan make_plan(kvdecode_s* h, int T_q = 1) {
    auto& c = h->plans[T_q];
    if (!c.valid) {
        const Plan p = compute_plan(h, T_q);
        c = kvdecode_s::CachedPlan{true, p.variant, p.tile, p.splits, p.chunk, p.lds_config};
    }
    return Plan{c.variant, c.tile, c.splits, c.chunk, c.lds_config};
}
void clear_plans(kvdecode_s* h) {
    for (auto& c : h->plans) c.valid = false;
}

Plan compute_plan(const kvdecode_s* h, int T_q) {
    Plan p;
    p.variant = resolve_variant(h, T_q);
    p.tile = p.variant == KVD_VARIANT_VALU   ? kvd::VALU_TILE
             : p.variant == KVD_VARIANT_XCHG ? kvd::XCHG_TILE
                                             : kvd::MFMA_TILE;
    p.lds_config = kvd::LDS_SHORT;
    const long long n_tiles = (h->d.capacity + p.tile - 1) / p.tile;  // tiles of a full cache
    // at most one split per tile, and no more than the launch grid holds
    const long long grid_cap = max_splits_for_grid(h, p.variant, T_q);
    const long long s_max = n_tiles < grid_cap ? n_tiles : grid_cap;
    auto clamp_splits = [&](long long s) {
        s = s > s_max ? s_max : s;
        return s < 1 ? 1 : s;  // (a grid that holds no split is refused before any launch)
    };
    // tiles are dealt round-robin: a split holds at most ceil(n_tiles / S)
    auto finish = [&](long long s) {
        s = clamp_splits(s);
        p.splits = (int)s;
        p.chunk = (int)((n_tiles + s - 1) / s * p.tile);
    };
    if (p.variant == KVD_VARIANT_LDS && h->d.head_dim == 256 && !is_fp8(h)) {
        const long long s = clamp_splits(h->forced_splits > 0
                                             ? h->forced_splits
                                             : plan_splits(h, shape_for(h, p.variant, kvd::LDS_LONG, T_q),
                                                           p.tile, n_tiles, T_q, s_max));
        if ((n_tiles + s - 1) / s >= kvd::LDS_LONG_MIN_TILES) {
            p.lds_config = kvd::LDS_LONG;
            finish(s);
            return p;
        }
    }
    if (h->forced_splits > 0) {
        finish(h->forced_splits);
        return p;
    }
    finish(plan_splits(h, shape_for(h, p.variant, kvd::LDS_SHORT, T_q), p.tile, n_tiles, T_q, s_max));
    return p;
}

int32_t hip_fail(hipError_t e) { return e == hipErrorOutOfMemory ? KVD_ENOMEM : KVD_EHIP; }

// Bind the handle to the current device on first use; later calls must run
// with the same device current.
int32_t ensure_device(kvdecode_s* h) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return KVD_EHIP;
    if (h->device >= 0) return dev == h->device ? KVD_OK : KVD_EINVAL;
    // err word; per sequence the attended length of the last step and the
    // rows its last append added; then the dispatch order the combine leaves
    // for the next partial pass (B entries and a flag, zero: not yet valid);
    // then the per-sequence arrival counters of single-split passes (zero
    // between launches)
    const size_t words = 2 + 4 * (size_t)h->d.batch;
    e = hipMalloc(reinterpret_cast<void**>(&h->err), words * sizeof(int));
    if (e != hipSuccess) return hip_fail(e);
    e = hipMemset(h->err, 0, words * sizeof(int));
    if (e != hipSuccess) {
        (void)hipFree(h->err);
        h->err = nullptr;
        return KVD_EHIP;
    }
    h->device = dev;
    return KVD_OK;
}

// Workspace for `splits` splits of B * Hq * T_q query rows (row_splits =
// splits * T_q; the capacity is kept in the same unit).
int32_t ensure_workspace(kvdecode_s* h, int row_splits) {
    const int splits = row_splits;
    if (splits <= h->ws_splits) return KVD_OK;
    if (h->o_part) (void)hipFree(h->o_part);
    if (h->lse_part) (void)hipFree(h->lse_part);
    h->o_part = nullptr;
    h->lse_part = nullptr;
    h->ws_splits = 0;
    const size_t rows = (size_t)h->d.batch * h->d.num_q_heads * (size_t)splits;
    const size_t part_elem = h->d.dtype == KVD_F32 ? sizeof(float) : sizeof(uint16_t);
    hipError_t e = hipMalloc(&h->o_part, rows * h->d.head_dim * part_elem);
    if (e != hipSuccess) return hip_fail(e);
    e = hipMalloc(reinterpret_cast<void**>(&h->lse_part), rows * sizeof(float));
    if (e != hipSuccess) {
        (void)hipFree(h->o_part);
        h->o_part = nullptr;
        return hip_fail(e);
    }
    h->ws_splits = splits;
    return KVD_OK;
}

void free_events(kvdecode_s* h) {
    for (hipEvent_t ev : h->ev_attend) (void)hipEventDestroy(ev);
    for (hipEvent_t ev : h->ev_append) (void)hipEventDestroy(ev);
    h->ev_attend.clear();
    h->ev_append.clear();
    h->comb_timed.clear();
    h->n_attend = h->n_append = 0;
}

int32_t ensure_events(kvdecode_s* h) {
    if (h->timing_cap <= 0 || !h->ev_attend.empty()) return KVD_OK;
    h->ev_attend.resize(4 * (size_t)h->timing_cap, nullptr);
    h->ev_append.resize(2 * (size_t)h->timing_cap, nullptr);
    h->comb_timed.assign((size_t)h->timing_cap, 0);
    for (auto* vec : {&h->ev_attend, &h->ev_append}) {
        for (hipEvent_t& ev : *vec) {
            // timing only: no system-scope fence (cache writeback) at record
            if (hipEventCreateWithFlags(&ev, hipEventDisableSystemFence) != hipSuccess) {
                ev = nullptr;
                free_events(h);
                return KVD_EHIP;
            }
        }
    }
    return KVD_OK;
}

// Device memory a step uses besides the caller's tensors: the sticky error
// word, per sequence the attended length (and the rows a several-token
// append added), the dispatch order the combine leaves for the next step
// (null: batch order, no sort), and the split partials.
struct Workspace {
    int* err;
    int* len_att;   // [B]
    int* n_new;     // [B]
    int* order;     // [B] + flag, or null
    int* seq_ctr;   // [B], zero between launches
    void* o_part;
    float* lse_part;
};

Workspace handle_workspace(const kvdecode_s* h) {
    const int B = h->d.batch;
    return Workspace{h->err, h->err + 1, h->err + 1 + B, h->err + 1 + 2 * B, h->err + 2 + 3 * B, h->o_part,
                     h->lse_part};
}

// A single-split plan of the LDS or VALU kernel writes the output in the
// partial pass; no combine launch follows (the combine exists only to merge
// splits).
bool single_pass(const kvdecode_s* h, const Plan& p) {
    return p.splits == 1 && ((p.variant == KVD_VARIANT_LDS && !is_fp8(h)) || p.variant == KVD_VARIANT_VALU);
}

int32_t launch_append_timed(kvdecode_s* h, const Workspace& ws, const void* k_new, const void* v_new,
                            hipStream_t st, int T_q = 1, bool may_time = true) {
    const bool timed = may_time && (h->timing_what & KVD_TIME_APPEND) && h->timing_cap > 0 &&
                       h->n_append < h->timing_cap;
    const kvd::Launch on = timed ? kvd::Launch(st, h->ev_append[2 * h->n_append], h->ev_append[2 * h->n_append + 1])
                                 : kvd::Launch(st);
    hipError_t e =
        is_fp8(h) ? kvd::launch_append_fp8(k_new, v_new, h->d.k_cache, h->d.v_cache, h->k_exp, h->v_exp, h->kv,
                                           h->d.lengths, ws.err, ws.n_new, h->d.batch, h->d.num_kv_heads,
                                           h->d.head_dim, h->d.capacity, T_q, on)
                  : kvd::launch_append(k_new, v_new, h->d.k_cache, h->d.v_cache, h->kv, h->d.lengths, ws.err,
                                       ws.n_new, h->d.batch, h->d.num_kv_heads, h->d.head_dim, h->d.capacity,
                                       T_q, h->elem, on);
    if (e != hipSuccess) return KVD_EHIP;
    if (timed) ++h->n_append;
    return KVD_OK;
}

// Host checks of a step (before any device work) and its plan.
int32_t check_step(kvdecode_s* h, const void* q, void* out, float scale, int T_q, Plan* plan) {
    if (!q || !out) return KVD_EINVAL;
    if (!aligned16(q) || !aligned16(out)) return KVD_EALIGN;
    if (!(scale > 0.f) || !isfinite(scale)) return KVD_EINVAL;
    const Plan p = make_plan(h, T_q);
    if (is_fp8(h) ? (p.variant != KVD_VARIANT_LDS && p.variant != KVD_VARIANT_WAVE && p.variant != KVD_VARIANT_XCHG)
                  : (p.variant != KVD_VARIANT_VALU && h->d.dtype != KVD_BF16))
        return KVD_EUNSUPPORTED;
    if (T_q > 1 && p.variant == KVD_VARIANT_MFMA) return KVD_EUNSUPPORTED;
    // Launch sizes: the partial pass (at its planned splits) and the
    // combine (one extra workgroup, and rows of B * Hq * T_q query rows, at
    // least one row per 256-thread workgroup) must fit 32-bit grids; the
    // kernels' int row arithmetic then fits too.
    const GridShape g = partial_grid(h, p.variant, T_q);
    const long long rows = (long long)h->d.batch * h->d.num_q_heads * T_q;
    if ((long long)g.threads * g.blocks_per_split * p.splits > GRID_ITEMS_MAX || (rows + 1) * 256 > GRID_ITEMS_MAX)
        return KVD_EINVAL;
    *plan = p;
    return KVD_OK;
}

// One step's launches on a given workspace: optionally the append kernel,
// the partial pass, the combine.  The LDS and VALU kernels fold a one-token
// append into the partial pass (the combine then advances lengths, or a
// one-split pass of those kernels does, with no combine), as do
// the fp8 wave and exchange kernels; the other kernels, and several new
// tokens, launch the append kernel first.  T_q > 1: a step with T_q new
// tokens per sequence (append then causal attend of their T_q queries); q
// and out then hold Hq * T_q rows.  may_time: record the timing events
// kvdecode_timing_enable asked for.
int32_t launch_step(kvdecode_s* h, const Plan& p, const Workspace& ws, const void* k_new, const void* v_new,
                    const void* q, void* out, float scale, hipStream_t st, int T_q, bool may_time) {
    const bool with_append = k_new != nullptr;
    const bool fused = with_append && T_q == 1 &&
                       (is_fp8(h) ? p.variant == KVD_VARIANT_WAVE || p.variant == KVD_VARIANT_XCHG
                                  : p.variant != KVD_VARIANT_MFMA);
    int32_t rc;
    if (with_append && !fused) {
        if ((rc = launch_append_timed(h, ws, k_new, v_new, st, T_q, may_time)) != KVD_OK) return rc;
    }

    kvd::PartialArgs a;
    a.q = q;
    a.k_cache = h->d.k_cache;
    a.v_cache = h->d.v_cache;
    a.lengths = h->d.lengths;
    a.o_part = ws.o_part;
    a.lse_part = ws.lse_part;
    a.err = ws.err;
    a.len_att = ws.len_att;
    a.k_new = fused ? k_new : nullptr;
    a.v_new = fused ? v_new : nullptr;
    a.B = h->d.batch;
    a.Hq = h->d.num_q_heads * T_q;
    a.Hkv = h->d.num_kv_heads;
    a.M = h->M * T_q;
    a.T_q = T_q;
    a.n_new = T_q > 1 ? ws.n_new : nullptr;
    a.order = ws.order;
    a.D = h->d.head_dim;
    a.T_cap = h->d.capacity;
    a.S = p.splits;
    a.scale_log2e = scale * kvd::LOG2E;
    a.lds_config = p.lds_config;
    a.kv = h->kv;
    a.k_exp = h->k_exp;
    a.v_exp = h->v_exp;
    a.m_init = h->unified ? h->unified_max * kvd::LOG2E : -INFINITY;
    a.tau = h->unified ? 64.f : 8.f;
    const bool one_pass = single_pass(h, p);
    a.out = one_pass ? out : nullptr;
    a.lengths_adv = one_pass && fused ? h->d.lengths : nullptr;
    a.seq_ctr = one_pass ? ws.seq_ctr : nullptr;

    kvd::CombineArgs c;
    c.o_part = ws.o_part;
    c.lse_part = ws.lse_part;
    c.len_att = ws.len_att;
    c.order = ws.order;
    c.lengths = h->d.lengths;
    c.fused_append = fused ? 1 : 0;
    c.out = out;
    c.B = a.B;
    c.Hq = a.Hq;
    c.D = a.D;
    c.T_cap = a.T_cap;
    c.tile = p.tile;
    c.S = p.splits;
    // Timed launches carry their events (the dispatch stamps them), so a
    // bracket asked for adds no command to the stream and measures the
    // kernel alone: ev[0], ev[1] the partial pass, ev[2], ev[3] the combine.
    const int what = h->timing_what;
    const bool timed = may_time && (what & (KVD_TIME_PARTIAL | KVD_TIME_COMBINE)) && h->timing_cap > 0 &&
                       h->n_attend < h->timing_cap;
    hipEvent_t* ev = timed ? &h->ev_attend[4 * h->n_attend] : nullptr;
    const kvd::Launch on_part = timed && (what & KVD_TIME_PARTIAL) ? kvd::Launch(st, ev[0], ev[1]) : kvd::Launch(st);
    const bool comb_timed = timed && (what & KVD_TIME_COMBINE) && !one_pass;
    const kvd::Launch on_comb = comb_timed ? kvd::Launch(st, ev[2], ev[3]) : kvd::Launch(st);
    hipError_t e = p.variant == KVD_VARIANT_WAVE   ? kvd::launch_partial_wave_fp8(a, on_part)
                   : p.variant == KVD_VARIANT_XCHG ? kvd::launch_partial_xchg(a, on_part)
                   : is_fp8(h)                     ? kvd::launch_partial_lds_fp8(a, on_part)
                   : p.variant == KVD_VARIANT_LDS  ? kvd::launch_partial_lds(a, on_part)
                   : p.variant == KVD_VARIANT_MFMA ? kvd::launch_partial_mfma(a, on_part)
                                                   : kvd::launch_partial_valu(a, h->d.dtype == KVD_BF16, on_part);
    if (e != hipSuccess) return KVD_EHIP;
    if (!one_pass) {
        e = kvd::launch_combine(c, h->d.dtype != KVD_F32, on_comb);  // fp8 caches give bf16 outputs
        if (e != hipSuccess) return KVD_EHIP;
    }
    if (timed) h->comb_timed[h->n_attend++] = comb_timed;
    return KVD_OK;
}

// One attend, optionally preceded by an append, on the handle's workspace
// (allocated here on first use).  Argument checks happen before any device
// work.
int32_t run_step(kvdecode_s* h, const void* k_new, const void* v_new, const void* q, void* out,
                 float scale, hipStream_t st, int T_q = 1) {
    Plan p;
    int32_t rc = check_step(h, q, out, scale, T_q, &p);
    if (rc != KVD_OK) return rc;
    if ((rc = ensure_device(h)) != KVD_OK) return rc;
    if ((rc = ensure_workspace(h, p.splits * T_q)) != KVD_OK) return rc;
    if ((rc = ensure_events(h)) != KVD_OK) return rc;
    return launch_step(h, p, handle_workspace(h), k_new, v_new, q, out, scale, st, T_q, true);
}

// --- allocation-free steps --------------------------------------------------
//
// kvdecode_append_attend_noalloc takes its workspace from this static device
// array instead of the handle's: one copy per GPU, loaded with the code
// object and held until the process ends, shared by every such call on that
// GPU.  Host code reaches it through the address hipGetSymbolAddress gives
// for the current device (the array's name is only a host-side stand-in),
// looked up once per device and kept in scratch_ptr.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)KVD_NOALLOC_SCRATCH_MIB << 20;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

// Device address of the current device's scratch array.
int32_t scratch_of(int dev, char** out) {
    if (dev < 0 || dev >= MAX_DEVICES) return KVD_EINVAL;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return KVD_EHIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = static_cast<char*>(g_scratch_ptr[dev]);
    return KVD_OK;
}

// Layout of one step's workspace in the scratch array: the error word; the
// per-sequence arrival counters of single-split passes, in a region of fixed
// place and size that nothing else uses, so they stay zero between launches
// whatever step ran before (the array starts zeroed and each launch leaves
// them zero); then [B] attended lengths and [B] appended-row counts, then
// the partials and their log-sum-exps, each 256-byte aligned.  No dispatch
// order is kept between calls (the array is shared): steps dispatch in
// batch order.
constexpr size_t NOALLOC_SEQ_CTR = 256;
struct ScratchLayout {
    size_t len_att, n_new, o_part, lse, total;
};
ScratchLayout scratch_layout(const kvdecode_s* h, const Plan& p) {
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t B = (size_t)h->d.batch;
    const size_t rows = B * h->d.num_q_heads * (size_t)p.splits;
    const size_t part_elem = h->d.dtype == KVD_F32 ? sizeof(float) : sizeof(uint16_t);
    ScratchLayout l;
    l.len_att = NOALLOC_SEQ_CTR + 65536 * sizeof(int);  // room for the largest batch a handle takes
    l.n_new = l.len_att + up(B * sizeof(int));
    l.o_part = l.n_new + up(B * sizeof(int));
    l.lse = l.o_part + up(rows * h->d.head_dim * part_elem);
    l.total = l.lse + up(rows * sizeof(float));
    return l;
}

// Read the sticky error word at `word` on stream st and clear it if set.
int32_t take_error_word(int* word, hipStream_t st, int* flag) {
    if (hipMemcpyAsync(flag, word, sizeof(int), hipMemcpyDeviceToHost, st) != hipSuccess) return KVD_EHIP;
    if (hipStreamSynchronize(st) != hipSuccess) return KVD_EHIP;
    if (*flag) {
        if (hipMemsetAsync(word, 0, sizeof(int), st) != hipSuccess) return KVD_EHIP;
        if (hipStreamSynchronize(st) != hipSuccess) return KVD_EHIP;
    }
    return KVD_OK;
}

}  // namespace

extern "C" {

const char* kvdecode_strerror(int32_t code) {
    switch (code) {
        case KVD_OK: return "success";
        case KVD_EINVAL: return "invalid argument";
        case KVD_EUNSUPPORTED: return "unsupported head_dim, dtype or variant";
        case KVD_EALIGN: return "pointer not 16-byte aligned";
        case KVD_ECAPACITY: return "append on a sequence already at cache capacity";
        case KVD_EHIP: return "HIP runtime error";
        case KVD_ENOMEM: return "out of memory";
        case KVD_ELENGTH: return "sequence length outside [0, capacity]";
        case KVD_EPAGE: return "block-table entry outside the page pool";
        case KVD_ESCRATCH: return "step needs more workspace than the allocation-free entry point's static buffer";
        default: return "unknown status code";
    }
}

namespace {

// Validation shared by both create calls; `h` is filled on success.
int32_t make_handle(const kvdecode_desc_t& d, const kvd::KvLayout& kv, kvdecode_t* out) {
    *out = nullptr;
    if (d.batch < 1 || d.num_q_heads < 1 || d.num_kv_heads < 1 || d.capacity < 1) return KVD_EINVAL;
    if (d.batch > 65535 || d.num_kv_heads > 65535 || d.num_q_heads > 65535) return KVD_EINVAL;
    if (d.capacity > (1 << 24)) return KVD_EINVAL;
    if (d.num_q_heads % d.num_kv_heads != 0) return KVD_EINVAL;
    if (d.head_dim != 64 && d.head_dim != 128 && d.head_dim != 256) return KVD_EUNSUPPORTED;
    if (d.dtype != KVD_F32 && d.dtype != KVD_BF16 && d.dtype != KVD_FP8_E4M3) return KVD_EUNSUPPORTED;
    if (!d.k_cache || !d.v_cache || !d.lengths) return KVD_EINVAL;
    if (!aligned16(d.k_cache) || !aligned16(d.v_cache) ||
        (reinterpret_cast<uintptr_t>(d.lengths) & 3u))
        return KVD_EALIGN;
    kvdecode_s* h = new (std::nothrow) kvdecode_s();
    if (!h) return KVD_ENOMEM;
    h->d = d;
    h->kv = kv;
    h->M = d.num_q_heads / d.num_kv_heads;
    h->elem = d.dtype == KVD_F32 ? 4 : (d.dtype == KVD_BF16 ? 2 : 1);
    {
        std::lock_guard<std::mutex> lk(g_mu);
        live().insert(h);
    }
    *out = h;
    return KVD_OK;
}

}  // namespace

int32_t kvdecode_create(const kvdecode_desc_t* desc, kvdecode_t* out) {
    if (!desc || !out) return KVD_EINVAL;
    if (desc->dtype == KVD_FP8_E4M3) return KVD_EUNSUPPORTED;  // kvdecode_create_fp8
    return make_handle(*desc, kvd::KvLayout{nullptr, 0, 0, 0}, out);
}

int32_t kvdecode_create_fp8(const kvdecode_fp8_desc_t* desc, kvdecode_t* out) {
    if (!desc || !out) return KVD_EINVAL;
    *out = nullptr;
    kvdecode_desc_t d = desc->cache;
    if (d.dtype != KVD_FP8_E4M3) return KVD_EUNSUPPORTED;
    if (d.capacity < 1 || d.capacity % 32 != 0) return KVD_EINVAL;
    if (!desc->k_exp || !desc->v_exp) return KVD_EINVAL;
    if (!aligned16(desc->k_exp) || !aligned16(desc->v_exp)) return KVD_EALIGN;
    const int32_t rc = make_handle(d, kvd::KvLayout{nullptr, 0, 0, 0}, out);
    if (rc == KVD_OK) {
        (*out)->k_exp = desc->k_exp;
        (*out)->v_exp = desc->v_exp;
    }
    return rc;
}

// The contiguous-equivalent descriptor and block-table layout of a paged
// descriptor, validated (dtype aside).
int32_t paged_desc(const kvdecode_paged_desc_t& p, kvdecode_desc_t* d, kvd::KvLayout* kv) {
    if (p.page_size < 32 || p.page_size > 65536 || (p.page_size & (p.page_size - 1))) return KVD_EINVAL;
    if (p.num_pages < 1 || p.max_pages < 1 || p.num_kv_heads < 1) return KVD_EINVAL;
    if ((long long)p.max_pages * p.page_size > (1 << 24)) return KVD_EINVAL;
    // every row index of the pool fits the kernels' 32-bit row arithmetic
    if ((long long)p.num_pages * p.num_kv_heads * p.page_size > (1LL << 31)) return KVD_EINVAL;
    if (!p.block_table) return KVD_EINVAL;
    if (reinterpret_cast<uintptr_t>(p.block_table) & 3u) return KVD_EALIGN;
    d->batch = p.batch;
    d->num_q_heads = p.num_q_heads;
    d->num_kv_heads = p.num_kv_heads;
    d->head_dim = p.head_dim;
    d->capacity = p.max_pages * p.page_size;
    d->dtype = p.dtype;
    d->k_cache = p.k_pages;
    d->v_cache = p.v_pages;
    d->lengths = p.lengths;
    int shift = 0;
    while ((1 << shift) < p.page_size) ++shift;
    *kv = kvd::KvLayout{p.block_table, shift, p.max_pages, p.num_pages};
    return KVD_OK;
}

int32_t kvdecode_create_paged(const kvdecode_paged_desc_t* desc, kvdecode_t* out) {
    if (!desc || !out) return KVD_EINVAL;
    *out = nullptr;
    kvdecode_desc_t d;
    kvd::KvLayout kv;
    const int32_t rc = paged_desc(*desc, &d, &kv);
    if (rc != KVD_OK) return rc;
    if (d.dtype == KVD_FP8_E4M3) return KVD_EUNSUPPORTED;  // kvdecode_create_fp8_paged
    return make_handle(d, kv, out);
}

int32_t kvdecode_create_fp8_paged(const kvdecode_fp8_paged_desc_t* desc, kvdecode_t* out) {
    if (!desc || !out) return KVD_EINVAL;
    *out = nullptr;
    kvdecode_desc_t d;
    kvd::KvLayout kv;
    int32_t rc = paged_desc(desc->pages, &d, &kv);
    if (rc != KVD_OK) return rc;
    if (d.dtype != KVD_FP8_E4M3) return KVD_EUNSUPPORTED;
    if (!desc->k_exp || !desc->v_exp) return KVD_EINVAL;
    if (!aligned16(desc->k_exp) || !aligned16(desc->v_exp)) return KVD_EALIGN;
    rc = make_handle(d, kv, out);
    if (rc == KVD_OK) {
        (*out)->k_exp = desc->k_exp;
        (*out)->v_exp = desc->v_exp;
    }
    return rc;
}

int32_t kvdecode_append(kvdecode_t h, const void* k_new, const void* v_new, void* stream) {
    if (!is_live(h)) return KVD_EINVAL;
    if (!k_new || !v_new) return KVD_EINVAL;
    if (!aligned16(k_new) || !aligned16(v_new)) return KVD_EALIGN;
    int32_t rc = ensure_device(h);
    if (rc != KVD_OK) return rc;
    if ((rc = ensure_events(h)) != KVD_OK) return rc;
    return launch_append_timed(h, handle_workspace(h), k_new, v_new, static_cast<hipStream_t>(stream));
}

int32_t kvdecode_attend(kvdecode_t h, const void* q, void* out, float scale, void* stream) {
    if (!is_live(h)) return KVD_EINVAL;
    return run_step(h, nullptr, nullptr, q, out, scale, static_cast<hipStream_t>(stream));
}

int32_t kvdecode_append_attend(kvdecode_t h, const void* k_new, const void* v_new, const void* q,
                               void* out, float scale, void* stream) {
    if (!is_live(h)) return KVD_EINVAL;
    if (!k_new || !v_new) return KVD_EINVAL;
    if (!aligned16(k_new) || !aligned16(v_new)) return KVD_EALIGN;
    return run_step(h, k_new, v_new, q, out, scale, static_cast<hipStream_t>(stream));
}

int32_t kvdecode_append_attend_multi(kvdecode_t h, int32_t n_tokens, const void* k_new,
                                     const void* v_new, const void* q, void* out, float scale,
                                     void* stream) {
    if (!is_live(h)) return KVD_EINVAL;
    if (n_tokens < 1 || n_tokens > KVD_MAX_NEW_TOKENS) return KVD_EINVAL;
    if (!k_new || !v_new) return KVD_EINVAL;
    if (!aligned16(k_new) || !aligned16(v_new)) return KVD_EALIGN;
    return run_step(h, k_new, v_new, q, out, scale, static_cast<hipStream_t>(stream), n_tokens);
}

int32_t kvdecode_append_attend_noalloc(kvdecode_t h, const void* k_new, const void* v_new, const void* q,
                                       void* out, float scale, void* stream) {
    if (!is_live(h)) return KVD_EINVAL;
    if (!k_new || !v_new) return KVD_EINVAL;
    if (!aligned16(k_new) || !aligned16(v_new)) return KVD_EALIGN;
    Plan p;
    int32_t rc = check_step(h, q, out, scale, 1, &p);
    if (rc != KVD_OK) return rc;
    const ScratchLayout l = scratch_layout(h, p);
    if (l.total > NOALLOC_SCRATCH_BYTES) return KVD_ESCRATCH;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return KVD_EHIP;
    char* base = nullptr;
    if ((rc = scratch_of(dev, &base)) != KVD_OK) return rc;
    const Workspace ws{reinterpret_cast<int*>(base),
                       reinterpret_cast<int*>(base + l.len_att),
                       reinterpret_cast<int*>(base + l.n_new),
                       nullptr,
                       reinterpret_cast<int*>(base + NOALLOC_SEQ_CTR),
                       base + l.o_part,
                       reinterpret_cast<float*>(base + l.lse)};
    h->noalloc_device = dev;
    return launch_step(h, p, ws, k_new, v_new, q, out, scale, static_cast<hipStream_t>(stream), 1, false);
}

int32_t kvdecode_status(kvdecode_t h, void* stream) {
    if (!is_live(h)) return KVD_EINVAL;
    if (h->device < 0 && h->noalloc_device < 0) return KVD_OK;
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return KVD_EINVAL;
    if ((h->device >= 0 && cur != h->device) || (h->noalloc_device >= 0 && cur != h->noalloc_device))
        return KVD_EINVAL;
    hipStream_t st = static_cast<hipStream_t>(stream);
    int flag = 0, rc;
    if (h->device >= 0 && (rc = take_error_word(h->err, st, &flag)) != KVD_OK) return rc;
    if (h->noalloc_device >= 0) {
        char* base = nullptr;
        int scratch_flag = 0;
        if ((rc = scratch_of(cur, &base)) != KVD_OK) return rc;
        if ((rc = take_error_word(reinterpret_cast<int*>(base), st, &scratch_flag)) != KVD_OK) return rc;
        flag |= scratch_flag;
    }
    if (flag & kvd::ERRBIT_CAPACITY) return KVD_ECAPACITY;
    if (flag & kvd::ERRBIT_LENGTH) return KVD_ELENGTH;
    if (flag & kvd::ERRBIT_PAGE) return KVD_EPAGE;
    return KVD_OK;
}

int32_t kvdecode_reserve(kvdecode_t h, int32_t max_new_tokens) {
    if (!is_live(h)) return KVD_EINVAL;
    if (max_new_tokens < 1 || max_new_tokens > KVD_MAX_NEW_TOKENS) return KVD_EINVAL;
    int32_t rc = ensure_device(h);
    if (rc != KVD_OK) return rc;
    // the workspace a step of T_q tokens needs grows with T_q, but its plan
    // may pick fewer splits: reserve the largest over 1..max_new_tokens
    int row_splits = 0;
    for (int t = 1; t <= max_new_tokens; ++t) {
        const int r = make_plan(h, t).splits * t;
        row_splits = r > row_splits ? r : row_splits;
    }
    if ((rc = ensure_workspace(h, row_splits)) != KVD_OK) return rc;
    return ensure_events(h);
}

int32_t kvdecode_set_unified_max(kvdecode_t h, int32_t enable, float phi) {
    if (!is_live(h)) return KVD_EINVAL;
    if (enable && !isfinite(phi)) return KVD_EINVAL;
    h->unified = enable != 0;
    h->unified_max = enable ? phi : 0.f;
    return KVD_OK;
}

int32_t kvdecode_set_num_splits(kvdecode_t h, int32_t n) {
    if (!is_live(h) || n < 0) return KVD_EINVAL;
    h->forced_splits = n;
    clear_plans(h);
    return KVD_OK;
}

int32_t kvdecode_set_variant(kvdecode_t h, int32_t variant) {
    if (!is_live(h)) return KVD_EINVAL;
    if (variant < KVD_VARIANT_AUTO || variant > KVD_VARIANT_XCHG) return KVD_EUNSUPPORTED;
    if (is_fp8(h)) {
        const bool ok = variant == KVD_VARIANT_AUTO || variant == KVD_VARIANT_LDS ||
                        ((variant == KVD_VARIANT_WAVE || variant == KVD_VARIANT_XCHG) && h->d.head_dim >= 128);
        if (!ok) return KVD_EUNSUPPORTED;
        h->variant_req = variant;
        clear_plans(h);
        return KVD_OK;
    }
    if (variant == KVD_VARIANT_WAVE || variant == KVD_VARIANT_XCHG) return KVD_EUNSUPPORTED;
    if ((variant == KVD_VARIANT_MFMA || variant == KVD_VARIANT_LDS) && h->d.dtype != KVD_BF16)
        return KVD_EUNSUPPORTED;
    if (variant == KVD_VARIANT_MFMA && h->kv.block_table) return KVD_EUNSUPPORTED;
    h->variant_req = variant;
    clear_plans(h);
    return KVD_OK;
}

int32_t kvdecode_get_plan(kvdecode_t h, int32_t* variant, int32_t* num_splits, int32_t* split_tokens) {
    return kvdecode_get_plan_multi(h, 1, variant, num_splits, split_tokens);
}

int32_t kvdecode_get_plan_multi(kvdecode_t h, int32_t n_tokens, int32_t* variant, int32_t* num_splits,
                                int32_t* split_tokens) {
    if (!is_live(h) || n_tokens < 1 || n_tokens > KVD_MAX_NEW_TOKENS) return KVD_EINVAL;
    const Plan p = make_plan(h, n_tokens);
    if (n_tokens > 1 && p.variant == KVD_VARIANT_MFMA) return KVD_EUNSUPPORTED;
    if (variant) *variant = p.variant;
    if (num_splits) *num_splits = p.splits;
    if (split_tokens) *split_tokens = p.chunk;
    return KVD_OK;
}

int32_t kvdecode_timing_enable(kvdecode_t h, int32_t max_calls, int32_t what) {
    if (!is_live(h) || max_calls < 0 || (what & ~KVD_TIME_ALL) != 0) return KVD_EINVAL;
    free_events(h);
    h->timing_what = what;
    h->timing_cap = what ? max_calls : 0;
    if (h->device >= 0) return ensure_events(h);
    return KVD_OK;
}

int32_t kvdecode_timing_read(kvdecode_t h, double* partial_ms, double* combine_ms, double* append_ms,
                             int32_t* n_attend, int32_t* n_append) {
    if (!is_live(h)) return KVD_EINVAL;
    double tp = 0, tc = 0, ta = 0;
    const int what = h->timing_what;
    for (int i = 0; i < h->n_attend; ++i) {
        hipEvent_t* ev = &h->ev_attend[4 * i];
        float a = 0, b = 0;
        if (what & KVD_TIME_PARTIAL) {
            if (hipEventSynchronize(ev[1]) != hipSuccess || hipEventElapsedTime(&a, ev[0], ev[1]) != hipSuccess)
                return KVD_EHIP;
        }
        if (h->comb_timed[i]) {
            if (hipEventSynchronize(ev[3]) != hipSuccess || hipEventElapsedTime(&b, ev[2], ev[3]) != hipSuccess)
                return KVD_EHIP;
        }
        tp += a;
        tc += b;
    }
    for (int i = 0; i < h->n_append; ++i) {
        float a = 0;
        if (hipEventSynchronize(h->ev_append[2 * i + 1]) != hipSuccess) return KVD_EHIP;
        if (hipEventElapsedTime(&a, h->ev_append[2 * i], h->ev_append[2 * i + 1]) != hipSuccess)
            return KVD_EHIP;
        ta += a;
    }
    if (partial_ms) *partial_ms = tp;
    if (combine_ms) *combine_ms = tc;
    if (append_ms) *append_ms = ta;
    if (n_attend) *n_attend = h->n_attend;
    if (n_append) *n_append = h->n_append;
    h->n_attend = h->n_append = 0;
    return KVD_OK;
}

int32_t kvdecode_destroy(kvdecode_t h) {
    {
        std::lock_guard<std::mutex> lk(g_mu);
        if (!h || !live().count(h)) return KVD_EINVAL;
        live().erase(h);
    }
    if (h->device >= 0) {
        int cur = -1;
        (void)hipGetDevice(&cur);
        if (cur != h->device) (void)hipSetDevice(h->device);
        (void)hipDeviceSynchronize();
        free_events(h);
        if (h->o_part) (void)hipFree(h->o_part);
        if (h->lse_part) (void)hipFree(h->lse_part);
        if (h->err) (void)hipFree(h->err);
        if (cur >= 0 && cur != h->device) (void)hipSetDevice(cur);
    }
    delete h;
    return KVD_OK;
}

}  // extern "C"
