/*
 * kvdecode.h -- C ABI of a single-GPU decode-attention library for AMD
 * Instinct MI355X (gfx950).
 *
 * The operation: during generation every sequence contributes one new token.
 * Its key and value projections are appended to the sequence's KV cache, and
 * its query -- one vector per query head -- attends over every cached token of
 * that sequence.  Many query heads share one key/value head (multiquery) or a
 * few (grouped-query); multi-head attention is the case Hq == Hkv.
 *
 * Passages that define it:
 *   - "All About Transformer Inference" (How To Scale Your Model, part 7),
 *     section "Transformer inference basics": the KV cache stores every past
 *     token's key/value projections; generation appends the new token's
 *     projections and computes only the new query against the cached keys.
 *   - same page, section "Implementation: JetStream": the engine interface
 *     (prefill produces a cache, insert places it into the generate batch,
 *     generate emits one token per batch item and appends the single-token
 *     KV cache).  Prefill and insert are the caller writing the cache tensors
 *     and lengths; this library provides the generate-side append and attend.
 *   - same page, section "Continuous batching": a KV buffer sized for a
 *     maximum batch and context length -- here [B, Hkv, T_cap, d] with a
 *     per-sequence valid length.
 *   - same page, section on tricks for generation throughput: ragged HBM
 *     reads (read only the valid prefix of each sequence) and grouped-query
 *     attention (Hkv KV heads, each shared by Hq/Hkv query heads).
 *   - same page, section "Sharding the KV cache": the grouped contraction --
 *     query heads reshaped row-major into [Hkv, M] groups, contracted with
 *     the keys over the head dimension, softmaxed over the sequence, and
 *     contracted with the values over the sequence -- and accumulating
 *     attention across sequence shards the way Flash Attention does.
 *   - "Efficiently Scaling Transformer Inference", section 3.3: multiquery
 *     attention keeps n_heads query heads and a single key/value head
 *     shared by all of them; during generation Q, K and V hold one token per
 *     example while the cache holds many.
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers owned by the caller, contiguous
 *     row-major, 16-byte aligned.  The library never frees them.  A handle
 *     stores the cache and length pointers given at creation: the caller keeps
 *     those allocations alive until kvdecode_destroy.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  append
 *     and attend are asynchronous on it; host-side validation happens first
 *     and a rejected call launches nothing.
 *   - q, k_new, v_new, out and both caches share the handle's dtype: fp32
 *     (KVD_F32) or bfloat16 (KVD_BF16).  Arithmetic is fp32 with fp32
 *     accumulation; bf16 outputs are rounded to nearest even.
 *   - Return values are KVD_OK (0) or a negative kvd_status_t code.
 *   - Calls that share one handle must be serialised by the caller (same
 *     stream, or ordered streams): attend uses the handle's workspace.
 */
#ifndef KVDECODE_H
#define KVDECODE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kvdecode_s* kvdecode_t;

/* Element types.  KVD_FP8_E4M3 is a cache type only (kvdecode_create_fp8,
 * kvdecode_create_fp8_paged):
 * q, k_new, v_new and out are then bf16. */
enum { KVD_F32 = 0, KVD_BF16 = 1, KVD_FP8_E4M3 = 2 };

typedef enum {
    KVD_OK = 0,
    KVD_EINVAL = -1,       /* bad argument (null, non-positive size, Hq % Hkv != 0, bad scale, unknown handle) */
    KVD_EUNSUPPORTED = -2, /* head_dim not in {64, 128, 256}, unknown dtype, or unknown variant */
    KVD_EALIGN = -3,       /* a pointer is not 16-byte aligned */
    KVD_ECAPACITY = -4,    /* (from kvdecode_status) an append found a sequence already at capacity */
    KVD_EHIP = -5,         /* a HIP runtime call or kernel launch failed */
    KVD_ENOMEM = -6,       /* host or device allocation failed */
    KVD_ELENGTH = -7,      /* (from kvdecode_status) an append or attend found lengths[b] outside [0, capacity] */
    KVD_EPAGE = -8,        /* (from kvdecode_status) a block-table entry in use was outside [0, num_pages) */
    KVD_ESCRATCH = -9      /* kvdecode_append_attend_noalloc: the step needs more workspace than its static buffer */
} kvd_status_t;

/* Kernel variants for the partial pass (kvdecode_set_variant).
 *   VALU: vector-ALU kernel, fp32 or bf16, one four-wave workgroup per
 *         (split, query head), each wave taking every fourth tile.
 *   MFMA: bf16 matrix-core kernel, one wave per 16 query heads, each wave
 *         loading K/V straight into registers.
 *   LDS:  bf16 matrix-core kernel, four waves per (split, KV head) sharing
 *         K/V tiles staged in LDS by direct global->LDS loads (for an fp8
 *         cache: its fp8 counterpart).
 *   WAVE: fp8 caches with d >= 128: four waves per (split, KV head[, group
 *         of up to 16 (d = 256) or 48 (d = 128) query rows]), each
 *         streaming its own tiles for all of the group's rows, merged in
 *         LDS at the end.
 *   XCHG: fp8 caches with d >= 128, for large query groups: four waves
 *         per (split, KV head[, group of up to 48 (d = 256) or 64 (d = 128)
 *         query rows]) split every 64-token tile, by tokens for the scores
 *         and by output columns for the values, and exchange the softmax
 *         weights through LDS, so each fp8 code is widened to bf16 once.
 * (Query rows: heads per KV head times the new tokens of the step.) */
enum { KVD_VARIANT_AUTO = 0, KVD_VARIANT_VALU = 1, KVD_VARIANT_MFMA = 2, KVD_VARIANT_LDS = 3,
       KVD_VARIANT_WAVE = 4, KVD_VARIANT_XCHG = 5 };

typedef struct {
    int32_t batch;        /* B  >= 1                                        */
    int32_t num_q_heads;  /* Hq >= 1, a multiple of num_kv_heads             */
    int32_t num_kv_heads; /* Hkv >= 1; M = Hq / Hkv query heads per KV head  */
    int32_t head_dim;     /* d in {64, 128, 256}                             */
    int32_t capacity;     /* T_cap >= 1: cache slots per (sequence, KV head) */
    int32_t dtype;        /* KVD_F32 or KVD_BF16                             */
    void* k_cache;        /* [B, Hkv, T_cap, d] keys   (device)              */
    void* v_cache;        /* [B, Hkv, T_cap, d] values (device)              */
    int32_t* lengths;     /* [B] valid tokens per sequence (device int32),
                             0 <= lengths[b] <= T_cap; slots >= lengths[b]
                             are never read and may hold anything (NaN)    */
} kvdecode_desc_t;

/*
 * Create a handle over caller-owned cache tensors.  Validates the
 * descriptor (KVD_EINVAL / KVD_EUNSUPPORTED / KVD_EALIGN) and makes no HIP
 * call: the device workspace (split partials, error flag) is allocated on
 * the first append or attend, on the device current at that call, and that
 * device is then bound to the handle (or earlier, by kvdecode_reserve).
 * Later calls never allocate unless kvdecode_set_num_splits asks for more
 * splits than any earlier plan.
 * Limits: B <= 65535, Hkv <= 65535, T_cap <= 2^24.
 */
int32_t kvdecode_create(const kvdecode_desc_t* desc, kvdecode_t* out);

/*
 * Paged KV cache: the caches of all sequences live in one pool of
 * fixed-size pages, and a block table maps each sequence's j-th block of
 * page_size tokens to a page of the pool, so a sequence holds only the pages
 * it needs and a batch slot can be refilled without moving other sequences'
 * caches.  ("All About Transformer Inference", section on tricks for
 * generation throughput -- paged attention, the cache as pages addressed
 * through a table -- and section "Continuous batching".)
 *
 * Token t of sequence b, KV head g is row
 *     (block_table[b * max_pages + t / page_size] * Hkv + g) * page_size
 *       + t % page_size
 * of the pool, i.e. a page holds page_size consecutive tokens of one
 * sequence for every KV head.  The capacity of every sequence is
 * max_pages * page_size tokens; entries of the block table are read only for
 * blocks holding valid tokens (and the block an append writes to), so the
 * rest of a row may hold anything.  An entry in use outside [0, num_pages)
 * is replaced by page 0 for memory safety and sets the sticky error
 * KVD_EPAGE.  Pages are not reference-counted: two sequences may share a
 * page only if neither appends into it.
 */
typedef struct {
    int32_t batch;        /* B  >= 1                                              */
    int32_t num_q_heads;  /* Hq >= 1, a multiple of num_kv_heads                   */
    int32_t num_kv_heads; /* Hkv >= 1                                              */
    int32_t head_dim;     /* d in {64, 128, 256}                                   */
    int32_t page_size;    /* tokens per page: a power of two in [32, 65536]        */
    int32_t num_pages;    /* pages in the pool, >= 1                               */
    int32_t max_pages;    /* block-table row length (blocks per sequence), >= 1    */
    int32_t dtype;        /* KVD_F32 or KVD_BF16                                   */
    void* k_pages;        /* [num_pages, Hkv, page_size, d] keys   (device)        */
    void* v_pages;        /* [num_pages, Hkv, page_size, d] values (device)        */
    int32_t* block_table; /* [B, max_pages] page of each block (device int32)      */
    int32_t* lengths;     /* [B] valid tokens per sequence (device int32),
                             0 <= lengths[b] <= max_pages * page_size             */
} kvdecode_paged_desc_t;

/*
 * fp8 KV cache: keys and values are stored as OCP FP8 E4M3 codes (one byte:
 * sign, 4 exponent bits with bias 7, 3 mantissa bits; largest finite value
 * 448; codes 0x7F and 0xFF are NaN) with one power-of-two scale per
 * (sequence, KV head, token): the stored row is codes * 2^e.  Half the
 * bytes of a bf16 cache per token, plus one exponent byte each for K and V.
 * ("All About Transformer Inference", section on tricks for generation
 * throughput: quantizing the KV cache to int8, int4 or fp8 saves memory
 * bandwidth; "Efficiently Scaling Transformer Inference", section 3.6:
 * quantized storage with bf16 arithmetic in the products.  The pages fix no
 * scale format; per-token power-of-two scales keep dequantization exact.)
 *
 * `cache` describes the codes: dtype KVD_FP8_E4M3, k_cache / v_cache
 * [B, Hkv, T_cap, d] uint8, capacity a multiple of 32.  q, k_new, v_new and
 * out are bf16.  Stored exponents lie in [-117, 119], the range in which
 * every code * 2^e is zero or a finite normal bf16 number, so attention
 * reads the dequantized cache exactly; an exponent outside it is read as
 * the nearest bound.  An append quantizes each new K (and V) row: e is the
 * smallest integer with max|x| <= 448 * 2^e (clamped to [-117, 119]; 0 for
 * an all-zero row) and each value becomes the code nearest to x * 2^-e
 * (ties to the even code; +-448 when e was clamped at 119, so values
 * beyond 448 * 2^119 saturate, and 0 below 2^-127 when it was clamped at
 * -117).  Products and sums are fp32, as for a bf16 cache.  Callers that
 * write the cache themselves (prefill) must follow the same format.  The
 * partial pass runs on the fp8 WAVE, XCHG or LDS kernel
 * (kvdecode_set_variant); kvdecode_create_fp8_paged takes the same format
 * in page pools.
 */
typedef struct {
    kvdecode_desc_t cache; /* dtype KVD_FP8_E4M3; caches hold the codes              */
    int8_t* k_exp;         /* [B, Hkv, T_cap] exponent of each key row (device)       */
    int8_t* v_exp;         /* [B, Hkv, T_cap] exponent of each value row (device)     */
} kvdecode_fp8_desc_t;

/*
 * Create a handle over a caller-owned fp8 cache.  Validation as for
 * kvdecode_create, plus KVD_EINVAL for a capacity that is not a multiple of
 * 32 or a null exponent array, KVD_EALIGN for an exponent array that is not
 * 16-byte aligned.  kvdecode_create and kvdecode_create_paged return
 * KVD_EUNSUPPORTED for dtype KVD_FP8_E4M3.
 */
int32_t kvdecode_create_fp8(const kvdecode_fp8_desc_t* desc, kvdecode_t* out);

/*
 * fp8 cache in page pools: the paged layout of kvdecode_create_paged (codes
 * in the pools, token t of sequence b at row (block_table[b][t / P] * Hkv +
 * g) * P + t mod P) with the exponents in pools of the same shape without
 * the last axis, so a token's exponent sits at the same row index.  Paging
 * after "All About Transformer Inference" (tricks for generation
 * throughput: paged attention), the format as for kvdecode_create_fp8.
 * Validation as for kvdecode_create_paged, KVD_EUNSUPPORTED unless dtype is
 * KVD_FP8_E4M3, KVD_EINVAL / KVD_EALIGN for a null or unaligned exponent
 * pool.
 */
typedef struct {
    kvdecode_paged_desc_t pages; /* dtype KVD_FP8_E4M3; the pools hold the codes        */
    int8_t* k_exp;               /* [num_pages, Hkv, page_size] key-row exponents      */
    int8_t* v_exp;               /* [num_pages, Hkv, page_size] value-row exponents    */
} kvdecode_fp8_paged_desc_t;

int32_t kvdecode_create_fp8_paged(const kvdecode_fp8_paged_desc_t* desc, kvdecode_t* out);

/*
 * Create a handle over a caller-owned paged cache.  Same validation and
 * lazy device binding as kvdecode_create; additionally KVD_EINVAL for a
 * page_size that is not a power of two in [32, 65536], num_pages or
 * max_pages < 1, max_pages * page_size > 2^24, or a pool of more than 2^31
 * rows.  Every call below works on the handle; the partial pass runs on the
 * LDS kernel (bf16) or the VALU kernel (fp32 or bf16) -- KVD_VARIANT_MFMA is
 * KVD_EUNSUPPORTED for a paged handle.
 */
int32_t kvdecode_create_paged(const kvdecode_paged_desc_t* desc, kvdecode_t* out);

/*
 * Bind the handle to the current device now and allocate everything its
 * current plan needs for steps of up to max_new_tokens new tokens per
 * sequence (1 for one-token decode; the draft length for
 * kvdecode_append_attend_multi): workspace, error flag, and the event slots
 * of kvdecode_timing_enable, which would otherwise happen on the first call
 * that needs them.  Lets a caller keep every hipMalloc out of its decode
 * loop.  KVD_EINVAL if max_new_tokens is outside 1..KVD_MAX_NEW_TOKENS or the
 * handle is already bound to another device; KVD_ENOMEM or KVD_EHIP if an
 * allocation fails.  Idempotent.
 */
int32_t kvdecode_reserve(kvdecode_t h, int32_t max_new_tokens);

/*
 * Append one token per sequence (the generate-side cache update).
 * k_new, v_new: [B, Hkv, d] device, handle dtype.  For each b with
 * lengths[b] < T_cap: K[b,g,lengths[b],:] = k_new[b,g,:] and likewise V for
 * every KV head g (a bit copy), then lengths[b] += 1.  A sequence already at
 * capacity is left unchanged (no write, no increment) and sets the handle's
 * sticky error, reported by kvdecode_status as KVD_ECAPACITY.
 */
int32_t kvdecode_append(kvdecode_t h, const void* k_new, const void* v_new, void* stream);

/*
 * Attend the new query over each sequence's valid cache prefix.
 * q: [B, Hq, d], out: [B, Hq, d] device, handle dtype; scale finite and > 0
 * (callers normally pass 1/sqrt(d)).  For query head h of sequence b, with
 * KV head g = floor(h / M) and n = lengths[b]:
 *     out[b,h,:] = sum_{t<n} softmax_t(scale * q[b,h,:] . K[b,g,t,:]) V[b,g,t,:]
 * and out[b,h,:] = 0 when n == 0.  Lengths are read on the device at run
 * time (no host synchronisation); a length outside [0, T_cap] is clamped
 * into range for memory safety and sets the sticky error KVD_ELENGTH.
 * Internally: a split-KV partial pass over (sequence, KV head, split) work
 * units, then a log-sum-exp combine of the splits.  A plan with one split
 * on the LDS or VALU kernel has nothing to merge: its partial pass writes
 * out directly and no combine is launched (the combine exists only to
 * merge the shards, "All About Transformer Inference", section "Sharding
 * the KV cache").
 */
int32_t kvdecode_attend(kvdecode_t h, const void* q, void* out, float scale, void* stream);

/*
 * One decode step: exactly kvdecode_append(h, k_new, v_new) followed by
 * kvdecode_attend(h, q, out, scale) -- same results, same cache contents,
 * same lengths update, same sticky errors -- in fewer launches: with the
 * LDS and VALU kernels the append is folded into the partial pass (the new
 * token's row is read from k_new/v_new directly and written to its cache
 * slot alongside), and with the fp8 WAVE and XCHG kernels the workgroups
 * owning the new token's tile quantize it into its slot before reading
 * that tile; the combine advances lengths (after a one-split pass of the
 * LDS or VALU kernel, the last of a sequence's workgroups to finish does).
 * The MFMA kernel and the fp8 LDS kernel run the append kernel first.
 * Same page, section "Implementation: JetStream": generate emits one token
 * per batch item and appends its single-token KV cache.
 */
int32_t kvdecode_append_attend(kvdecode_t h, const void* k_new, const void* v_new, const void* q,
                               void* out, float scale, void* stream);

/*
 * A step with several new tokens per sequence, as when a large model checks
 * n_tokens drafted tokens in one pass ("All About Transformer Inference",
 * appendix on speculative sampling: the drafted tokens are scored together
 * and share the KV cache load).  1 <= n_tokens <= KVD_MAX_NEW_TOKENS.
 *   k_new, v_new: [B, Hkv, n_tokens, d]; q, out: [B, Hq, n_tokens, d].
 * Each sequence with room for all n_tokens rows gets them at slots
 * lengths[b] .. lengths[b] + n_tokens - 1 (in order) and lengths[b]
 * advances by n_tokens; then query i of head h attends causally: over the
 * cached tokens and the new tokens 0 .. i.  A sequence without room is not
 * appended (sticky KVD_ECAPACITY) and all its queries attend over its
 * lengths[b] cached tokens.  Same dtype rules as kvdecode_append_attend;
 * every cache type and layout (fp32, bf16 or fp8; contiguous or paged), on
 * every kernel but KVD_VARIANT_MFMA (KVD_EUNSUPPORTED).  An fp8 cache
 * quantizes each new row as kvdecode_append does.  n_tokens = 1 gives
 * kvdecode_append_attend's results.
 */
enum { KVD_MAX_NEW_TOKENS = 16 };
int32_t kvdecode_append_attend_multi(kvdecode_t h, int32_t n_tokens, const void* k_new,
                                     const void* v_new, const void* q, void* out, float scale,
                                     void* stream);

/*
 * kvdecode_append_attend without any allocation, for callers that cannot
 * allocate device memory while they run: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 * results, cache update and sticky errors as kvdecode_append_attend, and it
 * calls no hipMalloc, hipFree or other allocating routine: the step's
 * workspace (split partials, their log-sum-exps, attended lengths, the
 * per-sequence counters of one-split passes -- zero when the array is
 * loaded and again after every step -- and the error word) is a static
 * device array of KVD_NOALLOC_SCRATCH_MIB MiB that
 * every GPU the library runs on holds until the process ends.  A step that
 * needs more (about B * Hq * splits * head_dim * 2 bytes of partials,
 * 4 bytes per element for fp32) returns KVD_ESCRATCH and launches nothing.
 * The handle's own workspace is not used, so a handle created by
 * kvdecode_create can take these steps without ever allocating.
 * Every call on one GPU shares that GPU's array: calls that overlap on a GPU
 * (on unordered streams, from any handle) race and must be serialised by
 * the caller.  The array keeps the last call's contents; the sticky error
 * word in it collects the errors of every such step on that GPU until a
 * kvdecode_status call on a handle that ran one reads and clears it.  Steps
 * dispatch the batch in its own order (the handle's length-sorted dispatch
 * order needs workspace kept between steps).  Timing events are not
 * recorded.  Argument checks and return codes otherwise as for
 * kvdecode_append_attend.
 */
enum { KVD_NOALLOC_SCRATCH_MIB = 32 };
int32_t kvdecode_append_attend_noalloc(kvdecode_t h, const void* k_new, const void* v_new, const void* q,
                                       void* out, float scale, void* stream);

/*
 * Synchronise `stream`, then report and clear the sticky device error:
 * KVD_OK, KVD_ECAPACITY, KVD_ELENGTH or KVD_EPAGE (in that order of
 * precedence when several occurred).  For a handle that ran allocation-free
 * steps it also reads and clears the error word of the current device's
 * static buffer (shared by every such step on that GPU).  Returns KVD_OK
 * without a device call if the handle has never touched a device.
 */
int32_t kvdecode_status(kvdecode_t h, void* stream);

/*
 * Force the split count of the attend pass (0 restores the automatic plan).
 * Each sequence's cache is cut into tiles of the partial kernel (32 tokens,
 * or 64 for the vector-ALU and fp8 exchange kernels) dealt round-robin to
 * the splits: split s owns tiles s, s+S, s+2S, ...  n is clamped to
 * [1, ceil(T_cap / tile)].
 * Used to check that results do not depend on the split.
 */
int32_t kvdecode_set_num_splits(kvdecode_t h, int32_t n);

/*
 * Asynchronous softmax with a unified maximum (FlashDecoding++, "Asynchronous
 * softmax with unified max value", as summarised on the blog-aggregator
 * page): with enable != 0 every partial softmax of the LDS kernels starts
 * from the same reference phi -- a bound on the attention logits
 * scale * q.k chosen by the caller -- instead of its own first scores, and
 * keeps it unless a score exceeds phi by more than 64 / log2(e) (the
 * overflow fallback: that wave's reference is raised and its partial sums
 * rescaled); a split whose first scores all lie more than that below phi
 * starts from its own maximum instead (the underflow fallback).  Results
 * are those of the default mode up to rounding for any finite phi; a good
 * phi removes every rescale.  enable = 0 restores the default (each split's
 * reference starts at its first scores, raised past a 2^8 headroom).  The
 * VALU and MFMA kernels keep exact running maxima and ignore the setting.
 * KVD_EINVAL for a non-finite phi.
 */
int32_t kvdecode_set_unified_max(kvdecode_t h, int32_t enable, float phi);

/*
 * Choose the partial-pass kernel: KVD_VARIANT_AUTO (LDS for bf16, VALU for
 * fp32; for fp8 with d >= 128 WAVE when one workgroup holds the whole query
 * group -- up to 16 rows per KV head at d = 256, 48 at d = 128 -- else
 * XCHG, and LDS at d = 64), KVD_VARIANT_VALU (fp32 or bf16),
 * KVD_VARIANT_MFMA (bf16), KVD_VARIANT_LDS (bf16 or fp8),
 * KVD_VARIANT_WAVE or KVD_VARIANT_XCHG (fp8, d >= 128);
 * KVD_EUNSUPPORTED otherwise.
 */
int32_t kvdecode_set_variant(kvdecode_t h, int32_t variant);

/*
 * Report the current plan: variant in use, number of splits per
 * (sequence, KV head) and the most tokens any split holds when the cache
 * is full.  Any pointer may be NULL.
 */
int32_t kvdecode_get_plan(kvdecode_t h, int32_t* variant, int32_t* num_splits,
                          int32_t* split_tokens);

/*
 * The plan of a step with n_tokens new tokens per sequence
 * (kvdecode_append_attend_multi; n_tokens = 1 is kvdecode_get_plan's):
 * variant, splits per (sequence, KV head) and the most tokens any split
 * holds when the cache is full.  A step's query rows grow with n_tokens,
 * so its plan can differ from the one-token plan.  KVD_EINVAL for
 * n_tokens outside 1..KVD_MAX_NEW_TOKENS, KVD_EUNSUPPORTED when the chosen
 * kernel takes one token per step (KVD_VARIANT_MFMA with n_tokens > 1).
 * Makes no device call.  Any output pointer may be NULL.
 */
int32_t kvdecode_get_plan_multi(kvdecode_t h, int32_t n_tokens, int32_t* variant, int32_t* num_splits,
                                int32_t* split_tokens);

/*
 * Kernel timing with HIP events.  `what` picks the brackets: KVD_TIME_PARTIAL
 * the partial-pass kernel of each attend, KVD_TIME_COMBINE its combine
 * kernel (zero for a one-split pass, which launches none), KVD_TIME_APPEND
 * a separate append kernel.  The events ride on the timed launches (HIP's
 * extended launch stamps them with the kernel's start and end), so timing
 * adds no command to the stream and a bracket holds its kernel alone, not
 * the gaps between launches.
 * kvdecode_timing_enable(h, n, what) allocates n event slots (n = 0 or
 * what = 0 disables and frees them); at most n attends (and n appends) are
 * timed before the slots are full.  KVD_EINVAL for n < 0 or unknown bits.
 * kvdecode_timing_read synchronises the recorded events, returns the summed
 * durations in milliseconds (0 for a bracket not asked for) and the number
 * of timed attends and appends, and resets the slots.  Any output pointer
 * may be NULL.
 */
enum { KVD_TIME_PARTIAL = 1, KVD_TIME_COMBINE = 2, KVD_TIME_APPEND = 4, KVD_TIME_ALL = 7 };
int32_t kvdecode_timing_enable(kvdecode_t h, int32_t max_calls, int32_t what);
int32_t kvdecode_timing_read(kvdecode_t h, double* partial_ms, double* combine_ms,
                             double* append_ms, int32_t* n_attend, int32_t* n_append);

/* Free the handle's workspace and events; never frees caller memory.
 * Synchronises the device the handle is bound to first. */
int32_t kvdecode_destroy(kvdecode_t h);

/* Static description of a status code. */
const char* kvdecode_strerror(int32_t code);

#ifdef __cplusplus
}
#endif

#endif /* KVDECODE_H */
