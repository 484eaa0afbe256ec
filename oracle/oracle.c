/*
 * oracle.c -- plain, slow, fp64 CPU oracle for single-token decode attention
 * over a KV cache with multiquery / grouped-query head sharing.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the GPU library; it includes only the C
 * standard library and pthreads.
 *
 * What it computes (the plain definition; no blocking, no splitting, no
 * base-2 exponentials):
 *
 *   For every sequence b and query head h, with group size M = Hq / Hkv and
 *   KV head g = floor(h / M):
 *     n      = lengths[b]                       (valid cached tokens)
 *     s_t    = scale * sum_j q[b,h,j] * K[b,g,t,j]          t = 0 .. n-1
 *     p      = softmax over t of s                 (max-subtracted exp)
 *     out[b,h,:] = sum_t p_t * V[b,g,t,:]
 *   and out[b,h,:] = 0 when n == 0.
 *
 * Sources (pages, not code):
 *   - Multiquery attention: every query head reads one shared key/value head
 *     ("Efficiently Scaling Transformer Inference", section 3.3 "Partitioning
 *     the attention layer").
 *   - Grouped-query attention: Hkv key/value heads each shared by Hq/Hkv query
 *     heads ("All About Transformer Inference", section on tricks for improving
 *     generation throughput and latency, GQA paragraph).
 *   - The grouped contraction: Q[B,N,H] is reshaped row-major to Q[B,K,M,H]
 *     (so query head h belongs to KV head floor(h/M)), contracted over H with
 *     K[B,S,K,H], softmaxed over S, contracted over S with V
 *     ("All About Transformer Inference", section "Sharding the KV cache",
 *     the full attention algorithm).
 *   - Decode semantics: the new token's query attends the cached keys and
 *     values of the tokens before it, which the cache holds
 *     ("All About Transformer Inference", section "Transformer inference
 *     basics", KV cache paragraph).
 *   - Ragged lengths: only the non-padding part of each sequence's cache is
 *     read ("All About Transformer Inference", section on tricks, ragged HBM
 *     reads and paged attention paragraph).
 *   - The scale 1/sqrt(d) is not printed on the pages; it is passed in.
 *
 * Input encodings: dtype 0 = IEEE binary32 (float*), dtype 1 = bfloat16 given
 * as raw 16-bit patterns (uint16_t*).  Both are widened to fp64 exactly.
 *
 * Build: gcc -O2 -shared -fPIC -pthread oracle.c -o liboracle.so -lm
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_ENOMEM (-2)

/* Exact widening of one stored element to fp64. */
static double widen(const void* base, int dtype, size_t idx) {
    if (dtype == 0) {
        return (double)((const float*)base)[idx];
    }
    uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

typedef struct {
    int B, Hq, Hkv, D, T_cap, dtype;
    const void* q;
    const void* k;
    const void* v;
    const int32_t* lengths;
    double scale;
    const int32_t* rows; /* flattened b*Hq + h, or NULL for all */
    int n_rows;
    double* out;         /* [n_rows, D] */
    int next;            /* shared work counter (guarded by mu) */
    pthread_mutex_t mu;
    int status;
} job_t;

/* One output row: out[b,h,:] for query head h of sequence b. */
static void attend_row(const job_t* J, int b, int h, double* s, double* o) {
    const int D = J->D;
    const int M = J->Hq / J->Hkv;
    const int g = h / M; /* row-major reshape of the head axis into [Hkv, M] */
    const int n = J->lengths[b];

    for (int j = 0; j < D; ++j) o[j] = 0.0;
    if (n == 0) return; /* empty sequence: zero row by convention */

    const size_t qoff = ((size_t)b * J->Hq + h) * (size_t)D;
    const size_t kvoff = ((size_t)b * J->Hkv + g) * (size_t)J->T_cap * (size_t)D;

    /* scores: contraction over the head dimension */
    for (int t = 0; t < n; ++t) {
        double acc = 0.0;
        for (int j = 0; j < D; ++j) {
            acc += widen(J->q, J->dtype, qoff + j) *
                   widen(J->k, J->dtype, kvoff + (size_t)t * D + j);
        }
        s[t] = J->scale * acc;
    }

    /* softmax over the sequence axis */
    double mx = s[0];
    for (int t = 1; t < n; ++t)
        if (s[t] > mx) mx = s[t];
    double z = 0.0;
    for (int t = 0; t < n; ++t) {
        s[t] = exp(s[t] - mx);
        z += s[t];
    }
    for (int t = 0; t < n; ++t) s[t] /= z;

    /* contraction over the sequence axis with the values */
    for (int t = 0; t < n; ++t) {
        const double p = s[t];
        for (int j = 0; j < D; ++j) {
            o[j] += p * widen(J->v, J->dtype, kvoff + (size_t)t * D + j);
        }
    }
}

static void* worker(void* arg) {
    job_t* J = (job_t*)arg;
    double* s = (double*)malloc(sizeof(double) * (size_t)(J->T_cap > 0 ? J->T_cap : 1));
    if (!s) {
        pthread_mutex_lock(&J->mu);
        J->status = ORACLE_ENOMEM;
        pthread_mutex_unlock(&J->mu);
        return NULL;
    }
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int r = J->next++;
        pthread_mutex_unlock(&J->mu);
        if (r >= J->n_rows) break;
        int flat = J->rows ? J->rows[r] : r;
        int b = flat / J->Hq, h = flat % J->Hq;
        attend_row(J, b, h, s, J->out + (size_t)r * J->D);
    }
    free(s);
    return NULL;
}

/*
 * Decode attention for the listed rows (flattened b*Hq + h), or for all
 * B*Hq rows when rows == NULL.  out receives n_rows x D doubles in the
 * order the rows are listed.  Returns 0, or a negative code for invalid
 * arguments (every length must lie in [0, T_cap]).
 */
int oracle_decode_attention(int B, int Hq, int Hkv, int D, int T_cap, int dtype,
                            const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* lengths, double scale,
                            const int32_t* rows, int n_rows, double* out,
                            int n_threads) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || T_cap < 0) return ORACLE_EINVAL;
    if (Hq % Hkv != 0) return ORACLE_EINVAL;
    if (dtype != 0 && dtype != 1) return ORACLE_EINVAL;
    if (!q || !k_cache || !v_cache || !lengths || !out) return ORACLE_EINVAL;
    for (int b = 0; b < B; ++b)
        if (lengths[b] < 0 || lengths[b] > T_cap) return ORACLE_EINVAL;
    if (!rows) n_rows = B * Hq;
    for (int r = 0; rows && r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= B * Hq) return ORACLE_EINVAL;
    if (n_threads < 1) n_threads = 1;
    if (n_threads > 256) n_threads = 256;

    job_t J;
    J.B = B; J.Hq = Hq; J.Hkv = Hkv; J.D = D; J.T_cap = T_cap; J.dtype = dtype;
    J.q = q; J.k = k_cache; J.v = v_cache; J.lengths = lengths; J.scale = scale;
    J.rows = rows; J.n_rows = n_rows; J.out = out; J.next = 0; J.status = ORACLE_OK;
    pthread_mutex_init(&J.mu, NULL);

    pthread_t tid[256];
    int started = 0;
    for (int i = 0; i < n_threads; ++i) {
        if (pthread_create(&tid[i], NULL, worker, &J) != 0) break;
        ++started;
    }
    if (started == 0) worker(&J);
    for (int i = 0; i < started; ++i) pthread_join(tid[i], NULL);
    pthread_mutex_destroy(&J.mu);
    return J.status;
}
