/*
 * oracle/ref_decode.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU oracle for grouped-query decode attention over a
 * paged KV cache. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. It shares no code, header, table
 * or helper with the HIP library under paged_kv_split_amd/.
 *
 * What it computes is the plain definition of the operation, not the
 * split/online algorithm that the GPU path uses. In exact arithmetic the
 * online-softmax recurrence (FlashQuant wiki "CUDA Kernels", section
 * "flash_attention.cu", Online Softmax) and the split merge (same page,
 * "split_k_reduce.cu", Algorithm) reach exactly this value:
 *
 *   for each sequence b and query head h:
 *     kvh  = h / (Hq / Hkv)                (same page, GQA Support)
 *     L    = context_lens[b]
 *     for t in [0, L):
 *       page = block_table[b][t / P], slot = t mod P
 *                                          (same page, "paged_decode.cu",
 *                                           Page Table Addressing)
 *       k_t  = K[page][slot][kvh][:],  v_t = V[page][slot][kvh][:]
 *       s_t  = scale * sum_d q[b][h][d] * k_t[d]
 *                                          (AstrAI "CUDA Kernels", Python
 *                                           Wrappers: scale 1/sqrt(head_dim))
 *     M = max_t s_t,  w_t = exp(s_t - M),  Z = sum_t w_t
 *     out[b][h][:] = sum_t w_t * v_t / Z
 *     lse[b][h]    = M + ln Z
 *   L == 0 gives out = 0 and lse = -inf (the empty-split sentinel and the
 *   zero-denominator guard of the FlashQuant page, taken together).
 *
 * KV element kinds:
 *   kind 0: bf16 bit patterns (uint16). bf16 -> double is exact.
 *   kind 1: OCP E4M3FN codes (uint8) with one fp32 scale per (token, kv head)
 *           and separate k_scale / v_scale arrays [num_pages][P][Hkv]
 *           (OASR "Kernel Layer", FP8 KV variants; DeepGEMM docs, section
 *           6.1, non-MX per-token fp32 kv scale). Dequantised value =
 *           decode(code) * scale, formed in double, which is exact.
 *
 * Everything is accumulated in double. Work is spread over (b, h) pairs on
 * POSIX threads; each pair is computed by the same sequential loop, so the
 * thread count does not change any result bit.
 */
#define _GNU_SOURCE
#include <math.h>
#include <pthread.h>
#include <sched.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef struct oracle_problem {
    int32_t batch;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t page_size;
    int32_t max_pages_per_seq;
    int32_t num_pages;
    int32_t kv_kind;      /* 0 = bf16 bits, 1 = e4m3fn codes + fp32 scales */
    double scale;
} oracle_problem;

/* bf16 is the upper half of an IEEE binary32; widening to double is exact. */
static double bf16_bits_to_double(uint16_t bits) {
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP 8-bit floating point, E4M3FN variant: 1 sign bit, 4 exponent bits with
 * bias 7, 3 mantissa bits; exponent field 0 encodes subnormals m/8 * 2^-6;
 * the all-ones pattern (exponent 15, mantissa 7) is NaN; there is no
 * infinity, so exponent 15 with mantissa 0..6 is an ordinary normal number
 * (largest finite magnitude 1.75 * 2^8 = 448). */
double oracle_e4m3fn_to_double(uint8_t code) {
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);            /* (m / 8) * 2^(1 - 7) */
    else
        mag = ldexp((double)(8 + m), e - 10);  /* (1 + m / 8) * 2^(e - 7) */
    return sign ? -mag : mag;
}

typedef struct oracle_job {
    const oracle_problem* p;
    const uint16_t* q;             /* bf16 bits [B][Hq][d] */
    const void* k;                 /* kind 0: uint16 bits, kind 1: uint8 codes */
    const void* v;
    const float* k_scale;          /* kind 1 only: [num_pages][P][Hkv] */
    const float* v_scale;
    const int32_t* block_table;    /* [B][max_pages_per_seq] */
    const int32_t* context_lens;   /* [B] */
    double* out;                   /* [B][Hq][d] */
    double* lse;                   /* [B][Hq] */
    int64_t next_pair;             /* shared work counter */
    pthread_mutex_t lock;
    int error;                     /* first error seen: 0 = none */
} oracle_job;

/* Element d of row (page, slot, kvh) of a pool, as an exact double. */
static double kv_element(const oracle_problem* p, const void* pool,
                         const float* scales, int64_t page, int64_t slot,
                         int64_t kvh, int64_t d) {
    int64_t row = (page * p->page_size + slot) * p->num_kv_heads + kvh;
    int64_t idx = row * p->head_dim + d;
    if (p->kv_kind == 0) return bf16_bits_to_double(((const uint16_t*)pool)[idx]);
    return oracle_e4m3fn_to_double(((const uint8_t*)pool)[idx]) * (double)scales[row];
}

/* One (b, h) pair, straight from the definition. Returns 0 or an error code. */
static int decode_pair(oracle_job* job, int64_t b, int64_t h, double* scores) {
    const oracle_problem* p = job->p;
    const int64_t D = p->head_dim;
    const int64_t group = p->num_q_heads / p->num_kv_heads;
    const int64_t kvh = h / group;
    const int64_t L = job->context_lens[b];
    const uint16_t* qrow = job->q + (b * p->num_q_heads + h) * D;
    double* orow = job->out + (b * p->num_q_heads + h) * D;
    double M, Z;
    int64_t t, d;

    if (L == 0) {
        for (d = 0; d < D; ++d) orow[d] = 0.0;
        job->lse[b * p->num_q_heads + h] = -INFINITY;
        return 0;
    }
    /* scores */
    for (t = 0; t < L; ++t) {
        int64_t logical = t / p->page_size;
        int64_t slot = t % p->page_size;
        int64_t page = job->block_table[b * p->max_pages_per_seq + logical];
        double dot = 0.0;
        if (page < 0 || page >= p->num_pages) return 3;
        for (d = 0; d < D; ++d)
            dot += bf16_bits_to_double(qrow[d]) *
                   kv_element(p, job->k, job->k_scale, page, slot, kvh, d);
        scores[t] = p->scale * dot;
    }
    /* softmax */
    M = scores[0];
    for (t = 1; t < L; ++t)
        if (scores[t] > M) M = scores[t];
    Z = 0.0;
    for (t = 0; t < L; ++t) {
        scores[t] = exp(scores[t] - M);   /* now the unnormalised weight w_t */
        Z += scores[t];
    }
    /* weighted sum of V rows */
    for (d = 0; d < D; ++d) orow[d] = 0.0;
    for (t = 0; t < L; ++t) {
        int64_t page = job->block_table[b * p->max_pages_per_seq + t / p->page_size];
        int64_t slot = t % p->page_size;
        for (d = 0; d < D; ++d)
            orow[d] += scores[t] * kv_element(p, job->v, job->v_scale, page, slot, kvh, d);
    }
    for (d = 0; d < D; ++d) orow[d] /= Z;
    job->lse[b * p->num_q_heads + h] = M + log(Z);
    return 0;
}

static void* worker(void* arg) {
    oracle_job* job = (oracle_job*)arg;
    const oracle_problem* p = job->p;
    const int64_t pairs = (int64_t)p->batch * p->num_q_heads;
    int64_t max_len = 1, b;
    double* scores;
    for (b = 0; b < p->batch; ++b)
        if (job->context_lens[b] > max_len) max_len = job->context_lens[b];
    scores = (double*)malloc((size_t)max_len * sizeof(double));
    if (!scores) {
        pthread_mutex_lock(&job->lock);
        if (!job->error) job->error = 4;
        pthread_mutex_unlock(&job->lock);
        return NULL;
    }
    for (;;) {
        int64_t pair;
        int rc;
        pthread_mutex_lock(&job->lock);
        pair = job->next_pair++;
        pthread_mutex_unlock(&job->lock);
        if (pair >= pairs) break;
        rc = decode_pair(job, pair / p->num_q_heads, pair % p->num_q_heads, scores);
        if (rc) {
            pthread_mutex_lock(&job->lock);
            if (!job->error) job->error = rc;
            pthread_mutex_unlock(&job->lock);
        }
    }
    free(scores);
    return NULL;
}

/* Number of CPUs this process may run on. */
int oracle_available_threads(void) {
    cpu_set_t set;
    CPU_ZERO(&set);
    if (sched_getaffinity(0, sizeof set, &set) == 0) {
        int n = CPU_COUNT(&set);
        if (n > 0) return n;
    }
    return 1;
}

/*
 * Returns 0 on success; 1 bad shape; 2 context length beyond the block table;
 * 3 block_table entry outside [0, num_pages); 4 out of memory.
 * threads <= 0 uses every CPU in the affinity mask. *threads_used receives
 * the number of threads started (may be NULL).
 */
int oracle_decode(const oracle_problem* p, const uint16_t* q, const void* k_pool,
                  const void* v_pool, const float* k_scale, const float* v_scale,
                  const int32_t* block_table, const int32_t* context_lens,
                  double* out, double* lse, int threads, int* threads_used) {
    oracle_job job;
    pthread_t* tids;
    int i, n, b;
    if (!p || !q || !k_pool || !v_pool || !block_table || !context_lens || !out || !lse) return 1;
    if (p->batch < 0 || p->num_q_heads <= 0 || p->num_kv_heads <= 0 || p->head_dim <= 0 ||
        p->page_size <= 0 || p->max_pages_per_seq < 0 || p->num_pages < 0)
        return 1;
    if (p->num_q_heads % p->num_kv_heads != 0) return 1;
    if (p->kv_kind != 0 && p->kv_kind != 1) return 1;
    if (p->kv_kind == 1 && (!k_scale || !v_scale)) return 1;
    for (b = 0; b < p->batch; ++b) {
        int64_t L = context_lens[b];
        if (L < 0) return 1;
        if (L > (int64_t)p->max_pages_per_seq * p->page_size) return 2;
    }
    memset(&job, 0, sizeof job);
    job.p = p;
    job.q = q;
    job.k = k_pool;
    job.v = v_pool;
    job.k_scale = k_scale;
    job.v_scale = v_scale;
    job.block_table = block_table;
    job.context_lens = context_lens;
    job.out = out;
    job.lse = lse;
    pthread_mutex_init(&job.lock, NULL);
    n = threads > 0 ? threads : oracle_available_threads();
    if ((int64_t)n > (int64_t)p->batch * p->num_q_heads) n = (int)((int64_t)p->batch * p->num_q_heads);
    if (n < 1) n = 1;
    tids = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)n);
    if (!tids) return 4;
    for (i = 0; i < n; ++i)
        if (pthread_create(&tids[i], NULL, worker, &job) != 0) break;
    if (i == 0) worker(&job);
    n = i > 0 ? i : 1;
    for (int j = 0; j < i; ++j) pthread_join(tids[j], NULL);
    free(tids);
    pthread_mutex_destroy(&job.lock);
    if (threads_used) *threads_used = n;
    return job.error;
}
