/*
 * pkv_oracle.c -- TEST INFRASTRUCTURE, NOT PRODUCT CODE.
 *
 * A plain, slow, obviously correct host implementation of paged-KV-cache
 * store and attention, in fp64.  It exists only so that tests, the smoke
 * check and the benchmark's CPU-baseline leg can judge the GPU kernels.  It
 * shares no code, header, table or helper with the GPU library and includes
 * nothing from it; the product path never calls it.
 *
 * Pages it follows (titles as printed on the pages):
 *   [NV2]  "Nano-vLLM Part 2: model internals, KV cache and tensor
 *          parallelism" (seekfood.cn/news/749872)
 *   [NVE]  "Nano-vLLM engine deep-dive: from 'it runs' to 'it runs well'"
 *          (mhpq.cn/news/130328)
 *   [LLM4] "LLM basics primer: from text to token, embedding, QKV and
 *          Transformer, part 4" (CSDN; qwbw.cn/news/156881)
 *
 * Layouts (the pages name the dimensions Block / Layer / K-V / Token in
 * [NV2] §05.2 but not their order; this is the reading taken):
 *   k_cache, v_cache : bf16 bits [num_blocks][num_kv_heads][block_size][head_dim]
 *                      (one array per layer and per K/V)
 *   k, v (new)       : bf16 bits [num_tokens][num_kv_heads][head_dim]
 *   slot_mapping     : int32 [num_tokens]; slot = block * block_size + offset,
 *                      slot < 0 means "no token here" (padding)
 *   q (decode)       : bf16 bits [num_seqs][num_q_heads][head_dim]
 *   q (prefill)      : bf16 bits [total_new][num_q_heads][head_dim], prompts packed
 *   block_tables     : int32 [num_seqs][max_blocks_per_seq]
 *   context_lens     : int32 [num_seqs], tokens in the cache AFTER the store
 *   out              : double [rows][num_q_heads][head_dim]
 *
 * Parity pins for every function live in tests/ (see the test file for the
 * list); none of them compares this file with itself.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#include "pkv_oracle.h"

/* A bf16 value is the upper 16 bits of an IEEE binary32; widen, then to double. */
static double bf16_bits_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * KV-cache bytes: 2 (one K and one V) x layers x KV heads (not query heads)
 * x head_dim x cached tokens x bytes per element.
 * [LLM4] §17.3 (general formula, "2 means K and V", "num_kv_heads is the KV
 * head count, not the Q head count") and §17.6 (cached_tokens is the sum of
 * every request's cached tokens).
 */
uint64_t pko_kv_bytes(int32_t num_layers, int32_t num_kv_heads, int32_t head_dim,
                      int64_t cached_tokens, int32_t bytes_per_element)
{
    if (num_layers < 0 || num_kv_heads < 0 || head_dim < 0 || cached_tokens < 0 ||
        bytes_per_element < 0)
        return 0;
    return (uint64_t)2 * (uint64_t)num_layers * (uint64_t)num_kv_heads *
           (uint64_t)head_dim * (uint64_t)cached_tokens * (uint64_t)bytes_per_element;
}

/*
 * Store: each new token's K and V go to the cache position its slot names.
 * [NVE] §2.1 (decode appends the new token's K and V to the cache), §2.2
 * (fixed-size blocks, managed "by block or by slot"); [NV2] §05.3 (a kernel
 * writes new K/V into the cache).  A slot below zero is skipped.  Slots that
 * repeat within one call, or that fall outside the pool, are rejected before
 * anything is written.
 */
int pko_store(const uint16_t *k, const uint16_t *v, const int32_t *slot_mapping,
              int32_t num_tokens, uint16_t *k_cache, uint16_t *v_cache,
              int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
              int32_t block_size)
{
    if (num_tokens < 0 || num_blocks < 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0)
        return PKO_ERR_ARG;
    if (num_tokens == 0)
        return PKO_OK;
    if (!k || !v || !slot_mapping || !k_cache || !v_cache)
        return PKO_ERR_ARG;

    int64_t num_slots = (int64_t)num_blocks * block_size;
    unsigned char *seen = calloc((size_t)(num_slots > 0 ? num_slots : 1), 1);
    if (!seen)
        return PKO_ERR_ALLOC;
    for (int32_t i = 0; i < num_tokens; ++i) {
        int32_t slot = slot_mapping[i];
        if (slot < 0)
            continue;
        if ((int64_t)slot >= num_slots) {
            free(seen);
            return PKO_ERR_RANGE;
        }
        if (seen[slot]) {
            free(seen);
            return PKO_ERR_DUPLICATE;
        }
        seen[slot] = 1;
    }
    free(seen);

    for (int32_t i = 0; i < num_tokens; ++i) {
        int32_t slot = slot_mapping[i];
        if (slot < 0)
            continue;
        int64_t block = slot / block_size;
        int64_t offset = slot % block_size;
        for (int32_t h = 0; h < num_kv_heads; ++h) {
            for (int32_t x = 0; x < head_dim; ++x) {
                int64_t src = ((int64_t)i * num_kv_heads + h) * head_dim + x;
                int64_t dst = ((block * num_kv_heads + h) * block_size + offset) * head_dim + x;
                k_cache[dst] = k[src];
                v_cache[dst] = v[src];
            }
        }
    }
    return PKO_OK;
}

/*
 * One query row against keys 0..n-1 of one sequence, read through its block
 * table:  out = softmax(scale * q . K^T) V, the scaled dot-product attention
 * of [NVE] §3 and [LLM4] §21.1, computed as its definition in fp64:
 *   score_t = scale * sum_x q[x] * K_t[x]
 *   M = max_t score_t          (the max subtraction of [NVE] §3.2)
 *   w_t = exp(score_t - M),  Z = sum_t w_t
 *   out[x] = sum_t w_t * V_t[x] / Z
 * Token t of the sequence lives in physical block block_table[t / block_size]
 * at offset t % block_size ([NVE] §2.2, [LLM4] §17.7 block table).  The K/V
 * head is the query head's group: kv = h / (num_q_heads / num_kv_heads)
 * ([LLM4] §21.1: grouped-query attention shares KV heads).  n == 0 gives 0.
 */
static void attend_one(const uint16_t *q_row, const uint16_t *k_cache,
                       const uint16_t *v_cache, const int32_t *block_table,
                       int32_t n, int32_t kv_head, int32_t num_kv_heads,
                       int32_t head_dim, int32_t block_size, double scale,
                       double *scores, double *out_row)
{
    for (int32_t x = 0; x < head_dim; ++x)
        out_row[x] = 0.0;
    if (n <= 0)
        return;

    for (int32_t t = 0; t < n; ++t) {
        int64_t block = block_table[t / block_size];
        int64_t offset = t % block_size;
        const uint16_t *key =
            k_cache + ((block * num_kv_heads + kv_head) * block_size + offset) * head_dim;
        double dot = 0.0;
        for (int32_t x = 0; x < head_dim; ++x)
            dot += bf16_bits_to_double(q_row[x]) * bf16_bits_to_double(key[x]);
        scores[t] = scale * dot;
    }

    double m = scores[0];
    for (int32_t t = 1; t < n; ++t)
        if (scores[t] > m)
            m = scores[t];

    double z = 0.0;
    for (int32_t t = 0; t < n; ++t) {
        scores[t] = exp(scores[t] - m);
        z += scores[t];
    }

    for (int32_t t = 0; t < n; ++t) {
        int64_t block = block_table[t / block_size];
        int64_t offset = t % block_size;
        const uint16_t *value =
            v_cache + ((block * num_kv_heads + kv_head) * block_size + offset) * head_dim;
        for (int32_t x = 0; x < head_dim; ++x)
            out_row[x] += scores[t] * bf16_bits_to_double(value[x]);
    }
    for (int32_t x = 0; x < head_dim; ++x)
        out_row[x] /= z;
}

/*
 * attend_one on a cache whose values are already fp64 (a dequantized FP8
 * cache, see pko_prefill_fp8): the same definition, the key and value rows
 * read from kd / vd, which hold [num_blocks][num_kv_heads][block_size]
 * [head_dim] doubles.
 */
static void attend_one_f64(const uint16_t *q_row, const double *kd, const double *vd,
                           const int32_t *block_table, int32_t n, int32_t kv_head,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           double scale, double *scores, double *out_row)
{
    for (int32_t x = 0; x < head_dim; ++x)
        out_row[x] = 0.0;
    if (n <= 0)
        return;

    for (int32_t t = 0; t < n; ++t) {
        int64_t row = ((int64_t)block_table[t / block_size] * num_kv_heads + kv_head) *
                          block_size + t % block_size;
        double dot = 0.0;
        for (int32_t x = 0; x < head_dim; ++x)
            dot += bf16_bits_to_double(q_row[x]) * kd[row * head_dim + x];
        scores[t] = scale * dot;
    }

    double m = scores[0];
    for (int32_t t = 1; t < n; ++t)
        if (scores[t] > m)
            m = scores[t];

    double z = 0.0;
    for (int32_t t = 0; t < n; ++t) {
        scores[t] = exp(scores[t] - m);
        z += scores[t];
    }

    for (int32_t t = 0; t < n; ++t) {
        int64_t row = ((int64_t)block_table[t / block_size] * num_kv_heads + kv_head) *
                          block_size + t % block_size;
        for (int32_t x = 0; x < head_dim; ++x)
            out_row[x] += scores[t] * vd[row * head_dim + x];
    }
    for (int32_t x = 0; x < head_dim; ++x)
        out_row[x] /= z;
}

/* ---- a minimal static thread split over independent (sequence, kv head) units ---- */

typedef struct {
    int mode; /* 0 = decode, 1 = prefill, 2 = prefill over fp64 kd / vd */
    const uint16_t *q, *k_cache, *v_cache;
    const double *kd, *vd;
    const int32_t *block_tables, *context_lens, *cu_new_lens;
    int32_t max_blocks_per_seq, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size;
    double scale;
    double *out;
    int32_t max_context_len;
    int nthreads, tid;
    int status;
} work_t;

static void run_unit(work_t *w, int32_t s, int32_t kvh, double *scores)
{
    int32_t group = w->num_q_heads / w->num_kv_heads;
    const int32_t *bt = w->block_tables + (int64_t)s * w->max_blocks_per_seq;
    int32_t ctx = w->context_lens[s];
    for (int32_t g = 0; g < group; ++g) {
        int32_t h = kvh * group + g;
        if (w->mode == 0) {
            const uint16_t *q_row = w->q + ((int64_t)s * w->num_q_heads + h) * w->head_dim;
            double *o = w->out + ((int64_t)s * w->num_q_heads + h) * w->head_dim;
            attend_one(q_row, w->k_cache, w->v_cache, bt, ctx, kvh, w->num_kv_heads,
                       w->head_dim, w->block_size, w->scale, scores, o);
        } else {
            /* Chunked causal prefill: prompt s has n new tokens after c cached
             * ones (c = ctx - n); new token i sits at position c + i and sees
             * keys 0..c+i inclusive -- it sees itself and what came before,
             * never what follows ([NVE] §3.2 causal mask; [LLM4] §22 steps 6-8,
             * where the middle token attends to the first and itself and the
             * later token's weight is exactly 0). */
            int32_t row0 = w->cu_new_lens[s];
            int32_t n = w->cu_new_lens[s + 1] - row0;
            int32_t c = ctx - n;
            for (int32_t i = 0; i < n; ++i) {
                const uint16_t *q_row =
                    w->q + ((int64_t)(row0 + i) * w->num_q_heads + h) * w->head_dim;
                double *o = w->out + ((int64_t)(row0 + i) * w->num_q_heads + h) * w->head_dim;
                if (w->mode != 2)
                    attend_one(q_row, w->k_cache, w->v_cache, bt, c + i + 1, kvh,
                               w->num_kv_heads, w->head_dim, w->block_size, w->scale, scores, o);
                else
                    attend_one_f64(q_row, w->kd, w->vd, bt, c + i + 1, kvh, w->num_kv_heads,
                                   w->head_dim, w->block_size, w->scale, scores, o);
            }
        }
    }
}

static void *thread_main(void *arg)
{
    work_t *w = (work_t *)arg;
    double *scores = malloc(sizeof(double) * (size_t)(w->max_context_len > 0 ? w->max_context_len : 1));
    if (!scores) {
        w->status = PKO_ERR_ALLOC;
        return NULL;
    }
    int64_t units = (int64_t)w->num_seqs * w->num_kv_heads;
    for (int64_t u = w->tid; u < units; u += w->nthreads)
        run_unit(w, (int32_t)(u / w->num_kv_heads), (int32_t)(u % w->num_kv_heads), scores);
    free(scores);
    return NULL;
}

int pko_default_threads(void)
{
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

static int run_threads(work_t *proto, int nthreads)
{
    if (nthreads <= 0)
        nthreads = pko_default_threads();
    int64_t units = (int64_t)proto->num_seqs * proto->num_kv_heads;
    if (units < nthreads)
        nthreads = units > 0 ? (int)units : 1;
    work_t *ws = calloc((size_t)nthreads, sizeof(work_t));
    pthread_t *th = calloc((size_t)nthreads, sizeof(pthread_t));
    if (!ws || !th) {
        free(ws);
        free(th);
        return PKO_ERR_ALLOC;
    }
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        ws[t] = *proto;
        ws[t].nthreads = nthreads;
        ws[t].tid = t;
        ws[t].status = PKO_OK;
        if (t == 0)
            continue;
        if (pthread_create(&th[t], NULL, thread_main, &ws[t]) != 0)
            break;
        started = t;
    }
    /* threads 1..started run in parallel; thread 0's share runs here, and any
     * share whose thread failed to start runs here too */
    thread_main(&ws[0]);
    for (int t = started + 1; t < nthreads; ++t)
        thread_main(&ws[t]);
    for (int t = 1; t <= started; ++t)
        pthread_join(th[t], NULL);
    int status = PKO_OK;
    for (int t = 0; t < nthreads; ++t)
        if (ws[t].status != PKO_OK)
            status = ws[t].status;
    free(ws);
    free(th);
    return status;
}

static int check_common(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                        const int32_t *block_tables, const int32_t *context_lens,
                        int32_t num_blocks, int32_t *max_ctx_out)
{
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0 || max_blocks_per_seq < 0 || num_blocks < 0)
        return PKO_ERR_ARG;
    if (num_q_heads % num_kv_heads != 0)
        return PKO_ERR_ARG;
    int32_t max_ctx = 0;
    for (int32_t s = 0; s < num_seqs; ++s) {
        int32_t ctx = context_lens[s];
        if (ctx < 0 || (int64_t)ctx > (int64_t)max_blocks_per_seq * block_size)
            return PKO_ERR_RANGE;
        int32_t used = (ctx + block_size - 1) / block_size;
        for (int32_t b = 0; b < used; ++b) {
            int32_t id = block_tables[(int64_t)s * max_blocks_per_seq + b];
            if (id < 0 || id >= num_blocks)
                return PKO_ERR_RANGE;
        }
        if (ctx > max_ctx)
            max_ctx = ctx;
    }
    *max_ctx_out = max_ctx;
    return PKO_OK;
}

int pko_decode(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
               int32_t num_blocks, const int32_t *block_tables, int32_t max_blocks_per_seq,
               const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
               int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
               double *out, int nthreads)
{
    int32_t max_ctx = 0;
    if (num_seqs > 0 && (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out))
        return PKO_ERR_ARG;
    int rc = check_common(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                          max_blocks_per_seq, block_tables, context_lens, num_blocks, &max_ctx);
    if (rc != PKO_OK || num_seqs == 0)
        return rc;
    work_t w;
    memset(&w, 0, sizeof w);
    w.mode = 0;
    w.q = q;
    w.k_cache = k_cache;
    w.v_cache = v_cache;
    w.block_tables = block_tables;
    w.context_lens = context_lens;
    w.max_blocks_per_seq = max_blocks_per_seq;
    w.num_seqs = num_seqs;
    w.num_q_heads = num_q_heads;
    w.num_kv_heads = num_kv_heads;
    w.head_dim = head_dim;
    w.block_size = block_size;
    w.scale = (double)scale;
    w.out = out;
    w.max_context_len = max_ctx;
    return run_threads(&w, nthreads);
}

int pko_prefill(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                int32_t num_blocks, const int32_t *block_tables, int32_t max_blocks_per_seq,
                const int32_t *cu_new_lens, const int32_t *context_lens, int32_t num_seqs,
                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                int32_t block_size, float scale, double *out, int nthreads)
{
    int32_t max_ctx = 0;
    if (num_seqs > 0 && (!q || !k_cache || !v_cache || !block_tables || !context_lens ||
                         !cu_new_lens || !out))
        return PKO_ERR_ARG;
    int rc = check_common(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                          max_blocks_per_seq, block_tables, context_lens, num_blocks, &max_ctx);
    if (rc != PKO_OK || num_seqs == 0)
        return rc;
    if (cu_new_lens[0] != 0)
        return PKO_ERR_ARG;
    for (int32_t s = 0; s < num_seqs; ++s) {
        int32_t n = cu_new_lens[s + 1] - cu_new_lens[s];
        if (n < 0 || n > context_lens[s])
            return PKO_ERR_ARG;
    }
    work_t w;
    memset(&w, 0, sizeof w);
    w.mode = 1;
    w.q = q;
    w.k_cache = k_cache;
    w.v_cache = v_cache;
    w.block_tables = block_tables;
    w.context_lens = context_lens;
    w.cu_new_lens = cu_new_lens;
    w.max_blocks_per_seq = max_blocks_per_seq;
    w.num_seqs = num_seqs;
    w.num_q_heads = num_q_heads;
    w.num_kv_heads = num_kv_heads;
    w.head_dim = head_dim;
    w.block_size = block_size;
    w.scale = (double)scale;
    w.out = out;
    w.max_context_len = max_ctx;
    return run_threads(&w, nthreads);
}


/* ------------------------------------------------------------------------ */
/* FP8 KV cache                                                             */
/* ------------------------------------------------------------------------ */

/*
 * [LLM4] §17.6 counts an FP8 KV cache at 1 byte per element and lists
 * "whether to use an FP8 KV cache" among the memory levers; it fixes neither
 * the 8-bit format nor the scaling.  Reading taken here: OCP FP8 E4M3 (sign,
 * 4 exponent bits with bias 7, 3 mantissa bits; no infinities; S.1111.111 is
 * NaN; largest finite magnitude 448; subnormals m * 2^-9), with one fp32 scale
 * per (token, KV head): scale = amax / 448 over the head's head_dim values
 * (1 when they are all zero) and code = E4M3(x / scale) rounded to nearest,
 * ties to even, after clamping x / scale to [-448, 448].  Both divisions are
 * fp32 (correctly rounded), so the codes and scales are exact integers/bits
 * to compare.  The cached value is decode(code) * scale.
 */

/* Value of an E4M3 code (NaN for the two NaN codes). */
double pko_fp8_decode(uint8_t code)
{
    int sign = code >> 7;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);              /* subnormal: (m / 8) * 2^-6 */
    else
        v = ldexp(8.0 + (double)m, e - 10);    /* (1 + m / 8) * 2^(e - 7) */
    return sign ? -v : v;
}

/* Nearest E4M3 code to y (|y| <= 448 and finite), ties to the even code:
 * the candidates are the two representable magnitudes around |y| on the
 * grid whose spacing is that of |y|'s binade. */
uint8_t pko_fp8_encode(float y)
{
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    double a = fabs((double)y);
    /* spacing of the grid containing a: 2^-9 below 2^-6, else 2^(e-3) */
    int e;
    double spacing;
    if (a < ldexp(1.0, -6)) {
        spacing = ldexp(1.0, -9);
    } else {
        frexp(a, &e);                          /* a in [2^(e-1), 2^e) */
        spacing = ldexp(1.0, e - 1 - 3);
    }
    double lo = floor(a / spacing) * spacing;  /* exact: a / spacing has few bits */
    double hi = lo + spacing;
    double pick;
    if (a - lo < hi - a)
        pick = lo;
    else if (a - lo > hi - a)
        pick = hi;
    else  /* tie: the candidate whose mantissa field is even */
        pick = ((long long)(lo / spacing) % 2 == 0) ? lo : hi;
    /* code of the picked magnitude (pick <= 448 because a <= 448) */
    for (int c = 0; c < 0x7f; ++c)
        if (pko_fp8_decode((uint8_t)c) == pick)
            return (uint8_t)(sign | c);
    return (uint8_t)(sign | 0x7e);             /* not reached */
}

static float bf16_bits_to_float(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Quantize one head row of head_dim bf16 values to codes + scale. */
static void quantize_row(const uint16_t *x, int32_t head_dim, uint8_t *codes, float *scale_out)
{
    float amax = 0.0f;
    for (int32_t i = 0; i < head_dim; ++i) {
        float a = fabsf(bf16_bits_to_float(x[i]));
        if (a > amax)
            amax = a;
    }
    float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
    for (int32_t i = 0; i < head_dim; ++i) {
        float y = bf16_bits_to_float(x[i]) / scale;
        if (y > 448.0f)
            y = 448.0f;
        if (y < -448.0f)
            y = -448.0f;
        codes[i] = pko_fp8_encode(y);
    }
    *scale_out = scale;
}

/*
 * Store into an FP8 cache: like pko_store, but each (token, KV head) row is
 * quantized as described above.  codes: uint8 [num_blocks][num_kv_heads]
 * [block_size][head_dim]; scales: float [num_blocks][num_kv_heads][block_size].
 */
int pko_store_fp8(const uint16_t *k, const uint16_t *v, const int32_t *slot_mapping,
                  int32_t num_tokens, uint8_t *k_codes, uint8_t *v_codes, float *k_scales,
                  float *v_scales, int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                  int32_t block_size)
{
    if (num_tokens < 0 || num_blocks < 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0)
        return PKO_ERR_ARG;
    if (num_tokens == 0)
        return PKO_OK;
    if (!k || !v || !slot_mapping || !k_codes || !v_codes || !k_scales || !v_scales)
        return PKO_ERR_ARG;
    int64_t num_slots = (int64_t)num_blocks * block_size;
    unsigned char *seen = calloc((size_t)(num_slots > 0 ? num_slots : 1), 1);
    if (!seen)
        return PKO_ERR_ALLOC;
    for (int32_t i = 0; i < num_tokens; ++i) {
        int32_t slot = slot_mapping[i];
        if (slot < 0)
            continue;
        if ((int64_t)slot >= num_slots || seen[slot]) {
            free(seen);
            return (int64_t)slot >= num_slots ? PKO_ERR_RANGE : PKO_ERR_DUPLICATE;
        }
        seen[slot] = 1;
    }
    free(seen);
    for (int32_t i = 0; i < num_tokens; ++i) {
        int32_t slot = slot_mapping[i];
        if (slot < 0)
            continue;
        int64_t block = slot / block_size, offset = slot % block_size;
        for (int32_t h = 0; h < num_kv_heads; ++h) {
            int64_t src = ((int64_t)i * num_kv_heads + h) * head_dim;
            int64_t row = (block * num_kv_heads + h) * block_size + offset;
            quantize_row(k + src, head_dim, k_codes + row * head_dim, k_scales + row);
            quantize_row(v + src, head_dim, v_codes + row * head_dim, v_scales + row);
        }
    }
    return PKO_OK;
}

/* Dequantize an FP8 cache into fp64 (value = decode(code) * scale). */
static void dequantize(const uint8_t *codes, const float *scales, int64_t rows, int32_t head_dim,
                       double *out)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int32_t x = 0; x < head_dim; ++x)
            out[r * head_dim + x] = pko_fp8_decode(codes[r * head_dim + x]) * (double)scales[r];
}

/*
 * Decode attention over an FP8 cache: the scaled dot-product attention of
 * pko_decode on the cached values decode(code) * scale, in fp64.  The cache
 * is dequantized up front into fp64 arrays and attention runs on those.
 */
int pko_decode_fp8(const uint16_t *q, const uint8_t *k_codes, const uint8_t *v_codes,
                   const float *k_scales, const float *v_scales, int32_t num_blocks,
                   const int32_t *block_tables, int32_t max_blocks_per_seq,
                   const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
                   double *out)
{
    int32_t max_ctx = 0;
    if (num_seqs > 0 && (!q || !k_codes || !v_codes || !k_scales || !v_scales ||
                         !block_tables || !context_lens || !out))
        return PKO_ERR_ARG;
    int rc = check_common(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                          max_blocks_per_seq, block_tables, context_lens, num_blocks, &max_ctx);
    if (rc != PKO_OK || num_seqs == 0)
        return rc;
    int64_t rows = (int64_t)num_blocks * num_kv_heads * block_size;
    double *kd = malloc(sizeof(double) * (size_t)(rows > 0 ? rows : 1) * head_dim);
    double *vd = malloc(sizeof(double) * (size_t)(rows > 0 ? rows : 1) * head_dim);
    double *scores = malloc(sizeof(double) * (size_t)(max_ctx > 0 ? max_ctx : 1));
    if (!kd || !vd || !scores) {
        free(kd);
        free(vd);
        free(scores);
        return PKO_ERR_ALLOC;
    }
    dequantize(k_codes, k_scales, rows, head_dim, kd);
    dequantize(v_codes, v_scales, rows, head_dim, vd);
    int32_t group = num_q_heads / num_kv_heads;
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int32_t *bt = block_tables + (int64_t)s * max_blocks_per_seq;
        int32_t n = context_lens[s];
        for (int32_t h = 0; h < num_q_heads; ++h) {
            int32_t kvh = h / group;
            const uint16_t *q_row = q + ((int64_t)s * num_q_heads + h) * head_dim;
            double *o = out + ((int64_t)s * num_q_heads + h) * head_dim;
            for (int32_t x = 0; x < head_dim; ++x)
                o[x] = 0.0;
            if (n <= 0)
                continue;
            for (int32_t t = 0; t < n; ++t) {
                int64_t row = ((int64_t)bt[t / block_size] * num_kv_heads + kvh) * block_size +
                              t % block_size;
                double dot = 0.0;
                for (int32_t x = 0; x < head_dim; ++x)
                    dot += bf16_bits_to_double(q_row[x]) * kd[row * head_dim + x];
                scores[t] = (double)scale * dot;
            }
            double m = scores[0];
            for (int32_t t = 1; t < n; ++t)
                if (scores[t] > m)
                    m = scores[t];
            double z = 0.0;
            for (int32_t t = 0; t < n; ++t) {
                scores[t] = exp(scores[t] - m);
                z += scores[t];
            }
            for (int32_t t = 0; t < n; ++t) {
                int64_t row = ((int64_t)bt[t / block_size] * num_kv_heads + kvh) * block_size +
                              t % block_size;
                for (int32_t x = 0; x < head_dim; ++x)
                    o[x] += scores[t] * vd[row * head_dim + x];
            }
            for (int32_t x = 0; x < head_dim; ++x)
                o[x] /= z;
        }
    }
    free(kd);
    free(vd);
    free(scores);
    return PKO_OK;
}


/*
 * Chunked causal prefill over an FP8 cache: pko_prefill's definition (new
 * token i of prompt s at position c + i sees keys 0 .. c + i, [NVE] §3.2,
 * [LLM4] §22) on the cached values decode(code) * scale of [LLM4] §17.6's
 * FP8 cache (the reading above pko_fp8_decode), in fp64.  The cache is
 * dequantized up front into fp64 arrays; the prompts' (sequence, KV head)
 * units then run on nthreads threads (0 = one per online CPU) as in
 * pko_prefill.  Arguments as pko_prefill, with pko_decode_fp8's cache.
 */
int pko_prefill_fp8(const uint16_t *q, const uint8_t *k_codes, const uint8_t *v_codes,
                    const float *k_scales, const float *v_scales, int32_t num_blocks,
                    const int32_t *block_tables, int32_t max_blocks_per_seq,
                    const int32_t *cu_new_lens, const int32_t *context_lens, int32_t num_seqs,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, float scale, double *out, int nthreads)
{
    int32_t max_ctx = 0;
    if (num_seqs > 0 && (!q || !k_codes || !v_codes || !k_scales || !v_scales ||
                         !block_tables || !context_lens || !cu_new_lens || !out))
        return PKO_ERR_ARG;
    int rc = check_common(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                          max_blocks_per_seq, block_tables, context_lens, num_blocks, &max_ctx);
    if (rc != PKO_OK || num_seqs == 0)
        return rc;
    if (cu_new_lens[0] != 0)
        return PKO_ERR_ARG;
    for (int32_t s = 0; s < num_seqs; ++s) {
        int32_t n = cu_new_lens[s + 1] - cu_new_lens[s];
        if (n < 0 || n > context_lens[s])
            return PKO_ERR_ARG;
    }
    int64_t rows = (int64_t)num_blocks * num_kv_heads * block_size;
    double *kd = malloc(sizeof(double) * (size_t)(rows > 0 ? rows : 1) * head_dim);
    double *vd = malloc(sizeof(double) * (size_t)(rows > 0 ? rows : 1) * head_dim);
    if (!kd || !vd) {
        free(kd);
        free(vd);
        return PKO_ERR_ALLOC;
    }
    dequantize(k_codes, k_scales, rows, head_dim, kd);
    dequantize(v_codes, v_scales, rows, head_dim, vd);
    work_t w;
    memset(&w, 0, sizeof w);
    w.mode = 2;
    w.q = q;
    w.kd = kd;
    w.vd = vd;
    w.block_tables = block_tables;
    w.context_lens = context_lens;
    w.cu_new_lens = cu_new_lens;
    w.max_blocks_per_seq = max_blocks_per_seq;
    w.num_seqs = num_seqs;
    w.num_q_heads = num_q_heads;
    w.num_kv_heads = num_kv_heads;
    w.head_dim = head_dim;
    w.block_size = block_size;
    w.scale = (double)scale;
    w.out = out;
    w.max_context_len = max_ctx;
    rc = run_threads(&w, nthreads);
    free(kd);
    free(vd);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Rotary position embedding                                                */
/* ------------------------------------------------------------------------ */

/* bf16 of a float, round to nearest, ties to even (NaN stays NaN). */
static uint16_t float_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)(((u >> 16) & 0x8000u) | 0x7fc0u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

/*
 * Rotary position embedding of rows of head_dim bf16 values, [NVE] §3.2 (RoPE
 * puts position into Q and K before attention) and [LLM4] §21.2 / §22 step 4
 * (no position vector is added; Q and K are rotated inside attention).  The
 * pages fix no formula; the reading taken is the rotation of element pairs
 * (i, i + d/2) by the angle whose cosine and sine the caller tabulates per
 * position:
 *   y[i]       = x[i] * c_i - x[i + d/2] * s_i
 *   y[i + d/2] = x[i + d/2] * c_i + x[i] * s_i,   i < d/2,
 *   c_i = cos_sin[p][i],  s_i = cos_sin[p][d/2 + i]   (fp32 table [positions][d])
 * every product and sum in fp32 (no fused multiply-add), the result rounded
 * to bf16 -- as a model materializes rotated q and k before attention.
 * rows: num_rows x heads rows of head_dim; positions[r] is row r's position.
 */
int pko_rope(const uint16_t *x, const int32_t *positions, int32_t num_rows, int32_t heads,
             int32_t head_dim, const float *cos_sin, int32_t max_positions, uint16_t *out)
{
    if (num_rows < 0 || heads <= 0 || head_dim <= 0 || head_dim % 2 || max_positions <= 0)
        return PKO_ERR_ARG;
    int32_t half = head_dim / 2;
    for (int32_t r = 0; r < num_rows; ++r) {
        int32_t p = positions[r];
        if (p < 0 || p >= max_positions)
            return PKO_ERR_RANGE;
        const float *c = cos_sin + (int64_t)p * head_dim;
        const float *sn = c + half;
        for (int32_t h = 0; h < heads; ++h) {
            const uint16_t *xr = x + ((int64_t)r * heads + h) * head_dim;
            uint16_t *yr = out + ((int64_t)r * heads + h) * head_dim;
            for (int32_t i = 0; i < half; ++i) {
                float x1 = bf16_bits_to_float(xr[i]);
                float x2 = bf16_bits_to_float(xr[i + half]);
                float a = x1 * c[i];
                float b = x2 * sn[i];
                float y1 = a - b;
                float e = x2 * c[i];
                float f = x1 * sn[i];
                float y2 = e + f;
                yr[i] = float_to_bf16_rne(y1);
                yr[i + half] = float_to_bf16_rne(y2);
            }
        }
    }
    return PKO_OK;
}

/*
 * Copy whole physical blocks: for each pair (src, dst) of copies [num_pairs][2]
 * and each of the num_pools pools ([num_blocks][block_bytes] bytes each),
 * block dst becomes a byte copy of block src.  This is the copy that
 * copy-on-write needs when a sequence writes into a block it shares ("Nano-vLLM
 * engine deep-dive", section 2.2; "LLM basics primer" part 4, section 17.7).
 * A pair with an id outside [0, num_blocks), or with src == dst, copies
 * nothing.  Two pairs with one dst, or a dst that is also some pair's src,
 * make the result depend on order: refused with PKO_ERR_DUPLICATE.
 */
int pko_copy_blocks(uint8_t *const *pools, int32_t num_pools, int64_t block_bytes,
                    int32_t num_blocks, const int32_t *copies, int32_t num_pairs)
{
    if (num_pools < 0 || block_bytes < 0 || num_blocks < 0 || num_pairs < 0)
        return PKO_ERR_ARG;
    if (num_pairs == 0 || num_pools == 0)
        return PKO_OK;
    if (!pools || !copies)
        return PKO_ERR_ARG;
    unsigned char *role = calloc((size_t)(num_blocks > 0 ? num_blocks : 1), 1);
    if (!role)
        return PKO_ERR_ALLOC;
    /* role bit 1: some pair's src; bit 2: some pair's dst */
    int rc = PKO_OK;
    for (int32_t i = 0; i < num_pairs && rc == PKO_OK; ++i) {
        int32_t src = copies[2 * i], dst = copies[2 * i + 1];
        if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst)
            continue;
        if ((role[dst] & 2) || (role[dst] & 1) || (role[src] & 2))
            rc = PKO_ERR_DUPLICATE;
        role[src] |= 1;
        role[dst] |= 2;
    }
    free(role);
    if (rc != PKO_OK)
        return rc;
    for (int32_t i = 0; i < num_pairs; ++i) {
        int32_t src = copies[2 * i], dst = copies[2 * i + 1];
        if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst)
            continue;
        for (int32_t p = 0; p < num_pools; ++p)
            memcpy(pools[p] + dst * block_bytes, pools[p] + src * block_bytes,
                   (size_t)block_bytes);
    }
    return PKO_OK;
}
