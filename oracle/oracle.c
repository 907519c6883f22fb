/*
 * oracle.c -- plain fp64 CPU oracle for batched paged-attention decode, its
 * multi-token causal form, and the multi-sequence KV-cache write.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header
 * or constant with the HIP library it checks, and it is written to be read,
 * not to be fast: every output row is computed straight from the definition.
 *
 * What is computed (PhotonInfer README, Korean translation, section
 * "Technical details > Paged attention", and "Key features > GPU-optimised
 * kernels"): the KV cache lives in fixed-size blocks; each sequence reaches
 * its tokens through its own block list; one query token per sequence
 * attends over that sequence's cached tokens; the softmax is the
 * numerically stable (max-subtracted) one.  The result is the plain
 * definition
 *
 *     out[b, hq, :] = sum_t softmax_t(scale * q[b, hq, :] . K_t) * V_t
 *
 * over the first L = context_lens[b] tokens of sequence b, gathered through
 * block_tables[b, :], evaluated in double precision from the exact values of
 * the stored bits.
 *
 * Pool layout: K and V pools are [num_blocks, num_kv_heads, block_size,
 * head_dim], row-major.  Token t of sequence b sits in physical block
 * block_tables[b, t / block_size] at offset t % block_size.
 * Query head hq reads kv head hq / (num_q_heads / num_kv_heads) (contiguous
 * grouping of query heads onto kv heads).
 *
 * Readings where the pages are silent: L <= 0 yields an all-zero row;
 * a write slot < 0 is padding and is skipped; a write slot at or beyond
 * num_blocks * block_size is skipped as well.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_F16 1
#define ORACLE_BF16 2

#define ORACLE_OK 0
#define ORACLE_BAD_ARGUMENT 1
#define ORACLE_BAD_BLOCK_ID 2
#define ORACLE_BAD_CONTEXT_LEN 3
#define ORACLE_NO_MEMORY 4

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits.  Written from the format's definition. */
double oracle_f16_to_f64(uint16_t bits)
{
    int sign = (bits >> 15) & 1;
    int expo = (bits >> 10) & 0x1f;
    int frac = bits & 0x3ff;
    double mag;
    if (expo == 0)
        mag = ldexp((double)frac, -24);              /* subnormal: frac * 2^-24 */
    else if (expo == 31)
        mag = frac ? NAN : INFINITY;
    else
        mag = ldexp((double)(1024 + frac), expo - 25); /* (1 + frac/2^10) * 2^(e-15) */
    return sign ? -mag : mag;
}

/* bfloat16 is the upper half of an IEEE binary32: 1 sign bit, 8 exponent
 * bits (bias 127), 7 fraction bits.  Decoded field by field as well. */
double oracle_bf16_to_f64(uint16_t bits)
{
    int sign = (bits >> 15) & 1;
    int expo = (bits >> 7) & 0xff;
    int frac = bits & 0x7f;
    double mag;
    if (expo == 0)
        mag = ldexp((double)frac, -133);             /* frac * 2^-7 * 2^-126 */
    else if (expo == 255)
        mag = frac ? NAN : INFINITY;
    else
        mag = ldexp((double)(128 + frac), expo - 134); /* (1 + frac/2^7) * 2^(e-127) */
    return sign ? -mag : mag;
}

static double load_elem(const void *base, int dtype, int64_t index)
{
    if (dtype == ORACLE_F32) {
        float f;
        memcpy(&f, (const char *)base + 4 * index, 4);
        return (double)f;
    }
    uint16_t h;
    memcpy(&h, (const char *)base + 2 * index, 2);
    return dtype == ORACLE_F16 ? oracle_f16_to_f64(h) : oracle_bf16_to_f64(h);
}

/* Decode n stored elements to double (used to check the decoders). */
void oracle_decode_array(const void *src, int dtype, int64_t n, double *dst)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = load_elem(src, dtype, i);
}

typedef struct {
    const void *q, *k_cache, *v_cache;
    /* optional appended token per sequence (NULL: none): rows of
     * [num_seqs][num_kv_heads][head_dim], token strides in elements */
    const void *k_new, *v_new;
    int64_t k_new_stride, v_new_stride;
    int dtype;
    const int32_t *block_tables;
    int32_t max_blocks_per_seq;
    const int32_t *context_lens;
    int32_t num_seqs, num_q_heads, num_kv_heads, head_dim;
    int32_t num_blocks, block_size;
    double scale;
    /* group-quantised INT8 pools (k_codes non-NULL): the K and V values are
     * code * scale (see the INT8 section below); q then has dtype q_dtype */
    const int8_t *k_codes, *v_codes;
    const float *k_scales, *v_scales;
    int32_t group_size;
    int q_dtype;
} decode_args;

/* Element dtype of q: the pools' dtype, or q_dtype over INT8 pools. */
static int query_dtype(const decode_args *a) { return a->k_codes ? a->q_dtype : a->dtype; }

static double int8_kv_elem(const decode_args *a, int is_value, int64_t blk, int h, int off, int d);

/* Index of element (block, head, offset, d) in a pool. */
static int64_t pool_index(const decode_args *a, int64_t block, int h, int off, int d)
{
    return ((block * a->num_kv_heads + h) * a->block_size + off) * (int64_t)a->head_dim + d;
}

/* Physical block holding logical token t of sequence b (-1 if invalid). */
static int64_t block_of(const decode_args *a, int b, int64_t t)
{
    int64_t blk = a->block_tables[(int64_t)b * a->max_blocks_per_seq + t / a->block_size];
    if (blk < 0 || blk >= a->num_blocks)
        return -1;
    return blk;
}

static int check_row(const decode_args *a, int b)
{
    int64_t L = a->context_lens[b];
    if (L > (int64_t)a->max_blocks_per_seq * a->block_size)
        return ORACLE_BAD_CONTEXT_LEN;
    for (int64_t t = 0; t < L; t += a->block_size)
        if (block_of(a, b, t) < 0)
            return ORACLE_BAD_BLOCK_ID;
    return ORACLE_OK;
}

/* Element d of the key (or value) of logical token t of sequence b, kv
 * head h: from the pool through the block table, except that with an
 * appended token the last position L_b - 1 comes from k_new (v_new). */
static double kv_elem(const decode_args *a, int is_value, int b, int h, int64_t t, int d)
{
    const void *app = is_value ? a->v_new : a->k_new;
    if (app && t == (int64_t)a->context_lens[b] - 1) {
        int64_t stride = is_value ? a->v_new_stride : a->k_new_stride;
        return load_elem(app, a->dtype, (int64_t)b * stride + (int64_t)h * a->head_dim + d);
    }
    int64_t blk = block_of(a, b, t);
    int off = (int)(t % a->block_size);
    if (a->k_codes)
        return int8_kv_elem(a, is_value, blk, h, off, d);
    return load_elem(is_value ? a->v_cache : a->k_cache, a->dtype, pool_index(a, blk, h, off, d));
}

/* scale * (q . K_t) for the tokens [t0, t1) of sequence b, kv head h. */
static void logits(const decode_args *a, int b, int hq, int h, int64_t t0, int64_t t1,
                   double *s)
{
    int64_t qbase = ((int64_t)b * a->num_q_heads + hq) * a->head_dim;
    for (int64_t t = t0; t < t1; ++t) {
        double dot = 0.0;
        for (int d = 0; d < a->head_dim; ++d)
            dot += load_elem(a->q, query_dtype(a), qbase + d) * kv_elem(a, 0, b, h, t, d);
        s[t - t0] = a->scale * dot;
    }
}

/* Softmax-weighted sum of V over the tokens [t0, t1): writes the normalised
 * row to o[0..D) and returns the max logit and the sum of exp(s - max). */
static void softmax_v(const decode_args *a, int b, int h, int64_t t0, int64_t t1,
                      double *s, double *o, double *m_out, double *l_out)
{
    int64_t n = t1 - t0;
    double m = -INFINITY;
    for (int64_t i = 0; i < n; ++i)
        if (s[i] > m)
            m = s[i];
    double l = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        s[i] = exp(s[i] - m); /* s now holds the unnormalised weights */
        l += s[i];
    }
    for (int d = 0; d < a->head_dim; ++d) {
        double acc = 0.0;
        for (int64_t i = 0; i < n; ++i)
            acc += s[i] * kv_elem(a, 1, b, h, t0 + i, d);
        o[d] = acc / l;
    }
    *m_out = m;
    *l_out = l;
}

static int decode_row(const decode_args *a, int b, int hq, int32_t partition_size,
                      double *out_row)
{
    int group = a->num_q_heads / a->num_kv_heads;
    int h = hq / group;
    int64_t L = a->context_lens[b];
    if (L <= 0) {
        for (int d = 0; d < a->head_dim; ++d)
            out_row[d] = 0.0;
        return ORACLE_OK;
    }
    int rc = check_row(a, b);
    if (rc != ORACLE_OK)
        return rc;
    double *s = (double *)malloc(sizeof(double) * (size_t)L);
    if (!s)
        return ORACLE_NO_MEMORY;
    if (partition_size <= 0) {
        /* The definition itself: one softmax over all L tokens. */
        double m, l;
        logits(a, b, hq, h, 0, L, s);
        softmax_v(a, b, h, 0, L, s, out_row, &m, &l);
    } else {
        /* The same result assembled from independent partitions of
         * partition_size tokens: partition j gives its max m_j, its sum l_j
         * and its normalised row o_j; with M = max_j m_j and
         * w_j = l_j exp(m_j - M), out = sum_j w_j o_j / sum_j w_j
         * (the log-sum-exp identity). */
        int64_t nparts = (L + partition_size - 1) / partition_size;
        double *pm = (double *)malloc(sizeof(double) * (size_t)nparts);
        double *pl = (double *)malloc(sizeof(double) * (size_t)nparts);
        double *po = (double *)malloc(sizeof(double) * (size_t)nparts * a->head_dim);
        if (!pm || !pl || !po) {
            free(pm); free(pl); free(po); free(s);
            return ORACLE_NO_MEMORY;
        }
        double M = -INFINITY;
        for (int64_t j = 0; j < nparts; ++j) {
            int64_t t0 = j * partition_size;
            int64_t t1 = t0 + partition_size < L ? t0 + partition_size : L;
            logits(a, b, hq, h, t0, t1, s);
            softmax_v(a, b, h, t0, t1, s, po + j * a->head_dim, &pm[j], &pl[j]);
            if (pm[j] > M)
                M = pm[j];
        }
        double wsum = 0.0;
        for (int64_t j = 0; j < nparts; ++j)
            wsum += pl[j] * exp(pm[j] - M);
        for (int d = 0; d < a->head_dim; ++d) {
            double acc = 0.0;
            for (int64_t j = 0; j < nparts; ++j)
                acc += pl[j] * exp(pm[j] - M) * po[j * a->head_dim + d];
            out_row[d] = acc / wsum;
        }
        free(pm); free(pl); free(po);
    }
    free(s);
    return ORACLE_OK;
}

static int decode_rows(const decode_args *ap, int32_t partition_size, const int32_t *rows,
                       int32_t n_rows, int32_t num_threads, double *out);

/*
 * Decode every (sequence, q head) row, or only the rows listed in `rows`
 * (n_rows pairs b, hq; then out is [n_rows, head_dim]).  out is double.
 * partition_size <= 0 evaluates the definition in one pass; > 0 assembles it
 * from partitions (a self-check of the split identity).  num_threads <= 0
 * leaves the OpenMP default.  Returns ORACLE_OK or the first error seen.
 */
static int decode_all(double *out, const void *q, const void *k_cache, const void *v_cache,
                      const void *k_new, const void *v_new, int64_t k_new_stride,
                      int64_t v_new_stride, int dtype, const int32_t *block_tables,
                      int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t num_seqs,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t num_blocks, int32_t block_size, double scale,
                      int32_t partition_size, const int32_t *rows, int32_t n_rows,
                      int32_t num_threads)
{
    if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
        return ORACLE_BAD_ARGUMENT;
    if (dtype < ORACLE_F32 || dtype > ORACLE_BF16 || num_seqs < 0 || num_kv_heads <= 0 ||
        num_q_heads <= 0 || num_q_heads % num_kv_heads != 0 || head_dim <= 0 ||
        block_size <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0)
        return ORACLE_BAD_ARGUMENT;
    decode_args a = {q, k_cache, v_cache, k_new, v_new, k_new_stride, v_new_stride,
                     dtype, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, num_blocks, block_size, scale};
    return decode_rows(&a, partition_size, rows, n_rows, num_threads, out);
}

/* decode_row for every row (or the listed rows) of the arguments in a. */
static int decode_rows(const decode_args *ap, int32_t partition_size, const int32_t *rows,
                       int32_t n_rows, int32_t num_threads, double *out)
{
    const decode_args a = *ap;
    const int32_t num_seqs = a.num_seqs, num_q_heads = a.num_q_heads, head_dim = a.head_dim;
    int64_t n = rows ? n_rows : (int64_t)num_seqs * num_q_heads;
    if (rows) {
        for (int64_t r = 0; r < n; ++r)
            if (rows[2 * r] < 0 || rows[2 * r] >= num_seqs || rows[2 * r + 1] < 0 ||
                rows[2 * r + 1] >= num_q_heads)
                return ORACLE_BAD_ARGUMENT;
    }
    int status = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1) num_threads(num_threads > 0 ? num_threads : omp_get_max_threads())
    for (int64_t r = 0; r < n; ++r) {
        int b = rows ? rows[2 * r] : (int)(r / num_q_heads);
        int hq = rows ? rows[2 * r + 1] : (int)(r % num_q_heads);
        int rc = decode_row(&a, b, hq, partition_size, out + r * head_dim);
        if (rc != ORACLE_OK) {
#pragma omp critical
            status = status == ORACLE_OK ? rc : status;
        }
    }
    return status;
}

int oracle_paged_attention_decode(double *out, const void *q, const void *k_cache,
                                  const void *v_cache, int dtype,
                                  const int32_t *block_tables, int32_t max_blocks_per_seq,
                                  const int32_t *context_lens, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t num_blocks, int32_t block_size, double scale,
                                  int32_t partition_size, const int32_t *rows, int32_t n_rows,
                                  int32_t num_threads)
{
    return decode_all(out, q, k_cache, v_cache, NULL, NULL, 0, 0, dtype, block_tables,
                      max_blocks_per_seq, context_lens, num_seqs, num_q_heads, num_kv_heads,
                      head_dim, num_blocks, block_size, scale, partition_size, rows, n_rows,
                      num_threads);
}

/*
 * Decode with one appended token per sequence: identical to the above
 * except that, for every sequence b with L_b >= 1, the key and value of its
 * last position L_b - 1 are k_new[b] and v_new[b] (rows [num_kv_heads]
 * [head_dim], token strides in elements) instead of the pool's contents.
 * When the new token has been stored at the slot of position L_b - 1, this
 * is exactly the plain decode of the updated pool.
 */
int oracle_paged_attention_decode_append(double *out, const void *q, const void *k_cache,
                                         const void *v_cache, const void *k_new,
                                         const void *v_new, int64_t k_new_stride,
                                         int64_t v_new_stride, int dtype,
                                         const int32_t *block_tables, int32_t max_blocks_per_seq,
                                         const int32_t *context_lens, int32_t num_seqs,
                                         int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t num_blocks,
                                         int32_t block_size, double scale,
                                         const int32_t *rows, int32_t n_rows, int32_t num_threads)
{
    if (!k_new || !v_new)
        return ORACLE_BAD_ARGUMENT;
    return decode_all(out, q, k_cache, v_cache, k_new, v_new, k_new_stride, v_new_stride,
                      dtype, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                      num_q_heads, num_kv_heads, head_dim, num_blocks, block_size, scale, 0,
                      rows, n_rows, num_threads);
}

/*
 * Multi-token causal paged attention: several new query tokens of a
 * sequence attend over its cache, each one up to its own position.  This is
 * the prefill of a chunk of a prompt, or the check of drafted tokens
 * (PhotonInfer README, Korean translation: "Continuous batching scheduler",
 * where a request advances token by token through num_computed_tokens, and
 * the speculative-decoding item of its "Roadmap"; JackerLab "vllm" tag page,
 * "Speculative Decoding": a large model checks several proposed tokens at
 * once).
 *
 * Sequence b owns the query rows [query_start[b], query_start[b+1]).  With
 * T = query_start[b+1] - query_start[b] and L = context_lens[b] (the tokens
 * in the cache, the T new ones included; their K and V are already in the
 * pools), query row r = query_start[b] + i sits at position p = L - T + i:
 *
 *     out[r, hq] = sum_{t <= p} softmax_t(scale * q[r, hq] . K_t) V_t.
 *
 * q and out are [num_query_tokens][num_q_heads][head_dim].  Every row is the
 * definition evaluated directly in double precision: the logits of the
 * p + 1 tokens, their maximum, the exponentials and their sum, the weighted
 * sum of V.
 */
static int prefill_row(const decode_args *a, const int32_t *query_start, int64_t r, int b,
                       int hq, double *out_row)
{
    int kvh = hq / (a->num_q_heads / a->num_kv_heads); /* contiguous grouping */
    int64_t T = (int64_t)query_start[b + 1] - query_start[b];
    int64_t i = r - query_start[b];
    int64_t p = (int64_t)a->context_lens[b] - T + i; /* this query's position */
    if (p < 0)
        return ORACLE_BAD_ARGUMENT; /* more new tokens than cached ones */
    int rc = check_row(a, b);
    if (rc != ORACLE_OK)
        return rc;
    int64_t n = p + 1;
    double *s = (double *)malloc(sizeof(double) * (size_t)n);
    if (!s)
        return ORACLE_NO_MEMORY;
    int64_t qbase = (r * a->num_q_heads + hq) * (int64_t)a->head_dim;
    for (int64_t t = 0; t < n; ++t) {
        double acc = 0.0;
        for (int e = 0; e < a->head_dim; ++e)
            acc += load_elem(a->q, query_dtype(a), qbase + e) * kv_elem(a, 0, b, kvh, t, e);
        s[t] = a->scale * acc;
    }
    double m, l;
    softmax_v(a, b, kvh, 0, n, s, out_row, &m, &l);
    free(s);
    return ORACLE_OK;
}

/*
 * Every (query row, q head) of a multi-token call, or only the pairs listed
 * in `rows` (n_rows pairs r, hq; out is then [n_rows, head_dim]).
 * query_start has num_seqs + 1 non-decreasing entries starting at 0; its
 * last entry is the number of query rows.
 */
int oracle_paged_attention_prefill(double *out, const void *q, const void *k_cache,
                                   const void *v_cache, int dtype, const int32_t *block_tables,
                                   int32_t max_blocks_per_seq, const int32_t *context_lens,
                                   const int32_t *query_start, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t num_blocks, int32_t block_size, double scale,
                                   const int32_t *rows, int32_t n_rows, int32_t num_threads)
{
    if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start)
        return ORACLE_BAD_ARGUMENT;
    if (dtype < ORACLE_F32 || dtype > ORACLE_BF16 || num_seqs < 0 || num_kv_heads <= 0 ||
        num_q_heads <= 0 || num_q_heads % num_kv_heads != 0 || head_dim <= 0 ||
        block_size <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 || query_start[0] != 0)
        return ORACLE_BAD_ARGUMENT;
    for (int b = 0; b < num_seqs; ++b)
        if (query_start[b + 1] < query_start[b])
            return ORACLE_BAD_ARGUMENT;
    int64_t num_rows = query_start[num_seqs];
    decode_args a = {q, k_cache, v_cache, NULL, NULL, 0, 0, dtype, block_tables,
                     max_blocks_per_seq, context_lens, num_seqs, num_q_heads, num_kv_heads,
                     head_dim, num_blocks, block_size, scale};
    int64_t n = rows ? n_rows : num_rows * num_q_heads;
    if (rows) {
        for (int64_t k = 0; k < n; ++k)
            if (rows[2 * k] < 0 || rows[2 * k] >= num_rows || rows[2 * k + 1] < 0 ||
                rows[2 * k + 1] >= num_q_heads)
                return ORACLE_BAD_ARGUMENT;
    }
    int status = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1) num_threads(num_threads > 0 ? num_threads : omp_get_max_threads())
    for (int64_t k = 0; k < n; ++k) {
        int64_t r = rows ? rows[2 * k] : k / num_q_heads;
        int hq = rows ? rows[2 * k + 1] : (int)(k % num_q_heads);
        int b = 0; /* the sequence whose query rows contain r */
        while (query_start[b + 1] <= r)
            ++b;
        int rc = prefill_row(&a, query_start, r, b, hq, out + k * head_dim);
        if (rc != ORACLE_OK) {
#pragma omp critical
            status = status == ORACLE_OK ? rc : status;
        }
    }
    return status;
}

/*
 * The multi-sequence KV-cache write (same README section: one batched
 * operation stores the new K/V rows of many sequences).  For each new token
 * i with slot s = slot_mapping[i] in [0, num_blocks * block_size):
 * block = s / block_size, offset = s % block_size, and for every kv head h
 * the head_dim elements k[i, h, :] are copied bit for bit to
 * k_cache[block, h, offset, :]; the same for v.  Rows of k and v are
 * token_stride elements apart, heads head_dim apart.  Every other byte of
 * both caches is left as it was.
 */
int oracle_kv_cache_write(const void *k, const void *v, int64_t k_token_stride,
                          int64_t v_token_stride, const int64_t *slot_mapping,
                          int32_t num_tokens, void *k_cache, void *v_cache, int32_t num_blocks,
                          int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                          int32_t elt_bytes)
{
    if (num_tokens < 0 || num_blocks <= 0 || block_size <= 0 || num_kv_heads <= 0 ||
        head_dim <= 0 || (elt_bytes != 2 && elt_bytes != 4))
        return ORACLE_BAD_ARGUMENT;
    if (num_tokens > 0 && (!k || !v || !slot_mapping || !k_cache || !v_cache))
        return ORACLE_BAD_ARGUMENT;
    size_t row = (size_t)head_dim * elt_bytes;
    for (int32_t i = 0; i < num_tokens; ++i) {
        int64_t s = slot_mapping[i];
        if (s < 0 || s >= (int64_t)num_blocks * block_size)
            continue;
        int64_t blk = s / block_size, off = s % block_size;
        for (int h = 0; h < num_kv_heads; ++h) {
            int64_t dst = ((blk * num_kv_heads + h) * block_size + off) * head_dim;
            memcpy((char *)k_cache + dst * elt_bytes,
                   (const char *)k + ((int64_t)i * k_token_stride + (int64_t)h * head_dim) * elt_bytes,
                   row);
            memcpy((char *)v_cache + dst * elt_bytes,
                   (const char *)v + ((int64_t)i * v_token_stride + (int64_t)h * head_dim) * elt_bytes,
                   row);
        }
    }
    return ORACLE_OK;
}

/*
 * Block movement for preemption and paging (PhotonInfer README, Korean
 * translation, "Continuous batching scheduler": requests can be PREEMPTED;
 * JackerLab "vllm" tag page, PagedAttention: KV pages move between GPU and
 * CPU memory).  A block is the contiguous run of block_bytes bytes that one
 * physical block holds in a pool ([num_blocks][num_kv_heads][block_size]
 * [head_dim], so block_bytes = num_kv_heads * block_size * head_dim * elt).
 * All three are bit copies; an id outside [0, num_blocks) skips its entry.
 */

/* For each pair i: block pairs[2i+1] of both pools becomes a copy of block
 * pairs[2i] (read before anything is written: sources and destinations
 * are taken from a snapshot of the pools). */
int oracle_copy_blocks(void *k_cache, void *v_cache, const int64_t *pairs, int32_t num_pairs,
                       int32_t num_blocks, int64_t block_bytes)
{
    if (num_pairs < 0 || num_blocks <= 0 || block_bytes <= 0)
        return ORACLE_BAD_ARGUMENT;
    if (num_pairs == 0)
        return ORACLE_OK;
    size_t pool = (size_t)num_blocks * (size_t)block_bytes;
    char *ks = (char *)malloc(pool), *vs = (char *)malloc(pool);
    if (!ks || !vs) {
        free(ks);
        free(vs);
        return ORACLE_NO_MEMORY;
    }
    memcpy(ks, k_cache, pool);
    memcpy(vs, v_cache, pool);
    for (int32_t i = 0; i < num_pairs; ++i) {
        int64_t src = pairs[2 * i], dst = pairs[2 * i + 1];
        if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks)
            continue;
        memcpy((char *)k_cache + dst * block_bytes, ks + src * block_bytes, (size_t)block_bytes);
        memcpy((char *)v_cache + dst * block_bytes, vs + src * block_bytes, (size_t)block_bytes);
    }
    free(ks);
    free(vs);
    return ORACLE_OK;
}

/* packed[i] = (K block ids[i], V block ids[i]): [n][2][block_bytes]; an
 * entry with an invalid id is left as it was. */
int oracle_gather_blocks(void *packed, const void *k_cache, const void *v_cache,
                         const int64_t *ids, int32_t n, int32_t num_blocks, int64_t block_bytes)
{
    if (n < 0 || num_blocks <= 0 || block_bytes <= 0)
        return ORACLE_BAD_ARGUMENT;
    for (int32_t i = 0; i < n; ++i) {
        int64_t id = ids[i];
        if (id < 0 || id >= num_blocks)
            continue;
        char *row = (char *)packed + (int64_t)i * 2 * block_bytes;
        memcpy(row, (const char *)k_cache + id * block_bytes, (size_t)block_bytes);
        memcpy(row + block_bytes, (const char *)v_cache + id * block_bytes, (size_t)block_bytes);
    }
    return ORACLE_OK;
}

/* The inverse: block ids[i] of the K and V pools take packed[i]. */
int oracle_scatter_blocks(void *k_cache, void *v_cache, const void *packed, const int64_t *ids,
                          int32_t n, int32_t num_blocks, int64_t block_bytes)
{
    if (n < 0 || num_blocks <= 0 || block_bytes <= 0)
        return ORACLE_BAD_ARGUMENT;
    for (int32_t i = 0; i < n; ++i) {
        int64_t id = ids[i];
        if (id < 0 || id >= num_blocks)
            continue;
        const char *row = (const char *)packed + (int64_t)i * 2 * block_bytes;
        memcpy((char *)k_cache + id * block_bytes, row, (size_t)block_bytes);
        memcpy((char *)v_cache + id * block_bytes, row + block_bytes, (size_t)block_bytes);
    }
    return ORACLE_OK;
}

/*
 * Float to the 16-bit formats, rounding to nearest with ties to even,
 * written from the formats' definitions in double arithmetic (every float
 * is exact in double; rint() rounds half to even in the default rounding
 * mode): find the quantum of the value's binade, count quanta, round.
 * Magnitudes at or past the midpoint above the largest finite value become
 * infinity; NaN becomes a quiet NaN with the sign and top payload bits.
 */
uint16_t oracle_f32_to_f16(float f)
{
    double x = (double)f;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x)) {
        uint32_t u;
        memcpy(&u, &f, 4);
        return (uint16_t)(sign | 0x7e00 | ((u >> 13) & 0x1ff));
    }
    if (a >= 65520.0) /* 65504 + half a quantum (2^5 / 2) and beyond */
        return sign | 0x7c00;
    if (a < ldexp(1.0, -14)) { /* subnormal binade: quantum 2^-24 */
        double q = rint(a / ldexp(1.0, -24));
        return (uint16_t)(sign | (uint16_t)q); /* q == 1024 is the smallest normal */
    }
    int e;
    frexp(a, &e); /* a = m 2^e, m in [0.5, 1): binade 2^(e-1) */
    int expo = e - 1;
    double q = rint(a / ldexp(1.0, expo - 10)); /* in [1024, 2048] */
    if (q == 2048.0) {
        q = 1024.0;
        expo += 1;
    }
    if (expo > 15)
        return sign | 0x7c00;
    return (uint16_t)(sign | ((expo + 15) << 10) | ((int)q - 1024));
}

uint16_t oracle_f32_to_bf16(float f)
{
    double x = (double)f;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x)) {
        uint32_t u;
        memcpy(&u, &f, 4);
        return (uint16_t)((u >> 16) | 0x40);
    }
    /* largest finite bf16: (2 - 2^-7) 2^127; halfway to 2^128 and beyond */
    if (a >= ldexp(2.0 - ldexp(1.0, -8), 127))
        return sign | 0x7f80;
    if (a < ldexp(1.0, -126)) { /* subnormal binade: quantum 2^-133 */
        double q = rint(a / ldexp(1.0, -133));
        return (uint16_t)(sign | (uint16_t)q);
    }
    int e;
    frexp(a, &e);
    int expo = e - 1;
    double q = rint(a / ldexp(1.0, expo - 7)); /* in [128, 256] */
    if (q == 256.0) {
        q = 128.0;
        expo += 1;
    }
    if (expo > 127)
        return sign | 0x7f80;
    return (uint16_t)(sign | ((expo + 127) << 7) | ((int)q - 128));
}

/*
 * The KV-cache write with the rotary position embedding applied to the new
 * keys (PhotonInfer README, Korean translation, "Key features >
 * GPU-optimised kernels": batched RoPE among the fused operations).  For
 * each token i with a valid slot (as in oracle_kv_cache_write) and a
 * position p = positions[i] in [0, max_position):
 *   V rows are stored unchanged;
 *   each K row x (head h) is stored as y with, for j < R/2 (R = rotary_dim),
 *     c = cos_sin[p][j], s = cos_sin[p][R/2 + j],
 *     y[j]       = x[j] c - x[j + R/2] s,
 *     y[j + R/2] = x[j + R/2] c + x[j] s,
 *   and y[d] = x[d] for d >= R,
 * each product and each sum rounded to float (no fused multiply-add), then
 * y rounded to nearest even into the pool dtype.  The table (cos then sin
 * of each position's angles, [max_position][R] floats) is the caller's:
 * the angle schedule (base, any frequency scaling) is not fixed here.  A
 * token whose position is outside the table is skipped.
 */
int oracle_kv_cache_write_rope(const void *k, const void *v, int64_t k_token_stride,
                               int64_t v_token_stride, const int64_t *slot_mapping,
                               const int32_t *positions, int32_t num_tokens, const float *cos_sin,
                               int32_t max_position, int32_t rotary_dim, void *k_cache,
                               void *v_cache, int32_t num_blocks, int32_t block_size,
                               int32_t num_kv_heads, int32_t head_dim, int dtype)
{
    if (num_tokens < 0 || num_blocks <= 0 || block_size <= 0 || num_kv_heads <= 0 ||
        head_dim <= 0 || dtype < ORACLE_F32 || dtype > ORACLE_BF16 || rotary_dim < 0 ||
        rotary_dim > head_dim || rotary_dim % 2 || max_position < 0)
        return ORACLE_BAD_ARGUMENT;
    int elt = dtype == ORACLE_F32 ? 4 : 2;
    int half = rotary_dim / 2;
    float *x = (float *)malloc(sizeof(float) * (size_t)head_dim);
    float *y = (float *)malloc(sizeof(float) * (size_t)head_dim);
    if (!x || !y) {
        free(x);
        free(y);
        return ORACLE_NO_MEMORY;
    }
    for (int32_t i = 0; i < num_tokens; ++i) {
        int64_t s = slot_mapping[i];
        int32_t p = positions[i];
        if (s < 0 || s >= (int64_t)num_blocks * block_size || p < 0 || p >= max_position)
            continue;
        int64_t blk = s / block_size;
        int64_t off = s - blk * block_size;
        const float *cs = cos_sin + (int64_t)p * rotary_dim;
        for (int h = 0; h < num_kv_heads; ++h) {
            int64_t dst = ((blk * num_kv_heads + h) * block_size + off) * head_dim;
            int64_t vsrc = (int64_t)i * v_token_stride + (int64_t)h * head_dim;
            memcpy((char *)v_cache + dst * elt, (const char *)v + vsrc * elt, (size_t)head_dim * elt);
            int64_t src = (int64_t)i * k_token_stride + (int64_t)h * head_dim;
            for (int d = 0; d < head_dim; ++d)
                x[d] = (float)load_elem(k, dtype, src + d);
            for (int d = 0; d < head_dim; ++d)
                y[d] = x[d];
            for (int j = 0; j < half; ++j) {
                float c = cs[j], sn = cs[half + j];
                float a = x[j] * c, b = x[j + half] * sn;
                float e = x[j + half] * c, f = x[j] * sn;
                y[j] = a - b;
                y[j + half] = e + f;
            }
            for (int d = 0; d < head_dim; ++d) {
                char *out = (char *)k_cache + (dst + d) * elt;
                if (dtype == ORACLE_F32) {
                    memcpy(out, &y[d], 4);
                } else {
                    uint16_t hb = dtype == ORACLE_F16 ? oracle_f32_to_f16(y[d])
                                                      : oracle_f32_to_bf16(y[d]);
                    memcpy(out, &hb, 2);
                }
            }
        }
    }
    free(x);
    free(y);
    return ORACLE_OK;
}

/* n floats to 16-bit bit patterns (to check the two conversions). */
void oracle_round_array(const float *src, int dtype, int64_t n, uint16_t *dst)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = dtype == ORACLE_F16 ? oracle_f32_to_f16(src[i]) : oracle_f32_to_bf16(src[i]);
}

/* ---------------------------------------------------------------------------
 * Group-quantised INT8 KV cache.
 *
 * PhotonInfer README (Korean translation), "Key features > GPU-optimised
 * kernels" and "Technical details > INT8 quantisation": quantisation to INT8
 * in groups, with a configurable group size of 32, 64 or 128.  The README
 * applies it to weights; here the same scheme stores the KV cache (a
 * reading: the pages do not quantise KV).  Each new token's row of one kv
 * head is cut into head_dim / group_size groups of consecutive elements, and
 * each group is stored as
 *
 *     amax = max_i |x_i|                   (float32, from the exact inputs)
 *     s    = amax / 127                    (one float32 division)
 *     c_i  = rint(x_i / s)                 (float32 division, ties to even)
 *
 * with c_i in [-127, 127] (s = 0 gives c_i = 0).  The cached value stands
 * for c_i * s.  Inputs are finite (non-finite inputs leave the codes
 * unspecified).
 *
 * Layouts.  The block_size * head_dim codes of one physical block and kv
 * head form one contiguous run of each code array, [num_blocks]
 * [num_kv_heads][block_size * head_dim] int8; inside it, tokens are taken
 * in tiles of 16 (token offset = 16 * tile + row) and the order is
 *   K code of (offset, d):  ((tile * 64 + 16 * jk + row) * (head_dim / 32)
 *                            + d / 32) * 8 + d % 8,     jk = (d % 32) / 8
 *   V code of (offset, d):  ((tile * 64 + 16 * jv + d % 16) * (head_dim / 16)
 *                            + d / 16) * 4 + row % 4,   jv = row / 4
 * (the order in which the matrix-core products consume them: lane
 * 16 * j + r of a 64-lane wave reads one contiguous run per tile).  The
 * scales are token-major:
 *   k_scales, v_scales
 *             float32 [num_blocks][num_kv_heads][block_size][head_dim/group_size]
 * ------------------------------------------------------------------------- */

static int64_t int8_code_index(const decode_args *a, int is_value, int64_t blk, int h, int off,
                               int d)
{
    int64_t base = (blk * a->num_kv_heads + h) * (int64_t)a->block_size * a->head_dim;
    int tile = off / 16, row = off % 16;
    if (!is_value) {
        int jk = (d % 32) / 8;
        return base + (((int64_t)tile * 64 + 16 * jk + row) * (a->head_dim / 32) + d / 32) * 8 +
               d % 8;
    }
    int jv = row / 4;
    return base + (((int64_t)tile * 64 + 16 * jv + d % 16) * (a->head_dim / 16) + d / 16) * 4 +
           row % 4;
}

static int64_t int8_scale_index(int32_t num_kv_heads, int32_t block_size, int32_t groups,
                                int64_t blk, int h, int off, int g)
{
    return ((blk * num_kv_heads + h) * block_size + off) * groups + g;
}

/* The value an INT8 pool holds for element d: code * scale, in double. */
static double int8_kv_elem(const decode_args *a, int is_value, int64_t blk, int h, int off, int d)
{
    const int8_t *codes = is_value ? a->v_codes : a->k_codes;
    const float *scales = is_value ? a->v_scales : a->k_scales;
    int groups = a->head_dim / a->group_size;
    double c = (double)codes[int8_code_index(a, is_value, blk, h, off, d)];
    double s = (double)scales[int8_scale_index(a->num_kv_heads, a->block_size, groups, blk, h, off,
                                               d / a->group_size)];
    return c * s;
}

/* One group: n float32 values -> n codes and the group's scale. */
float oracle_quantize_group(const float *x, int32_t n, int8_t *codes)
{
    float amax = 0.0f;
    for (int32_t i = 0; i < n; ++i) {
        float m = fabsf(x[i]);
        if (m > amax)
            amax = m;
    }
    float s = amax / 127.0f;
    for (int32_t i = 0; i < n; ++i) {
        float c = s > 0.0f ? rintf(x[i] / s) : 0.0f;
        if (c > 127.0f)
            c = 127.0f;
        if (c < -127.0f)
            c = -127.0f;
        codes[i] = (int8_t)c;
    }
    return s;
}

/*
 * The batched write into INT8 pools: for each new token i whose slot
 * s = slot_mapping[i] lies in [0, num_blocks * block_size) (others are
 * skipped), every kv head's K and V rows (dtype elements, token strides in
 * elements, heads head_dim apart) are quantised group by group and stored at
 * block s / block_size, offset s % block_size of the four arrays.  Every
 * other byte is left as it was.
 */
int oracle_kv_cache_write_int8(const void *k, const void *v, int64_t k_token_stride,
                               int64_t v_token_stride, int dtype, const int64_t *slot_mapping,
                               int32_t num_tokens, int8_t *k_codes, int8_t *v_codes,
                               float *k_scales, float *v_scales, int32_t num_blocks,
                               int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                               int32_t group_size)
{
    if (num_tokens < 0 || num_blocks <= 0 || block_size <= 0 || num_kv_heads <= 0 ||
        head_dim <= 0 || group_size <= 0 || head_dim % group_size || dtype < ORACLE_F32 ||
        dtype > ORACLE_BF16)
        return ORACLE_BAD_ARGUMENT;
    if (num_tokens > 0 && (!k || !v || !slot_mapping || !k_codes || !v_codes || !k_scales ||
                           !v_scales))
        return ORACLE_BAD_ARGUMENT;
    decode_args a;
    memset(&a, 0, sizeof a);
    a.num_kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    a.block_size = block_size;
    int groups = head_dim / group_size;
    float *x = (float *)malloc(sizeof(float) * (size_t)group_size);
    int8_t *c = (int8_t *)malloc((size_t)group_size);
    if (!x || !c) {
        free(x); free(c);
        return ORACLE_NO_MEMORY;
    }
    for (int32_t i = 0; i < num_tokens; ++i) {
        int64_t s = slot_mapping[i];
        if (s < 0 || s >= (int64_t)num_blocks * block_size)
            continue;
        int64_t blk = s / block_size;
        int off = (int)(s % block_size);
        for (int h = 0; h < num_kv_heads; ++h) {
            for (int is_value = 0; is_value < 2; ++is_value) {
                const void *src = is_value ? v : k;
                int64_t row = (int64_t)i * (is_value ? v_token_stride : k_token_stride) +
                              (int64_t)h * head_dim;
                int8_t *codes = is_value ? v_codes : k_codes;
                float *scales = is_value ? v_scales : k_scales;
                for (int g = 0; g < groups; ++g) {
                    for (int e = 0; e < group_size; ++e)
                        x[e] = (float)load_elem(src, dtype, row + (int64_t)g * group_size + e);
                    scales[int8_scale_index(num_kv_heads, block_size, groups, blk, h, off, g)] =
                        oracle_quantize_group(x, group_size, c);
                    for (int e = 0; e < group_size; ++e)
                        codes[int8_code_index(&a, is_value, blk, h, off, g * group_size + e)] = c[e];
                }
            }
        }
    }
    free(x);
    free(c);
    return ORACLE_OK;
}

/*
 * Decode over INT8 pools: the plain definition evaluated on the values the
 * pools stand for (code * scale, exact in double), with q stored as q_dtype
 * (float32, fp16 or bf16 bits).  Row selection, partition_size
 * and threads as for oracle_paged_attention_decode.
 */
int oracle_paged_attention_decode_int8(double *out, const void *q, int q_dtype,
                                       const int8_t *k_codes, const int8_t *v_codes,
                                       const float *k_scales, const float *v_scales,
                                       const int32_t *block_tables, int32_t max_blocks_per_seq,
                                       const int32_t *context_lens, int32_t num_seqs,
                                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int32_t num_blocks, int32_t block_size, int32_t group_size,
                                       double scale, int32_t partition_size, const int32_t *rows,
                                       int32_t n_rows, int32_t num_threads)
{
    if (!out || !q || !k_codes || !v_codes || !k_scales || !v_scales || !block_tables ||
        !context_lens)
        return ORACLE_BAD_ARGUMENT;
    if (q_dtype < ORACLE_F32 || q_dtype > ORACLE_BF16 || num_seqs < 0 || num_kv_heads <= 0 ||
        num_q_heads <= 0 || num_q_heads % num_kv_heads != 0 || head_dim <= 0 ||
        group_size <= 0 || head_dim % group_size || block_size <= 0 || max_blocks_per_seq <= 0 ||
        num_blocks <= 0)
        return ORACLE_BAD_ARGUMENT;
    decode_args a;
    memset(&a, 0, sizeof a);
    a.q = q;
    a.k_cache = k_codes;
    a.v_cache = v_codes;
    a.dtype = q_dtype;
    a.block_tables = block_tables;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.context_lens = context_lens;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    a.num_blocks = num_blocks;
    a.block_size = block_size;
    a.scale = scale;
    a.k_codes = k_codes;
    a.v_codes = v_codes;
    a.k_scales = k_scales;
    a.v_scales = v_scales;
    a.group_size = group_size;
    a.q_dtype = q_dtype;
    return decode_rows(&a, partition_size, rows, n_rows, num_threads, out);
}
