/*
 * oracle.c -- plain CPU reference for batched attention over a paged KV cache
 * with a sliding-window mask, the merge of two (output, LSE) partials, and the
 * two steps on either side of it: writing new key/value rows into the cache
 * and building the page table from a request-to-page map.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark do.  It shares no code, header or table with the HIP
 * kernels.
 *
 * Every quantity is computed in IEEE double precision, straight from the
 * definition, one (query token, query head) row at a time, with no tiling,
 * no online rescaling and no reordering beyond what the definition states.
 *
 * Sources (the web pages this follows):
 *  [PR31501]  sglang PR "[flashinfer] Pass window_left at plan time for the
 *             SWA paged prefill wrapper", section "What".
 *  [FIB]      sglang python/sglang/srt/layers/attention/flashinfer_backend.py,
 *             functions named below.
 *  [PR234]    AMD-Ecosystem/flashinfer PR "fix(rocm): correct AITER decode
 *             backend gaps -- sliding window, CUDA graph, return_lse",
 *             sections "Why each fix" 1 (sliding window) and 3 (return_lse).
 */
#define _POSIX_C_SOURCE 200809L
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_BF16 0
#define ORACLE_FP32 1
#define ORACLE_FP16 2
#define ORACLE_FP8_E4M3 3
#define ORACLE_FP8_E5M2 4

/* Exact widening of one stored element to double.  bf16 is the upper half of
 * an IEEE binary32, so shifting its 16 bits up gives the same value.  An IEEE
 * binary16 with exponent field e and fraction f is (1 + f/1024) * 2^(e-15)
 * for 0 < e < 31, f * 2^-24 for e = 0 (subnormal), +-inf or NaN for e = 31. */
static double load_elem(const void *base, int dtype, int64_t idx)
{
    if (dtype == ORACLE_BF16) {
        uint32_t u = (uint32_t)((const uint16_t *)base)[idx] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    if (dtype == ORACLE_FP16) {
        const uint16_t h = ((const uint16_t *)base)[idx];
        const int e = (h >> 10) & 31, f = h & 1023;
        double v;
        if (e == 0)
            v = ldexp((double)f, -24);
        else if (e == 31)
            v = f ? NAN : INFINITY;
        else
            v = ldexp((double)(1024 + f), e - 25);
        return (h >> 15) ? -v : v;
    }
    if (dtype == ORACLE_FP8_E4M3 || dtype == ORACLE_FP8_E5M2) {
        /* OCP 8-bit floats.  E4M3 ("fn"): exponent bias 7, subnormals
         * f/8 * 2^-6, no infinities, S.1111.111 is NaN.  E5M2: the upper byte
         * of an IEEE binary16 (bias 15, subnormals f/4 * 2^-14, inf/NaN at
         * exponent 31). */
        const uint8_t x = ((const uint8_t *)base)[idx];
        const int e4 = dtype == ORACLE_FP8_E4M3;
        const int mbits = e4 ? 3 : 2, bias = e4 ? 7 : 15;
        const int e = (x & 0x7f) >> mbits, f = x & ((1 << mbits) - 1);
        double v;
        if (e4 && e == 15 && f == 7)
            v = NAN;
        else if (!e4 && e == 31)
            v = f ? NAN : INFINITY;
        else if (e == 0)
            v = ldexp((double)f, 1 - bias - mbits);
        else
            v = ldexp((double)((1 << mbits) + f), e - bias - mbits);
        return (x & 0x80) ? -v : v;
    }
    return (double)((const float *)base)[idx];
}

/* The stored elements src[0 .. n-1] widened to double (the reading every
 * input of the oracle goes through). */
void oracle_widen(int32_t dtype, const void *src, int64_t n, double *dst)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = load_elem(src, dtype, i);
}

/* Number of keys held by request b of a CSR page table: all pages but the
 * last are full, the last holds kv_last_page_len[b] slots.  (The argument
 * names are the ones [FIB] fast_prefill_plan takes: paged_kv_indptr,
 * paged_kv_indices, paged_kv_last_page_len.) */
static int64_t request_kv_len(const int32_t *kv_indptr, const int32_t *kv_last_page_len,
                              int32_t page_size, int32_t b)
{
    int64_t npages = (int64_t)kv_indptr[b + 1] - kv_indptr[b];
    if (npages <= 0)
        return 0;
    return (npages - 1) * (int64_t)page_size + kv_last_page_len[b];
}

/* Flat element offset of logical key j of request b, KV head hk, dim 0, in an
 * NHD cache [num_pages, page_size, H_kv, D]: page id from the CSR indices,
 * slot = j mod page_size. */
static int64_t key_offset(const int32_t *kv_indptr, const int32_t *kv_indices,
                          int32_t page_size, int32_t num_kv_heads, int32_t head_dim,
                          int32_t b, int64_t j, int32_t hk)
{
    int64_t page = kv_indices[(int64_t)kv_indptr[b] + j / page_size];
    int64_t slot = j % page_size;
    return ((page * page_size + slot) * num_kv_heads + hk) * (int64_t)head_dim;
}

/* Visibility of key j to the query at absolute position p.
 * Window ([PR234] "Why each fix" 1; [FIB] _build_swa_prefix_custom_mask):
 * window_left = W >= 0 lets position p see keys p-W .. p, i.e. W+1 keys;
 * W = -1 switches the window off.  Causality: keys after p are hidden.
 * key_lo/key_hi only restrict the key range (used to split a request). */
static int key_visible(int64_t j, int64_t p, int32_t causal, int32_t window_left,
                       int64_t key_lo, int64_t key_hi)
{
    if (j < key_lo || j >= key_hi)
        return 0;
    if (causal && j > p)
        return 0;
    if (window_left >= 0 && j < p - (int64_t)window_left)
        return 0;
    return 1;
}

/* Arguments of one oracle_paged_attention call, shared by its threads. */
struct attention_call {
    int32_t batch;
    const int32_t *qo_indptr, *kv_indptr, *kv_indices, *kv_last_page_len;
    int32_t page_size, num_qo_heads, num_kv_heads, head_dim, causal, window_left;
    double sm_scale, soft_cap;
    int32_t in_dtype, kv_dtype;
    const void *q;
    double k_scale, v_scale;
    const void *k_cache, *v_cache;
    const int64_t *rows;
    int64_t count, nnz_qo, max_kv, key_lo, key_hi;
    double *o, *lse;
    /* the next output row to take (threads claim rows one at a time) */
    pthread_mutex_t lock;
    int64_t next_row;
    int failed;
};

/*
 * One output row r: every query head of query token t = rows[r] (or t = r).
 * s holds max_kv logits and acc head_dim sums (scratch of the calling thread).
 */
static void attention_row(const struct attention_call *c, int64_t r, double *s, double *acc)
{
    const int32_t batch = c->batch, page_size = c->page_size, num_qo_heads = c->num_qo_heads;
    const int32_t num_kv_heads = c->num_kv_heads, head_dim = c->head_dim, causal = c->causal;
    const int32_t window_left = c->window_left, in_dtype = c->in_dtype, kv_dtype = c->kv_dtype;
    const int32_t *qo_indptr = c->qo_indptr, *kv_indptr = c->kv_indptr;
    const int32_t *kv_indices = c->kv_indices, *kv_last_page_len = c->kv_last_page_len;
    const double sm_scale = c->sm_scale, soft_cap = c->soft_cap;
    const double k_scale = c->k_scale, v_scale = c->v_scale;
    const void *q = c->q, *k_cache = c->k_cache, *v_cache = c->v_cache;
    const int64_t *rows = c->rows;
    const int64_t key_lo = c->key_lo, key_hi = c->key_hi;
    double *o = c->o, *lse = c->lse;
    const int32_t group = num_qo_heads / num_kv_heads;

    const int64_t t = rows ? rows[r] : r;
    if (t < 0 || t >= c->nnz_qo)
        return;
    int32_t b = 0;
    while (b + 1 < batch && qo_indptr[b + 1] <= t)
        ++b;
    const int64_t kv_len = request_kv_len(kv_indptr, kv_last_page_len, page_size, b);
    const int64_t qo_len = (int64_t)qo_indptr[b + 1] - qo_indptr[b];
    const int64_t p = (kv_len - qo_len) + (t - qo_indptr[b]);

    const int64_t out_row = rows ? r : t;
    for (int32_t h = 0; h < num_qo_heads; ++h) {
        const int32_t hk = h / group;
        const int64_t qoff = (t * num_qo_heads + h) * (int64_t)head_dim;
        const int64_t ooff = (out_row * num_qo_heads + h) * (int64_t)head_dim;

        /* logits of the visible keys, and their maximum */
        double m = -INFINITY;
        for (int64_t j = 0; j < kv_len; ++j) {
            if (!key_visible(j, p, causal, window_left, key_lo, key_hi))
                continue;
            const int64_t koff = key_offset(kv_indptr, kv_indices, page_size, num_kv_heads,
                                            head_dim, b, j, hk);
            double dot = 0.0;
            for (int32_t d = 0; d < head_dim; ++d)
                dot += load_elem(q, in_dtype, qoff + d) *
                       (k_scale * load_elem(k_cache, kv_dtype, koff + d));
            s[j] = sm_scale * dot;
            if (soft_cap > 0.0)
                s[j] = soft_cap * tanh(s[j] / soft_cap);
            if (s[j] > m)
                m = s[j];
        }

        for (int32_t d = 0; d < head_dim; ++d)
            acc[d] = 0.0;
        double l = 0.0;
        if (m != -INFINITY) {
            for (int64_t j = 0; j < kv_len; ++j) {
                if (!key_visible(j, p, causal, window_left, key_lo, key_hi))
                    continue;
                const double w = exp(s[j] - m);
                l += w;
                const int64_t voff = key_offset(kv_indptr, kv_indices, page_size,
                                                num_kv_heads, head_dim, b, j, hk);
                for (int32_t d = 0; d < head_dim; ++d)
                    acc[d] += w * (v_scale * load_elem(v_cache, kv_dtype, voff + d));
            }
        }
        double *orow = o + ooff;
        if (l > 0.0) {
            for (int32_t d = 0; d < head_dim; ++d)
                orow[d] = acc[d] / l;
            lse[out_row * num_qo_heads + h] = m + log(l);
        } else {
            for (int32_t d = 0; d < head_dim; ++d)
                orow[d] = 0.0;
            lse[out_row * num_qo_heads + h] = -INFINITY;
        }
    }
}

/* A worker: claims output rows one at a time until none is left.  Every row is
 * computed by exactly one thread, with the same arithmetic as a single thread
 * would use; only the order in which rows are finished changes. */
static void *attention_worker(void *arg)
{
    struct attention_call *c = (struct attention_call *)arg;
    double *s = (double *)malloc(sizeof(double) * (size_t)(c->max_kv > 0 ? c->max_kv : 1));
    double *acc = (double *)malloc(sizeof(double) * (size_t)c->head_dim);
    if (!s || !acc) {
        pthread_mutex_lock(&c->lock);
        c->failed = 1;
        pthread_mutex_unlock(&c->lock);
        free(s);
        free(acc);
        return NULL;
    }
    for (;;) {
        pthread_mutex_lock(&c->lock);
        const int64_t r = c->failed ? c->count : c->next_row++;
        pthread_mutex_unlock(&c->lock);
        if (r >= c->count)
            break;
        attention_row(c, r, s, acc);
    }
    free(s);
    free(acc);
    return NULL;
}

/*
 * Attention of every query row (or of the listed rows) over its request's
 * paged keys.
 *
 *  Request b holds qo_len_b = qo_indptr[b+1]-qo_indptr[b] queries and kv_len_b
 *  keys; its queries are the last qo_len_b positions of the sequence, so query
 *  i sits at p = (kv_len_b - qo_len_b) + i.  This is how the extend step with a
 *  cached prefix lines up ([FIB] call_begin_forward builds qo_indptr from
 *  seq_len - prefix_len; forward_extend writes the new keys to the cache before
 *  the paged kernel reads them).  A decode request is qo_len_b = 1, p =
 *  kv_len_b - 1.  A request with no keys may still carry queries (a padded
 *  decode slot); they see nothing.
 *
 *  Query head h reads KV head h / (H_q / H_kv) (grouped-query heads share
 *  contiguous groups).
 *
 *  Keys and values are read as k_scale * k and v_scale * v from a cache of
 *  type kv_dtype ([FIB] forward_extend / forward_decode pass k_scale and
 *  v_scale with the cache; an 8-bit cache holds K / k_scale and V / v_scale).
 *
 *  s_j   = sm_scale * sum_d q[d] * k_j[d]                for visible j
 *  s_j  <- soft_cap * tanh(s_j / soft_cap)   when soft_cap > 0 (the logits
 *          soft cap [FIB] forward_extend / forward_decode pass to the
 *          wrappers as logits_soft_cap; the pages do not print its formula,
 *          this is the tanh cap of the scaled logits)
 *  m     = max_j s_j,  l = sum_j exp(s_j - m)
 *  o     = sum_j exp(s_j - m) / l * v_j
 *  lse   = m + ln(l)          (natural log; the log-sum-exp of the logits)
 *  empty visible set: o = 0, lse = -inf.
 *
 *  Inputs are read in their stored type (ORACLE_BF16 as raw 16-bit words,
 *  ORACLE_FP32) and widened exactly.  o is [nnz_qo, H_q, D] double, lse is
 *  [nnz_qo, H_q] double.  rows (may be NULL) lists the global query-token
 *  indices to compute; then o and lse are compact, [n_rows, H_q, D] and
 *  [n_rows, H_q], row r holding query token rows[r].
 *
 *  n_threads > 1 computes the rows on that many POSIX threads (each row by one
 *  thread, unchanged arithmetic: the results are bit-identical).
 *
 *  Returns 0 on success, -1 on a malformed layout, -2 when out of memory.
 */
int oracle_paged_attention(int32_t batch, const int32_t *qo_indptr, const int32_t *kv_indptr,
                           const int32_t *kv_indices, const int32_t *kv_last_page_len,
                           int32_t page_size, int32_t num_qo_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t causal, int32_t window_left,
                           double sm_scale, double soft_cap, int32_t in_dtype, const void *q,
                           int32_t kv_dtype, double k_scale, double v_scale,
                           const void *k_cache, const void *v_cache, const int64_t *rows,
                           int64_t n_rows, int64_t key_lo, int64_t key_hi, double *o,
                           double *lse, int32_t n_threads)
{
    if (batch < 0 || page_size <= 0 || num_kv_heads <= 0 || num_qo_heads % num_kv_heads)
        return -1;
    struct attention_call c;
    memset(&c, 0, sizeof c);
    c.batch = batch;
    c.qo_indptr = qo_indptr;
    c.kv_indptr = kv_indptr;
    c.kv_indices = kv_indices;
    c.kv_last_page_len = kv_last_page_len;
    c.page_size = page_size;
    c.num_qo_heads = num_qo_heads;
    c.num_kv_heads = num_kv_heads;
    c.head_dim = head_dim;
    c.causal = causal;
    c.window_left = window_left;
    c.sm_scale = sm_scale;
    c.soft_cap = soft_cap;
    c.in_dtype = in_dtype;
    c.kv_dtype = kv_dtype;
    c.q = q;
    c.k_scale = k_scale;
    c.v_scale = v_scale;
    c.k_cache = k_cache;
    c.v_cache = v_cache;
    c.rows = rows;
    c.nnz_qo = qo_indptr[batch];
    c.count = rows ? n_rows : c.nnz_qo;
    c.key_lo = key_lo;
    c.key_hi = key_hi;
    c.o = o;
    c.lse = lse;

    for (int32_t b = 0; b < batch; ++b) {
        int64_t n = request_kv_len(kv_indptr, kv_last_page_len, page_size, b);
        int64_t nq = (int64_t)qo_indptr[b + 1] - qo_indptr[b];
        if (nq < 0 || (nq > n && n > 0))
            return -1;
        if (n > c.max_kv)
            c.max_kv = n;
    }

    if (pthread_mutex_init(&c.lock, NULL) != 0)
        return -2;
    int32_t nt = n_threads < 1 ? 1 : n_threads;
    if ((int64_t)nt > c.count)
        nt = c.count > 0 ? (int32_t)c.count : 1;
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nt);
    int32_t started = 0;
    if (tid)
        for (; started < nt - 1; ++started)
            if (pthread_create(&tid[started], NULL, attention_worker, &c) != 0)
                break;
    attention_worker(&c); /* the calling thread works too */
    for (int32_t i = 0; i < started; ++i)
        pthread_join(tid[i], NULL);
    free(tid);
    pthread_mutex_destroy(&c.lock);
    return c.failed ? -2 : 0;
}

/*
 * Combine two attention partials over disjoint key sets A and B into the
 * partial over A u B (the (v_a, s_a, v_b, s_b) -> (v, s) combine that [FIB]
 * _safe_merge_state dispatches; the per-call LSE it consumes is what [PR234]
 * "Why each fix" 3 asks the decode path to return).
 *
 *  With s_x = ln sum_{j in X} exp(logit_j) and v_x the softmax-weighted mean of
 *  the values over X:
 *    s = ln(exp(s_a) + exp(s_b))   evaluated as  M + ln(exp(s_a-M) + exp(s_b-M)),
 *                                   M = max(s_a, s_b)
 *    v = exp(s_a - s) * v_a + exp(s_b - s) * v_b
 *  Two empty partials (s_a = s_b = -inf) give v = 0, s = -inf; one empty
 *  partial leaves the other unchanged.
 *
 *  v_* are [n, H, D] and s_* are [n, H], all double.
 */
void oracle_merge_state(int64_t n, int32_t num_heads, int32_t head_dim, const double *v_a,
                        const double *s_a, const double *v_b, const double *s_b, double *v_out,
                        double *s_out)
{
    for (int64_t i = 0; i < n * num_heads; ++i) {
        const double a = s_a[i], b = s_b[i];
        const double M = a > b ? a : b;
        const double *va = v_a + i * head_dim, *vb = v_b + i * head_dim;
        double *vo = v_out + i * head_dim;
        if (M == -INFINITY) {
            for (int32_t d = 0; d < head_dim; ++d)
                vo[d] = 0.0;
            s_out[i] = -INFINITY;
            continue;
        }
        const double s = M + log(exp(a - M) + exp(b - M));
        const double wa = exp(a - s), wb = exp(b - s);
        for (int32_t d = 0; d < head_dim; ++d)
            vo[d] = wa * va[d] + wb * vb[d];
        s_out[i] = s;
    }
}

/*
 * Writing new keys and values into the cache ([FIB] forward_extend and
 * forward_decode call token_to_kv_pool.set_kv_buffer with the batch's cache
 * locations before the paged attention reads them).
 *
 * The cache is viewed as num_slots rows of row_bytes bytes (slot = page *
 * page_size + position in the page).  Row i of k_new / v_new goes to slot
 * loc[i]; a loc outside [0, num_slots) writes nothing and is counted.
 * Returns the number of such skipped rows.
 */
int64_t oracle_append_kv(int64_t n, const int64_t *loc, int64_t row_bytes, const uint8_t *k_new,
                         const uint8_t *v_new, int64_t num_slots, uint8_t *k_cache,
                         uint8_t *v_cache)
{
    int64_t skipped = 0;
    for (int64_t i = 0; i < n; ++i) {
        const int64_t s = loc[i];
        if (s < 0 || s >= num_slots) {
            ++skipped;
            continue;
        }
        memcpy(k_cache + s * row_bytes, k_new + i * row_bytes, (size_t)row_bytes);
        memcpy(v_cache + s * row_bytes, v_new + i * row_bytes, (size_t)row_bytes);
    }
    return skipped;
}

/*
 * Rounding to the 8-bit cache formats (the cast of set_kv_buffer when the
 * pool holds 8-bit floats): round to nearest, ties to even mantissa.  E4M3
 * ("fn", bias 7, 3 mantissa bits, largest 448, no infinities): a value that
 * rounds past 448, an infinity or a NaN becomes NaN (S.1111.111).  E5M2 (bias
 * 15, 2 mantissa bits, largest 57344): a value that rounds past 57344 becomes
 * +-inf, a NaN stays NaN.  Subnormals are kept (steps of 2^-9 and 2^-16).
 */
/* binade of a > 0: the e with 2^e <= a < 2^(e+1) */
static int binade(double a)
{
    int e = (int)floor(log2(a));
    if (ldexp(1.0, e) > a)
        --e;
    if (ldexp(1.0, e + 1) <= a)
        ++e;
    return e;
}

/* a >= 0 rounded to the grid of a float format with mbits mantissa bits and
 * smallest normal exponent emin (subnormal steps below it), ties to even */
static double round_to_grid(double a, int mbits, int emin)
{
    if (a == 0.0)
        return 0.0;
    int e = binade(a);
    if (e < emin)
        e = emin;
    const double q = ldexp(1.0, e - mbits); /* the step of that binade */
    double r = floor(a / q);                /* a / q is exact: q is 2^k */
    const double frac = a / q - r;
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0))
        r += 1.0;
    return r * q;
}

static uint8_t round_to_fp8(double v, int e4)
{
    const int mbits = e4 ? 3 : 2, bias = e4 ? 7 : 15;
    const uint8_t sign = signbit(v) ? 0x80 : 0;
    if (isnan(v))
        return (uint8_t)(sign | 0x7f);
    const double a = fabs(v);
    /* E4M3: 464 ties to 448 (even); above it the value rounds onto the NaN
     * pattern.  E5M2: 61440 ties to 65536 (even), i.e. overflows to inf. */
    if (e4 ? (a > 464.0) : (a >= 61440.0))
        return (uint8_t)(sign | (e4 ? 0x7f : 0x7c));
    const double r = round_to_grid(a, mbits, 1 - bias);
    if (r == 0.0)
        return sign;
    const int e = binade(r);
    if (e < 1 - bias) /* subnormal: r = f * 2^(1 - bias - mbits) */
        return (uint8_t)(sign | (int)ldexp(r, bias - 1 + mbits));
    const int f = (int)ldexp(r, mbits - e) - (1 << mbits);
    return (uint8_t)(sign | ((e + bias) << mbits) | f);
}

/* RNE to bf16 or IEEE half (fp32: unchanged) */
static double round_to_16(double v, int dtype)
{
    if (isnan(v) || isinf(v) || dtype == ORACLE_FP32)
        return v;
    const double a = fabs(v), sv = signbit(v) ? -1.0 : 1.0;
    if (dtype == ORACLE_BF16) /* 8 exponent bits: overflow only past fp32's range */
        return sv * round_to_grid(a, 7, -126);
    if (a >= 65520.0) /* half: 65520 ties to 65536 (even), i.e. inf */
        return sv * INFINITY;
    return sv * round_to_grid(a, 10, -14);
}

/* The 8-bit encoding of one stored element x of in_dtype divided by scale the
 * way set_kv_buffer does it: the quotient in fp32 (a correctly rounded single
 * division), rounded to in_dtype, then to the 8-bit format. */
uint8_t oracle_quantize(int32_t in_dtype, double x, float scale, int32_t kv_dtype)
{
    const float y = (float)x / scale;
    return round_to_fp8(round_to_16((double)y, in_dtype), kv_dtype == ORACLE_FP8_E4M3);
}

/* oracle_quantize over n stored elements */
void oracle_quantize_many(int32_t in_dtype, const void *src, int64_t n, float scale,
                          int32_t kv_dtype, uint8_t *dst)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = oracle_quantize(in_dtype, load_elem(src, in_dtype, i), scale, kv_dtype);
}

/*
 * Writing new keys and values into an 8-bit cache: row i of k_new / v_new
 * (in_dtype, elems per row) goes to slot loc[i], each element quantized as
 * oracle_quantize with k_scale / v_scale.  Out-of-pool slots are skipped and
 * counted (returned).
 */
int64_t oracle_append_kv_quant(int64_t n, const int64_t *loc, int64_t elems, int32_t in_dtype,
                               const void *k_new, const void *v_new, int64_t num_slots,
                               int32_t kv_dtype, float k_scale, float v_scale, uint8_t *k_cache,
                               uint8_t *v_cache)
{
    int64_t skipped = 0;
    for (int64_t i = 0; i < n; ++i) {
        const int64_t s = loc[i];
        if (s < 0 || s >= num_slots) {
            ++skipped;
            continue;
        }
        for (int64_t e = 0; e < elems; ++e) {
            k_cache[s * elems + e] =
                oracle_quantize(in_dtype, load_elem(k_new, in_dtype, i * elems + e), k_scale,
                                kv_dtype);
            v_cache[s * elems + e] =
                oracle_quantize(in_dtype, load_elem(v_new, in_dtype, i * elems + e), v_scale,
                                kv_dtype);
        }
    }
    return skipped;
}

/*
 * Building the page table on the device ([FIB] call_begin_forward: kv_indptr
 * is the running sum of the per-request lengths, and the gather
 * create_flashinfer_kv_indices_triton copies, for request b, entries
 * start[b] .. start[b] + len[b] - 1 of row slot[b] of the request-to-page map
 * into kv_indices from kv_indptr[b] on).
 *
 *  map      [map_rows, map_cols] int32     start  [batch] or NULL (all 0)
 *  slot     [batch] rows of the map        len    [batch] entries per request
 *  kv_indptr [batch + 1] (out)             kv_indices [capacity] (out)
 *
 * A negative len counts as 0; an entry whose source lies outside the map is
 * written as -1; an entry past `capacity` is not written.  Each of these is
 * counted in the return value.
 */
int64_t oracle_build_kv_indices(int32_t batch, const int32_t *map, int64_t map_rows,
                                int64_t map_cols, const int32_t *slot, const int32_t *start,
                                const int32_t *len, int32_t *kv_indptr, int32_t *kv_indices,
                                int64_t capacity)
{
    int64_t errors = 0;
    kv_indptr[0] = 0;
    for (int32_t b = 0; b < batch; ++b) {
        int64_t n = len[b];
        if (n < 0) {
            ++errors;
            n = 0;
        }
        kv_indptr[b + 1] = (int32_t)(kv_indptr[b] + n);
        const int64_t s0 = start ? start[b] : 0;
        for (int64_t j = 0; j < n; ++j) {
            const int64_t dst = (int64_t)kv_indptr[b] + j;
            if (dst >= capacity) {
                ++errors;
                continue;
            }
            const int64_t col = s0 + j;
            if (slot[b] < 0 || slot[b] >= map_rows || col < 0 || col >= map_cols) {
                ++errors;
                kv_indices[dst] = -1;
            } else {
                kv_indices[dst] = map[(int64_t)slot[b] * map_cols + col];
            }
        }
    }
    return errors;
}
