/*
 * pkv_oracle.c -- CPU reference ("oracle") for attention over a paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or constant with
 * the HIP library: it has its own argument conventions, written from the
 * pages' description of the method, and it is deliberately plain and slow.
 *
 * What it computes (all arithmetic in IEEE fp64; bf16/fp32 inputs are widened
 * exactly):
 *
 *  - Routing.  Logical token j of sequence b lives in physical page
 *    block_table[b][j / page_size] at slot j % page_size.  The page table maps
 *    (logical batch, logical block) -> physical page [unsloth scripts commit
 *    page, "Why this works" item 1; mini-infer 06 "True PagedAttention", §1,
 *    block_table argument].  Inside a page the element (slot, kv head, dim)
 *    sits at page*s_page + head*s_head + slot*s_tok + dim (element strides;
 *    the dim stride is 1), which covers both the head-major "HND" pool of the
 *    FlashInfer PR #9451 analysis (§1 domain check) and the
 *    (num_blocks, block_size, num_kv_heads, head_dim) block tensor of
 *    mini-infer 06 §1.
 *
 *  - Append.  Each new K/V token of sequence b is copied bit for bit into
 *    logical position cache_seqlens[b] + t, i.e. written in place into the
 *    page the table routes that position to, before attention reads the pool
 *    [mini-infer 06, §1, the three things flash_attn_with_kvcache does].
 *
 *  - Rotary position embedding (optional, before the append).  The new
 *    token's q and k head vectors are rotated pair by pair by the angle of
 *    its position, from caller-given cos/sin tables, in the half-split or the
 *    interleaved pair layout [mini-infer 06, §3]; see pkvref_rope.
 *
 *  - Attention.  For query row i of request r (kv_len keys, q_len queries,
 *    end-aligned causal), the row sees keys 0 .. kv_len - q_len + i, i.e.
 *    kv_len - q_len + i + 1 keys [FlashInfer PR #9451 analysis, §1, the
 *    causal work bound].  Decode is the q_len == 1 case: the single query sees
 *    all kv_len keys, including the token appended in the same step.  Query
 *    head h reads KV head h / (num_q_heads / num_kv_heads) (consecutive
 *    grouping of the GQA ratio, §1 domain check).  The row's output is plain
 *    softmax attention, evaluated in two passes over the page walk:
 *        s_j = scale * sum_d q[d] * K_j[d]           (pass 1, M = max_j s_j)
 *        w_j = exp(s_j - M), Z = sum_j w_j,
 *        out[d] = sum_j w_j V_j[d] / Z,  lse = M + ln Z   (pass 2)
 *    A row with no visible key returns out = 0 and lse = -inf (the pages call
 *    a NaN from a fully masked row a bug: flex-vs-vLLM results page,
 *    "What broke").
 *
 * Every entry point returns 0 on success and a positive code naming the first
 * violated precondition otherwise; on failure no output is written.
 */
#include "pkv_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* element access                                                            */
/* ------------------------------------------------------------------------ */

static size_t elem_bytes(int dtype) { return dtype == PKVREF_BF16 ? 2u : 4u; }

/* Exact widening of one stored element to fp64.  A bf16 value is the top 16
 * bits of the fp32 value with the same sign, exponent and leading mantissa
 * bits, so shifting it up by 16 reproduces it exactly. */
static double load_elem(const void *base, int64_t idx, int dtype)
{
    if (dtype == PKVREF_BF16) {
        uint16_t h;
        memcpy(&h, (const char *)base + (size_t)idx * 2u, 2);
        uint32_t u = (uint32_t)h << 16;
        float f;
        memcpy(&f, &u, 4);
        return (double)f;
    } else {
        float f;
        memcpy(&f, (const char *)base + (size_t)idx * 4u, 4);
        return (double)f;
    }
}

static void copy_elem(void *dst, int64_t di, const void *src, int64_t si, int dtype)
{
    size_t es = elem_bytes(dtype);
    memcpy((char *)dst + (size_t)di * es, (const char *)src + (size_t)si * es, es);
}

/* ------------------------------------------------------------------------ */
/* routing                                                                   */
/* ------------------------------------------------------------------------ */

/* Element offset of (token j of sequence b, kv head g, dim 0) in the pool. */
static int64_t token_offset(const pkvref_pool *pool, const int32_t *block_table,
                            int bt_cols, int b, int64_t j, int g)
{
    int64_t logical_block = j / pool->page_size;
    int64_t slot = j % pool->page_size;
    int64_t page = block_table[(int64_t)b * bt_cols + logical_block];
    return page * pool->s_page + (int64_t)g * pool->s_head + slot * pool->s_tok;
}

/* Checks that every block a sequence of length len touches is a real page
 * (1 .. num_pages-1; page 0 is the reserved padding page) and that the table
 * has enough columns.  Returns 0 or an error code. */
static int check_row_pages(const pkvref_pool *pool, const int32_t *block_table,
                           int bt_cols, int b, int64_t len)
{
    int64_t nblocks = (len + pool->page_size - 1) / pool->page_size;
    if (nblocks > bt_cols)
        return PKVREF_E_TABLE_COLS;
    for (int64_t blk = 0; blk < nblocks; ++blk) {
        int32_t page = block_table[(int64_t)b * bt_cols + blk];
        if (page < 1 || page >= pool->num_pages)
            return PKVREF_E_PAGE_RANGE;
    }
    return 0;
}

static int check_pool(const pkvref_pool *pool)
{
    if (!pool)
        return PKVREF_E_ARG;
    if (pool->dtype != PKVREF_F32 && pool->dtype != PKVREF_BF16)
        return PKVREF_E_ARG;
    if (pool->num_pages < 1 || pool->page_size < 1 || pool->num_kv_heads < 1 ||
        pool->head_dim < 1)
        return PKVREF_E_ARG;
    if (pool->s_page < 0 || pool->s_head < 0 || pool->s_tok < 0)
        return PKVREF_E_ARG;
    return 0;
}

int pkvref_route(const pkvref_pool *pool, const int32_t *block_table, int bt_cols,
                 const int32_t *seqlens, int batch, int max_len, int64_t *offsets)
{
    int rc = check_pool(pool);
    if (rc)
        return rc;
    if (batch < 0 || max_len < 0 || !offsets)
        return PKVREF_E_ARG;
    for (int b = 0; b < batch; ++b) {
        if (seqlens[b] < 0 || seqlens[b] > max_len)
            return PKVREF_E_LENGTH;
        rc = check_row_pages(pool, block_table, bt_cols, b, seqlens[b]);
        if (rc)
            return rc;
    }
    for (int b = 0; b < batch; ++b)
        for (int64_t j = 0; j < max_len; ++j)
            offsets[(int64_t)b * max_len + j] =
                j < seqlens[b] ? token_offset(pool, block_table, bt_cols, b, j, 0) : -1;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* append                                                                    */
/* ------------------------------------------------------------------------ */

int pkvref_append(const pkvref_pool *pool, void *k_cache, void *v_cache,
                  const void *k_new, const void *v_new, const int32_t *block_table,
                  int bt_cols, const int32_t *cache_seqlens, const int32_t *new_indptr,
                  int batch, int total_new, int32_t *seqlens_out)
{
    int rc = check_pool(pool);
    if (rc)
        return rc;
    if (batch < 0 || total_new < 0 || !k_cache || !v_cache)
        return PKVREF_E_ARG;
    /* preconditions first, so that a failure writes nothing */
    for (int b = 0; b < batch; ++b) {
        int64_t n_new = new_indptr ? new_indptr[b + 1] - new_indptr[b] : 1;
        if (n_new < 0 || cache_seqlens[b] < 0)
            return PKVREF_E_LENGTH;
        rc = check_row_pages(pool, block_table, bt_cols, b, cache_seqlens[b] + n_new);
        if (rc)
            return rc;
    }
    if (new_indptr ? (new_indptr[0] != 0 || new_indptr[batch] != total_new)
                   : (total_new != batch))
        return PKVREF_E_INDPTR;

    const int H = pool->num_kv_heads, D = pool->head_dim;
    for (int b = 0; b < batch; ++b) {
        int64_t first = new_indptr ? new_indptr[b] : b;
        int64_t n_new = new_indptr ? new_indptr[b + 1] - new_indptr[b] : 1;
        for (int64_t t = 0; t < n_new; ++t) {
            int64_t pos = (int64_t)cache_seqlens[b] + t;
            for (int g = 0; g < H; ++g) {
                int64_t dst = token_offset(pool, block_table, bt_cols, b, pos, g);
                int64_t src = ((first + t) * H + g) * (int64_t)D;
                for (int d = 0; d < D; ++d) {
                    copy_elem(k_cache, dst + d, k_new, src + d, pool->dtype);
                    copy_elem(v_cache, dst + d, v_new, src + d, pool->dtype);
                }
            }
        }
        if (seqlens_out)
            seqlens_out[b] = (int32_t)(cache_seqlens[b] + n_new);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* rotary position embedding                                                 */
/* ------------------------------------------------------------------------ */

/* Round an fp64 value to the nearest bf16 value, ties to even, and return
 * its bit pattern.  bf16 keeps 8 significant bits and fp32's exponent range:
 * the value is scaled so that its rounding quantum becomes 1, rounded to the
 * nearest integer with ties to even (rint in the default rounding mode), and
 * scaled back, both scalings being exact powers of two.  Values below the
 * smallest normal (2^-126) share the subnormal quantum 2^-133; results of
 * magnitude 2^128 or more are infinities. */
static uint16_t round_to_bf16(double v)
{
    float f;
    if (isnan(v)) {
        f = (float)v;
    } else if (v == 0.0 || isinf(v)) {
        f = (float)v;
    } else {
        int e;
        frexp(v, &e);                        /* 2^(e-1) <= |v| < 2^e */
        int qexp = (e < -125 ? -125 : e) - 8; /* quantum 2^qexp: 8 significant bits */
        double r = ldexp(rint(ldexp(v, -qexp)), qexp);
        f = fabs(r) >= ldexp(1.0, 128) ? (r > 0 ? INFINITY : -INFINITY) : (float)r; /* exact */
    }
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

/* Store an fp64 value as one element of the given dtype, rounded to nearest
 * with ties to even. */
static void store_rounded(void *base, int64_t idx, int dtype, double v)
{
    if (dtype == PKVREF_BF16) {
        uint16_t h = round_to_bf16(v);
        memcpy((char *)base + (size_t)idx * 2u, &h, 2);
    } else {
        float f = (float)v;
        memcpy((char *)base + (size_t)idx * 4u, &f, 4);
    }
}

/* Rotary position embedding of a token's head vectors (the rotation Qwen's
 * attention applies to q and k before the paged call: mini-infer 06 "True
 * PagedAttention", §3, which also names the two cos/sin layouts).  The
 * head_dim values of a head form head_dim/2 pairs: pair i is (i, i +
 * head_dim/2) in the half-split layout and (2i, 2i+1) in the interleaved
 * one.  At position p pair i is turned by the angle whose cosine and sine
 * are cos_table[p][i] and sin_table[p][i]:
 *     a' = a cos - b sin,   b' = b cos + a sin,
 * computed in fp64 from the exactly widened values and rounded once to the
 * element dtype.  x is [rows, heads, head_dim], rotated in place; row r is at
 * position positions[r]. */
int pkvref_rope(int dtype, void *x, int64_t rows, int heads, int head_dim,
                const int32_t *positions, const float *cos_table, const float *sin_table,
                int64_t table_rows, int interleaved)
{
    if ((dtype != PKVREF_F32 && dtype != PKVREF_BF16) || rows < 0 || heads < 1 || head_dim < 2 ||
        head_dim % 2 || !x || !positions || !cos_table || !sin_table)
        return PKVREF_E_ARG;
    for (int64_t r = 0; r < rows; ++r)
        if (positions[r] < 0 || positions[r] >= table_rows)
            return PKVREF_E_LENGTH;
    const int half = head_dim / 2;
    for (int64_t r = 0; r < rows; ++r) {
        const float *c = cos_table + (int64_t)positions[r] * half;
        const float *s = sin_table + (int64_t)positions[r] * half;
        for (int h = 0; h < heads; ++h) {
            int64_t base = (r * heads + h) * (int64_t)head_dim;
            for (int i = 0; i < half; ++i) {
                int64_t ia = base + (interleaved ? 2 * i : i);
                int64_t ib = base + (interleaved ? 2 * i + 1 : i + half);
                double a = load_elem(x, ia, dtype), b = load_elem(x, ib, dtype);
                double ci = (double)c[i], si = (double)s[i];
                double ra = a * ci - b * si;
                double rb = b * ci + a * si;
                store_rounded(x, ia, dtype, ra);
                store_rounded(x, ib, dtype, rb);
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* attention                                                                 */
/* ------------------------------------------------------------------------ */

/* One query row: q_row (dtype elements, head_dim long) against the first
 * n_visible keys of sequence b, kv head g.  scores is caller scratch of at
 * least n_visible doubles. */
static void attend_row(const pkvref_pool *pool, const void *k_cache, const void *v_cache,
                       const int32_t *block_table, int bt_cols, int b, int g,
                       const void *q, int64_t q_index, int64_t n_visible, double scale,
                       double *scores, double *out_row, double *lse_out)
{
    const int D = pool->head_dim;
    for (int d = 0; d < D; ++d)
        out_row[d] = 0.0;
    if (n_visible <= 0) {
        *lse_out = -INFINITY;
        return;
    }
    /* pass 1: scores and their maximum, walking the row's pages in order */
    double m = -INFINITY;
    for (int64_t j = 0; j < n_visible; ++j) {
        int64_t base = token_offset(pool, block_table, bt_cols, b, j, g);
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += load_elem(q, q_index + d, pool->dtype) * load_elem(k_cache, base + d, pool->dtype);
        scores[j] = scale * dot;
        if (scores[j] > m)
            m = scores[j];
    }
    /* pass 2: normalised weights applied to V */
    double z = 0.0;
    for (int64_t j = 0; j < n_visible; ++j) {
        double w = exp(scores[j] - m);
        z += w;
        int64_t base = token_offset(pool, block_table, bt_cols, b, j, g);
        for (int d = 0; d < D; ++d)
            out_row[d] += w * load_elem(v_cache, base + d, pool->dtype);
    }
    for (int d = 0; d < D; ++d)
        out_row[d] /= z;
    *lse_out = m + log(z);
}

/* Work description shared by the worker threads of one attention call. */
typedef struct {
    const pkvref_pool *pool;
    const void *q, *k_cache, *v_cache;
    const int32_t *block_table, *kv_lens, *qo_indptr;
    int bt_cols, batch, num_q_heads, causal;
    double scale;
    double *out, *lse;
    int64_t *pair_counts;      /* [batch, num_q_heads] or NULL */
    const int32_t *row_request; /* query token -> request */
    int64_t n_units;           /* query tokens * num_q_heads */
    int64_t next;              /* next unit to hand out (atomic) */
    int64_t max_kv;
} attn_job;

static void *attn_worker(void *arg)
{
    attn_job *job = (attn_job *)arg;
    const int D = job->pool->head_dim;
    const int group = job->num_q_heads / job->pool->num_kv_heads;
    double *scores = (double *)malloc(sizeof(double) * (size_t)(job->max_kv > 0 ? job->max_kv : 1));
    if (!scores)
        return (void *)1;
    for (;;) {
        int64_t unit = __atomic_fetch_add(&job->next, 1, __ATOMIC_RELAXED);
        if (unit >= job->n_units)
            break;
        int64_t token = unit / job->num_q_heads;
        int h = (int)(unit % job->num_q_heads);
        int r = job->row_request[token];
        int64_t q_len = job->qo_indptr[r + 1] - job->qo_indptr[r];
        int64_t i = token - job->qo_indptr[r];
        int64_t kv = job->kv_lens[r];
        int64_t visible = job->causal ? kv - q_len + i + 1 : kv;
        int g = h / group;
        attend_row(job->pool, job->k_cache, job->v_cache, job->block_table, job->bt_cols, r, g,
                   job->q, (token * job->num_q_heads + h) * (int64_t)D, visible, job->scale,
                   scores, job->out + unit * D, job->lse + unit);
        if (job->pair_counts)
            __atomic_fetch_add(&job->pair_counts[(int64_t)r * job->num_q_heads + h],
                               visible > 0 ? visible : 0, __ATOMIC_RELAXED);
    }
    free(scores);
    return NULL;
}

static int run_attention(attn_job *job, int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    pthread_t tids[256];
    int started = 0, failed = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&tids[started], NULL, attn_worker, job) != 0)
            break;
        ++started;
    }
    if (attn_worker(job) != NULL)
        failed = 1;
    for (int t = 0; t < started; ++t) {
        void *ret = NULL;
        pthread_join(tids[t], &ret);
        if (ret != NULL)
            failed = 1;
    }
    return failed ? PKVREF_E_ALLOC : 0;
}

int pkvref_prefill(const pkvref_pool *pool, double *out, double *lse, const void *q,
                   int num_q_heads, const void *k_cache, const void *v_cache,
                   const int32_t *block_table, int bt_cols, const int32_t *kv_lens,
                   const int32_t *qo_indptr, int batch, int causal, double scale,
                   int64_t *pair_counts, int nthreads)
{
    int rc = check_pool(pool);
    if (rc)
        return rc;
    if (batch < 0 || num_q_heads < 1 || !out || !lse || !qo_indptr)
        return PKVREF_E_ARG;
    if (num_q_heads % pool->num_kv_heads != 0)
        return PKVREF_E_ARG;
    if (qo_indptr[0] != 0)
        return PKVREF_E_INDPTR;
    int64_t max_kv = 0;
    for (int r = 0; r < batch; ++r) {
        int64_t q_len = qo_indptr[r + 1] - qo_indptr[r];
        if (q_len < 0)
            return PKVREF_E_INDPTR;
        /* end-aligned causal prefill needs 0 < q_len <= kv_len; a request
         * with no query rows is allowed and produces nothing */
        if (kv_lens[r] < 0 || (causal && q_len > kv_lens[r]))
            return PKVREF_E_LENGTH;
        rc = check_row_pages(pool, block_table, bt_cols, r, kv_lens[r]);
        if (rc)
            return rc;
        if (kv_lens[r] > max_kv)
            max_kv = kv_lens[r];
    }
    int64_t total_q = qo_indptr[batch];
    int32_t *row_request = (int32_t *)malloc(sizeof(int32_t) * (size_t)(total_q > 0 ? total_q : 1));
    if (!row_request)
        return PKVREF_E_ALLOC;
    for (int r = 0; r < batch; ++r)
        for (int64_t t = qo_indptr[r]; t < qo_indptr[r + 1]; ++t)
            row_request[t] = r;
    if (pair_counts)
        memset(pair_counts, 0, sizeof(int64_t) * (size_t)batch * (size_t)num_q_heads);

    attn_job job;
    memset(&job, 0, sizeof job);
    job.pool = pool;
    job.q = q;
    job.k_cache = k_cache;
    job.v_cache = v_cache;
    job.block_table = block_table;
    job.kv_lens = kv_lens;
    job.qo_indptr = qo_indptr;
    job.bt_cols = bt_cols;
    job.batch = batch;
    job.num_q_heads = num_q_heads;
    job.causal = causal;
    job.scale = scale;
    job.out = out;
    job.lse = lse;
    job.pair_counts = pair_counts;
    job.row_request = row_request;
    job.n_units = total_q * num_q_heads;
    job.next = 0;
    job.max_kv = max_kv;
    rc = run_attention(&job, nthreads);
    free(row_request);
    return rc;
}

int pkvref_decode(const pkvref_pool *pool, double *out, double *lse, const void *q,
                  int num_q_heads, const void *k_cache, const void *v_cache,
                  const int32_t *block_table, int bt_cols, const int32_t *seqlens,
                  int batch, double scale, int nthreads)
{
    if (batch < 0)
        return PKVREF_E_ARG;
    /* decode = one query token per sequence that sees every cached key */
    int32_t *indptr = (int32_t *)malloc(sizeof(int32_t) * (size_t)(batch + 1));
    if (!indptr)
        return PKVREF_E_ALLOC;
    for (int b = 0; b <= batch; ++b)
        indptr[b] = b;
    int rc = pkvref_prefill(pool, out, lse, q, num_q_heads, k_cache, v_cache, block_table,
                            bt_cols, seqlens, indptr, batch, /*causal=*/0, scale, NULL,
                            nthreads);
    free(indptr);
    return rc;
}
