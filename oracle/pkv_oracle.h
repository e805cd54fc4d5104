/*
 * pkv_oracle.h -- CPU fp64 reference for paged KV attention (test
 * infrastructure; see pkv_oracle.c for what is computed and why).
 *
 * All pointers are host pointers.  Tensors are dense and row-major unless a
 * stride says otherwise:
 *   q           [tokens, num_q_heads, head_dim]            (dtype)
 *   k_new/v_new [total_new, num_kv_heads, head_dim]        (dtype)
 *   k/v cache   element (page, kv head, slot, dim) at
 *               page*s_page + head*s_head + slot*s_tok + dim
 *   block_table [batch, bt_cols] int32, physical page per logical block
 *   out         [tokens, num_q_heads, head_dim] fp64
 *   lse         [tokens, num_q_heads] fp64 (natural log)
 */
#ifndef PKV_ORACLE_H
#define PKV_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { PKVREF_F32 = 0, PKVREF_BF16 = 1 };

enum {
    PKVREF_OK = 0,
    PKVREF_E_ARG = 1,        /* bad scalar argument or null pointer */
    PKVREF_E_PAGE_RANGE = 2, /* a touched block maps outside 1..num_pages-1 */
    PKVREF_E_TABLE_COLS = 3, /* a sequence needs more blocks than the table has */
    PKVREF_E_LENGTH = 4,     /* negative length, or q_len > kv_len when causal */
    PKVREF_E_INDPTR = 5,     /* indptr not starting at 0 / not matching totals */
    PKVREF_E_ALLOC = 6       /* host allocation failed */
};

typedef struct {
    int32_t dtype;        /* PKVREF_F32 or PKVREF_BF16 */
    int32_t num_pages;    /* physical pages in the pool, page 0 included */
    int32_t page_size;    /* tokens per page */
    int32_t num_kv_heads;
    int32_t head_dim;
    int64_t s_page, s_head, s_tok; /* element strides; the dim stride is 1 */
} pkvref_pool;

int pkvref_route(const pkvref_pool *pool, const int32_t *block_table, int bt_cols,
                 const int32_t *seqlens, int batch, int max_len, int64_t *offsets);

int pkvref_append(const pkvref_pool *pool, void *k_cache, void *v_cache,
                  const void *k_new, const void *v_new, const int32_t *block_table,
                  int bt_cols, const int32_t *cache_seqlens, const int32_t *new_indptr,
                  int batch, int total_new, int32_t *seqlens_out);

/* Rotary position embedding of x [rows, heads, head_dim] (dtype elements) in
 * place: row r at position positions[r] < table_rows; cos_table and
 * sin_table are fp32 [table_rows, head_dim/2]; interleaved selects pairs
 * (2i, 2i+1) instead of (i, i + head_dim/2). */
int pkvref_rope(int dtype, void *x, int64_t rows, int heads, int head_dim,
                const int32_t *positions, const float *cos_table, const float *sin_table,
                int64_t table_rows, int interleaved);

int pkvref_decode(const pkvref_pool *pool, double *out, double *lse, const void *q,
                  int num_q_heads, const void *k_cache, const void *v_cache,
                  const int32_t *block_table, int bt_cols, const int32_t *seqlens,
                  int batch, double scale, int nthreads);

int pkvref_prefill(const pkvref_pool *pool, double *out, double *lse, const void *q,
                   int num_q_heads, const void *k_cache, const void *v_cache,
                   const int32_t *block_table, int bt_cols, const int32_t *kv_lens,
                   const int32_t *qo_indptr, int batch, int causal, double scale,
                   int64_t *pair_counts, int nthreads);

#ifdef __cplusplus
}
#endif

#endif /* PKV_ORACLE_H */
