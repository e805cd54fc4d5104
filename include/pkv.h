/*
 * pkv.h -- C ABI of libpkv: attention over a paged KV cache on AMD Instinct
 * MI355X (gfx950).
 *
 * The KV cache is one pool of fixed-size physical pages per layer for K and
 * one for V.  Each sequence owns a row of `block_table` that maps its logical
 * blocks to physical pages; logical token j of sequence b lives in page
 * block_table[b][j / page_size] at slot j % page_size.  This is the routing
 * of the flash_attn `block_table` / `cache_seqlens` call described in
 * mini-infer 06 "True PagedAttention" §1 and of the page table in the
 * unsloth scripts commit page ("Why this works", item 1).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument is a DEVICE pointer unless its comment says
 *    "host".  All buffers are owned by the caller; the library allocates and
 *    frees nothing, keeps no state between calls and never reads device
 *    memory back to the host, so calls never synchronise the stream and are
 *    safe to capture in a HIP graph.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *    work is enqueued on it asynchronously.
 *  - Only host scalars and pointer nullness are checked.  Device-resident
 *    metadata (tables, lengths, indptr) is the caller's contract; on the host
 *    it can be checked with pkv_validate_host / pkv_validate_append_host.
 *    Violating it is undefined behaviour (out-of-bounds device accesses).
 *  - Return value: PKV_OK, or an error code; on an error nothing has been
 *    enqueued except for PKV_ELAUNCH (the launch itself failed).
 *
 * Pool layout (pkv_cache_desc)
 * ----------------------------
 * Element (page, kv_head, slot, dim) of a pool is at element offset
 *     page * s_page + kv_head * s_head + slot * s_tok + dim
 * from the pool base; the dim stride is 1.  The head-major "HND" layout of
 * the FlashInfer PR #9451 analysis (§1 domain check) is
 * [num_pages, num_kv_heads, page_size, head_dim] (s_tok = head_dim,
 * s_head = page_size*head_dim); the flash_attn block tensor
 * (num_blocks, block_size, num_kv_heads, head_dim) of mini-infer 06 §1 is
 * "NHD" (s_head = head_dim, s_tok = num_kv_heads*head_dim).  K and V pools
 * share one descriptor.  Page 0 is reserved: tables never need to route a
 * live token to it, and unused table entries may hold 0.
 *
 * Supported: dtype PKV_BF16 or PKV_F32; page_size 16, 32, 64, 128 or 256
 * (the 256-token blocks of mini-infer 06 §1 included; other sizes, and pools
 * with num_pages * page_size above 2^31 - 1 tokens, give PKV_EUNSUPPORTED --
 * the kernels walk every page as page_size / 16 runs of 16 consecutive
 * slots, so the arithmetic and the results are those of 16-token pages
 * whose table entries are expanded); head_dim 64, 128 or 256; a GQA ratio G = num_q_heads / num_kv_heads from 1 to 16 (this covers
 * the ratios {1, 2, 4, 8, 16} of the FlashInfer PR #9451 analysis, §1, and
 * the 48/8 = 6 of its D=256 workload); strides multiples of 8 elements and
 * all pointers 16-byte aligned.  Query head h reads KV head h / G.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 3

typedef enum pkv_status {
    PKV_OK = 0,
    PKV_EINVAL = 1,        /* null pointer, non-positive size, inconsistent sizes */
    PKV_EUNSUPPORTED = 2,  /* dtype, head_dim, page_size, GQA ratio, stride or alignment */
    PKV_EWORKSPACE = 3,    /* workspace missing or smaller than the query says */
    PKV_ELAUNCH = 4,       /* a kernel launch failed (hipGetLastError) */
    PKV_EDEVICE = 5,       /* no usable HIP device / device query failed */
    PKV_EVALIDATE = 6      /* pkv_validate_*: a device-data precondition is violated */
} pkv_status;

typedef enum pkv_dtype { PKV_F32 = 0, PKV_BF16 = 1 } pkv_dtype;

typedef struct pkv_cache_desc {
    int32_t dtype;        /* pkv_dtype of the pools, q, new K/V and out */
    int32_t num_pages;    /* physical pages per pool, page 0 included */
    int32_t page_size;    /* tokens per page: 16, 32, 64, 128 or 256 */
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t reserved;     /* must be 0 */
    int64_t s_page;       /* element strides of the pool; dim stride is 1 */
    int64_t s_head;
    int64_t s_tok;
} pkv_cache_desc;

/* PKV_ABI_VERSION of the loaded library. */
int32_t pkv_abi_version(void);

/* Static text for a status code (never NULL). */
const char *pkv_status_string(pkv_status status);

/*
 * pkv_append -- write each step's new K/V into the pool in place.
 *
 * The write half of flash_attn_with_kvcache(k=, v=, cache_seqlens, block_table)
 * in mini-infer 06 §1 (new keys are stored at the current cache length, in the
 * block the table routes that position to), and the in-graph
 * `k_cache[addr] = k_val` of the unsloth scripts commit page ("Files").
 *
 *   k_new, v_new   [total_new, num_kv_heads, head_dim], dense, dtype of the pool
 *   block_table    int32 [batch, bt_cols]
 *   cache_seqlens  int32 [batch]: tokens already cached (pre-append length L_b)
 *   new_indptr     int32 [batch+1], new_indptr[0] = 0, new_indptr[batch] =
 *                  total_new: sequence b appends rows new_indptr[b] ..
 *                  new_indptr[b+1]-1.  NULL means one token per sequence
 *                  (total_new must equal batch).
 *   seqlens_out    int32 [batch] or NULL: receives L_b + tokens appended, the
 *                  attended length for the following attention call.  Must not
 *                  alias cache_seqlens.
 * A padding row (cache_seqlens[b] = -1, the fixed-size batch slots of a
 * captured decode graph: unsloth scripts commit page, "Why this works" item
 * 3) writes nothing and keeps seqlens_out[b] = -1; its new_indptr range may
 * hold rows, which are ignored.
 * Token t of sequence b goes to logical position L_b + t; its page must be a
 * real page (1..num_pages-1) and no two appended tokens may share a slot.  The
 * copy is bit-exact; no other byte of either pool is written.
 */
pkv_status pkv_append(const pkv_cache_desc *cache, void *k_cache, void *v_cache,
                      const void *k_new, const void *v_new, const int32_t *block_table,
                      int32_t bt_cols, const int32_t *cache_seqlens, const int32_t *new_indptr,
                      int32_t batch, int32_t total_new, int32_t *seqlens_out, void *stream);

/*
 * pkv_append_rope -- pkv_append with the rotary position embedding of the
 * new tokens fused in: each new token's k is rotated before it is stored,
 * and its q (when given) is rotated in place for the attention call that
 * follows.  mini-infer 06 §3 applies this rotation to q and k right before
 * the paged flash_attn call, and notes the two cos/sin layouts in use.
 *
 * A head vector's head_dim values form head_dim/2 pairs: pair i is
 * (i, i + head_dim/2) when rope_interleaved == 0 (the half-split layout of
 * Qwen-style rotate_half) and (2i, 2i+1) otherwise (the interleaved layout).
 * Token t of sequence b is at position p = L_b + t, and its pair i turns by
 * the angle of cos/sin table row p:
 *     a' = a * rope_cos[p][i] - b * rope_sin[p][i]
 *     b' = b * rope_cos[p][i] + a * rope_sin[p][i]
 * evaluated in fp64 from the exact values and stored rounded to nearest
 * (ties to even) in the pool's dtype.  V is stored unrotated.
 *
 *   rope_cos, rope_sin  float [rope_rows, head_dim/2], device, 16-byte aligned;
 *                       every position L_b + t must be < rope_rows (a larger
 *                       position reads row rope_rows - 1: stays in bounds,
 *                       gives a wrong rotation)
 *   q                   [total_new, num_q_heads, head_dim] or NULL: rotated in
 *                       place, row new_indptr[b] + t by position L_b + t
 * The other arguments, the padding-row rule (L_b = -1: nothing rotated or
 * written) and the errors are those of pkv_append.
 */
pkv_status pkv_append_rope(const pkv_cache_desc *cache, void *k_cache, void *v_cache,
                           const void *k_new, const void *v_new, void *q, int32_t num_q_heads,
                           const float *rope_cos, const float *rope_sin, int32_t rope_rows,
                           int32_t rope_interleaved, const int32_t *block_table, int32_t bt_cols,
                           const int32_t *cache_seqlens, const int32_t *new_indptr, int32_t batch,
                           int32_t total_new, int32_t *seqlens_out, void *stream);

/*
 * pkv_decode_workspace_bytes -- device workspace pkv_decode_attn needs for
 * these sizes on the current device (bytes; 0 only for invalid arguments).
 * Depends on the descriptor, batch, num_q_heads and the device (its CU count
 * and the decode kernel's occupancy), never on the lengths: max_kv_len is
 * accepted and ignored, so one workspace serves every step of a batch shape
 * however the lengths grow or shrink.
 *
 * Layout: one int32 arrival counter per (sequence, kv head) at the start,
 * then the partial results of rows split across workers, then the plan
 * region that pkv_decode_plan writes.  The counter region must be zero
 * before a call: zero-fill the workspace before its
 * first use (pkv_decode_workspace_reset, or any fill of zeros), and again
 * when it is reused for a different batch or kv-head count.  Every call that
 * completes leaves it zero.  A launch that did not complete (an aborted or
 * faulted stream) can leave counters non-zero, which would corrupt the
 * merges of later calls: reset the workspace after any such error.  Calls
 * that run concurrently must not share a workspace.
 */
size_t pkv_decode_workspace_bytes(const pkv_cache_desc *cache, int32_t batch, int32_t num_q_heads,
                                  int32_t max_kv_len);

/*
 * pkv_decode_workspace_reset -- enqueue a zero fill of the counter region of
 * a decode workspace for `batch` rows (the first bytes of `workspace`), by a
 * small kernel on `stream` (no memset node, so it may be recorded into a
 * graph).  PKV_EWORKSPACE when the buffer is missing or too small for the
 * counters.
 */
pkv_status pkv_decode_workspace_reset(const pkv_cache_desc *cache, int32_t batch, void *workspace,
                                      size_t workspace_bytes, void *stream);

/*
 * pkv_decode_plan -- the split of a decode step's work, computed once for
 * all the decode calls of the step.
 *
 * Every layer of a decode step attends over the same block_table and
 * cache_seqlens, so how the (row, kv head, page) units are cut across the
 * split workers is the same for each layer's call; mini-infer 06 §5 makes
 * the same point for its per-step metadata (computed once, shared by every
 * layer).  This call enqueues one small kernel on `stream` that reads
 * cache_seqlens and writes that cut into the plan region of `workspace`.
 * A later pkv_decode_attn / _ex or pkv_append_decode_attn / _ex call given
 * the same workspace reads the plan together with its own lengths, and uses
 * it only if the plan was made for the same number of KV heads, batch,
 * max_kv_len, worker count and mode (`fused`) and every row's
 * cache_seqlens value still equals the planned one; otherwise the call plans
 * on its own, as it does without this call.  The cut depends on nothing
 * else, so results are bit-identical either way: the plan only saves the
 * calls the work of cutting.  It holds no page ids (each call reads the
 * table it is given, which may change freely between plan and call).
 *
 *   cache_seqlens  int32 [batch] on the device, as the calls will get it
 *                  (pre-append lengths when fused = 1)
 *   max_kv_len     as the calls will pass it
 *   fused          1: plan pkv_append_decode_attn calls; 0: pkv_decode_attn
 *   workers        as the calls will pass it (0 = automatic)
 *   workspace      a decode workspace of pkv_decode_workspace_bytes_ex(...,
 *                  workers) bytes; only its plan region is written
 * Only bf16 pools use a plan: for fp32 pools (fused = 0) the call checks its
 * arguments and enqueues nothing.  pkv_append_decode_attn_noalloc never uses
 * one.  A plan stays in the workspace until the next pkv_decode_plan on it
 * (pkv_decode_workspace_reset does not clear it).  The plan call must be
 * ordered before the calls that use it (same stream), like every use of a
 * workspace.
 * Errors: PKV_EINVAL (fused not 0 or 1, negative sizes, NULL cache_seqlens,
 * num_q_heads not a multiple of the KV heads), PKV_EUNSUPPORTED (descriptor,
 * more than 16 query heads per KV head, fused = 1 on fp32 pools, max_kv_len
 * above 2^28), PKV_EWORKSPACE (workspace
 * missing, misaligned or smaller than the query for this worker count),
 * PKV_ELAUNCH, PKV_EDEVICE; batch = 0 returns PKV_OK and enqueues nothing.
 */
pkv_status pkv_decode_plan(const pkv_cache_desc *cache, int32_t num_q_heads, const int32_t *cache_seqlens,
                           int32_t batch, int32_t max_kv_len, int32_t fused, void *workspace,
                           size_t workspace_bytes, int32_t workers, void *stream);

/*
 * pkv_decode_attn -- GQA decode attention, one query token per sequence.
 *
 * The attend half of flash_attn_with_kvcache in mini-infer 06 §1 (the
 * split-KV path it profiles in §6): query b attends the first
 * cache_seqlens[b] tokens of its row (the token appended in the same step
 * included), softmax(scale * q k^T) v, without gathering pages.
 *
 *   out            [batch, num_q_heads, head_dim], dtype of the pool
 *   lse            float [batch, num_q_heads] or NULL: natural-log
 *                  log-sum-exp of the scaled scores (-inf for an empty row)
 *   q              [batch, num_q_heads, head_dim], dtype of the pool
 *   cache_seqlens  int32 [batch]: ATTENDED length n_b (after append); 0 (or a
 *                  padding row's -1) gives out = 0 and lse = -inf for that
 *                  row, and nothing of the row (q, table) is read
 *   max_kv_len     host upper bound of cache_seqlens (no device read-back is
 *                  made to find it; mini-infer 06 §5); must satisfy
 *                  max_kv_len <= bt_cols * page_size; above 2^28 the call
 *                  returns PKV_EUNSUPPORTED
 *   workspace      device buffer of at least pkv_decode_workspace_bytes(...)
 * Long rows are split across workers and merged by a log-sum-exp combine;
 * every row's result depends only on its logical keys, not on which physical
 * pages hold them.
 */
pkv_status pkv_decode_attn(const pkv_cache_desc *cache, void *out, float *lse, const void *q,
                           int32_t num_q_heads, const void *k_cache, const void *v_cache,
                           const int32_t *block_table, int32_t bt_cols,
                           const int32_t *cache_seqlens, int32_t batch, int32_t max_kv_len,
                           float scale, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Same as pkv_decode_attn with an explicit number of split workers (0 =
 * automatic: one wave per resident slot of the device, and on the device
 * fewer for small calls so that each keeps at least 8 (16-token page, kv
 * head) units; with bf16 and head_dim 128, calls of fewer than 64 such units
 * per compute unit use at most three waves per compute unit, which measured
 * faster than four there).  A count > 0
 * is used as given (capped at the call's page count; work is cut in equal
 * shares of pages plus a fixed charge per row and kv head, so with many
 * workers some shares hold no page and those workers do nothing).  For tests of split
 * invariance and for tuning; the workspace must be sized with
 * pkv_decode_workspace_bytes_ex and the same count.
 */
size_t pkv_decode_workspace_bytes_ex(const pkv_cache_desc *cache, int32_t batch,
                                     int32_t num_q_heads, int32_t max_kv_len, int32_t workers);
pkv_status pkv_decode_attn_ex(const pkv_cache_desc *cache, void *out, float *lse, const void *q,
                              int32_t num_q_heads, const void *k_cache, const void *v_cache,
                              const int32_t *block_table, int32_t bt_cols,
                              const int32_t *cache_seqlens, int32_t batch, int32_t max_kv_len,
                              float scale, void *workspace, size_t workspace_bytes,
                              int32_t workers, void *stream);

/*
 * pkv_append_decode_attn -- one decode step in one launch: append each
 * sequence's new token to the pool and attend it with the cached ones.
 *
 * The same result as pkv_append (one token per sequence) followed by
 * pkv_decode_attn on the lengths it returns: flash_attn_with_kvcache's
 * in-place write of the new k/v at the row's current length, then attention
 * over the updated row (mini-infer 06 §1).  Folding the cache write into the
 * attention call is what the unsloth scripts page does inside its captured
 * decode step ("Why this works"); here it removes the separate append launch.
 *
 *   k_cache, v_cache  the pools (written: one slot per sequence and kv head)
 *   k_new, v_new      [batch, num_kv_heads, head_dim], dtype of the pool
 *   cache_seqlens     int32 [batch]: PRE-append length L_b; the new token goes
 *                     to position L_b and the row attends L_b + 1 keys
 *   seqlens_out       int32 [batch] or NULL: the new length of each row,
 *                     L_b + 1 where the token was stored and L_b where it
 *                     was not (see below); must not alias cache_seqlens
 *   max_kv_len        host upper bound of L_b + 1 (<= bt_cols * page_size)
 *   workspace         as for pkv_decode_attn (same size query)
 * Padding rows: cache_seqlens[b] = -1 marks a batch slot that takes no part
 * in the step (the fixed-size batch buckets of a captured decode graph:
 * unsloth scripts commit page, "Why this works" item 3).  Nothing of the row
 * is read (q, k_new, v_new, its table row may hold anything, NaN included),
 * nothing is written to the pools, out = 0, lse = -inf and seqlens_out[b]
 * stays -1.  No page needs to be reserved for such a slot.
 * Preconditions (checked on the host by pkv_validate_decode_step_host):
 * L_b + 1 <= max_kv_len, the slot's page is a real page (1..num_pages-1) and
 * no two sequences share a slot.  Where they are violated the call stays in
 * bounds and reports it: a row with L_b + 1 > max_kv_len attends its first
 * max_kv_len keys and stores nothing; a row whose slot page is not a real
 * page attends its new token but does not store it.  Either way its
 * seqlens_out entry stays L_b.  The written bytes are a bit copy of k_new /
 * v_new.  Only PKV_BF16 is supported.
 */
pkv_status pkv_append_decode_attn(const pkv_cache_desc *cache, void *out, float *lse,
                                  const void *q, int32_t num_q_heads, void *k_cache,
                                  void *v_cache, const void *k_new, const void *v_new,
                                  const int32_t *block_table, int32_t bt_cols,
                                  const int32_t *cache_seqlens, int32_t *seqlens_out,
                                  int32_t batch, int32_t max_kv_len, float scale,
                                  void *workspace, size_t workspace_bytes, void *stream);
/* With an explicit split-worker count, as pkv_decode_attn_ex. */
pkv_status pkv_append_decode_attn_ex(const pkv_cache_desc *cache, void *out, float *lse,
                                     const void *q, int32_t num_q_heads, void *k_cache,
                                     void *v_cache, const void *k_new, const void *v_new,
                                     const int32_t *block_table, int32_t bt_cols,
                                     const int32_t *cache_seqlens, int32_t *seqlens_out,
                                     int32_t batch, int32_t max_kv_len, float scale,
                                     void *workspace, size_t workspace_bytes, int32_t workers,
                                     void *stream);

/*
 * pkv_append_decode_attn_noalloc -- pkv_append_decode_attn (automatic worker
 * count) for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  It
 * takes no workspace: the library keeps one fixed array of 32 MiB in device
 * memory on each GPU it runs on (from module load until the process ends)
 * and uses it as the workspace.  The call allocates and frees nothing; it
 * enqueues a small fill kernel that clears the array's arrival counters, then
 * the decode launch.  Arguments, results and preconditions are those of
 * pkv_append_decode_attn.
 *   Limit: the workspace this call would need (pkv_decode_workspace_bytes for
 *   the same batch, num_q_heads and descriptor) must fit in 32 MiB, otherwise
 *   PKV_EWORKSPACE and nothing is enqueued.
 *   Every call on one GPU shares that GPU's array: calls that may overlap in
 *   time on one GPU (different streams, threads or processes' graphs without
 *   ordering) race on it and must not be issued; calls ordered on one stream
 *   are safe.
 */
pkv_status pkv_append_decode_attn_noalloc(const pkv_cache_desc *cache, void *out, float *lse,
                                          const void *q, int32_t num_q_heads, void *k_cache,
                                          void *v_cache, const void *k_new, const void *v_new,
                                          const int32_t *block_table, int32_t bt_cols,
                                          const int32_t *cache_seqlens, int32_t *seqlens_out,
                                          int32_t batch, int32_t max_kv_len, float scale,
                                          void *stream);

/*
 * pkv_prefill_workspace_bytes / pkv_prefill_attn -- causal (chunked) prefill
 * over the paged pool.
 *
 * Request r has q_r = qo_indptr[r+1] - qo_indptr[r] query rows (its newest
 * tokens, already appended) and kv_lens[r] keys.  With causal != 0 the
 * causal mask is end-aligned: query row i (0-based) sees keys
 * 0 .. kv_r - q_r + i, i.e. kv_r - q_r + i + 1 of them (FlashInfer PR #9451
 * analysis, §1 work bound); causal == 0 lets every row see all kv_r keys.
 *
 *   out        [total_q, num_q_heads, head_dim], dtype of the pool
 *   lse        float [total_q, num_q_heads] or NULL
 *   q          [total_q, num_q_heads, head_dim]
 *   kv_lens    int32 [batch]: keys of each request, chunk included
 *   qo_indptr  int32 [batch+1], device: ragged query offsets, qo_indptr[0] = 0,
 *              qo_indptr[batch] = total_q, 0 <= q_r (<= kv_r when causal)
 *   max_q      host upper bound of q_r; max_kv_len host upper bound of kv_r
 *   workspace  NULL, or device memory of at least pkv_prefill_workspace_bytes
 *              (same arguments, same current device), 16-byte aligned and
 *              zero-filled before its first use; each call leaves it ready
 *              for the next.  Calls that share one must not overlap.
 * Only PKV_BF16 is supported by this entry point.
 *
 * Key splits: a call whose (request, 128-row query tile, query head)
 * workgroups number at most the device's CUs, and whose longest request has
 * more than 960 keys, may cut each workgroup's keys into S pieces when it is
 * given a workspace.  S (at most 16, at most one piece per 512 keys, at most
 * three rounds of pieces over the CUs) minimises rounds x piece length, with
 * 512 keys added to each piece for its start-up and merge.  The pieces'
 * partial rows meet in the workspace (one 128 x (head_dim + 2) fp32 record
 * per piece: up to ~100 MB at head_dim 256 on 256 CUs) and are merged in a
 * fixed piece order, so results are deterministic.  They equal the unsplit
 * results up to rounding (the online softmax rescales at other points), not
 * bit for bit.
 * pkv_prefill_workspace_bytes returns 0 when the call would not split; the
 * workspace may then be NULL.  Without a workspace (NULL) the keys are never
 * split and no error is returned; a workspace smaller than needed gives
 * PKV_EWORKSPACE.
 */
size_t pkv_prefill_workspace_bytes(const pkv_cache_desc *cache, int32_t batch,
                                   int32_t num_q_heads, int32_t total_q, int32_t max_q,
                                   int32_t max_kv_len);
pkv_status pkv_prefill_attn(const pkv_cache_desc *cache, void *out, float *lse, const void *q,
                            int32_t num_q_heads, const void *k_cache, const void *v_cache,
                            const int32_t *block_table, int32_t bt_cols, const int32_t *kv_lens,
                            const int32_t *qo_indptr, int32_t batch, int32_t total_q,
                            int32_t max_q, int32_t max_kv_len, int32_t causal, float scale,
                            void *workspace, size_t workspace_bytes, void *stream);
/*
 * As pkv_prefill_attn, with the query rows per workgroup chosen by the caller
 * (the outputs of 128 and 192 are the same; only the speed differs):
 *   rows_per_workgroup  0: the library's choice (what pkv_prefill_attn does);
 *                       128: 8 waves of 16 rows;
 *                       192: 12 waves of 16 rows.
 * Any other value gives PKV_EINVAL.  The library takes 192 once the call has
 * enough 192-row workgroups (ceil(total_q / 192) * num_q_heads of them): at
 * least one and a half per CU at head_dim 256, more than one per CU at
 * head_dim 64 and 128; else 128.  A call that splits its keys (see above)
 * runs 128.  With 128 or 192 the keys are never split and the workspace is
 * not used.
 */
pkv_status pkv_prefill_attn_ex(const pkv_cache_desc *cache, void *out, float *lse, const void *q,
                               int32_t num_q_heads, const void *k_cache, const void *v_cache,
                               const int32_t *block_table, int32_t bt_cols, const int32_t *kv_lens,
                               const int32_t *qo_indptr, int32_t batch, int32_t total_q,
                               int32_t max_q, int32_t max_kv_len, int32_t causal, float scale,
                               void *workspace, size_t workspace_bytes, int32_t rows_per_workgroup,
                               void *stream);

/*
 * pkv_mixed_workspace_bytes / pkv_mixed_attn -- chunked prefill and decode
 * rows of one batch in ONE launch.
 *
 * The flex-vs-vLLM results page ("What's left on the table", chunked
 * prefill) names the separate prefill pass as the main penalty left at large
 * batch; a serving step that runs new-prompt chunks and decode rows over one
 * pool does both here in one kernel launch, whose work list holds the
 * chunks' query tiles and then the decode rows (one workgroup per decode row
 * and KV head, that KV head's query heads computed together).
 *
 * The batch is ordered: requests 0 .. num_prefill-1 are prefill chunks, the
 * remaining batch - num_prefill requests are decode rows.
 *   qo_indptr  int32 [batch+1], device: request r's query rows are
 *              qo_indptr[r] .. qo_indptr[r+1]-1; a decode row has exactly one
 *              (so the decode rows are the last batch - num_prefill query rows)
 *   kv_lens    int32 [batch]: keys of each request, its new tokens included
 *              (append them first, e.g. with one pkv_append over new_indptr =
 *              qo_indptr)
 *   max_q      host upper bound of the chunks' q_r
 * Chunk rows are causal, end-aligned: row i of a chunk sees keys
 * 0 .. kv_r - q_r + i (FlashInfer PR #9451 analysis, §1); a decode row sees
 * all kv_r keys (0 keys: out = 0, lse = -inf).  The chunks take
 * pkv_prefill_attn's tiling and, given a workspace, its key splits: the
 * chunk rows are bit for bit those of pkv_prefill_attn on the chunks (same
 * max_q and max_kv_len) called with a workspace exactly when this call gets
 * one.  The decode rows equal pkv_decode_attn's up to rounding order.  bf16,
 * head_dim 64 or 128 only (PKV_EUNSUPPORTED otherwise).
 * Two launches: a decode row in that launch is one workgroup per KV head,
 * not split across workgroups, so a row of many keys would hold the launch,
 * and many rows queue for the CUs.  With max_kv_len above 8192, or (given a
 * workspace) with more than 2 x CUs decode-row workgroups (decode rows x
 * Hkv), the call therefore enqueues two launches instead: the chunks as
 * pkv_prefill_attn and the decode rows as pkv_decode_attn (bit for bit those
 * calls' results).
 *   workspace  NULL, or a device buffer of pkv_mixed_workspace_bytes(...)
 *              bytes, 16-byte aligned, zero-filled before its first use like a
 *              decode workspace (each call leaves it ready for the next; calls
 *              sharing one must not overlap): the decode rows'
 *              pkv_decode_attn workspace, then room for any key split of the
 *              chunks (three records of 128 rows per CU: ~51 MB at head_dim
 *              128 on 256 CUs).  The size depends on the current device; 0
 *              for invalid arguments.
 *              Without one the chunks never split, and calls with decode rows
 *              and max_kv_len above 8192 return PKV_EWORKSPACE; one smaller
 *              than the size gives PKV_EWORKSPACE.
 */
size_t pkv_mixed_workspace_bytes(const pkv_cache_desc *cache, int32_t batch, int32_t num_prefill,
                                 int32_t num_q_heads);
pkv_status pkv_mixed_attn(const pkv_cache_desc *cache, void *out, float *lse, const void *q,
                          int32_t num_q_heads, const void *k_cache, const void *v_cache,
                          const int32_t *block_table, int32_t bt_cols, const int32_t *kv_lens,
                          const int32_t *qo_indptr, int32_t batch, int32_t num_prefill,
                          int32_t total_q, int32_t max_q, int32_t max_kv_len, float scale,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * pkv_route -- debug/test entry point, not on the hot path: the element
 * offset (kv head 0, dim 0) of every logical token, as the kernels compute it.
 *   offsets  int64 [batch, max_len]: offsets[b][j] for j < seqlens[b], -1 after
 */
pkv_status pkv_route(const pkv_cache_desc *cache, const int32_t *block_table, int32_t bt_cols,
                     const int32_t *seqlens, int32_t batch, int32_t max_len, int64_t *offsets,
                     void *stream);

/*
 * pkv_validate_host -- host-side check of the device-data preconditions of an
 * attention call, on HOST copies of the metadata (the fail-closed metadata
 * consistency rules of the FlashInfer PR #9451 analysis, §1).
 *   block_table  host int32 [batch, bt_cols]; kv_lens host int32 [batch]
 *   qo_indptr    host int32 [batch+1] or NULL (decode)
 * Checks: 0 <= kv_r <= max_kv_len <= bt_cols*page_size; every block a row
 * touches is a page in 1..num_pages-1; with qo_indptr: qo_indptr[0] == 0,
 * non-decreasing, qo_indptr[batch] == total_q, q_r <= max_q and, when causal,
 * 0 < q_r <= kv_r.  Returns PKV_OK or PKV_EVALIDATE and writes a message into
 * msg (host, may be NULL).
 */
pkv_status pkv_validate_host(const pkv_cache_desc *cache, const int32_t *block_table,
                             int32_t bt_cols, const int32_t *kv_lens, const int32_t *qo_indptr,
                             int32_t batch, int32_t total_q, int32_t max_q, int32_t max_kv_len,
                             int32_t causal, char *msg, size_t msg_len);

/*
 * pkv_validate_decode_step_host -- host-side check of the preconditions of
 * pkv_append_decode_attn on HOST copies: 0 <= L_b and L_b + 1 <= max_kv_len
 * <= bt_cols*page_size; every block of the L_b + 1 attended keys is a page
 * in 1..num_pages-1; no two rows append into the same (page, slot).  Padding
 * rows (L_b = -1) are skipped.
 *   block_table  host int32 [batch, bt_cols]; cache_seqlens host int32 [batch]
 * Returns PKV_OK or PKV_EVALIDATE with a message in msg (host, may be NULL).
 */
pkv_status pkv_validate_decode_step_host(const pkv_cache_desc *cache, const int32_t *block_table,
                                         int32_t bt_cols, const int32_t *cache_seqlens, int32_t batch,
                                         int32_t max_kv_len, char *msg, size_t msg_len);

/*
 * pkv_validate_append_host -- host-side check of pkv_append's preconditions
 * on HOST copies: every target position routes to a page in
 * 1..num_pages-1, the table is wide enough, new_indptr is consistent, and no
 * two appended tokens target the same (page, slot).  Padding rows
 * (cache_seqlens[b] = -1) write nothing and are skipped.
 */
pkv_status pkv_validate_append_host(const pkv_cache_desc *cache, const int32_t *block_table,
                                    int32_t bt_cols, const int32_t *cache_seqlens,
                                    const int32_t *new_indptr, int32_t batch, int32_t total_new,
                                    char *msg, size_t msg_len);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
