// internal.hpp -- host-side interfaces between the C ABI (pkv_api.hip) and the
// kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace pkv {

// Pool geometry after the ABI checks (element strides, dim stride 1).
// The kernels walk keys in 16-token sub-pages; a page of page_size tokens
// holds page_size / 16 of them (page_shift = log2 of that).
struct PoolGeom {
    int dtype;       // 0 = fp32, 1 = bf16
    int num_pages;
    int page_size;   // 16, 32, 64, 128 or 256
    int page_shift;  // log2(page_size / 16)
    int hkv;
    int head_dim;
    int64_t s_page, s_head, s_tok;
    int elem_bytes() const { return dtype == 1 ? 2 : 4; }
};

hipError_t launch_append(const PoolGeom &g, void *k_cache, void *v_cache, const void *k_new,
                         const void *v_new, const int32_t *block_table, int bt_cols,
                         const int32_t *cache_seqlens, const int32_t *new_indptr, int batch,
                         int total_new, int32_t *seqlens_out, hipStream_t stream);

// Append with the rotary position embedding of the new tokens' k (stored) and,
// when q is given, q (rotated in place).
hipError_t launch_append_rope(const PoolGeom &g, void *k_cache, void *v_cache, const void *k_new,
                              const void *v_new, void *q, int hq, const float *rope_cos, const float *rope_sin,
                              int rope_rows, int interleaved, const int32_t *block_table, int bt_cols,
                              const int32_t *cache_seqlens, const int32_t *new_indptr, int batch, int total_new,
                              int32_t *seqlens_out, hipStream_t stream);

hipError_t launch_route(const PoolGeom &g, const int32_t *block_table, int bt_cols,
                        const int32_t *seqlens, int batch, int max_len, int64_t *offsets,
                        hipStream_t stream);

// Decode: split-K over a flattened (sequence, kv head, page) space.
struct DecodeArgs {
    const void *q;
    void *out;
    float *lse;
    const void *k_cache;
    const void *v_cache;
    int64_t s_page, s_head, s_tok;
    const int32_t *block_table;
    int32_t bt_cols;
    const int32_t *seqlens;
    int32_t batch, hq, hkv;
    int32_t max_kv;     // host bound on seqlens; longer rows are cut to it
    int32_t num_pages;  // page ids are clamped into 0..num_pages-1
    int32_t page_shift; // log2(page_size / 16): 16-token sub-page j is in table column j >> page_shift
    float scale_log2;   // softmax scale times log2(e)
    int32_t workers;    // split workers (one wave each)
    int32_t fixed_workers;  // 1: the caller fixed the count (no cap by page count)
    // Automatic count only: a call with fewer than mid_pages (page, kv head)
    // units uses at most mid_workers waves (0: no such cap).
    int32_t mid_workers;
    int64_t mid_pages;
    float *part_o;      // [(record workers + batch*hkv) * group * head_dim]
    float *part_ml;     // [(record workers + batch*hkv) * group * 2]
    int32_t *arrivals;  // [batch*hkv]: pieces finished per split row; zero between calls
    // Fused append (bf16 only): when fused is 1, seqlens holds the pre-append
    // lengths L, each row attends L+1 keys, and the token at position L is taken
    // from k_new / v_new [batch, hkv, head_dim] and written into the pool.
    int32_t fused;
    const void *k_new;
    const void *v_new;
    int32_t *seqlens_out;  // nullable (fused mode only): L+1 where the token was stored, else L
    // Nullable: a plan of the cut for calls of this shape (written by
    // launch_decode_plan, taken only where it matches the call's lengths).
    int32_t *plan;
};

// Fills a.mid_workers / a.mid_pages for an automatic worker count of
// `w_rec` waves on `device` (zero when the caller fixed the count).
void decode_mid_cap(int device, const PoolGeom &g, int w_rec, DecodeArgs &a);

// Workers the decode kernel uses on `device` when the caller asks for
// `requested` (0 = automatic); never more than `max_pages_bound` (< 0: no
// bound).  -1 when the device cannot be queried.
int decode_workers(int device, const PoolGeom &g, int hq, int64_t max_pages_bound, int requested);
// Bytes of the arrival-counter region at the start of the decode workspace.
size_t decode_counter_bytes(const PoolGeom &g, int batch);
// Whole decode workspace for `record_workers` (the uncapped worker count).
size_t decode_workspace(const PoolGeom &g, int batch, int hq, int record_workers);
// Launches the decode kernel on args.workers waves; the workspace layout
// (counters, then records for record_workers + batch*hkv pieces, then the
// plan region) is derived here and fills args.arrivals / part_o / part_ml,
// and args.plan when use_plan.
hipError_t launch_decode(const PoolGeom &g, DecodeArgs args, void *workspace, int record_workers, bool use_plan,
                         hipStream_t stream);
// Writes the plan of calls shaped as args into the workspace's plan region
// (one wave per worker; args.workers of them).
hipError_t launch_decode_plan(const PoolGeom &g, DecodeArgs args, void *workspace, int record_workers,
                              hipStream_t stream);
// Fills a.arrivals / part_o / part_ml / plan from the workspace layout.
void decode_workspace_layout(const PoolGeom &g, DecodeArgs &a, void *workspace, int record_workers);
// Zero `words` int32 values at p with a fill kernel (no memset node, so the
// call can be recorded into a graph).
hipError_t launch_zero_words(int32_t *p, int64_t words, hipStream_t stream);

// Per-device facts of the current device, cached after the first query
// (thread-safe).  CU count, or -1 when the device cannot be queried.
int current_device_cus();
// Raise a kernel's dynamic LDS limit to `bytes` once per device (thread-safe);
// `done` holds one bit per device already set.
hipError_t set_smem_once(const void *kernel, int bytes, std::atomic<uint64_t> &done);

// Prefill (bf16, MFMA).
struct PrefillArgs {
    const void *q;
    void *out;
    float *lse;
    const void *k_cache;
    const void *v_cache;
    int64_t s_page, s_head, s_tok;
    const int32_t *block_table;
    int32_t bt_cols;
    const int32_t *kv_lens;
    const int32_t *qo_indptr;
    int32_t batch, hq, hkv, total_q, max_q, max_kv;
    int32_t num_pages;  // page ids are clamped into 0..num_pages-1
    int32_t page_shift; // log2(page_size / 16)
    int32_t causal;
    float scale_log2;
    int32_t wg_rows;  // query rows per workgroup: 0 = the library's choice, else 128 or (head_dim 256) 192
    // Key splits (set by launch_prefill; 1 = none): each (request, query tile,
    // head) workgroup's key tiles are cut into `splits` pieces, whose partial
    // rows meet as fp32 records in `part` and are merged by the piece that
    // counts last in `arrivals` (one counter per workgroup; zero between calls).
    int32_t splits;
    float *part;
    int32_t *arrivals;
};
// Workspace of a prefill call with the library's tiling: the key-split
// records and counters when the call splits (see launch_prefill), else 0.
size_t prefill_workspace(const PoolGeom &g, int batch, int hq, int total_q, int max_q, int max_kv);
// Bytes that hold the key split of any call on the current device (at most
// three records per CU, and counters): what a caller that cannot size its
// workspace from max_q and max_kv reserves.
size_t prefill_split_region_max(int head_dim);
// Launches the prefill kernel.  With the library's tiling (args.wg_rows 0) and
// a workspace, a call of at most one round of workgroups over long keys runs
// with its keys split (args' split fields are set here), as far as the
// workspace holds the records (prefill_workspace bytes hold the best split);
// without one it runs unsplit.
hipError_t launch_prefill(const PoolGeom &g, const PrefillArgs &args, void *workspace, size_t workspace_bytes,
                          hipStream_t stream);

// Chunked prefill and one-row requests in one launch (bf16, head_dim 64 or
// 128): a's requests 0 .. a.batch-1 as query tiles, then n_rows1 one-row
// requests first_row1 .. first_row1+n_rows1-1 (a.total_q counts the rows of
// both) packed by KV head.  The chunks take launch_prefill's tiling and, with
// a workspace, its key splits.
hipError_t launch_mixed(const PoolGeom &g, const PrefillArgs &a, int n_rows1, int first_row1, void *workspace,
                        size_t workspace_bytes, hipStream_t stream);

}  // namespace pkv
