// append.hip -- in-place write of new K/V tokens into the paged pool, the
// debug routing kernel and a word fill.
//
// The append is the write half of flash_attn_with_kvcache in mini-infer 06
// "True PagedAttention" §1: token t of sequence b goes to logical position
// cache_seqlens[b] + t, i.e. page block_table[b][pos / 16], slot pos % 16.
// Each thread moves one 16-byte chunk of one (token, kv head) row of K and
// the same chunk of V, so a row of head_dim elements is written by
// head_dim*elem/16 consecutive lanes (coalesced on both sides).
#include "common.hpp"
#include "internal.hpp"

namespace pkv {

namespace {

// Sequence that owns appended row t: the b with indptr[b] <= t < indptr[b+1].
__device__ __forceinline__ int owner_of(const int32_t *indptr, int batch, int t) {
    int lo = 0, hi = batch;  // answer in [lo, hi)
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (indptr[mid] <= t) lo = mid; else hi = mid;
    }
    return lo;
}

__global__ __launch_bounds__(256) void append_kernel(
    char *__restrict__ k_cache, char *__restrict__ v_cache, const char *__restrict__ k_new,
    const char *__restrict__ v_new, const int32_t *__restrict__ block_table, int bt_cols,
    const int32_t *__restrict__ cache_seqlens, const int32_t *__restrict__ new_indptr, int batch,
    int num_pages, int hkv, int row_bytes, int64_t s_page_b, int64_t s_head_b, int64_t s_tok_b,
    int64_t total_chunks, int32_t *__restrict__ seqlens_out) {
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    if (seqlens_out) {
        for (int64_t b = tid; b < batch; b += stride) {
            int n_new = new_indptr ? new_indptr[b + 1] - new_indptr[b] : 1;
            seqlens_out[b] = cache_seqlens[b] + n_new;
        }
    }
    const int chunks_per_row = row_bytes >> 4;
    for (int64_t c = tid; c < total_chunks; c += stride) {
        const int64_t row = c / chunks_per_row;            // (token, kv head)
        const int chunk = (int)(c - row * chunks_per_row);
        const int t = (int)(row / hkv);
        const int g = (int)(row - (int64_t)t * hkv);
        int b, t_local;
        if (new_indptr) {
            b = owner_of(new_indptr, batch, t);
            t_local = t - new_indptr[b];
        } else {
            b = t;
            t_local = 0;
        }
        const int pos = cache_seqlens[b] + t_local;
        const int blk = pos >> 4;
        if (pos < 0 || blk >= bt_cols) continue;  // outside the row: write nothing
        const int page = block_table[(int64_t)b * bt_cols + blk];
        if (page < 1 || page >= num_pages) continue;  // page 0 is reserved
        const int slot = pos & (kPage - 1);
        const int64_t dst = page * s_page_b + g * s_head_b + slot * s_tok_b + chunk * 16;
        const int64_t src = row * row_bytes + chunk * 16;
        st16(k_cache + dst, ld16(k_new + src));
        st16(v_cache + dst, ld16(v_new + src));
    }
}

__global__ __launch_bounds__(256) void route_kernel(const int32_t *__restrict__ block_table,
                                                    int bt_cols, const int32_t *__restrict__ seqlens,
                                                    int batch, int max_len, int64_t s_page,
                                                    int64_t s_tok, int64_t *__restrict__ offsets) {
    const int64_t total = (int64_t)batch * max_len;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int b = (int)(i / max_len);
        const int j = (int)(i - (int64_t)b * max_len);
        int64_t off = -1;
        if (j < seqlens[b]) {
            const int page = block_table[(int64_t)b * bt_cols + (j >> 4)];
            off = page * s_page + (j & (kPage - 1)) * s_tok;
        }
        offsets[i] = off;
    }
}

// Zero fill of a word range (the decode workspace's arrival counters).
__global__ __launch_bounds__(256) void zero_words_kernel(int32_t *__restrict__ p, int64_t words) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

int grid_for(int64_t work, int block) {
    int64_t g = (work + block - 1) / block;
    if (g < 1) g = 1;
    if (g > 65536) g = 65536;
    return (int)g;
}

}  // namespace

hipError_t launch_append(const PoolGeom &g, void *k_cache, void *v_cache, const void *k_new,
                         const void *v_new, const int32_t *block_table, int bt_cols,
                         const int32_t *cache_seqlens, const int32_t *new_indptr, int batch,
                         int total_new, int32_t *seqlens_out, hipStream_t stream) {
    const int es = g.elem_bytes();
    const int row_bytes = g.head_dim * es;
    const int64_t total_chunks = (int64_t)total_new * g.hkv * (row_bytes / 16);
    const int64_t work = total_chunks > batch ? total_chunks : batch;
    hipLaunchKernelGGL(append_kernel, dim3(grid_for(work, 256)), dim3(256), 0, stream,
                       (char *)k_cache, (char *)v_cache, (const char *)k_new, (const char *)v_new,
                       block_table, bt_cols, cache_seqlens, new_indptr, batch, g.num_pages, g.hkv, row_bytes,
                       g.s_page * es, g.s_head * es, g.s_tok * es, total_chunks, seqlens_out);
    return hipGetLastError();
}

hipError_t launch_route(const PoolGeom &g, const int32_t *block_table, int bt_cols,
                        const int32_t *seqlens, int batch, int max_len, int64_t *offsets,
                        hipStream_t stream) {
    hipLaunchKernelGGL(route_kernel, dim3(grid_for((int64_t)batch * max_len, 256)), dim3(256), 0,
                       stream, block_table, bt_cols, seqlens, batch, max_len, g.s_page, g.s_tok,
                       offsets);
    return hipGetLastError();
}

hipError_t launch_zero_words(int32_t *p, int64_t words, hipStream_t stream) {
    if (words <= 0) return hipSuccess;
    hipLaunchKernelGGL(zero_words_kernel, dim3(grid_for(words, 256)), dim3(256), 0, stream, p, words);
    return hipGetLastError();
}

}  // namespace pkv
