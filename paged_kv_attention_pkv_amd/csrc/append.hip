// append.hip -- in-place write of new K/V tokens into the paged pool, the
// debug routing kernel and a word fill.
//
// The append is the write half of flash_attn_with_kvcache in mini-infer 06
// "True PagedAttention" §1: token t of sequence b goes to logical position
// cache_seqlens[b] + t, i.e. page block_table[b][pos / 16], slot pos % 16.
// Each thread moves one 16-byte chunk of one (token, kv head) row of K and
// the same chunk of V, so a row of head_dim elements is written by
// head_dim*elem/16 consecutive lanes (coalesced on both sides).
#include <math.h>

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
    int num_pages, int log2_page, int hkv, int row_bytes, int64_t s_page_b, int64_t s_head_b, int64_t s_tok_b,
    int64_t total_chunks, int32_t *__restrict__ seqlens_out) {
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    if (seqlens_out) {
        for (int64_t b = tid; b < batch; b += stride) {
            const int n_new = new_indptr ? new_indptr[b + 1] - new_indptr[b] : 1;
            const int L = cache_seqlens[b];
            seqlens_out[b] = L < 0 ? L : L + n_new;  // a padding row (L < 0) keeps its length
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
        const int L = cache_seqlens[b];
        const int pos = L + t_local;
        const int blk = pos >> log2_page;
        if (L < 0 || blk >= bt_cols) continue;  // a padding row, or outside the row: write nothing
        const int page = block_table[(int64_t)b * bt_cols + blk];
        if (page < 1 || page >= num_pages) continue;  // page 0 is reserved
        const int slot = pos & ((1 << log2_page) - 1);
        const int64_t dst = page * s_page_b + g * s_head_b + slot * s_tok_b + chunk * 16;
        const int64_t src = row * row_bytes + chunk * 16;
        st16(k_cache + dst, ld16(k_new + src));
        st16(v_cache + dst, ld16(v_new + src));
    }
}

__global__ __launch_bounds__(256) void route_kernel(const int32_t *__restrict__ block_table,
                                                    int bt_cols, const int32_t *__restrict__ seqlens,
                                                    int batch, int max_len, int log2_page, int64_t s_page,
                                                    int64_t s_tok, int64_t *__restrict__ offsets) {
    const int64_t total = (int64_t)batch * max_len;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int b = (int)(i / max_len);
        const int j = (int)(i - (int64_t)b * max_len);
        int64_t off = -1;
        if (j < seqlens[b]) {
            const int page = block_table[(int64_t)b * bt_cols + (j >> log2_page)];
            off = page * s_page + (j & ((1 << log2_page) - 1)) * s_tok;
        }
        offsets[i] = off;
    }
}

// ---------------------------------------------------------------------------
// append with rotary position embedding
// ---------------------------------------------------------------------------
//
// The rotation Qwen's attention applies to the new token's q and k before the
// paged call (mini-infer 06 "True PagedAttention", §3), fused into the
// append: the head vector's values form D/2 pairs -- (i, i + D/2) in the
// half-split layout, (2i, 2i+1) in the interleaved one -- and pair i of a
// token at position p turns by the angle whose cosine and sine are
// cos_table[p][i], sin_table[p][i]:  a' = a cos - b sin, b' = b cos + a sin.
// The new token's position is its logical index L_b + t.  The rotation is
// evaluated in fp64 from the exactly widened values (every product of a bf16
// or fp32 value with an fp32 table entry is exact in fp64, so the result is
// the correctly rounded fp64 difference whatever the contraction) and stored
// once, rounded to nearest with ties to even.
//
// A thread takes 16 + 16 bytes of one head row: P = 16 / elem pairs.
// Half-split: A = dims P*c .., B = dims D/2 + P*c .., pair e = (A[e], B[e]).
// Interleaved: A = dims 2P*c .., B = the next P dims, pair e = (x[2e], x[2e+1])
// of the 2P values A:B.  Either way the pairs are i = P*c + e, whose table
// entries are contiguous.

// (bf16_bits_rne, the rounding, is in common.hpp.)

template <int ES>
struct RopeElems;
template <>
struct RopeElems<2> {  // bf16: 8 values per 16 bytes
    static constexpr int P = 8;
    __device__ static __forceinline__ double get(const u32x4 &x, int e) {
        const uint32_t w = x[e >> 1];
        return (double)bf16_bits_to_f32((e & 1) ? (w >> 16) : (w & 0xffffu));
    }
    __device__ static __forceinline__ void put(u32x4 &x, int e, double v) {
        const uint32_t h = bf16_bits_rne(v);
        uint32_t w = x[e >> 1];
        w = (e & 1) ? ((w & 0xffffu) | (h << 16)) : ((w & 0xffff0000u) | h);
        x[e >> 1] = w;
    }
};
template <>
struct RopeElems<4> {  // fp32: 4 values per 16 bytes
    static constexpr int P = 4;
    __device__ static __forceinline__ double get(const u32x4 &x, int e) { return (double)__uint_as_float(x[e]); }
    __device__ static __forceinline__ void put(u32x4 &x, int e, double v) { x[e] = __float_as_uint((float)v); }
};

// Rotate the pairs held in (a, b) by the table row entries cs / sn (P each).
template <int ES>
__device__ __forceinline__ void rotate_pairs(u32x4 &a, u32x4 &b, const float *cs, const float *sn, bool interleaved) {
    using E = RopeElems<ES>;
    constexpr int P = E::P;
    u32x4 ra = a, rb = b;
#pragma unroll
    for (int e = 0; e < P; ++e) {
        double x, y;
        if (interleaved) {
            x = (2 * e < P) ? E::get(a, 2 * e) : E::get(b, 2 * e - P);
            y = (2 * e + 1 < P) ? E::get(a, 2 * e + 1) : E::get(b, 2 * e + 1 - P);
        } else {
            x = E::get(a, e);
            y = E::get(b, e);
        }
        const double c = (double)cs[e], s = (double)sn[e];
        const double rx = x * c - y * s;
        const double ry = y * c + x * s;
        if (interleaved) {
            if (2 * e < P) E::put(ra, 2 * e, rx); else E::put(rb, 2 * e - P, rx);
            if (2 * e + 1 < P) E::put(ra, 2 * e + 1, ry); else E::put(rb, 2 * e + 1 - P, ry);
        } else {
            E::put(ra, e, rx);
            E::put(rb, e, ry);
        }
    }
    a = ra;
    b = rb;
}

template <int ES>
__global__ __launch_bounds__(256) void rope_append_kernel(
    char *__restrict__ k_cache, char *__restrict__ v_cache, const char *__restrict__ k_new,
    const char *__restrict__ v_new, char *__restrict__ q, int hq, const float *__restrict__ rope_cos,
    const float *__restrict__ rope_sin, int rope_rows, int interleaved, const int32_t *__restrict__ block_table,
    int bt_cols, const int32_t *__restrict__ cache_seqlens, const int32_t *__restrict__ new_indptr, int batch,
    int num_pages, int log2_page, int hkv, int head_dim, int64_t s_page_b, int64_t s_head_b, int64_t s_tok_b,
    int64_t total_units, int32_t *__restrict__ seqlens_out) {
    constexpr int P = RopeElems<ES>::P;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    if (seqlens_out) {
        for (int64_t b = tid; b < batch; b += stride) {
            const int n_new = new_indptr ? new_indptr[b + 1] - new_indptr[b] : 1;
            const int L = cache_seqlens[b];
            seqlens_out[b] = L < 0 ? L : L + n_new;
        }
    }
    const int half = head_dim / 2;
    const int slots = half / P;       // threads per head row
    const int heads = hkv + (q ? hq : 0);  // kv heads first, then query heads
    const int row_bytes = head_dim * ES;
    for (int64_t u = tid; u < total_units; u += stride) {
        const int64_t row = u / slots;  // (token, head)
        const int c = (int)(u - row * slots);
        const int t = (int)(row / heads);
        const int h = (int)(row - (int64_t)t * heads);
        int b, t_local;
        if (new_indptr) {
            b = owner_of(new_indptr, batch, t);
            t_local = t - new_indptr[b];
        } else {
            b = t;
            t_local = 0;
        }
        const int L = cache_seqlens[b];
        if (L < 0) continue;  // a padding row: nothing is rotated or written
        const int pos = L + t_local;
        const int prow = pos < rope_rows ? pos : rope_rows - 1;  // in bounds (positions past the table are a precondition violation)
        const float *cs = rope_cos + (int64_t)prow * half + P * c;
        const float *sn = rope_sin + (int64_t)prow * half + P * c;
        const int offa = interleaved ? 2 * P * c : P * c;       // elements
        const int offb = interleaved ? 2 * P * c + P : half + P * c;
        if (h >= hkv) {  // query head: rotated in place
            char *qr = q + ((int64_t)t * hq + (h - hkv)) * row_bytes;
            u32x4 a = ld16(qr + offa * ES), bb = ld16(qr + offb * ES);
            rotate_pairs<ES>(a, bb, cs, sn, interleaved);
            st16(qr + offa * ES, a);
            st16(qr + offb * ES, bb);
            continue;
        }
        const int blk = pos >> log2_page;
        if (blk >= bt_cols) continue;  // outside the row: write nothing
        const int page = block_table[(int64_t)b * bt_cols + blk];
        if (page < 1 || page >= num_pages) continue;  // page 0 is reserved
        const int slot = pos & ((1 << log2_page) - 1);
        const int64_t dst = page * s_page_b + h * s_head_b + slot * s_tok_b;
        const int64_t src = ((int64_t)t * hkv + h) * row_bytes;
        u32x4 a = ld16(k_new + src + offa * ES), bb = ld16(k_new + src + offb * ES);
        const u32x4 va = ld16(v_new + src + offa * ES), vb = ld16(v_new + src + offb * ES);
        rotate_pairs<ES>(a, bb, cs, sn, interleaved);
        st16(k_cache + dst + offa * ES, a);
        st16(k_cache + dst + offb * ES, bb);
        st16(v_cache + dst + offa * ES, va);
        st16(v_cache + dst + offb * ES, vb);
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
                       block_table, bt_cols, cache_seqlens, new_indptr, batch, g.num_pages, g.page_shift + 4, g.hkv,
                       row_bytes,
                       g.s_page * es, g.s_head * es, g.s_tok * es, total_chunks, seqlens_out);
    return hipGetLastError();
}

hipError_t launch_route(const PoolGeom &g, const int32_t *block_table, int bt_cols,
                        const int32_t *seqlens, int batch, int max_len, int64_t *offsets,
                        hipStream_t stream) {
    hipLaunchKernelGGL(route_kernel, dim3(grid_for((int64_t)batch * max_len, 256)), dim3(256), 0,
                       stream, block_table, bt_cols, seqlens, batch, max_len, g.page_shift + 4, g.s_page, g.s_tok,
                       offsets);
    return hipGetLastError();
}

hipError_t launch_append_rope(const PoolGeom &g, void *k_cache, void *v_cache, const void *k_new,
                              const void *v_new, void *q, int hq, const float *rope_cos, const float *rope_sin,
                              int rope_rows, int interleaved, const int32_t *block_table, int bt_cols,
                              const int32_t *cache_seqlens, const int32_t *new_indptr, int batch, int total_new,
                              int32_t *seqlens_out, hipStream_t stream) {
    const int es = g.elem_bytes();
    const int P = 16 / es;
    const int slots = g.head_dim / 2 / P;
    const int heads = g.hkv + (q ? hq : 0);
    const int64_t total_units = (int64_t)total_new * heads * slots;
    const int64_t work = total_units > batch ? total_units : batch;
    if (es == 2)
        hipLaunchKernelGGL(rope_append_kernel<2>, dim3(grid_for(work, 256)), dim3(256), 0, stream, (char *)k_cache,
                           (char *)v_cache, (const char *)k_new, (const char *)v_new, (char *)q, hq, rope_cos,
                           rope_sin, rope_rows, interleaved, block_table, bt_cols, cache_seqlens, new_indptr, batch,
                           g.num_pages, g.page_shift + 4, g.hkv, g.head_dim, g.s_page * es, g.s_head * es, g.s_tok * es, total_units,
                           seqlens_out);
    else
        hipLaunchKernelGGL(rope_append_kernel<4>, dim3(grid_for(work, 256)), dim3(256), 0, stream, (char *)k_cache,
                           (char *)v_cache, (const char *)k_new, (const char *)v_new, (char *)q, hq, rope_cos,
                           rope_sin, rope_rows, interleaved, block_table, bt_cols, cache_seqlens, new_indptr, batch,
                           g.num_pages, g.page_shift + 4, g.hkv, g.head_dim, g.s_page * es, g.s_head * es, g.s_tok * es, total_units,
                           seqlens_out);
    return hipGetLastError();
}

hipError_t launch_zero_words(int32_t *p, int64_t words, hipStream_t stream) {
    if (words <= 0) return hipSuccess;
    hipLaunchKernelGGL(zero_words_kernel, dim3(grid_for(words, 256)), dim3(256), 0, stream, p, words);
    return hipGetLastError();
}

}  // namespace pkv
