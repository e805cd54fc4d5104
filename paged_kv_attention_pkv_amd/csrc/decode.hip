// decode.hip -- GQA decode attention over the paged KV pool (gfx950).
//
// What is computed: for every sequence b and query head h, softmax attention
// of q[b,h] over the first cache_seqlens[b] keys of its block_table row,
// reading KV head h / G (G = Hq / Hkv) -- the attend half of
// flash_attn_with_kvcache in mini-infer 06 "True PagedAttention" §1, run by a
// split-KV kernel in its profile (§6).
//
// Work decomposition ("stream-K" over pages).  The pages of all
// (sequence, kv head) segments are laid end to end, sequence-major, and cut
// into `workers` equal ranges, one per wavefront.  A wave walks its range,
// which may start and end inside a segment; every maximal run of one segment
// is a "piece".  A piece that covers a whole segment writes the final output;
// otherwise it writes an unnormalised partial (o, m, l) record, and the wave
// that covers a segment's first page records which workers hold its pieces.
// The combine kernel merges the pieces of split segments with the
// log-sum-exp rule.  Equal page counts per wave keep every CU busy to the end
// for any length mix (uniform or log-uniform up to 32k tokens), at a cost of
// one partial record per piece.  A row's result depends only on its logical
// keys, never on where its pages live.
//
// Per page pair, one wave (bf16 path):
//   S^T[16 tok x 16] = K[16 tok x D] . Q^T[D x 16]     (D/32 MFMA 16x16x32 per page)
//   O^T[D x 16]     += V^T[D x 32 tok] . P^T[32 tok x 16]  (D/16 MFMA 16x16x32)
// The 16 MFMA columns are query heads of one KV head (G <= 16 of them; the
// rest are zero), so every K/V byte is loaded once and used by all G heads.
// A lane (quad = lane/16, col = lane%16) loads K[token col][32kc + 8quad ..]
// (16 B) for the A operand and V[token 4quad+e][DPL*col ..] (DPL = D/16
// elements), which it transposes in registers (v_perm) into the V^T operand;
// the PV token order within a page pair is chosen so that the P^T operand is
// exactly the S^T accumulator layout, so no data crosses lanes except the
// row-max/row-sum reductions of the online softmax (fp32, exp2 with the
// softmax scale folded into log2 units).  Masked tokens (past the row length,
// including stale or NaN-poisoned slots) get score -inf and V = 0.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace pkv {

namespace {

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// ---------------------------------------------------------------------------
// worker geometry
// ---------------------------------------------------------------------------

// Attended length of row b, cut to the host bound so that every table read
// stays inside the row (max_kv <= bt_cols * 16 is checked on the host).
__device__ __forceinline__ int row_len(const DecodeArgs &a, int b) {
    const int n = a.seqlens[b];
    return n < 0 ? 0 : (n > a.max_kv ? a.max_kv : n);
}

// Physical page of logical block blk of a row, clamped into the pool.
__device__ __forceinline__ int page_of(const DecodeArgs &a, const int32_t *bt, int blk) {
    const int p = bt[blk];
    return p < 0 ? 0 : (p >= a.num_pages ? a.num_pages - 1 : p);
}

struct Range {
    int64_t f0, f1, total;
    int workers;
};

// Total pages (over all sequences and kv heads) and this wave's share.
__device__ __forceinline__ bool worker_range(const DecodeArgs &a, int w, Range &r) {
    const int l = lane_id();
    int64_t pages = 0;
    for (int base = 0; base < a.batch; base += kWave) {
        const int b = base + l;
        const int n = b < a.batch ? row_len(a, b) : 0;
        pages += ceil_div(n, kPage);
    }
    const int64_t total = uniform64(wave_sum64(pages)) * a.hkv;
    const int64_t wmax = total < (int64_t)a.workers ? total : (int64_t)a.workers;
    if ((int64_t)w >= wmax) return false;
    r.total = total;
    r.workers = (int)wmax;
    r.f0 = (int64_t)w * total / wmax;
    r.f1 = (int64_t)(w + 1) * total / wmax;
    return true;
}

// Sequence b whose segments contain flat page index f, and the flat index of
// its first page (kv head 0, page 0).
__device__ __forceinline__ void locate(const DecodeArgs &a, int64_t f, int &b_out,
                                       int64_t &start_out) {
    const int l = lane_id();
    int64_t run = 0;
    for (int base = 0; base < a.batch; base += kWave) {
        const int b = base + l;
        const int n = b < a.batch ? row_len(a, b) : 0;
        const int64_t np = (int64_t)ceil_div(n, kPage) * a.hkv;
        const int64_t incl = wave_incl_scan64(np);
        const int64_t tot = uniform64(__shfl(incl, kWave - 1, kWave));
        if (run + tot > f) {
            const uint64_t hit = __ballot(run + incl > f);
            const int first = uniform((int)__builtin_ctzll(hit));
            b_out = base + first;
            start_out = run + uniform64(__shfl(incl - np, first, kWave));
            return;
        }
        run += tot;
    }
    b_out = a.batch - 1;  // not reached for f < total
    start_out = run;
}

// ---------------------------------------------------------------------------
// bf16 engine: MFMA 16x16x32 bf16, two pages per step
// ---------------------------------------------------------------------------

template <int D>
struct EngBf16 {
    static constexpr int KC = D / 32;   // QK MFMAs per page
    static constexpr int DPL = D / 16;  // V elements per lane per token = PV MFMAs per step
    static constexpr int VW = DPL / 2;  // dwords per lane per V token row

    u32x4 qop[KC];
    f32x4 acc[DPL];
    float m, l;
    int G, quad, col;

    __device__ __forceinline__ void init(const DecodeArgs &a, int b, int g) {
        G = a.hq / a.hkv;
        const int ln = lane_id();
        quad = ln >> 4;
        col = ln & 15;
        const int qc = col < G ? col : G - 1;  // lanes past the group read nothing
        const uint16_t *q = (const uint16_t *)a.q + ((int64_t)b * a.hq + (int64_t)g * G + qc) * D;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            u32x4 z = {0u, 0u, 0u, 0u};
            qop[kc] = col < G ? ld16(q + 32 * kc + 8 * quad) : z;
        }
#pragma unroll
        for (int j = 0; j < DPL; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        m = kNegInf;
        l = 0.f;
    }

    __device__ __forceinline__ void load_v(const uint16_t *page, int64_t s_tok, uint32_t (&v)[4][VW]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint16_t *src = page + (int64_t)(4 * quad + e) * s_tok + DPL * col;
            if constexpr (VW == 2) {
                u32x2 x = ld8(src);
                v[e][0] = x[0];
                v[e][1] = x[1];
            } else {
#pragma unroll
                for (int c = 0; c < VW / 4; ++c) {
                    u32x4 x = ld16(src + 8 * c);
                    v[e][4 * c + 0] = x[0];
                    v[e][4 * c + 1] = x[1];
                    v[e][4 * c + 2] = x[2];
                    v[e][4 * c + 3] = x[3];
                }
            }
        }
    }

    __device__ __forceinline__ void run(const DecodeArgs &a, int b, int g, int n, int p0, int p1) {
        const int32_t *bt = a.block_table + (int64_t)b * a.bt_cols;
        const uint16_t *kbase = (const uint16_t *)a.k_cache + (int64_t)g * a.s_head;
        const uint16_t *vbase = (const uint16_t *)a.v_cache + (int64_t)g * a.s_head;
        const int64_t s_tok = a.s_tok, s_page = a.s_page;
        const float c = a.scale_log2;
        for (int pp = p0; pp < p1; pp += 2) {
            const bool has_b = pp + 1 < p1;
            const int pa = page_of(a, bt, pp);
            const int pb = has_b ? page_of(a, bt, pp + 1) : pa;
            const uint16_t *ka = kbase + (int64_t)pa * s_page;
            const uint16_t *kb = kbase + (int64_t)pb * s_page;
            const uint16_t *va = vbase + (int64_t)pa * s_page;
            const uint16_t *vb = vbase + (int64_t)pb * s_page;

            u32x4 kA[KC], kB[KC];
            uint32_t vA[4][VW], vB[4][VW];
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) kA[kc] = ld16(ka + (int64_t)col * s_tok + 32 * kc + 8 * quad);
            load_v(va, s_tok, vA);
            if (has_b) {
#pragma unroll
                for (int kc = 0; kc < KC; ++kc)
                    kB[kc] = ld16(kb + (int64_t)col * s_tok + 32 * kc + 8 * quad);
                load_v(vb, s_tok, vB);
            } else {
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) kB[kc] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int w = 0; w < VW; ++w) vB[e][w] = 0u;
            }

            // scores, S^T layout: lane holds tokens 4quad+i of head col
            f32x4 sA = {0.f, 0.f, 0.f, 0.f}, sB = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                sA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kA[kc]),
                                                             __builtin_bit_cast(bf16x8, qop[kc]), sA, 0, 0, 0);
                sB = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kB[kc]),
                                                             __builtin_bit_cast(bf16x8, qop[kc]), sB, 0, 0, 0);
            }
            const int vcA = min(n - pp * kPage, kPage);
            const int vcB = has_b ? min(n - (pp + 1) * kPage, kPage) : 0;
            float x[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[i] = (4 * quad + i < vcA) ? sA[i] * c : kNegInf;
                x[4 + i] = (4 * quad + i < vcB) ? sB[i] * c : kNegInf;
            }
            float mx = x[0];
#pragma unroll
            for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
            mx = fmaxf(mx, shfl_xor(mx, 16));
            mx = fmaxf(mx, shfl_xor(mx, 32));
            const float mn = fmaxf(m, mx);
            const float alpha = fast_exp2(m - mn);
            float p[8], sum = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                p[i] = fast_exp2(x[i] - mn);
                sum += p[i];
            }
            l = l * alpha + sum;
            m = mn;
#pragma unroll
            for (int j = 0; j < DPL; ++j) acc[j] *= alpha;

            // V rows of masked tokens may hold anything (stale data, NaN): zero them
            if (vcA < kPage) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (4 * quad + e >= vcA)
#pragma unroll
                        for (int w = 0; w < VW; ++w) vA[e][w] = 0u;
            }
            if (has_b && vcB < kPage) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (4 * quad + e >= vcB)
#pragma unroll
                        for (int w = 0; w < VW; ++w) vB[e][w] = 0u;
            }

            // P^T operand: k-slot 8quad+e <-> page A token 4quad+e (e<4), page B token 4quad+e-4
            const u32x4 pop = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                               pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
            const bf16x8 pb8 = __builtin_bit_cast(bf16x8, pop);
#pragma unroll
            for (int j = 0; j < DPL; ++j) {
                const int w = j >> 1;
                u32x4 vop;
                if ((j & 1) == 0) {
                    vop = u32x4{pack_lo16(vA[0][w], vA[1][w]), pack_lo16(vA[2][w], vA[3][w]),
                                pack_lo16(vB[0][w], vB[1][w]), pack_lo16(vB[2][w], vB[3][w])};
                } else {
                    vop = u32x4{pack_hi16(vA[0][w], vA[1][w]), pack_hi16(vA[2][w], vA[3][w]),
                                pack_hi16(vB[0][w], vB[1][w]), pack_hi16(vB[2][w], vB[3][w])};
                }
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vop), pb8,
                                                                 acc[j], 0, 0, 0);
            }
        }
    }

    // acc[j][i] is O^T[dim DPL*(4quad+i) + j][head col].
    __device__ __forceinline__ float row_sum() const {
        float t = l + shfl_xor(l, 16);
        return t + shfl_xor(t, 32);
    }

    __device__ __forceinline__ void store_final(const DecodeArgs &a, int b, int g) {
        const float lt = row_sum();
        if (col >= G) return;
        const int h = g * G + col;
        const float inv = 1.f / lt;
        uint16_t *o = (uint16_t *)a.out + ((int64_t)b * a.hq + h) * D;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t wv[VW];
#pragma unroll
            for (int w = 0; w < VW; ++w)
                wv[w] = pack_bf16x2(acc[2 * w][i] * inv, acc[2 * w + 1][i] * inv);
            uint16_t *dst = o + DPL * (4 * quad + i);
            if constexpr (VW == 2) {
                *reinterpret_cast<u32x2 *>(dst) = u32x2{wv[0], wv[1]};
            } else {
#pragma unroll
                for (int c4 = 0; c4 < VW / 4; ++c4)
                    st16(dst + 8 * c4, u32x4{wv[4 * c4], wv[4 * c4 + 1], wv[4 * c4 + 2], wv[4 * c4 + 3]});
            }
        }
        if (quad == 0 && a.lse) a.lse[(int64_t)b * a.hq + h] = (m + log2f(lt)) * kLn2;
    }

    __device__ __forceinline__ void store_partial(const DecodeArgs &a, int64_t rec) {
        const float lt = row_sum();
        if (col >= G) return;
        float *o = a.part_o + (rec * G + col) * D;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float *dst = o + DPL * (4 * quad + i);
#pragma unroll
            for (int j4 = 0; j4 < DPL / 4; ++j4)
                *reinterpret_cast<f32x4 *>(dst + 4 * j4) =
                    f32x4{acc[4 * j4][i], acc[4 * j4 + 1][i], acc[4 * j4 + 2][i], acc[4 * j4 + 3][i]};
        }
        if (quad == 0) *reinterpret_cast<f32x2 *>(a.part_ml + (rec * G + col) * 2) = f32x2{m, lt};
    }
};

// ---------------------------------------------------------------------------
// fp32 engine: MFMA 16x16x4 f32, one page per step
// ---------------------------------------------------------------------------

template <int D>
struct EngF32 {
    static constexpr int KC = D / 4;   // QK MFMAs per page
    static constexpr int DC = D / 16;  // output dim chunks

    float qop[KC];
    f32x4 acc[DC];
    float m, l;
    int G, quad, col;

    __device__ __forceinline__ void init(const DecodeArgs &a, int b, int g) {
        G = a.hq / a.hkv;
        const int ln = lane_id();
        quad = ln >> 4;
        col = ln & 15;
        const int qc = col < G ? col : G - 1;
        const float *q = (const float *)a.q + ((int64_t)b * a.hq + (int64_t)g * G + qc) * D;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) qop[kc] = col < G ? q[4 * kc + quad] : 0.f;
#pragma unroll
        for (int j = 0; j < DC; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        m = kNegInf;
        l = 0.f;
    }

    __device__ __forceinline__ void run(const DecodeArgs &a, int b, int g, int n, int p0, int p1) {
        const int32_t *bt = a.block_table + (int64_t)b * a.bt_cols;
        const float *kbase = (const float *)a.k_cache + (int64_t)g * a.s_head;
        const float *vbase = (const float *)a.v_cache + (int64_t)g * a.s_head;
        const float c = a.scale_log2;
        for (int p = p0; p < p1; ++p) {
            const int phys = page_of(a, bt, p);
            const float *kp = kbase + (int64_t)phys * a.s_page;
            const float *vp = vbase + (int64_t)phys * a.s_page;
            f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
                s = __builtin_amdgcn_mfma_f32_16x16x4f32(kp[(int64_t)col * a.s_tok + 4 * kc + quad], qop[kc],
                                                          s, 0, 0, 0);
            const int vc = min(n - p * kPage, kPage);
            float x[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = (4 * quad + i < vc) ? s[i] * c : kNegInf;
            float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
            mx = fmaxf(mx, shfl_xor(mx, 16));
            mx = fmaxf(mx, shfl_xor(mx, 32));
            const float mn = fmaxf(m, mx);
            const float alpha = fast_exp2(m - mn);
            float pr[4], sum = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pr[i] = fast_exp2(x[i] - mn);
                sum += pr[i];
            }
            l = l * alpha + sum;
            m = mn;
#pragma unroll
            for (int j = 0; j < DC; ++j) acc[j] *= alpha;
            // PV: MFMA i takes k-slot quad <-> token 4quad+i
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = 4 * quad + i < vc;
                const float *vrow = vp + (int64_t)(4 * quad + i) * a.s_tok;
#pragma unroll
                for (int dc = 0; dc < DC; ++dc) {
                    const float v = ok ? vrow[16 * dc + col] : 0.f;
                    acc[dc] = __builtin_amdgcn_mfma_f32_16x16x4f32(v, pr[i], acc[dc], 0, 0, 0);
                }
            }
        }
    }

    // acc[dc][i] is O^T[dim 16dc + 4quad + i][head col].
    __device__ __forceinline__ float row_sum() const {
        float t = l + shfl_xor(l, 16);
        return t + shfl_xor(t, 32);
    }

    __device__ __forceinline__ void store_final(const DecodeArgs &a, int b, int g) {
        const float lt = row_sum();
        if (col >= G) return;
        const int h = g * G + col;
        float *o = (float *)a.out + ((int64_t)b * a.hq + h) * D;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc)
            *reinterpret_cast<f32x4 *>(o + 16 * dc + 4 * quad) = acc[dc] / lt;
        if (quad == 0 && a.lse) a.lse[(int64_t)b * a.hq + h] = (m + log2f(lt)) * kLn2;
    }

    __device__ __forceinline__ void store_partial(const DecodeArgs &a, int64_t rec) {
        const float lt = row_sum();
        if (col >= G) return;
        float *o = a.part_o + (rec * G + col) * D;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) *reinterpret_cast<f32x4 *>(o + 16 * dc + 4 * quad) = acc[dc];
        if (quad == 0) *reinterpret_cast<f32x2 *>(a.part_ml + (rec * G + col) * 2) = f32x2{m, lt};
    }
};

// ---------------------------------------------------------------------------
// kernels
// ---------------------------------------------------------------------------

template <class Eng>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeArgs a) {
    const int w = blockIdx.x;
    Range r;
    if (!worker_range(a, w, r)) return;
    int b;
    int64_t seq_start;
    locate(a, r.f0, b, seq_start);
    int n = uniform(row_len(a, b));
    int np = ceil_div(n, kPage);
    const int64_t off = r.f0 - seq_start;
    int g = (int)(off / np);
    int p0 = (int)(off - (int64_t)g * np);
    int64_t f = r.f0;
    Eng eng;
    for (;;) {
        const int64_t seg_start = f - p0;
        const int64_t left = r.f1 - f;
        const int p1 = left < (int64_t)(np - p0) ? p0 + (int)left : np;
        const int64_t s = (int64_t)b * a.hkv + g;
        eng.init(a, b, g);
        eng.run(a, b, g, n, p0, p1);
        if (p0 == 0 && lane_id() == 0) {
            const int64_t w_last = ((seg_start + np) * r.workers - 1) / r.total;
            a.meta[2 * s] = w;
            a.meta[2 * s + 1] = (int)(w_last - w + 1);
        }
        if (p0 == 0 && p1 == np)
            eng.store_final(a, b, g);
        else
            eng.store_partial(a, (int64_t)w + s);
        f += p1 - p0;
        if (f >= r.f1) break;
        p0 = 0;
        if (++g == a.hkv) {
            g = 0;
            do {
                ++b;
                n = uniform(row_len(a, b));
                np = ceil_div(n, kPage);
            } while (np == 0);
        }
    }
}

// One workgroup per (sequence, kv head): merge split pieces; write empty rows.
template <typename OutT>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a, int D) {
    const int s = blockIdx.x;
    const int b = s / a.hkv;
    const int g = s - b * a.hkv;
    const int G = a.hq / a.hkv;
    const int n = row_len(a, b);
    OutT *out = (OutT *)a.out;
    if (n <= 0) {
        for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
            const int c = idx / D, d = idx - (idx / D) * D;
            out[((int64_t)b * a.hq + g * G + c) * D + d] = OutT(0.f);
            if (d == 0 && a.lse) a.lse[(int64_t)b * a.hq + g * G + c] = kNegInf;
        }
        return;
    }
    const int w0 = a.meta[2 * s];
    const int cnt = a.meta[2 * s + 1];
    if (cnt <= 1) return;
    // records hold ids w + s with w < workers; anything else is not ours
    if (w0 < 0 || (int64_t)w0 + cnt > a.workers) return;
    for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
        const int c = idx / D, d = idx - (idx / D) * D;
        float M = kNegInf;
        for (int k = 0; k < cnt; ++k) {
            const int64_t rec = (int64_t)w0 + k + s;
            M = fmaxf(M, a.part_ml[(rec * G + c) * 2]);
        }
        float num = 0.f, den = 0.f;
        for (int k = 0; k < cnt; ++k) {
            const int64_t rec = (int64_t)w0 + k + s;
            const float wgt = fast_exp2(a.part_ml[(rec * G + c) * 2] - M);
            num += wgt * a.part_o[(rec * G + c) * D + d];
            den += wgt * a.part_ml[(rec * G + c) * 2 + 1];
        }
        out[((int64_t)b * a.hq + g * G + c) * D + d] = OutT(num / den);
        if (d == 0 && a.lse) a.lse[(int64_t)b * a.hq + g * G + c] = (M + log2f(den)) * kLn2;
    }
}

template <class Eng>
const void *split_kernel_ptr() {
    return reinterpret_cast<const void *>(&decode_split_kernel<Eng>);
}

const void *pick_split_kernel(int dtype, int d) {
    if (dtype == 1) {
        if (d == 64) return split_kernel_ptr<EngBf16<64>>();
        if (d == 128) return split_kernel_ptr<EngBf16<128>>();
        if (d == 256) return split_kernel_ptr<EngBf16<256>>();
    } else {
        if (d == 64) return split_kernel_ptr<EngF32<64>>();
        if (d == 128) return split_kernel_ptr<EngF32<128>>();
        if (d == 256) return split_kernel_ptr<EngF32<256>>();
    }
    return nullptr;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct DeviceInfo {
    int cus = 0;
    int occ[2][3] = {{0, 0, 0}, {0, 0, 0}};  // resident split waves per CU [dtype][d]
};
constexpr int kMaxDevices = 64;
DeviceInfo g_info[kMaxDevices];

int dim_index(int d) { return d == 64 ? 0 : (d == 128 ? 1 : 2); }

}  // namespace

int decode_workers(int device, const PoolGeom &g, int hq, int64_t max_pages_bound, int requested) {
    (void)hq;
    int64_t w = requested;
    if (w <= 0) {
        if (device < 0 || device >= kMaxDevices) return -1;
        DeviceInfo &info = g_info[device];
        if (info.cus == 0) {
            int cus = 0;
            if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess)
                return -1;
            info.cus = cus;
        }
        int &occ = info.occ[g.dtype == 1 ? 1 : 0][dim_index(g.head_dim)];
        if (occ == 0) {
            int blocks = 0;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, pick_split_kernel(g.dtype, g.head_dim),
                                                             kWave, 0) != hipSuccess || blocks <= 0)
                blocks = 8;
            occ = blocks > 16 ? 16 : blocks;
        }
        w = (int64_t)info.cus * occ;
    }
    if (max_pages_bound >= 0 && w > max_pages_bound) w = max_pages_bound;
    if (w < 1) w = 1;
    if (w > (1 << 22)) w = 1 << 22;
    return (int)w;
}

size_t decode_workspace(const PoolGeom &g, int batch, int hq, int workers) {
    const int G = hq / g.hkv;
    const size_t recs = (size_t)workers + (size_t)batch * g.hkv;
    return align256(recs * G * g.head_dim * sizeof(float)) + align256(recs * G * 2 * sizeof(float)) +
           align256((size_t)batch * g.hkv * 2 * sizeof(int32_t));
}

hipError_t launch_decode(const PoolGeom &g, DecodeArgs a, int max_kv_len, hipStream_t stream) {
    const int G = a.hq / a.hkv;
    const size_t recs = (size_t)a.workers + (size_t)a.batch * a.hkv;
    char *ws = (char *)a.part_o;
    a.part_ml = (float *)(ws + align256(recs * G * g.head_dim * sizeof(float)));
    a.meta = (int32_t *)((char *)a.part_ml + align256(recs * G * 2 * sizeof(float)));
    if (max_kv_len > 0) {
        const void *k = pick_split_kernel(g.dtype, g.head_dim);
        void *args[] = {&a};
        hipError_t e = hipLaunchKernel(k, dim3(a.workers), dim3(kWave), args, 0, stream);
        if (e != hipSuccess) return e;
    }
    if (g.dtype == 1)
        hipLaunchKernelGGL(decode_combine_kernel<__bf16>, dim3(a.batch * a.hkv), dim3(256), 0, stream, a,
                           g.head_dim);
    else
        hipLaunchKernelGGL(decode_combine_kernel<float>, dim3(a.batch * a.hkv), dim3(256), 0, stream, a,
                           g.head_dim);
    return hipGetLastError();
}

}  // namespace pkv
