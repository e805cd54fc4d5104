// decode.hip -- GQA decode attention over the paged KV pool (gfx950).
//
// What is computed: for every sequence b and query head h, softmax attention
// of q[b,h] over the first cache_seqlens[b] keys of its block_table row,
// reading KV head h / G (G = Hq / Hkv) -- the attend half of
// flash_attn_with_kvcache in mini-infer 06 "True PagedAttention" §1, run by a
// split-KV kernel in its profile (§6).
//
// Work decomposition ("stream-K" over pages), one kernel launch.  The pages
// of all (sequence, kv head) segments are laid end to end, sequence-major,
// and cut into `workers` equal ranges, one per wavefront.  A wave walks its
// range, which may start and end inside a segment; every maximal run of one
// segment is a "piece".  A piece that covers a whole segment writes the
// final output.  Otherwise it writes an unnormalised (o, m, l) record to the
// workspace and counts itself in the segment's arrival counter; the piece
// that arrives last merges every record of the segment, in piece order (so
// the result does not depend on which piece came last), writes the output
// and resets the counter to zero for the next call.  Equal page counts per
// wave keep every CU busy to the end for any mix of lengths.  Rows with no
// keys are written (0, lse = -inf) by the waves in a round-robin.
//
// Per page pair, one wave (bf16 path):
//   S^T[16 tok x 16]  = K[16 tok x D] . Q^T[D x 16]        (D/32 MFMA 16x16x32 per page)
//   O^T[D x 16]      += V^T[D x 32 tok] . P^T[32 tok x 16]  (D/16 MFMA 16x16x32)
// The 16 MFMA columns are the query heads of one KV head (G <= 16 of them;
// the rest are zero), so every K/V byte is loaded once and serves all G
// heads.  A lane (quad = lane/16, col = lane%16) loads K[token col][32kc +
// 8quad ..] (16 B) for the A operand and V[token 4quad+e][DPL*col ..]
// (DPL = D/16 elements), which it transposes in registers (v_perm) into the
// V^T operand; the PV token order inside a page pair is chosen so that the
// P^T operand is exactly the S^T accumulator layout.  No data crosses lanes
// except the row max / row sum of the online softmax (fp32, exp2 with the
// softmax scale folded into log2 units).  Masked tokens (past the row length,
// stale or NaN-poisoned slots) get score -inf and V = 0.  The next page
// pair's K/V loads are issued before the current pair is computed (two
// register buffers), and the row's block-table entries are read 64 at a time
// into one register, so no table read sits in front of a page load.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

// Tuning knobs (compile time): prefetch the next page pair into a second
// register buffer; resident waves per SIMD the bf16 kernel is register-capped to.
#ifndef PKV_DECODE_PREFETCH
#define PKV_DECODE_PREFETCH 1
#endif
#ifndef PKV_DECODE_WAVES_PER_EU
#define PKV_DECODE_WAVES_PER_EU 1
#endif

namespace pkv {

namespace {

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// ---------------------------------------------------------------------------
// rows, pages, workers
// ---------------------------------------------------------------------------

// Attended length of row b, cut to the host bound so that every table read
// stays inside the row (max_kv <= bt_cols * 16 is checked on the host).
__device__ __forceinline__ int row_len(const DecodeArgs &a, int b) {
    const int n = a.seqlens[b];
    return n < 0 ? 0 : (n > a.max_kv ? a.max_kv : n);
}

__device__ __forceinline__ int clamp_page(const DecodeArgs &a, int p) {
    return p < 0 ? 0 : (p >= a.num_pages ? a.num_pages - 1 : p);
}

// Partial records travel between waves on different XCDs (each with its own
// L2).  They are written and read with agent-scope atomic accesses, which the
// compiler emits as agent-coherent (sc1) loads and stores, so no cache-wide
// write-back or invalidate (what an agent-scope fence costs on this chip) is
// needed; a wave waits for its record stores to complete before it counts
// itself in the segment's arrival counter.
__device__ __forceinline__ void st_shared2(float *p, float x, float y) {
    const uint64_t v = (uint64_t)__builtin_bit_cast(uint32_t, x) | ((uint64_t)__builtin_bit_cast(uint32_t, y) << 32);
    __hip_atomic_store(reinterpret_cast<uint64_t *>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x2 ld_shared2(const float *p) {
    const uint64_t v =
        __hip_atomic_load(reinterpret_cast<const uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return f32x2{__builtin_bit_cast(float, (uint32_t)v), __builtin_bit_cast(float, (uint32_t)(v >> 32))};
}
__device__ __forceinline__ void wait_stores_complete() { __builtin_amdgcn_s_waitcnt(0); }

// Zero output and -inf lse for a row without keys (b wave-uniform).
template <typename OutT>
__device__ void zero_row(const DecodeArgs &a, int b, int D) {
    OutT *out = (OutT *)a.out + (int64_t)b * a.hq * D;
    for (int i = lane_id(); i < a.hq * D; i += kWave) out[i] = OutT(0.f);
    if (a.lse)
        for (int h = lane_id(); h < a.hq; h += kWave) a.lse[(int64_t)b * a.hq + h] = kNegInf;
}

struct Range {
    int64_t f0, f1, total;
    int workers;
};

// Total pages over all segments and this wave's share; empty rows are
// zero-filled here, row b by worker b mod workers.
template <typename OutT>
__device__ __forceinline__ bool worker_range(const DecodeArgs &a, int w, int D, Range &r) {
    const int l = lane_id();
    int64_t pages = 0;
    for (int base = 0; base < a.batch; base += kWave) {
        const int b = base + l;
        const int n = b < a.batch ? row_len(a, b) : -1;
        pages += n > 0 ? ceil_div(n, kPage) : 0;
        uint64_t empty = __ballot(n == 0 && b % a.workers == w);
        while (empty) {
            const int e = uniform((int)__builtin_ctzll(empty));
            empty &= empty - 1;
            zero_row<OutT>(a, base + e, D);
        }
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
__device__ __forceinline__ void locate(const DecodeArgs &a, int64_t f, int &b_out, int64_t &start_out) {
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

// Worker whose range holds flat page p.
__device__ __forceinline__ int64_t worker_of(int64_t p, const Range &r) {
    return ((p + 1) * r.workers - 1) / r.total;
}

// Merge the partial records of split segment s (pieces of workers wf ..
// wf+cnt-1, record ids w + s) in piece order and write its output rows.  A
// lane owns 8 consecutive outputs of one head; pieces are taken 8 at a time
// with every load of a batch issued before any is used (two memory round
// trips per batch), and batches are folded with the log-sum-exp rule.
template <typename OutT, int D>
__device__ void merge_segment(const DecodeArgs &a, int64_t s, int b, int g, int64_t wf, int cnt) {
    constexpr int kBatch = 8;
    const int G = a.hq / a.hkv;
    OutT *out = (OutT *)a.out + ((int64_t)b * a.hq + (int64_t)g * G) * D;
    for (int base = lane_id() * 8; base < G * D; base += kWave * 8) {
        const int c = base / D;
        const int d0 = base - c * D;
        float M = kNegInf, den = 0.f;
        float num[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int k0 = 0; k0 < cnt; k0 += kBatch) {
            const int nb = min(kBatch, cnt - k0);
            f32x2 ml[kBatch];
            f32x2 o[kBatch][4];
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                if (k < nb) {
                    const int64_t rec = (wf + k0 + k + s) * G + c;
                    ml[k] = ld_shared2(a.part_ml + rec * 2);
#pragma unroll
                    for (int t = 0; t < 4; ++t) o[k][t] = ld_shared2(a.part_o + rec * D + d0 + 2 * t);
                }
            }
            float Mb = M;
#pragma unroll
            for (int k = 0; k < kBatch; ++k)
                if (k < nb) Mb = fmaxf(Mb, ml[k][0]);
            const float r = fast_exp2(M - Mb);
            den *= r;
#pragma unroll
            for (int t = 0; t < 8; ++t) num[t] *= r;
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                if (k < nb) {
                    const float wgt = fast_exp2(ml[k][0] - Mb);
                    den += wgt * ml[k][1];
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        num[2 * t] += wgt * o[k][t][0];
                        num[2 * t + 1] += wgt * o[k][t][1];
                    }
                }
            }
            M = Mb;
        }
        const float inv = 1.f / den;
#pragma unroll
        for (int t = 0; t < 8; ++t) out[base + t] = OutT(num[t] * inv);
        if (d0 == 0 && a.lse) a.lse[(int64_t)b * a.hq + (int64_t)g * G + c] = (M + log2f(den)) * kLn2;
    }
}

// ---------------------------------------------------------------------------
// bf16 engine: MFMA 16x16x32 bf16, two pages per step, one pair prefetched
// ---------------------------------------------------------------------------

template <int D>
struct EngBf16 {
    using Out = __bf16;
    static constexpr int KC = D / 32;   // QK MFMAs per page
    static constexpr int DPL = D / 16;  // V elements per lane per token = PV MFMAs per pair
    static constexpr int VW = DPL / 2;  // dwords per lane per V token row

    struct Buf {
        u32x4 kA[KC], kB[KC];
        uint32_t vA[4][VW], vB[4][VW];
    };

    u32x4 qop[KC];
    f32x4 acc[DPL];
    float m, l;
    int G, quad, col;
    uint32_t koff;     // lane's byte offset in a page for K (token col, dims 8quad..)
    uint32_t voff[4];  // lane's byte offsets for V (token 4quad+e, dims DPL*col..)

    __device__ __forceinline__ void init(const DecodeArgs &a, int b, int g) {
        G = a.hq / a.hkv;
        const int ln = lane_id();
        quad = ln >> 4;
        col = ln & 15;
        const uint32_t st = (uint32_t)a.s_tok * 2u;
        koff = col * st + 16u * quad;
#pragma unroll
        for (int e = 0; e < 4; ++e) voff[e] = (4u * quad + e) * st + 2u * DPL * col;
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

    // kp / vp are wave-uniform page bases and the lane parts zero-extended
    // 32-bit byte offsets, so the loads use scalar-base + vector-offset
    // addressing and need no per-lane 64-bit address registers.
    __device__ __forceinline__ void load_page(const uint16_t *kp, const uint16_t *vp, u32x4 (&k)[KC],
                                              uint32_t (&v)[4][VW]) {
        const char *kb = (const char *)kp;
        const char *vb = (const char *)vp;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) k[kc] = ld16(kb + (uint64_t)koff + 64 * kc);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint16_t *src = (const uint16_t *)(vb + (uint64_t)voff[e]);
            if constexpr (VW == 2) {
                u32x2 x = ld8(src);
                v[e][0] = x[0];
                v[e][1] = x[1];
            } else {
#pragma unroll
                for (int c4 = 0; c4 < VW / 4; ++c4) {
                    u32x4 x = ld16(src + 8 * c4);
                    v[e][4 * c4 + 0] = x[0];
                    v[e][4 * c4 + 1] = x[1];
                    v[e][4 * c4 + 2] = x[2];
                    v[e][4 * c4 + 3] = x[3];
                }
            }
        }
    }

    // Loads of pages pa and pb (pb == pa when the pair has one page).
    __device__ __forceinline__ void issue(const DecodeArgs &a, const uint16_t *kbase, const uint16_t *vbase, int pa,
                                          int pb, Buf &buf) {
        load_page(kbase + (int64_t)pa * a.s_page, vbase + (int64_t)pa * a.s_page, buf.kA, buf.vA);
        load_page(kbase + (int64_t)pb * a.s_page, vbase + (int64_t)pb * a.s_page, buf.kB, buf.vB);
    }

    // One page pair: vcA / vcB valid tokens in the two pages (vcB = 0 for a
    // pair with one page).
    __device__ __forceinline__ void compute(Buf &buf, int vcA, int vcB, float c) {
        f32x4 sA = {0.f, 0.f, 0.f, 0.f}, sB = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            sA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, buf.kA[kc]),
                                                         __builtin_bit_cast(bf16x8, qop[kc]), sA, 0, 0, 0);
            sB = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, buf.kB[kc]),
                                                         __builtin_bit_cast(bf16x8, qop[kc]), sB, 0, 0, 0);
        }
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
                    for (int w = 0; w < VW; ++w) buf.vA[e][w] = 0u;
        }
        if (vcB < kPage) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (4 * quad + e >= vcB)
#pragma unroll
                    for (int w = 0; w < VW; ++w) buf.vB[e][w] = 0u;
        }

        // P^T operand: k-slot 8quad+e <-> page A token 4quad+e (e<4), page B token 4quad+e-4
        const u32x4 pop = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                           pack_bf16x2(p[6], p[7])};
        const bf16x8 pb8 = __builtin_bit_cast(bf16x8, pop);
#pragma unroll
        for (int j = 0; j < DPL; ++j) {
            const int w = j >> 1;
            u32x4 vop;
            if ((j & 1) == 0) {
                vop = u32x4{pack_lo16(buf.vA[0][w], buf.vA[1][w]), pack_lo16(buf.vA[2][w], buf.vA[3][w]),
                            pack_lo16(buf.vB[0][w], buf.vB[1][w]), pack_lo16(buf.vB[2][w], buf.vB[3][w])};
            } else {
                vop = u32x4{pack_hi16(buf.vA[0][w], buf.vA[1][w]), pack_hi16(buf.vA[2][w], buf.vA[3][w]),
                            pack_hi16(buf.vB[0][w], buf.vB[1][w]), pack_hi16(buf.vB[2][w], buf.vB[3][w])};
            }
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vop), pb8, acc[j], 0, 0, 0);
        }
    }

    __device__ __forceinline__ void run(const DecodeArgs &a, int b, int g, int n, int p0, int p1) {
        const int32_t *bt = a.block_table + (int64_t)b * a.bt_cols;
        const uint16_t *kbase = (const uint16_t *)a.k_cache + (int64_t)g * a.s_head;
        const uint16_t *vbase = (const uint16_t *)a.v_cache + (int64_t)g * a.s_head;
        const float c = a.scale_log2;
        const int ln = lane_id();
        Buf b0, b1;
        // pages in chunks of 64: the chunk's table entries sit one per lane
        for (int c0 = p0; c0 < p1; c0 += kWave) {
            const int cn = min(p1 - c0, kWave);
            const int tb = ln < cn ? bt[c0 + ln] : 0;
            const int npairs = (cn + 1) >> 1;
            auto pages_of = [&](int i, int &pa, int &pb) {
                pa = clamp_page(a, __builtin_amdgcn_readlane(tb, 2 * i));
                pb = 2 * i + 1 < cn ? clamp_page(a, __builtin_amdgcn_readlane(tb, 2 * i + 1)) : pa;
            };
            auto valid = [&](int i, int &va, int &vb) {
                const int first = (c0 + 2 * i) * kPage;
                va = min(n - first, kPage);
                vb = 2 * i + 1 < cn ? min(n - first - kPage, kPage) : 0;
            };
            int pa, pb, va, vb;
#if !PKV_DECODE_PREFETCH
            for (int i = 0; i < npairs; ++i) {
                pages_of(i, pa, pb);
                issue(a, kbase, vbase, pa, pb, b0);
                valid(i, va, vb);
                compute(b0, va, vb, c);
            }
            continue;
#endif
            pages_of(0, pa, pb);
            issue(a, kbase, vbase, pa, pb, b0);
            // Two buffers in turn; the next pair's loads are issued before the
            // current pair is computed, and no load is left unconsumed at the
            // end, so the compiler's wait counts stay exact across iterations.
            // The scheduling barriers keep the loads ahead of the compute.
            for (int i = 0;; i += 2) {
                valid(i, va, vb);
                if (i + 1 < npairs) {
                    pages_of(i + 1, pa, pb);
                    __builtin_amdgcn_sched_barrier(0);
                    issue(a, kbase, vbase, pa, pb, b1);
                    __builtin_amdgcn_sched_barrier(0);
                    compute(b0, va, vb, c);
                } else {
                    compute(b0, va, vb, c);
                    break;
                }
                valid(i + 1, va, vb);
                if (i + 2 < npairs) {
                    pages_of(i + 2, pa, pb);
                    __builtin_amdgcn_sched_barrier(0);
                    issue(a, kbase, vbase, pa, pb, b0);
                    __builtin_amdgcn_sched_barrier(0);
                    compute(b1, va, vb, c);
                } else {
                    compute(b1, va, vb, c);
                    break;
                }
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
            for (int w = 0; w < VW; ++w) wv[w] = pack_bf16x2(acc[2 * w][i] * inv, acc[2 * w + 1][i] * inv);
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
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < DPL; j += 2) st_shared2(o + DPL * (4 * quad + i) + j, acc[j][i], acc[j + 1][i]);
        if (quad == 0) st_shared2(a.part_ml + (rec * G + col) * 2, m, lt);
    }
};

// ---------------------------------------------------------------------------
// fp32 engine: MFMA 16x16x4 f32, one page per step
// ---------------------------------------------------------------------------

template <int D>
struct EngF32 {
    using Out = float;
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
            const int phys = clamp_page(a, bt[p]);
            const float *kp = kbase + (int64_t)phys * a.s_page;
            const float *vp = vbase + (int64_t)phys * a.s_page;
            f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
                s = __builtin_amdgcn_mfma_f32_16x16x4f32(kp[(int64_t)col * a.s_tok + 4 * kc + quad], qop[kc], s, 0, 0,
                                                          0);
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
        for (int dc = 0; dc < DC; ++dc) *reinterpret_cast<f32x4 *>(o + 16 * dc + 4 * quad) = acc[dc] / lt;
        if (quad == 0 && a.lse) a.lse[(int64_t)b * a.hq + h] = (m + log2f(lt)) * kLn2;
    }

    __device__ __forceinline__ void store_partial(const DecodeArgs &a, int64_t rec) {
        const float lt = row_sum();
        if (col >= G) return;
        float *o = a.part_o + (rec * G + col) * D;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
            st_shared2(o + 16 * dc + 4 * quad, acc[dc][0], acc[dc][1]);
            st_shared2(o + 16 * dc + 4 * quad + 2, acc[dc][2], acc[dc][3]);
        }
        if (quad == 0) st_shared2(a.part_ml + (rec * G + col) * 2, m, lt);
    }
};

// ---------------------------------------------------------------------------
// kernel
// ---------------------------------------------------------------------------

// Resident waves per SIMD the register allocation is capped to (head_dim <= 128).
template <class Eng, int D>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(D <= 128 ? PKV_DECODE_WAVES_PER_EU : 1)))
void decode_kernel(DecodeArgs a) {
    using OutT = typename Eng::Out;
    const int w = blockIdx.x;
    Range r;
    if (!worker_range<OutT>(a, w, D, r)) return;
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
        if (p0 == 0 && p1 == np) {
            eng.store_final(a, b, g);
        } else {
            eng.store_partial(a, (int64_t)w + s);
            const int64_t wf = worker_of(seg_start, r);
            const int cnt = (int)(worker_of(seg_start + np - 1, r) - wf + 1);
            wait_stores_complete();  // the record is visible before it is counted
            int prior = 0;
            if (lane_id() == 0)
                prior = __hip_atomic_fetch_add(a.arrivals + s, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            prior = __shfl(prior, 0, kWave);
            if (prior == cnt - 1) {  // last piece of this segment: merge all of them
                merge_segment<OutT, D>(a, s, b, g, wf, cnt);
                if (lane_id() == 0)
                    __hip_atomic_store(a.arrivals + s, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
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

const void *pick_kernel(int dtype, int d) {
    if (dtype == 1) {
        if (d == 64) return reinterpret_cast<const void *>(&decode_kernel<EngBf16<64>, 64>);
        if (d == 128) return reinterpret_cast<const void *>(&decode_kernel<EngBf16<128>, 128>);
        if (d == 256) return reinterpret_cast<const void *>(&decode_kernel<EngBf16<256>, 256>);
    } else {
        if (d == 64) return reinterpret_cast<const void *>(&decode_kernel<EngF32<64>, 64>);
        if (d == 128) return reinterpret_cast<const void *>(&decode_kernel<EngF32<128>, 128>);
        if (d == 256) return reinterpret_cast<const void *>(&decode_kernel<EngF32<256>, 256>);
    }
    return nullptr;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct DeviceInfo {
    int cus = 0;
    int occ[2][3] = {{0, 0, 0}, {0, 0, 0}};  // resident decode waves per CU [dtype][d]
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
            if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) return -1;
            info.cus = cus;
        }
        int &occ = info.occ[g.dtype == 1 ? 1 : 0][dim_index(g.head_dim)];
        if (occ == 0) {
            int blocks = 0;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, pick_kernel(g.dtype, g.head_dim), kWave, 0) !=
                    hipSuccess ||
                blocks <= 0)
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

// Workspace: partial records (o: G*D fp32, (m, l): 2 fp32) for up to
// workers + batch*hkv pieces, then one arrival counter per (sequence, kv
// head).  The counters must be zero before the first call; every call leaves
// them zero.
size_t decode_workspace(const PoolGeom &g, int batch, int hq, int workers) {
    const int G = hq / g.hkv;
    const size_t recs = (size_t)workers + (size_t)batch * g.hkv;
    return align256(recs * G * g.head_dim * sizeof(float)) + align256(recs * G * 2 * sizeof(float)) +
           align256((size_t)batch * g.hkv * sizeof(int32_t));
}

hipError_t launch_decode(const PoolGeom &g, DecodeArgs a, int max_kv_len, hipStream_t stream) {
    (void)max_kv_len;
    const int G = a.hq / a.hkv;
    const size_t recs = (size_t)a.workers + (size_t)a.batch * a.hkv;
    char *ws = (char *)a.part_o;
    a.part_ml = (float *)(ws + align256(recs * G * g.head_dim * sizeof(float)));
    a.arrivals = (int32_t *)((char *)a.part_ml + align256(recs * G * 2 * sizeof(float)));
    const void *k = pick_kernel(g.dtype, g.head_dim);
    void *args[] = {&a};
    hipError_t e = hipLaunchKernel(k, dim3(a.workers), dim3(kWave), args, 0, stream);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace pkv
