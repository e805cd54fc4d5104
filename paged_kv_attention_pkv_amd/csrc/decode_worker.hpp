// decode_worker.hpp -- device code of the bf16 split decode worker (included
// by decode.hip).  What it computes and how the work is cut is
// described at the top of decode.hip.
#pragma once

#include <math.h>

#include "common.hpp"
#include "internal.hpp"

// Fewest pages a split worker is given when the library picks the count.
constexpr int64_t kMinPagesPerWorker = 8;
// Virtual pages charged for each segment start when ranges are cut.
constexpr int kSegCostPages = 4;

namespace pkv {

namespace {

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();
constexpr int kStage = 2048;  // page ids of its range a wave keeps in LDS at a time

// ---------------------------------------------------------------------------
// rows, segments, workers
// ---------------------------------------------------------------------------

// Attended length for a raw cache length (cut to the host bound, so that
// every table read stays inside the row: max_kv <= bt_cols * 16 is checked
// on the host).  In fused-append mode the raw length is the pre-append one.
__device__ __forceinline__ int attended(const DecodeArgs &a, int raw) {
    if (raw < 0) return 0;
    if (a.fused) return raw >= a.max_kv ? a.max_kv : raw + 1;
    return raw > a.max_kv ? a.max_kv : raw;
}

// Fused mode: the row's last attended key is the new token (not cut away).
__device__ __forceinline__ int fresh_token(const DecodeArgs &a, int raw) {
    return a.fused && raw >= 0 && raw < a.max_kv;
}

__device__ __forceinline__ int raw_len(const DecodeArgs &a, int b) { return b < a.batch ? a.seqlens[b] : -1; }

__device__ __forceinline__ int clamp_page(const DecodeArgs &a, int p) {
    return p < 0 ? 0 : (p >= a.num_pages ? a.num_pages - 1 : p);
}

// Raw lengths of 64 consecutive rows, one per lane (rows past the batch: -1),
// and, as left by plan() for rows 0..63, the inclusive prefix sum of their
// page counts.
struct RowLens {
    int base, raw, incl;
    __device__ __forceinline__ int get(const DecodeArgs &a, int b) {
        if (b < base || b >= base + kWave) {
            base = b & ~(kWave - 1);
            raw = raw_len(a, base + lane_id());
        }
        return __builtin_amdgcn_readlane(raw, b - base);
    }
};

// One (sequence, kv head) segment of the page space.
struct Seg {
    int b, g, n, np, fresh;  // row, kv head, attended length, pages, new-token flag
    int64_t f;               // position of its page 0 on the cost line (see plan)
};

__device__ __forceinline__ void seg_row(const DecodeArgs &a, Seg &s, int raw) {
    s.n = attended(a, raw);
    s.np = ceil_div(s.n, kPage);
    s.fresh = fresh_token(a, raw);
}

// The next non-empty segment (the caller knows one exists).
__device__ __forceinline__ void seg_next(const DecodeArgs &a, Seg &s, RowLens &rl) {
    s.f += s.np + kSegCostPages;
    if (++s.g == a.hkv) {
        s.g = 0;
        do {
            ++s.b;
            seg_row(a, s, rl.get(a, s.b));
        } while (s.n == 0 && s.b < a.batch);
    }
}

// Partial records travel between waves on different XCDs through
// agent-coherent accesses (st_agent2 / ld_agent2); a wave waits for its
// record stores to complete before it counts itself in the segment's
// arrival counter.
__device__ __forceinline__ void wait_stores_complete() { __builtin_amdgcn_s_waitcnt(0); }
// LDS writes of this wave become visible to all its lanes: wait for them and
// keep the compiler from moving LDS accesses across.
__device__ __forceinline__ void wave_lds_sync() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
}

// Zero output and -inf lse for a row without keys (b wave-uniform).
template <typename OutT>
__device__ void zero_row(const DecodeArgs &a, int b, int D) {
    OutT *out = (OutT *)a.out + (int64_t)b * a.hq * D;
    for (int i = lane_id(); i < a.hq * D; i += kWave) out[i] = OutT(0.f);
    if (a.lse)
        for (int h = lane_id(); h < a.hq; h += kWave) a.lse[(int64_t)b * a.hq + h] = kNegInf;
}

struct Range {
    int64_t f0, f1;  // its pages lie in [f0, f1): the first page positions at or after its two cuts
    int64_t total;   // length of the cost line
    int workers;
};

// Work is measured on a "cost line": the non-empty segments in flat order,
// each as kSegCostPages virtual positions (the extra time a segment start
// brings: a new query row, a piece to settle after the range) followed by one
// position per page.  Waves take equal shares of the line, so a range that
// starts a segment holds that many fewer pages.  Page p of the i-th non-empty
// segment sits at (pages of the segments before) + kSegCostPages * (i + 1) + p.
// Cursors, page-id staging and piece bookkeeping all count in these positions.

// Pages and positions of the rows of one 64-row chunk (one lane per row,
// inclusive prefix over the chunk, per kv head).
__device__ __forceinline__ int chunk_cost(const DecodeArgs &a, int raw, int incl) {
    const int np = ceil_div(attended(a, raw), kPage);
    const uint64_t ne = __ballot(np > 0);
    const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(ne >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)ne, 0));
    return incl + kSegCostPages * (below + (np > 0 ? 1 : 0));
}

// First page position at or after each of x0 < x1 (x1 may be the line's
// length), and the segment of the first into s.  One pass over the row
// lengths: rows 0..63 from `rl` (as left by plan), further chunks read if
// needed.
__device__ __forceinline__ void locate2(const DecodeArgs &a, int64_t x0, int64_t x1, const RowLens &rl, Seg &s,
                                        int64_t &f0, int64_t &f1) {
    const int l = lane_id();
    int64_t run = 0;  // positions of the rows before this chunk
    bool need0 = true;
    f1 = x1;  // x1 at the line's end
    for (int base = 0; base < a.batch; base += kWave) {
        int raw = rl.raw, incl = rl.incl;
        if (base > 0) {
            raw = raw_len(a, base + l);
            incl = wave_incl_scan32(ceil_div(attended(a, raw), kPage));
        }
        const int cincl = chunk_cost(a, raw, incl);
        const int64_t tot = run + (int64_t)__builtin_amdgcn_readlane(cincl, kWave - 1) * a.hkv;
        // the first row whose positions end past x has pages (an empty row has none)
        if (need0 && tot > x0) {
            const int first = uniform((int)__builtin_ctzll(__ballot(run + (int64_t)cincl * a.hkv > x0)));
            s.b = base + first;
            seg_row(a, s, __builtin_amdgcn_readlane(raw, first));
            const int per = s.np + kSegCostPages;
            const int64_t start = run + (int64_t)(__builtin_amdgcn_readlane(cincl, first) - per) * a.hkv;
            s.g = (int)((x0 - start) / per);
            s.f = start + (int64_t)s.g * per + kSegCostPages;
            f0 = x0 > s.f ? x0 : s.f;
            need0 = false;
        }
        if (tot > x1) {
            const int first = uniform((int)__builtin_ctzll(__ballot(run + (int64_t)cincl * a.hkv > x1)));
            const int np = ceil_div(attended(a, __builtin_amdgcn_readlane(raw, first)), kPage);
            const int per = np + kSegCostPages;
            const int64_t start = run + (int64_t)(__builtin_amdgcn_readlane(cincl, first) - per) * a.hkv;
            const int64_t e = start + ((x1 - start) / per) * per + kSegCostPages;
            f1 = x1 > e ? x1 : e;
            return;
        }
        run = tot;
    }
}

// The per-row chores of worker w for the 64 rows from `base` (raw lengths one
// per lane): rows are handed out round-robin (row b to worker b mod workers);
// a row without keys gets zero output and -inf lse, and in fused mode a row
// whose token is not stored keeps its length (the others get theirs from the
// wave that writes the token, in the splice).
template <typename OutT>
__device__ __forceinline__ void row_chores(const DecodeArgs &a, int w, int D, int base, int raw) {
    const int b = base + lane_id();
    const bool mine = b < a.batch && b % a.workers == w;
    if (mine && a.seqlens_out && !fresh_token(a, raw)) a.seqlens_out[b] = raw;
    uint64_t empty = __ballot(mine && attended(a, raw) == 0);
    while (empty) {
        const int e = uniform((int)__builtin_ctzll(empty));
        empty &= empty - 1;
        zero_row<OutT>(a, base + e, D);
    }
}

// Pages of all rows (one kv head) and the number of rows with pages, with
// the chores of worker w when kChores.  The first 64 raw lengths and their
// page prefix sums stay in `rl`.
template <typename OutT, bool kChores>
__device__ __forceinline__ void count_rows(const DecodeArgs &a, int w, int D, RowLens &rl, int64_t &pages,
                                           int &rows) {
    pages = 0;
    rows = 0;
    for (int base = 0; base < a.batch; base += kWave) {
        const int raw = raw_len(a, base + lane_id());
        const int n = attended(a, raw);
        const int incl = wave_incl_scan32(ceil_div(n, kPage));
        if (base == 0) {
            rl.base = 0;
            rl.raw = raw;
            rl.incl = incl;
        }
        pages += __builtin_amdgcn_readlane(incl, kWave - 1);
        rows += __builtin_popcountll(__ballot(n > 0));
        if constexpr (kChores) row_chores<OutT>(a, w, D, base, raw);
    }
}

// Line length and the share of wave w, with the segment its range starts in.
// The range is [f0, f1) with f0 and f1 the first page positions at or after
// the two cuts, so a walk stops where the next segment would start at or past
// f1.  False when the wave has no pages.
__device__ __forceinline__ bool cut_range(const DecodeArgs &a, int w, int64_t pages, int rows, const RowLens &rl,
                                          Range &r, Seg &s) {
    const int64_t total = pages * a.hkv;
    // Small calls use fewer waves, so each keeps at least kMinPagesPerWorker
    // pages (a segment cut into many tiny pieces costs more in merges than
    // the extra waves gain).  A count the caller fixed is used as given.
    const int64_t by_pages = total / kMinPagesPerWorker > 0 ? total / kMinPagesPerWorker : 1;
    int64_t wmax = by_pages < (int64_t)a.workers ? by_pages : (int64_t)a.workers;
    if (a.fixed_workers) wmax = total < (int64_t)a.workers ? total : (int64_t)a.workers;
    else if (a.mid_workers > 0 && total < a.mid_pages && wmax > a.mid_workers) wmax = a.mid_workers;
    if ((int64_t)w >= wmax) return false;
    const int64_t len = total + (int64_t)kSegCostPages * rows * a.hkv;
    r.total = len;
    r.workers = (int)wmax;
    locate2(a, (int64_t)w * len / wmax, (int64_t)(w + 1) * len / wmax, rl, s, r.f0, r.f1);
    return r.f0 < r.f1;
}

// Everything a wave needs before its first page: the chores, the line and
// its range.  The first 64 raw lengths stay in `rl`.  False when the wave has
// no pages.
template <typename OutT>
__device__ __forceinline__ bool plan(const DecodeArgs &a, int w, int D, RowLens &rl, Range &r, Seg &s) {
    int64_t pages;
    int rows;
    count_rows<OutT, true>(a, w, D, rl, pages, rows);
    return cut_range(a, w, pages, rows, rl, r, s);
}

// ---------------------------------------------------------------------------
// a plan computed once for several calls
// ---------------------------------------------------------------------------
//
// The cut depends only on the row lengths and on the call's shape (batch, kv
// heads, max_kv, fused mode, worker counts), so the decode calls of one step
// (one per layer, all on the same table and lengths) share it.
// decode_plan_kernel writes it to the plan region of a workspace:
//   words 0..15            header: kPlanMagic and the shape (plan_word)
//   kPlanHdr ..            the raw length of every row, as planned
//   kPlanHdr + lens_words  one record of kPlanRec words per worker: has
//                          pages, workers, line length, f0, f1, and the
//                          first segment (b, g, n, np, fresh, f)
// A call given a plan reads the header, its record and every row's length
// and planned length together (one round trip), and takes the record only if
// every header word and every length agree with its own; otherwise it plans
// as without one.  Either way it walks the same range.
constexpr int kPlanMagic = 0x504b5650;
constexpr int kPlanHdr = 64;  // words (256 bytes)
constexpr int kPlanRec = 16;  // words per worker

__device__ __forceinline__ int64_t plan_lens_words(int batch) { return ((int64_t)batch + 63) & ~(int64_t)63; }

// Header word k (0..15) of a plan for the call `a`.
__device__ __forceinline__ int plan_word(const DecodeArgs &a, int k) {
    switch (k) {
        case 0: return kPlanMagic;
        case 1: return a.batch;
        case 2: return a.hkv;
        case 3: return a.max_kv;
        case 4: return a.fused;
        case 5: return a.workers;
        case 6: return a.fixed_workers;
        case 7: return a.mid_workers;
        case 8: return (int)(uint32_t)a.mid_pages;
        case 9: return (int)(a.mid_pages >> 32);
        default: return 0;
    }
}

__device__ __forceinline__ int64_t lanes64(int v, int k) {
    return (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane(v, k + 1) << 32) |
                     (uint32_t)__builtin_amdgcn_readlane(v, k));
}

// plan() through the plan at a.plan when it matches the call (see above).
template <typename OutT>
__device__ __forceinline__ bool plan_or_load(const DecodeArgs &a, int w, int D, RowLens &rl, Range &r, Seg &s) {
    if (!a.plan) return plan<OutT>(a, w, D, rl, r, s);
    const int l = lane_id();
    const int32_t *lens = a.plan + kPlanHdr;
    const int32_t *recs = lens + plan_lens_words(a.batch);
    const int hv = a.plan[l & 15];
    const int rv = recs[(int64_t)w * kPlanRec + (l & 15)];
    const int raw = raw_len(a, l);
    const int cp = l < a.batch ? lens[l] : -1;
    bool ok = __ballot((l < 16 && hv != plan_word(a, l)) || raw != cp) == 0;
    for (int base = kWave; ok && base < a.batch; base += kWave) {
        const int b = base + l;
        ok = __ballot(raw_len(a, b) != (b < a.batch ? lens[b] : -1)) == 0;
    }
    if (!ok) return plan<OutT>(a, w, D, rl, r, s);
    rl.base = 0;
    rl.raw = raw;
    rl.incl = 0;  // read by the cut only
    row_chores<OutT>(a, w, D, 0, raw);
    for (int base = kWave; base < a.batch; base += kWave) row_chores<OutT>(a, w, D, base, raw_len(a, base + l));
    if (!__builtin_amdgcn_readlane(rv, 0)) return false;
    r.workers = __builtin_amdgcn_readlane(rv, 1);
    r.total = lanes64(rv, 2);
    r.f0 = lanes64(rv, 4);
    r.f1 = lanes64(rv, 6);
    s.b = __builtin_amdgcn_readlane(rv, 8);
    s.g = __builtin_amdgcn_readlane(rv, 9);
    s.n = __builtin_amdgcn_readlane(rv, 10);
    s.np = __builtin_amdgcn_readlane(rv, 11);
    s.fresh = __builtin_amdgcn_readlane(rv, 12);
    s.f = lanes64(rv, 13);
    return true;
}

// Writes the plan of a call shaped as `a` (one wave per worker, w = its
// index): its record, the lengths of rows 64w.. (and every further
// 64*workers), and from wave 0 the header.
__device__ __forceinline__ void write_plan(const DecodeArgs &a, int w) {
    RowLens rl;
    int64_t pages;
    int rows;
    count_rows<float, false>(a, w, 0, rl, pages, rows);
    Range r;
    Seg s;
    const bool has = cut_range(a, w, pages, rows, rl, r, s);
    const int l = lane_id();
    int32_t *lens = a.plan + kPlanHdr;
    int32_t *recs = lens + plan_lens_words(a.batch);
    if (l < 16) {
        int v = 0;
        if (has) {
            switch (l) {
                case 0: v = 1; break;
                case 1: v = r.workers; break;
                case 2: v = (int)(uint32_t)r.total; break;
                case 3: v = (int)(r.total >> 32); break;
                case 4: v = (int)(uint32_t)r.f0; break;
                case 5: v = (int)(r.f0 >> 32); break;
                case 6: v = (int)(uint32_t)r.f1; break;
                case 7: v = (int)(r.f1 >> 32); break;
                case 8: v = s.b; break;
                case 9: v = s.g; break;
                case 10: v = s.n; break;
                case 11: v = s.np; break;
                case 12: v = s.fresh; break;
                case 13: v = (int)(uint32_t)s.f; break;
                case 14: v = (int)(s.f >> 32); break;
                default: v = 0;
            }
        }
        recs[(int64_t)w * kPlanRec + l] = v;
    }
    for (int64_t base = (int64_t)w * kWave; base < a.batch; base += (int64_t)a.workers * kWave) {
        const int b = (int)base + l;
        if (b < a.batch) lens[b] = a.seqlens[b];
    }
    if (w == 0 && l < 16) a.plan[l] = plan_word(a, l);
}

// Worker whose range holds the page at position x.
__device__ __forceinline__ int64_t worker_of(int64_t x, const Range &r) {
    return ((x + 1) * r.workers - 1) / r.total;
}

// ---------------------------------------------------------------------------
// partial records and their merge
// ---------------------------------------------------------------------------
//
// A record holds the G x D unnormalised outputs of one piece as D/8 blocks,
// one per store instruction of the engine: block t holds, at pair index
// t*4G + quad*G + col, the two fp32 values the lane (quad, col) stores with
// it, so each instruction writes one contiguous run and the merge reads the
// record with consecutive lanes on consecutive pairs.  Eng::dim_of(t, quad)
// gives the (even) output dim of such a pair.  (m, l) per head follow in a
// second array.

template <typename OutT>
__device__ __forceinline__ void store_out_pair(OutT *p, float x, float y);
template <>
__device__ __forceinline__ void store_out_pair<__bf16>(__bf16 *p, float x, float y) {
    *reinterpret_cast<uint32_t *>(p) = pack_bf16x2(x, y);
}
template <>
__device__ __forceinline__ void store_out_pair<float>(float *p, float x, float y) {
    *reinterpret_cast<f32x2 *>(p) = f32x2{x, y};
}

// One split segment to merge: pieces of workers wf .. wf+cnt-1, record ids
// w + s, output row b, kv head g.
struct MergeJob {
    int64_t s, wf;
    int b, g, cnt;
};

// Merge the partial records of NJ split segments (NJ = 1, or 2 when their
// pieces fit in one batch) in piece order and write their output rows.
// Pieces are taken 8 at a time with every load of a batch issued before any
// is used, so two segments merged together have all their loads in flight at
// once.  A segment's arithmetic (batches, order of the folds) is the same
// whether it is merged alone or beside another, so results do not depend on
// which wave merges it.  Batches are folded with the log-sum-exp rule.  The
// merging wave's own piece (piece own_piece of job own_job) may come from
// LDS (own_o, own_ml: the same record layout and values) instead of memory.
template <typename OutT, class Eng, int D, int NJ>
__device__ void merge_jobs(const DecodeArgs &a, const MergeJob *job, int own_job = -1, int own_piece = -1,
                           const float *own_o = nullptr, const float *own_ml = nullptr) {
    constexpr int kBatch = 8, kPairs = 4;
    const int G = a.hq / a.hkv;
    const int npairs = G * D / 2;
    const int64_t ostride = (int64_t)G * D;
    const int c0 = job[0].cnt;
    const int total = NJ == 1 ? c0 : c0 + job[NJ - 1].cnt;
    for (int u0 = 0; u0 < npairs; u0 += kWave * kPairs) {
        int uu[kPairs], col[kPairs], dim[kPairs];
        float M[NJ][kPairs], den[NJ][kPairs], n0[NJ][kPairs], n1[NJ][kPairs];
#pragma unroll
        for (int k = 0; k < kPairs; ++k) {
            const int u = u0 + k * kWave + lane_id();
            uu[k] = u < npairs ? u : npairs - 1;
            const int t = uu[k] / (4 * G);
            const int rem = uu[k] - t * 4 * G;
            const int quad = rem / G;
            col[k] = rem - quad * G;
            dim[k] = Eng::dim_of(t, quad);
#pragma unroll
            for (int jj = 0; jj < NJ; ++jj) {
                M[jj][k] = kNegInf;
                den[jj][k] = n0[jj][k] = n1[jj][k] = 0.f;
            }
        }
        for (int k0 = 0; k0 < total; k0 += kBatch) {
            const int nb = min(kBatch, total - k0);
            f32x2 ml[kBatch][kPairs], o[kBatch][kPairs];
            int owner[kBatch];  // job of batch entry j (wave-uniform)
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const int q = k0 + j;
                owner[j] = j >= nb ? -1 : (NJ == 2 && q >= c0 ? 1 : 0);
                if (j < nb) {
                    const int piece = owner[j] == 0 ? q : q - c0;
                    if (owner[j] == own_job && piece == own_piece) {
#pragma unroll
                        for (int k = 0; k < kPairs; ++k) {
                            ml[j][k] = *reinterpret_cast<const f32x2 *>(own_ml + col[k] * 2);
                            o[j][k] = *reinterpret_cast<const f32x2 *>(own_o + 2 * uu[k]);
                        }
                    } else {
                        const int64_t rec = owner[j] == 0 ? job[0].wf + piece + job[0].s
                                                          : job[NJ - 1].wf + piece + job[NJ - 1].s;
#pragma unroll
                        for (int k = 0; k < kPairs; ++k) {
                            ml[j][k] = ld_agent2(a.part_ml + (rec * G + col[k]) * 2);
                            o[j][k] = ld_agent2(a.part_o + rec * ostride + 2 * uu[k]);
                        }
                    }
                }
            }
#pragma unroll
            for (int k = 0; k < kPairs; ++k) {
#pragma unroll
                for (int jj = 0; jj < NJ; ++jj) {
                    float Mb = M[jj][k];
#pragma unroll
                    for (int j = 0; j < kBatch; ++j)
                        if (owner[j] == jj) Mb = fmaxf(Mb, ml[j][k][0]);
                    const float r = fast_exp2(M[jj][k] - Mb);
                    den[jj][k] *= r;
                    n0[jj][k] *= r;
                    n1[jj][k] *= r;
#pragma unroll
                    for (int j = 0; j < kBatch; ++j) {
                        if (owner[j] == jj) {
                            const float wgt = fast_exp2(ml[j][k][0] - Mb);
                            den[jj][k] = fmaf(wgt, ml[j][k][1], den[jj][k]);
                            n0[jj][k] = fmaf(wgt, o[j][k][0], n0[jj][k]);
                            n1[jj][k] = fmaf(wgt, o[j][k][1], n1[jj][k]);
                        }
                    }
                    M[jj][k] = Mb;
                }
            }
        }
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) {
            const int b = job[jj].b;
            OutT *out = (OutT *)a.out + ((int64_t)b * a.hq + (int64_t)job[jj].g * G) * D;
#pragma unroll
            for (int k = 0; k < kPairs; ++k) {
                if (u0 + k * kWave + lane_id() < npairs) {
                    const float inv = 1.f / den[jj][k];
                    store_out_pair<OutT>(out + (int64_t)col[k] * D + dim[k], n0[jj][k] * inv, n1[jj][k] * inv);
                    if (dim[k] == 0 && a.lse)
                        a.lse[(int64_t)b * a.hq + (int64_t)job[jj].g * G + col[k]] =
                            (M[jj][k] + log2f(den[jj][k])) * kLn2;
                }
            }
        }
    }
}

// Split pieces a wave leaves for the merge (at most its first and its last).
struct Pending {
    int n;
    MergeJob job[2];
    int state[2];  // kStored, kSaved or kHeld
    int prior[2];  // the count before this piece's arrival (lane 0)
    int check;     // held job: its arrival count read ahead (lane 0), -1 if not read
};
// kStored: record written, not yet counted.  kSaved: the range's first
// piece, its state copied aside in the engine's registers (record stores are
// agent-coherent and complete only at memory; loads issued behind them wait
// for that, so a record written mid-range stalls the page stream).  kHeld:
// the range's last piece, still in the engine's accumulators.
constexpr int kStored = 0, kSaved = 1, kHeld = 2;

__device__ __forceinline__ void pending_init(Pending &p) {
    p.n = 0;
    p.check = -1;
}

__device__ __forceinline__ void pending_add(Pending &p, int64_t s, int b, int g, int64_t wf, int cnt, int state) {
    const MergeJob j{s, wf, b, g, cnt};
    if (p.n == 0) {
        p.job[0] = j;
        p.state[0] = state;
    } else {
        p.job[1] = j;
        p.state[1] = state;
    }
    ++p.n;
}

__device__ __forceinline__ int count_arrival(const DecodeArgs &a, int64_t s) {
    int prior = 0;
    if (lane_id() == 0) prior = __hip_atomic_fetch_add(a.arrivals + s, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return prior;
}

// Read ahead the arrival count of the segment of the wave's last piece
// (issued behind the last pair's loads, looked at after the range).
__device__ __forceinline__ int peek_arrivals(const DecodeArgs &a, int64_t s) {
    int v = 0;
    if (lane_id() == 0) v = __hip_atomic_load(a.arrivals + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return v;
}

// After the range: write the saved record, then count the pieces (once
// their record stores have completed); the piece that completes a segment's
// count merges it.  A held last piece whose segment has every other piece
// counted already (as read ahead) is merged straight from the registers,
// through LDS, with no record written and no count taken.  When the wave
// merges both of its segments, the two merges run as one.
template <typename OutT, class Eng, int D>
__device__ void settle(const DecodeArgs &a, Eng &eng, Pending &p, int w, float *own_o, float *own_ml) {
    if (p.n == 0) return;
    if constexpr (Eng::kHolds) {
        if (p.state[0] == kSaved) {
            eng.store_saved(a, (int64_t)w + p.job[0].s);
            p.state[0] = kStored;
        }
    }
    const int H = (p.n == 2 ? p.state[1] : p.state[0]) == kHeld ? p.n - 1 : -1;
    const MergeJob &hj = H == 1 ? p.job[1] : p.job[0];
    bool fast = false;
    if constexpr (Eng::kHolds) {
        if (H >= 0) {
            const int seen = __shfl(p.check >= 0 ? p.check : peek_arrivals(a, hj.s), 0, kWave);
            fast = seen == hj.cnt - 1;
            if (fast) {
                eng.stage_record(own_o, own_ml);
                wave_lds_sync();  // the record's lanes are read back by other lanes of this wave
            } else {
                eng.store_partial(a, (int64_t)w + hj.s);
                if (H == 1)
                    p.state[1] = kStored;
                else
                    p.state[0] = kStored;
            }
        }
    }
    const bool st0 = p.state[0] == kStored, st1 = p.n == 2 && p.state[1] == kStored;
    if (st0 || st1) wait_stores_complete();  // the records are visible before they are counted
    if (st0) p.prior[0] = count_arrival(a, p.job[0].s);
    if (st1) p.prior[1] = count_arrival(a, p.job[1].s);
    bool last[2];
    last[0] = (H == 0 && fast) || __shfl(p.prior[0], 0, kWave) == p.job[0].cnt - 1;
    last[1] = p.n == 2 && ((H == 1 && fast) || __shfl(p.prior[1], 0, kWave) == p.job[1].cnt - 1);
    const int own_job = fast ? H : -1;
    const int own_piece = fast ? (int)((int64_t)w - hj.wf) : -1;
    if (p.n == 2 && last[0] && last[1] && p.job[0].cnt + p.job[1].cnt <= 8) {
        merge_jobs<OutT, Eng, D, 2>(a, p.job, own_job, own_piece, own_o, own_ml);
    } else {
        if (last[0]) merge_jobs<OutT, Eng, D, 1>(a, &p.job[0], own_job == 0 ? 0 : -1, own_piece, own_o, own_ml);
        if (p.n == 2 && last[1])
            merge_jobs<OutT, Eng, D, 1>(a, &p.job[1], own_job == 1 ? 0 : -1, own_piece, own_o, own_ml);
    }
    if (lane_id() == 0) {
        if (last[0]) __hip_atomic_store(a.arrivals + p.job[0].s, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (last[1]) __hip_atomic_store(a.arrivals + p.job[1].s, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ---------------------------------------------------------------------------
// bf16 stream: cursor over the wave's range, page pairs, MFMA 16x16x32 bf16
// ---------------------------------------------------------------------------

// Position of the next page to load.
struct Cursor {
    Seg s;
    int p, pend, pstart;  // next page, end of the piece in this segment, first page of the piece
    int live;
    __device__ __forceinline__ int64_t f() const { return s.f + p; }
};

// One page pair as the compute side sees it (wave-uniform).
struct Desc {
    int b, g, n, np, pa;
    // bit 0: two pages; bit 1: last pair of its piece; bit 2: the piece covers
    // the whole segment; bit 3 (fused mode): the pair's last token is the new one
    int flags;
    int ida, idb;
    int raw_last;  // table entry of the pair's last page (unclamped)
    int64_t segf;  // position of its segment's page 0
    __device__ __forceinline__ int npg() const { return 1 + (flags & 1); }
    __device__ __forceinline__ bool last() const { return flags & 2; }
    __device__ __forceinline__ bool whole() const { return flags & 4; }
    __device__ __forceinline__ bool newtok() const { return flags & 8; }
};

// Fill ids[i] with the table entry of the page at position c.f() + i, for
// i < min(kStage, f1 - c.f()) (0 at virtual positions): one pass of coalesced
// table reads, eight 64-entry chunks at a time with all loads of a group
// issued before any is used.
//
// With pages of more than 16 tokens (SUB), position p of a segment is the
// 16-token sub-page p of its row: table column p >> page_shift, sub-page
// p & (2^page_shift - 1) of that page, and ids[i] holds (page << page_shift)
// | sub-page, with entries outside the pool taken as page 0.
template <bool SUB>
__device__ void stage(const DecodeArgs &a, int *ids, const Cursor &c, int64_t f1, RowLens &rl) {
    const int64_t f0 = c.f();
    const int len = (int)(f1 - f0 < kStage ? f1 - f0 : kStage);
    const int l = lane_id();
    Seg s = c.s;
    for (int c0 = 0; c0 < len; c0 += 8 * kWave) {
        const int64_t gend = f0 + (c0 + 8 * kWave < len ? c0 + 8 * kWave : len);
        int64_t off[8];
        int sub[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) off[u] = -1;
        for (;;) {  // the segments overlapping [f0 + c0, gend)
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int64_t fl = f0 + c0 + u * kWave + l;
                if (fl < gend && fl >= s.f && fl < s.f + s.np) {
                    if constexpr (SUB) {
                        off[u] = (int64_t)s.b * a.bt_cols + ((fl - s.f) >> a.page_shift);
                        sub[u] = (int)(fl - s.f) & ((1 << a.page_shift) - 1);
                    } else {
                        off[u] = (int64_t)s.b * a.bt_cols + (fl - s.f);
                    }
                }
            }
            if (s.f + s.np >= gend) break;
            seg_next(a, s, rl);
        }
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = off[u] >= 0 ? a.block_table[off[u]] : 0;
        if constexpr (SUB) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int pg = v[u] >= 0 && v[u] < a.num_pages ? v[u] : 0;
                v[u] = off[u] >= 0 ? (pg << a.page_shift) | sub[u] : 0;
            }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = c0 + u * kWave + l;
            if (i < len) ids[i] = v[u];
        }
    }
}

// The next pair at the cursor, then advance.  Restages the id window when
// the cursor has run past it.
template <bool SUB>
__device__ __forceinline__ void take(const DecodeArgs &a, Cursor &c, int *ids, int64_t &fbase, int64_t f1,
                                     RowLens &rl, Desc &d) {
    if (__builtin_expect(c.f() - fbase >= kStage, 0)) {
        fbase = c.f();
        stage<SUB>(a, ids, c, f1, rl);
    }
    const int64_t i = c.f() - fbase;
    d.b = c.s.b;
    d.g = c.s.g;
    d.n = c.s.n;
    d.np = c.s.np;
    d.pa = c.p;
    d.segf = c.s.f;
    const int npg = (c.p + 1 < c.pend && i + 1 < kStage) ? 2 : 1;
    d.flags = (npg - 1) | (c.p + npg == c.pend ? 2 : 0) | (c.pstart == 0 && c.pend == c.s.np ? 4 : 0) |
              (c.s.fresh && c.p + npg == c.s.np ? 8 : 0);
    const int ra = uniform(ids[i]);
    const int rb = npg == 2 ? uniform(ids[i + 1]) : ra;
    if constexpr (SUB) {  // staged in range
        d.ida = ra;
        d.idb = rb;
    } else {
        d.ida = clamp_page(a, ra);
        d.idb = clamp_page(a, rb);
    }
    d.raw_last = rb;
    c.p += npg;
    if (__builtin_expect(c.p == c.pend, 0)) {
        if (c.f() + kSegCostPages >= f1) {  // stopped inside a segment, or the next one starts at or past f1
            c.live = 0;
        } else {
            seg_next(a, c.s, rl);
            c.p = c.pstart = 0;
            c.pend = (int)(c.s.np < f1 - c.s.f ? c.s.np : f1 - c.s.f);
        }
    }
}

template <int D, bool SUB>
struct Bf16 {
    using Out = __bf16;
    static constexpr bool kHolds = true;  // can hold its last piece for a merge from registers
    static constexpr int KC = D / 32;   // QK MFMAs per page
    static constexpr int DPL = D / 16;  // V elements per lane per token = PV MFMAs per pair
    static constexpr int VW = DPL / 2;  // dwords per lane per V token row

    struct Buf {
        u32x4 q[KC];
        u32x4 kA[KC], kB[KC];
        uint32_t vA[4][VW], vB[4][VW];
        u32x4 kn[KC];     // fused append: the new token's K (lanes col == slot)
        uint32_t vn[VW];  // and V (lanes quad == slot / 4)
    };

    f32x4 acc[DPL];
    float m, l;
    f32x4 sacc[DPL];  // the range's first split piece, written after the range
    float sm, sl;
    int G, quad, col;
    uint32_t koff;     // lane's byte offset in a page for K (token col, dims 8quad..)
    uint32_t voff[4];  // lane's byte offsets for V (token 4quad+e, dims DPL*col..)

    // Output dim of record pair (t, quad): acc[2jj][i], acc[2jj+1][i] with t = i*VW + jj.
    __device__ static __forceinline__ int dim_of(int t, int quad) {
        const int i = t / VW, jj = t - i * VW;
        return DPL * (4 * quad + i) + 2 * jj;
    }

    __device__ __forceinline__ void reset() {
#pragma unroll
        for (int j = 0; j < DPL; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        m = kNegInf;
        l = 0.f;
    }

    __device__ __forceinline__ void init(const DecodeArgs &a) {
        G = a.hq / a.hkv;
        const int ln = lane_id();
        quad = ln >> 4;
        col = ln & 15;
        const uint32_t st = (uint32_t)a.s_tok * 2u;
        koff = col * st + 16u * quad;
#pragma unroll
        for (int e = 0; e < 4; ++e) voff[e] = (4u * quad + e) * st + 2u * DPL * col;
        reset();
    }

    // kb / vb are wave-uniform page bases and the lane parts zero-extended
    // 32-bit byte offsets, so the loads use scalar-base + vector-offset
    // addressing and need no per-lane 64-bit address registers.
    // Page loads carry the non-temporal hint: every K/V byte is read once per
    // call, and with the hint the caches stop holding lines that will not be
    // read again (measured: 36-layer long-context workload 5.5 -> 6.0 TB/s,
    // B = 64 step 50.3 -> 46.9 us).
    __device__ __forceinline__ void load_page(const char *kb, const char *vb, u32x4 (&k)[KC],
                                              uint32_t (&v)[4][VW]) {
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) k[kc] = ld16_stream(kb + (uint64_t)koff + 64 * kc);
#pragma unroll
        for (int e = 0; e < 4; ++e) load_vrow(vb + (uint64_t)voff[e], v[e]);
    }

    __device__ __forceinline__ static void load_vrow(const char *src, uint32_t (&v)[VW]) {
        if constexpr (VW == 2) {
            const u32x2 x = ld8_stream(src);
            v[0] = x[0];
            v[1] = x[1];
        } else {
#pragma unroll
            for (int c4 = 0; c4 < VW / 4; ++c4) {
                const u32x4 x = ld16_stream(src + 16 * c4);
                v[4 * c4 + 0] = x[0];
                v[4 * c4 + 1] = x[1];
                v[4 * c4 + 2] = x[2];
                v[4 * c4 + 3] = x[3];
            }
        }
    }

    __device__ __forceinline__ static void store_vrow(char *dst, const uint32_t (&v)[VW]) {
        if constexpr (VW == 2) {
            *reinterpret_cast<u32x2 *>(dst) = u32x2{v[0], v[1]};
        } else {
#pragma unroll
            for (int c4 = 0; c4 < VW / 4; ++c4)
                st16(dst + 16 * c4, u32x4{v[4 * c4], v[4 * c4 + 1], v[4 * c4 + 2], v[4 * c4 + 3]});
        }
    }

    // Loads of pair d: K and V of its pages, the query rows of (b, g) and, in
    // fused mode, the new token.
    // Byte offset of a staged page id (with SUB: page and 16-token sub-page).
    __device__ static __forceinline__ int64_t page_bytes(const DecodeArgs &a, int id, int64_t ps) {
        if constexpr (SUB)
            return (int64_t)(id >> a.page_shift) * ps + (int64_t)(id & ((1 << a.page_shift) - 1)) * kPage * a.s_tok * 2;
        else
            return (int64_t)id * ps;
    }

    __device__ __forceinline__ void issue(const DecodeArgs &a, const Desc &d, Buf &buf) {
        const int64_t hoff = (int64_t)d.g * a.s_head * 2;
        const char *kc = (const char *)a.k_cache + hoff;
        const char *vc = (const char *)a.v_cache + hoff;
        const int64_t ps = a.s_page * 2;
        const int64_t pa = page_bytes(a, d.ida, ps), pb = page_bytes(a, d.idb, ps);
        load_page(kc + pa, vc + pa, buf.kA, buf.vA);
        load_page(kc + pb, vc + pb, buf.kB, buf.vB);
        const int qc = col < G ? col : G - 1;  // lanes past the group read nothing
        const char *q = (const char *)a.q + ((int64_t)d.b * a.hq + (int64_t)d.g * G + qc) * D * 2;
#pragma unroll
        for (int kc2 = 0; kc2 < KC; ++kc2) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            buf.q[kc2] = col < G ? ld16(q + 64 * kc2 + 16 * quad) : z;
        }
        if (__builtin_expect(d.newtok(), 0)) {
            const int slot = (d.n - 1) & (kPage - 1);
            const int64_t row = ((int64_t)d.b * a.hkv + d.g) * D * 2;
            if (col == slot) {
#pragma unroll
                for (int kc2 = 0; kc2 < KC; ++kc2)
                    buf.kn[kc2] = ld16((const char *)a.k_new + row + 64 * kc2 + 16 * quad);
            }
            if (quad == (slot >> 2)) load_vrow((const char *)a.v_new + row + 2 * DPL * col, buf.vn);
        }
    }

    // Fused mode: put the new token into the pair's registers in place of
    // its (stale) slot and write it into the pool.
    __device__ __forceinline__ void splice(const DecodeArgs &a, const Desc &d, Buf &buf) {
        const int slot = (d.n - 1) & (kPage - 1);
        const int e = slot & 3;
        const bool inB = d.npg() == 2;
        const int last_page = SUB ? d.raw_last >> a.page_shift : d.raw_last;
        const bool writable = last_page >= 1 && last_page < a.num_pages;
        // the new length counts the token only where it was stored
        if (d.g == 0 && lane_id() == 0 && a.seqlens_out) a.seqlens_out[d.b] = writable ? d.n : d.n - 1;
        const int64_t base = (int64_t)d.g * a.s_head * 2 + page_bytes(a, d.raw_last, a.s_page * 2);
        if (col == slot) {
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                if (inB)
                    buf.kB[kc] = buf.kn[kc];
                else
                    buf.kA[kc] = buf.kn[kc];
                if (writable) st16((char *)a.k_cache + base + koff + 64 * kc, buf.kn[kc]);
            }
        }
        if (quad == (slot >> 2)) {
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                if (e2 == e) {
#pragma unroll
                    for (int w = 0; w < VW; ++w) {
                        if (inB)
                            buf.vB[e2][w] = buf.vn[w];
                        else
                            buf.vA[e2][w] = buf.vn[w];
                    }
                    if (writable) store_vrow((char *)a.v_cache + base + voff[e2], buf.vn);
                }
            }
        }
    }

    __device__ __forceinline__ void compute(const DecodeArgs &a, Buf &buf, const Desc &d, float c) {
        if (__builtin_expect(d.newtok(), 0)) splice(a, d, buf);
        const int vcA = min(d.n - d.pa * kPage, kPage);
        const int vcB = d.npg() == 2 ? min(d.n - (d.pa + 1) * kPage, kPage) : 0;
        f32x4 sA = {0.f, 0.f, 0.f, 0.f}, sB = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            sA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, buf.kA[kc]),
                                                         __builtin_bit_cast(bf16x8, buf.q[kc]), sA, 0, 0, 0);
            sB = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, buf.kB[kc]),
                                                         __builtin_bit_cast(bf16x8, buf.q[kc]), sB, 0, 0, 0);
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
        const float mn = fmaxf(m, rows4_max(mx));
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

    // acc[j][i] is O^T[dim DPL*(4quad+i) + j][head col].
    __device__ __forceinline__ void store_final(const DecodeArgs &a, int b, int g) {
        const float lt = rows4_sum(l);
        if (col >= G) return;
        const int h = g * G + col;
        const float inv = 1.f / lt;
        uint16_t *o = (uint16_t *)a.out + ((int64_t)b * a.hq + h) * D;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t wv[VW];
#pragma unroll
            for (int w = 0; w < VW; ++w) wv[w] = pack_bf16x2(acc[2 * w][i] * inv, acc[2 * w + 1][i] * inv);
            store_vrow((char *)(o + DPL * (4 * quad + i)), wv);
        }
        if (quad == 0 && a.lse) a.lse[(int64_t)b * a.hq + h] = (m + log2f(lt)) * kLn2;
    }

    __device__ __forceinline__ void store_record(const DecodeArgs &a, int64_t rec, const f32x4 (&o4)[DPL], float mm,
                                                 float ll) {
        const float lt = rows4_sum(ll);
        if (col >= G) return;
        float *o = a.part_o + rec * G * D;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int jj = 0; jj < VW; ++jj)
                st_agent2(o + ((i * VW + jj) * 4 * G + quad * G + col) * 2, o4[2 * jj][i], o4[2 * jj + 1][i]);
        if (quad == 0) st_agent2(a.part_ml + (rec * G + col) * 2, mm, lt);
    }
    __device__ __forceinline__ void store_partial(const DecodeArgs &a, int64_t rec) { store_record(a, rec, acc, m, l); }

    __device__ __forceinline__ void save() {
#pragma unroll
        for (int j = 0; j < DPL; ++j) sacc[j] = acc[j];
        sm = m;
        sl = l;
    }
    __device__ __forceinline__ void store_saved(const DecodeArgs &a, int64_t rec) { store_record(a, rec, sacc, sm, sl); }

    // The same record, values and layout, written to LDS (o: G*D floats, ml: 2G).
    __device__ __forceinline__ void stage_record(float *o, float *ml) {
        const float lt = rows4_sum(l);
        if (col >= G) return;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int jj = 0; jj < VW; ++jj)
                *reinterpret_cast<f32x2 *>(o + ((i * VW + jj) * 4 * G + quad * G + col) * 2) =
                    f32x2{acc[2 * jj][i], acc[2 * jj + 1][i]};
        if (quad == 0) *reinterpret_cast<f32x2 *>(ml + col * 2) = f32x2{m, lt};
    }
};

// End of a piece: its output, or its record (then the merge is pending).
// A split piece with more pages to follow (the range's first) is copied
// aside in registers; the range's last split piece stays in the
// accumulators.  settle() deals with both after the range.
template <class Eng>
__device__ __forceinline__ void finish_piece(const DecodeArgs &a, Eng &eng, const Desc &d, int w, const Range &r,
                                             Pending &pend, bool more) {
    if (d.whole()) {
        eng.store_final(a, d.b, d.g);
    } else {
        const int64_t s = (int64_t)d.b * a.hkv + d.g;
        const int64_t wf = worker_of(d.segf, r);
        const int cnt = (int)(worker_of(d.segf + d.np - 1, r) - wf + 1);
        if (more) {
            eng.save();
            pending_add(pend, s, d.b, d.g, wf, cnt, kSaved);
        } else {
            pending_add(pend, s, d.b, d.g, wf, cnt, kHeld);
            return;
        }
    }
    eng.reset();
}

// LDS one worker wave uses: its range's page ids, and the record of its held
// piece for a merge from registers (G <= 16 heads of D values, then (m, l)).
template <int D>
struct WorkerLds {
    static constexpr int kIdsBytes = kStage * 4;
    static constexpr int kBytes = kIdsBytes + 16 * D * 4 + 2 * 16 * 4;
};

// One split worker (a single wave, worker index w) of the bf16 decode over
// its range of the cost line; lds points at WorkerLds<D>::kBytes bytes of
// this wave's own LDS (16-byte aligned).  The wave synchronises only with
// itself, so several workers may share a workgroup.
template <int D, bool SUB>
__device__ __forceinline__ void decode_bf16_worker(const DecodeArgs &a, int w, char *lds) {
    using Eng = Bf16<D, SUB>;
    int *ids = reinterpret_cast<int *>(lds);
    float *own_o = reinterpret_cast<float *>(lds + WorkerLds<D>::kIdsBytes);
    float *own_ml = own_o + 16 * D;
    RowLens rl;
    Range r;
    Cursor cur;
    if (!plan_or_load<__bf16>(a, w, D, rl, r, cur.s)) return;
    cur.p = cur.pstart = (int)(r.f0 - cur.s.f);
    cur.pend = (int)(cur.s.np < r.f1 - cur.s.f ? cur.s.np : r.f1 - cur.s.f);
    cur.live = 1;
    int64_t fbase = r.f0;
    stage<SUB>(a, ids, cur, r.f1, rl);
    Eng eng;
    eng.init(a);
    Pending pend;
    pending_init(pend);
    const float c = a.scale_log2;
    Desc d0, d1;
    take<SUB>(a, cur, ids, fbase, r.f1, rl, d0);
    if constexpr (D >= 256) {
        // One pair in flight: its loads, then its compute.  Two pair buffers
        // (~200 registers each at head_dim 256) would spill the engine to
        // scratch; a pair is 32 KB here, so the waves keep enough bytes in
        // flight without the second buffer (measured: 388 -> 103 us per call
        // at B = 64, Hq 16 / Hkv 8).
        typename Eng::Buf b0;
        for (;;) {
            eng.issue(a, d0, b0);
            if (__builtin_expect(!cur.live && !d0.whole(), 0))
                pend.check = peek_arrivals(a, (int64_t)d0.b * a.hkv + d0.g);
            eng.compute(a, b0, d0, c);
            const bool more = cur.live;
            if (__builtin_expect(d0.last(), 0)) finish_piece(a, eng, d0, w, r, pend, more);
            if (!more) break;
            take<SUB>(a, cur, ids, fbase, r.f1, rl, d0);
        }
        settle<__bf16, Eng, D>(a, eng, pend, w, own_o, own_ml);
        return;
    }
    typename Eng::Buf b0, b1;
    eng.issue(a, d0, b0);
    // Two buffers in turn: the next pair's loads are issued before the
    // current pair is computed, and no load is left unconsumed at the end, so
    // the compiler's wait counts stay exact across iterations.  The
    // scheduling barriers keep the loads ahead of the compute.
    // After the last pair's loads, the arrival count of its segment is read
    // ahead when its piece is split (it is then the range's held piece).
    // Piece ends, id restages and the last-pair read are rare: they are
    // marked so, which keeps the per-pair path straight-line code.
    if (__builtin_expect(!cur.live && !d0.whole(), 0)) pend.check = peek_arrivals(a, (int64_t)d0.b * a.hkv + d0.g);
    for (;;) {
        if (cur.live) {
            take<SUB>(a, cur, ids, fbase, r.f1, rl, d1);
            __builtin_amdgcn_sched_barrier(0);
            eng.issue(a, d1, b1);
            if (__builtin_expect(!cur.live && !d1.whole(), 0)) pend.check = peek_arrivals(a, (int64_t)d1.b * a.hkv + d1.g);
            __builtin_amdgcn_sched_barrier(0);
            eng.compute(a, b0, d0, c);
            if (__builtin_expect(d0.last(), 0)) finish_piece(a, eng, d0, w, r, pend, true);
        } else {
            eng.compute(a, b0, d0, c);
            if (__builtin_expect(d0.last(), 0)) finish_piece(a, eng, d0, w, r, pend, false);
            break;
        }
        if (cur.live) {
            take<SUB>(a, cur, ids, fbase, r.f1, rl, d0);
            __builtin_amdgcn_sched_barrier(0);
            eng.issue(a, d0, b0);
            if (__builtin_expect(!cur.live && !d0.whole(), 0)) pend.check = peek_arrivals(a, (int64_t)d0.b * a.hkv + d0.g);
            __builtin_amdgcn_sched_barrier(0);
            eng.compute(a, b1, d1, c);
            if (__builtin_expect(d1.last(), 0)) finish_piece(a, eng, d1, w, r, pend, true);
        } else {
            eng.compute(a, b1, d1, c);
            if (__builtin_expect(d1.last(), 0)) finish_piece(a, eng, d1, w, r, pend, false);
            break;
        }
    }
    settle<__bf16, Eng, D>(a, eng, pend, w, own_o, own_ml);
}

}  // namespace

}  // namespace pkv
