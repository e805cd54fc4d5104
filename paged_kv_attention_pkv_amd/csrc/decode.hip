// decode.hip -- GQA decode attention over the paged KV pool (gfx950).
//
// What is computed: for every sequence b and query head h, softmax attention
// of q[b,h] over the first n_b keys of its block_table row, reading KV head
// h / G (G = Hq / Hkv) -- the attend half of flash_attn_with_kvcache in
// mini-infer 06 "True PagedAttention" §1, run there by a split-KV kernel
// (§6).  Optionally (bf16) the step's new token is appended in the same
// launch: the cache lengths are then the pre-append lengths L, each row
// attends L+1 keys, and the token at position L comes from k_new / v_new and
// is written into its page slot -- the in-place write of §1 folded into the
// attention call, as the unsloth scripts page does inside its captured
// decode step ("Why this works").
//
// Work decomposition ("stream-K" over pages), one kernel launch.  The pages
// of all (sequence, kv head) segments are laid end to end, sequence-major,
// and cut into ranges of equal cost, one per wavefront: `workers` of them, or
// fewer on small calls (each wave keeps at least kMinPagesPerWorker pages; the
// count is decided on the device from the lengths, with no host read-back).
// A segment costs its pages plus a few virtual ones for the work its start
// brings, so a range that starts a segment holds fewer pages.  A wave walks its
// range as one stream of page pairs that crosses segment boundaries without
// draining: the next pair's loads are always in flight while the current one
// is computed.  Every maximal run of one segment inside a range is a
// "piece".  A piece that covers a whole segment writes the final output;
// otherwise it writes an unnormalised (o, m, l) record to the workspace.
// After its range, a wave counts each of its (at most two) split pieces in
// the segment's arrival counter; the piece that arrives last merges every
// record of the segment in piece order (so the result does not depend on
// which piece came last), writes the output and resets the counter to zero
// for the next call.  A wave whose last piece finds, by a read issued with
// its last loads, every other piece already counted merges without writing
// or counting that piece.  Equal costs per wave keep every CU busy to the
// end for any mix of lengths.  Rows with no keys are written (0, lse = -inf)
// by the waves in a round-robin.
//
// A wave first stages the physical page ids of its range in LDS (one
// coalesced pass over the block table), so no table read ever sits in front
// of a page load.
//
// Per page pair, one wave (bf16):
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
// softmax scale folded into log2 units), done with row-swap permutes.
// Masked tokens (past the row length, stale or NaN-poisoned slots) get score
// -inf and V = 0.  The query rows travel with each pair's loads (they hit in
// cache after the first pair of a segment), so the register buffers of a
// pair are self-contained.
#include <math.h>

#include <atomic>

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
    if (a.k_new) return raw >= a.max_kv ? a.max_kv : raw + 1;
    return raw > a.max_kv ? a.max_kv : raw;
}

// Fused mode: the row's last attended key is the new token (not cut away).
__device__ __forceinline__ int fresh_token(const DecodeArgs &a, int raw) {
    return a.k_new && raw >= 0 && raw < a.max_kv;
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

// Line length and this wave's share, with the segment its range starts in.
// The range is [f0, f1) with f0 and f1 the first page positions at or after
// the two cuts, so a walk stops where the next segment would start at or past
// f1.  Rows are handed out round-robin (row b to worker b mod workers) for
// the per-row chores: zero fill of rows without keys, and in fused mode the
// new lengths.  The first 64 raw lengths stay in `rl`.  False when the wave
// has no pages.
template <typename OutT>
__device__ __forceinline__ bool plan(const DecodeArgs &a, int w, int D, RowLens &rl, Range &r, Seg &s) {
    const int l = lane_id();
    int64_t pages = 0;  // pages of all rows, one kv head
    int rows = 0;       // rows with pages
    for (int base = 0; base < a.batch; base += kWave) {
        const int b = base + l;
        const int raw = raw_len(a, b);
        const int n = attended(a, raw);
        const int incl = wave_incl_scan32(ceil_div(n, kPage));
        if (base == 0) {
            rl.base = 0;
            rl.raw = raw;
            rl.incl = incl;
        }
        pages += __builtin_amdgcn_readlane(incl, kWave - 1);
        rows += __builtin_popcountll(__ballot(n > 0));
        const bool mine = b < a.batch && b % a.workers == w;
        // a row whose token is not appended keeps its length; the others get
        // theirs from the wave that writes the token (splice)
        if (mine && a.seqlens_out && !fresh_token(a, raw)) a.seqlens_out[b] = raw;
        uint64_t empty = __ballot(mine && n == 0);
        while (empty) {
            const int e = uniform((int)__builtin_ctzll(empty));
            empty &= empty - 1;
            zero_row<OutT>(a, base + e, D);
        }
    }
    const int64_t total = pages * a.hkv;
    // Small calls use fewer waves, so each keeps at least kMinPagesPerWorker
    // pages (a segment cut into many tiny pieces costs more in merges than
    // the extra waves gain).  A count the caller fixed is used as given.
    const int64_t by_pages = total / kMinPagesPerWorker > 0 ? total / kMinPagesPerWorker : 1;
    int64_t wmax = by_pages < (int64_t)a.workers ? by_pages : (int64_t)a.workers;
    if (a.fixed_workers) wmax = total < (int64_t)a.workers ? total : (int64_t)a.workers;
    if ((int64_t)w >= wmax) return false;
    const int64_t len = total + (int64_t)kSegCostPages * rows * a.hkv;
    r.total = len;
    r.workers = (int)wmax;
    locate2(a, (int64_t)w * len / wmax, (int64_t)(w + 1) * len / wmax, rl, s, r.f0, r.f1);
    return r.f0 < r.f1;
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
                            ml[j][k] = ld_shared2(a.part_ml + (rec * G + col[k]) * 2);
                            o[j][k] = ld_shared2(a.part_o + rec * ostride + 2 * uu[k]);
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
                __syncthreads();
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
__device__ void stage(const DecodeArgs &a, int *ids, const Cursor &c, int64_t f1, RowLens &rl) {
    const int64_t f0 = c.f();
    const int len = (int)(f1 - f0 < kStage ? f1 - f0 : kStage);
    const int l = lane_id();
    Seg s = c.s;
    for (int c0 = 0; c0 < len; c0 += 8 * kWave) {
        const int64_t gend = f0 + (c0 + 8 * kWave < len ? c0 + 8 * kWave : len);
        int64_t off[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) off[u] = -1;
        for (;;) {  // the segments overlapping [f0 + c0, gend)
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int64_t fl = f0 + c0 + u * kWave + l;
                if (fl < gend && fl >= s.f && fl < s.f + s.np) off[u] = (int64_t)s.b * a.bt_cols + (fl - s.f);
            }
            if (s.f + s.np >= gend) break;
            seg_next(a, s, rl);
        }
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = off[u] >= 0 ? a.block_table[off[u]] : 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = c0 + u * kWave + l;
            if (i < len) ids[i] = v[u];
        }
    }
}

// The next pair at the cursor, then advance.  Restages the id window when
// the cursor has run past it.
__device__ __forceinline__ void take(const DecodeArgs &a, Cursor &c, int *ids, int64_t &fbase, int64_t f1,
                                     RowLens &rl, Desc &d) {
    if (__builtin_expect(c.f() - fbase >= kStage, 0)) {
        fbase = c.f();
        stage(a, ids, c, f1, rl);
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
    d.ida = clamp_page(a, ra);
    d.idb = clamp_page(a, rb);
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

template <int D>
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
    __device__ __forceinline__ void issue(const DecodeArgs &a, const Desc &d, Buf &buf) {
        const int64_t hoff = (int64_t)d.g * a.s_head * 2;
        const char *kc = (const char *)a.k_cache + hoff;
        const char *vc = (const char *)a.v_cache + hoff;
        const int64_t ps = a.s_page * 2;
        load_page(kc + d.ida * ps, vc + d.ida * ps, buf.kA, buf.vA);
        load_page(kc + d.idb * ps, vc + d.idb * ps, buf.kB, buf.vB);
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
        const bool writable = d.raw_last >= 1 && d.raw_last < a.num_pages;
        // the new length counts the token only where it was stored
        if (d.g == 0 && lane_id() == 0 && a.seqlens_out) a.seqlens_out[d.b] = writable ? d.n : d.n - 1;
        const int64_t base = (int64_t)d.g * a.s_head * 2 + (int64_t)d.raw_last * a.s_page * 2;
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
                st_shared2(o + ((i * VW + jj) * 4 * G + quad * G + col) * 2, o4[2 * jj][i], o4[2 * jj + 1][i]);
        if (quad == 0) st_shared2(a.part_ml + (rec * G + col) * 2, mm, lt);
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

template <int D>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1)))
void decode_bf16_kernel(DecodeArgs a) {
    using Eng = Bf16<D>;
    __shared__ int ids[kStage];
    __shared__ __align__(16) float own_o[16 * D];  // the held piece's record for a merge from registers (G <= 16)
    __shared__ __align__(16) float own_ml[2 * 16];
    const int w = blockIdx.x;
    RowLens rl;
    Range r;
    Cursor cur;
    if (!plan<__bf16>(a, w, D, rl, r, cur.s)) return;
    cur.p = cur.pstart = (int)(r.f0 - cur.s.f);
    cur.pend = (int)(cur.s.np < r.f1 - cur.s.f ? cur.s.np : r.f1 - cur.s.f);
    cur.live = 1;
    int64_t fbase = r.f0;
    stage(a, ids, cur, r.f1, rl);
    Eng eng;
    eng.init(a);
    Pending pend;
    pending_init(pend);
    const float c = a.scale_log2;
    typename Eng::Buf b0, b1;
    Desc d0, d1;
    take(a, cur, ids, fbase, r.f1, rl, d0);
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
            take(a, cur, ids, fbase, r.f1, rl, d1);
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
            take(a, cur, ids, fbase, r.f1, rl, d0);
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

// ---------------------------------------------------------------------------
// fp32: MFMA 16x16x4 f32, one page per step (no fused append)
// ---------------------------------------------------------------------------

template <int D>
struct EngF32 {
    static constexpr bool kHolds = false;
    using Out = float;
    static constexpr int KC = D / 4;   // QK MFMAs per page
    static constexpr int DC = D / 16;  // output dim chunks

    float qop[KC];
    f32x4 acc[DC];
    float m, l;
    int G, quad, col;

    // Output dim of record pair (t, quad): acc[dc][2ii], acc[dc][2ii+1] with t = 2dc + ii.
    __device__ static __forceinline__ int dim_of(int t, int quad) { return 16 * (t >> 1) + 4 * quad + 2 * (t & 1); }

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
            const float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
            const float mn = fmaxf(m, rows4_max(mx));
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
    __device__ __forceinline__ void store_final(const DecodeArgs &a, int b, int g) {
        const float lt = rows4_sum(l);
        if (col >= G) return;
        const int h = g * G + col;
        float *o = (float *)a.out + ((int64_t)b * a.hq + h) * D;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) *reinterpret_cast<f32x4 *>(o + 16 * dc + 4 * quad) = acc[dc] / lt;
        if (quad == 0 && a.lse) a.lse[(int64_t)b * a.hq + h] = (m + log2f(lt)) * kLn2;
    }

    __device__ __forceinline__ void store_partial(const DecodeArgs &a, int64_t rec) {
        const float lt = rows4_sum(l);
        if (col >= G) return;
        float *o = a.part_o + rec * G * D;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
            st_shared2(o + ((2 * dc) * 4 * G + quad * G + col) * 2, acc[dc][0], acc[dc][1]);
            st_shared2(o + ((2 * dc + 1) * 4 * G + quad * G + col) * 2, acc[dc][2], acc[dc][3]);
        }
        if (quad == 0) st_shared2(a.part_ml + (rec * G + col) * 2, m, lt);
    }
};

template <int D>
__global__ __launch_bounds__(64) void decode_f32_kernel(DecodeArgs a) {
    using Eng = EngF32<D>;
    const int w = blockIdx.x;
    RowLens rl;
    Range r;
    Seg s;
    if (!plan<float>(a, w, D, rl, r, s)) return;
    int p0 = (int)(r.f0 - s.f);
    Eng eng;
    Pending pend;
    pending_init(pend);
    for (;;) {
        const int64_t left = r.f1 - (s.f + p0);
        const int p1 = left < (int64_t)(s.np - p0) ? p0 + (int)left : s.np;
        eng.init(a, s.b, s.g);
        eng.run(a, s.b, s.g, s.n, p0, p1);
        if (p0 == 0 && p1 == s.np) {
            eng.store_final(a, s.b, s.g);
        } else {
            const int64_t seg = (int64_t)s.b * a.hkv + s.g;
            eng.store_partial(a, (int64_t)w + seg);
            const int64_t wf = worker_of(s.f, r);
            pending_add(pend, seg, s.b, s.g, wf, (int)(worker_of(s.f + s.np - 1, r) - wf + 1), kStored);
        }
        if (s.f + p1 + kSegCostPages >= r.f1) break;
        seg_next(a, s, rl);
        p0 = 0;
    }
    settle<float, Eng, D>(a, eng, pend, w, nullptr, nullptr);
}

const void *pick_kernel(int dtype, int d) {
    if (dtype == 1) {
        if (d == 64) return reinterpret_cast<const void *>(&decode_bf16_kernel<64>);
        if (d == 128) return reinterpret_cast<const void *>(&decode_bf16_kernel<128>);
        if (d == 256) return reinterpret_cast<const void *>(&decode_bf16_kernel<256>);
    } else {
        if (d == 64) return reinterpret_cast<const void *>(&decode_f32_kernel<64>);
        if (d == 128) return reinterpret_cast<const void *>(&decode_f32_kernel<128>);
        if (d == 256) return reinterpret_cast<const void *>(&decode_f32_kernel<256>);
    }
    return nullptr;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Lazily filled per-device launch facts.  Several host threads may launch on
// one device at once: each field is written with the same value by whichever
// thread gets there first, through relaxed atomics.
struct DeviceInfo {
    std::atomic<int> cus{0};
    std::atomic<int> occ[2][3] = {{{0}, {0}, {0}}, {{0}, {0}, {0}}};  // resident decode waves per CU [dtype][d]
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
        int cus = info.cus.load(std::memory_order_relaxed);
        if (cus == 0) {
            if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus <= 0)
                return -1;
            info.cus.store(cus, std::memory_order_relaxed);
        }
        std::atomic<int> &occ_slot = info.occ[g.dtype == 1 ? 1 : 0][dim_index(g.head_dim)];
        int occ = occ_slot.load(std::memory_order_relaxed);
        if (occ == 0) {
            int blocks = 0;
            int cur = -1;
            // the occupancy query is answered for the current device
            if (hipGetDevice(&cur) != hipSuccess || cur != device ||
                hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, pick_kernel(g.dtype, g.head_dim), kWave, 0) !=
                    hipSuccess ||
                blocks <= 0)
                return -1;
            occ = blocks > 16 ? 16 : blocks;
            occ_slot.store(occ, std::memory_order_relaxed);
        }
        w = (int64_t)cus * occ;
    }
    if (max_pages_bound >= 0 && w > max_pages_bound) w = max_pages_bound;
    if (w < 1) w = 1;
    if (w > (1 << 22)) w = 1 << 22;
    return (int)w;
}

// Workspace: one int32 arrival counter per (sequence, kv head) first, then
// the partial records (o: G*D fp32, (m, l): 2 fp32) for up to
// `record_workers` + batch*hkv pieces.  `record_workers` is the worker count
// before any cap by the call's page count, so the size and the layout depend
// on the batch shape and the device only, never on the lengths.  The
// counters must be zero before a call; every call that completes leaves them
// zero.
size_t decode_workspace(const PoolGeom &g, int batch, int hq, int record_workers) {
    const int G = hq / g.hkv;
    const size_t recs = (size_t)record_workers + (size_t)batch * g.hkv;
    return decode_counter_bytes(g, batch) + align256(recs * G * g.head_dim * sizeof(float)) +
           align256(recs * G * 2 * sizeof(float));
}

size_t decode_counter_bytes(const PoolGeom &g, int batch) { return align256((size_t)batch * g.hkv * sizeof(int32_t)); }

hipError_t launch_decode(const PoolGeom &g, DecodeArgs a, void *workspace, int record_workers, hipStream_t stream) {
    const int G = a.hq / a.hkv;
    const size_t recs = (size_t)record_workers + (size_t)a.batch * a.hkv;
    char *ws = (char *)workspace;
    a.arrivals = (int32_t *)ws;
    a.part_o = (float *)(ws + decode_counter_bytes(g, a.batch));
    a.part_ml = (float *)((char *)a.part_o + align256(recs * G * g.head_dim * sizeof(float)));
    const void *k = pick_kernel(g.dtype, g.head_dim);
    void *args[] = {&a};
    hipError_t e = hipLaunchKernel(k, dim3(a.workers), dim3(kWave), args, 0, stream);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace pkv
