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
// The cut depends only on the lengths and the call's shape, so the calls of
// one decode step (one per layer) may share it: decode_plan_kernel writes it
// to the workspace once, and a call takes its range from there when the
// plan matches it exactly (decode_worker.hpp, plan_or_load).
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

#include "decode_worker.hpp"

namespace pkv {

namespace {

// SUB: pages of more than 16 tokens (page ids staged with their sub-page)
template <int D, bool SUB>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1)))
void decode_bf16_kernel(DecodeArgs a) {
    __shared__ __align__(16) char lds[WorkerLds<D>::kBytes];
    decode_bf16_worker<D, SUB>(a, blockIdx.x, lds);
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
            // 16-token sub-page p: table column p >> page_shift, then its sub-page
            const int phys = clamp_page(a, bt[p >> a.page_shift]);
            const int64_t soff = (int64_t)(p & ((1 << a.page_shift) - 1)) * kPage * a.s_tok;
            const float *kp = kbase + (int64_t)phys * a.s_page + soff;
            const float *vp = vbase + (int64_t)phys * a.s_page + soff;
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
            st_agent2(o + ((2 * dc) * 4 * G + quad * G + col) * 2, acc[dc][0], acc[dc][1]);
            st_agent2(o + ((2 * dc + 1) * 4 * G + quad * G + col) * 2, acc[dc][2], acc[dc][3]);
        }
        if (quad == 0) st_agent2(a.part_ml + (rec * G + col) * 2, m, lt);
    }
};

// The plan of a call shaped as `a` (see write_plan).
__global__ __launch_bounds__(64) void decode_plan_kernel(DecodeArgs a) { write_plan(a, blockIdx.x); }

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

const void *pick_kernel(int dtype, int d, bool sub = false) {
    if (dtype == 1) {
        if (d == 64) return sub ? reinterpret_cast<const void *>(&decode_bf16_kernel<64, true>)
                                : reinterpret_cast<const void *>(&decode_bf16_kernel<64, false>);
        if (d == 128) return sub ? reinterpret_cast<const void *>(&decode_bf16_kernel<128, true>)
                                 : reinterpret_cast<const void *>(&decode_bf16_kernel<128, false>);
        if (d == 256) return sub ? reinterpret_cast<const void *>(&decode_bf16_kernel<256, true>)
                                 : reinterpret_cast<const void *>(&decode_bf16_kernel<256, false>);
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

// Mid-sized calls: on the bf16 head_dim 128 kernel (one wave per SIMD, four
// per CU) a call of fewer than 64 (page, kv head) units per CU runs faster on
// three waves per CU than on four (measured over batch 8..64 of two length
// mixes: up to 10% at 9000-12000 units, within 1% elsewhere); larger calls
// keep four.  Smaller calls are cut further by the pages-per-worker floor.
void decode_mid_cap(int device, const PoolGeom &g, int w_rec, DecodeArgs &a) {
    a.mid_workers = 0;
    a.mid_pages = 0;
    if (a.fixed_workers || g.dtype != 1 || g.head_dim != 128 || device < 0 || device >= kMaxDevices) return;
    const int cus = g_info[device].cus.load(std::memory_order_relaxed);
    if (cus <= 0 || w_rec != 4 * cus) return;
    a.mid_workers = 3 * cus;
    a.mid_pages = 64 * (int64_t)cus;
}

// Workspace: one int32 arrival counter per (sequence, kv head) first, then
// the partial records (o: G*D fp32, (m, l): 2 fp32) for up to
// `record_workers` + batch*hkv pieces, then the plan region (header, the
// planned length of every row, one record per worker; decode_worker.hpp).
// `record_workers` is the worker count before any cap by the call's page
// count, so the size and the layout depend on the batch shape and the device
// only, never on the lengths.  The counters must be zero before a call; every
// call that completes leaves them zero.
static size_t decode_records_end(const PoolGeom &g, int batch, int hq, int record_workers) {
    const int G = hq / g.hkv;
    const size_t recs = (size_t)record_workers + (size_t)batch * g.hkv;
    return decode_counter_bytes(g, batch) + align256(recs * G * g.head_dim * sizeof(float)) +
           align256(recs * G * 2 * sizeof(float));
}

static size_t decode_plan_bytes(int batch, int record_workers) {
    return (size_t)kPlanHdr * 4 + align256((size_t)batch * 4) + align256((size_t)record_workers * kPlanRec * 4);
}

size_t decode_workspace(const PoolGeom &g, int batch, int hq, int record_workers) {
    return decode_records_end(g, batch, hq, record_workers) + decode_plan_bytes(batch, record_workers);
}

size_t decode_counter_bytes(const PoolGeom &g, int batch) { return align256((size_t)batch * g.hkv * sizeof(int32_t)); }

void decode_workspace_layout(const PoolGeom &g, DecodeArgs &a, void *workspace, int record_workers) {
    const int G = a.hq / a.hkv;
    const size_t recs = (size_t)record_workers + (size_t)a.batch * a.hkv;
    char *ws = (char *)workspace;
    a.arrivals = (int32_t *)ws;
    a.part_o = (float *)(ws + decode_counter_bytes(g, a.batch));
    a.part_ml = (float *)((char *)a.part_o + align256(recs * G * g.head_dim * sizeof(float)));
    a.plan = (int32_t *)(ws + decode_records_end(g, a.batch, a.hq, record_workers));
}

hipError_t launch_decode(const PoolGeom &g, DecodeArgs a, void *workspace, int record_workers, bool use_plan,
                         hipStream_t stream) {
    decode_workspace_layout(g, a, workspace, record_workers);
    if (!use_plan) a.plan = nullptr;
    const void *k = pick_kernel(g.dtype, g.head_dim, g.page_shift > 0);
    void *args[] = {&a};
    hipError_t e = hipLaunchKernel(k, dim3(a.workers), dim3(kWave), args, 0, stream);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

hipError_t launch_decode_plan(const PoolGeom &g, DecodeArgs a, void *workspace, int record_workers,
                              hipStream_t stream) {
    decode_workspace_layout(g, a, workspace, record_workers);
    void *args[] = {&a};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&decode_plan_kernel), dim3(a.workers), dim3(kWave),
                                   args, 0, stream);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace pkv
