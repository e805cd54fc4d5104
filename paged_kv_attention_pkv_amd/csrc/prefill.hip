// prefill.hip -- causal (chunked) prefill attention over the paged KV pool
// (bf16, MFMA, gfx950).
//
// What is computed: request r has q_r query rows (its newest tokens, already
// appended to the pool) and kv_r keys.  With the causal flag, query row i
// (0-based) sees keys 0 .. kv_r - q_r + i -- the end-aligned mask whose pair
// count q(2kv - q + 1)/2 the FlashInfer PR #9451 analysis uses as the work
// measure (§1) -- otherwise all kv_r keys.  Each row's output is softmax
// attention over the visible keys read through block_table, query head h
// reading KV head h / G.
//
// Kernel.  One workgroup (4 waves) per (request, tile of 128 query rows,
// query head); wave w owns query rows 32w .. 32w+31 of the tile.  Keys are
// walked in tiles of 32 (two pages).  Per key tile, for every wave:
//   S^T[32 key x 32 q]  = K[32 x D] . Q^T[D x 32]        (D/16 MFMA 32x32x16)
//   O^T[D x 32 q]      += V^T[D x 32 key] . P^T[32 key x 32 q]  (D/16 MFMA)
// Query rows sit on lanes (lane % 32) so the softmax statistics of a row live
// in two lanes (lane and lane ^ 32); scores carry the softmax scale folded
// into log2 units and use exp2.  Q stays in registers for the whole walk.
// The key tile is staged in LDS twice over: K as [key][dim] and V transposed
// as [dim][key] (the PV contraction runs over keys), both row-padded against
// bank conflicts, double-buffered, with the next tile's global loads in
// flight while the current one is computed.  Keys at or past kv_r (tail
// slots of the last page, which may hold anything) are written to LDS as
// zeros, and masked scores get -inf.  Tiles are scheduled longest first
// (causal rows late in a request see the most keys).
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace pkv {

namespace {

constexpr float kLn2f = 0.6931471805599453f;
constexpr float kNegInff = -__builtin_inff();

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;            // waves per workgroup
constexpr int kRowsPerWave = 32;     // query rows per wave
constexpr int kBM = kWaves * kRowsPerWave;  // query rows per workgroup
constexpr int kBN = 32;              // keys per tile (two pages)
constexpr int kThreads = kWaves * kWave;

template <int D>
struct Smem {
    static constexpr int KSTRIDE = D + 8;    // bf16 elements per K row (16 B pad)
    static constexpr int VSTRIDE = kBN + 4;  // bf16 elements per V^T row (8 B pad)
    static constexpr int KELEMS = kBN * KSTRIDE;
    static constexpr int VELEMS = D * VSTRIDE;
    static constexpr int BUF = KELEMS + VELEMS;  // one stage
    static constexpr int BYTES = 2 * BUF * 2;    // two stages of bf16
};

// Global loads of one key tile: thread t holds chunks t + kThreads*i
// (8 dims each) of K and of V; keys past kv are zero.
template <int D>
struct TileRegs {
    static constexpr int CHUNKS = kBN * D / 8 / kThreads;  // per thread
    u32x4 k[CHUNKS], v[CHUNKS];
};

template <int D>
__device__ __forceinline__ void load_tile(const PrefillArgs &a, const int32_t *bt, int g, int tile, int kv,
                                          TileRegs<D> &t) {
    const int tid = threadIdx.x;
    const int blk0 = tile * 2;
    const int nblk = (kv + kPage - 1) / kPage;
    int page[2];
    page[0] = blk0 < nblk ? bt[blk0] : 0;
    page[1] = blk0 + 1 < nblk ? bt[blk0 + 1] : 0;
#pragma unroll
    for (int u = 0; u < 2; ++u) page[u] = page[u] < 0 ? 0 : (page[u] >= a.num_pages ? a.num_pages - 1 : page[u]);
#pragma unroll
    for (int i = 0; i < TileRegs<D>::CHUNKS; ++i) {
        const int c = tid + kThreads * i;
        const int key = c / (D / 8);
        const int d8 = c - key * (D / 8);
        const int j = tile * kBN + key;
        u32x4 z = {0u, 0u, 0u, 0u};
        if (j < kv) {
            const int pg = page[key >> 4];
            const int64_t off = pg * a.s_page + g * a.s_head + (int64_t)(key & 15) * a.s_tok + d8 * 8;
            t.k[i] = ld16((const uint16_t *)a.k_cache + off);
            t.v[i] = ld16((const uint16_t *)a.v_cache + off);
        } else {
            t.k[i] = z;
            t.v[i] = z;
        }
    }
}

template <int D>
__device__ __forceinline__ void store_tile(uint16_t *buf, const TileRegs<D> &t) {
    using S = Smem<D>;
    const int tid = threadIdx.x;
    uint16_t *ks = buf;
    uint16_t *vt = buf + S::KELEMS;
#pragma unroll
    for (int i = 0; i < TileRegs<D>::CHUNKS; ++i) {
        const int c = tid + kThreads * i;
        const int key = c / (D / 8);
        const int d8 = c - key * (D / 8);
        *reinterpret_cast<u32x4 *>(ks + key * S::KSTRIDE + d8 * 8) = t.k[i];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            vt[(d8 * 8 + 2 * w) * S::VSTRIDE + key] = (uint16_t)(t.v[i][w] & 0xffffu);
            vt[(d8 * 8 + 2 * w + 1) * S::VSTRIDE + key] = (uint16_t)(t.v[i][w] >> 16);
        }
    }
}

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_kernel(PrefillArgs a, int n_qtiles) {
    using S = Smem<D>;
    constexpr int KS = D / 16;  // k-steps of the QK contraction
    constexpr int DB = D / 32;  // 32-dim blocks of the output
    extern __shared__ __align__(16) uint16_t smem[];

    // grid: (request, tile, head) with tiles reversed (longest first)
    const int per_req = n_qtiles * a.hq;
    const int r = blockIdx.x / per_req;
    const int rem = blockIdx.x - r * per_req;
    const int qt = n_qtiles - 1 - rem / a.hq;
    const int h = rem - (rem / a.hq) * a.hq;
    // metadata is clamped so that every access stays inside the buffers
    const int q0 = min(max(a.qo_indptr[r], 0), a.total_q);
    const int q_len = min(max(a.qo_indptr[r + 1] - q0, 0), a.total_q - q0);
    if (qt * kBM >= q_len) return;
    const int kv = min(max(a.kv_lens[r], 0), a.max_kv);
    const int G = a.hq / a.hkv;
    const int g = h / G;
    const int32_t *bt = a.block_table + (int64_t)r * a.bt_cols;

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int half = lane >> 5;
    const int col = lane & 31;
    // this lane's query row (rows past q_len repeat the last row and are not stored)
    const int i_row = qt * kBM + wave * kRowsPerWave + col;
    const bool row_ok = i_row < q_len;
    const int i_eff = row_ok ? i_row : q_len - 1;
    const int limit = a.causal ? kv - q_len + i_eff : kv - 1;  // last visible key

    // key tiles the workgroup walks, and the last one this wave needs
    const int i_last_wg = min(qt * kBM + kBM, q_len) - 1;
    const int last_key_wg = a.causal ? kv - q_len + i_last_wg : kv - 1;
    const int n_tiles = last_key_wg / kBN + 1;
    const int wave_first = qt * kBM + wave * kRowsPerWave;
    const int i_last_wave = min(wave_first + kRowsPerWave, q_len) - 1;
    const int last_key_wave = wave_first >= q_len ? -1 : (a.causal ? kv - q_len + i_last_wave : kv - 1);
    if (kv == 0 || (a.causal && kv < q_len)) {
        // no visible key (only reachable without the causal flag): 0 and -inf
        if (row_ok) {
            uint16_t *orow = (uint16_t *)a.out + ((int64_t)(q0 + i_row) * a.hq + h) * D;
            for (int d = half; d < D; d += 2) orow[d] = 0;
            if (half == 0 && a.lse) a.lse[(int64_t)(q0 + i_row) * a.hq + h] = kNegInff;
        }
        return;
    }

    // Q^T operand: lane holds Q[row][16ks + 8half .. +7] for every k-step
    u32x4 qop[KS];
    {
        const uint16_t *qrow = (const uint16_t *)a.q + ((int64_t)(q0 + i_eff) * a.hq + h) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qop[ks] = ld16(qrow + 16 * ks + 8 * half);
    }
    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
    float m = kNegInff, l = 0.f;
    const float c = a.scale_log2;

    TileRegs<D> regs;
    load_tile<D>(a, bt, g, 0, kv, regs);
    store_tile<D>(smem, regs);
    __syncthreads();
    for (int tile = 0; tile < n_tiles; ++tile) {
        uint16_t *cur = smem + (tile & 1) * S::BUF;
        uint16_t *nxt = smem + ((tile + 1) & 1) * S::BUF;
        const bool more = tile + 1 < n_tiles;
        if (more) load_tile<D>(a, bt, g, tile + 1, kv, regs);

        if (tile * kBN <= last_key_wave) {
            const uint16_t *ks = cur;
            const uint16_t *vt = cur + S::KELEMS;
            // S^T = K . Q^T
            f32x16 s = f32x16{};
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                const u32x4 kop = *reinterpret_cast<const u32x4 *>(ks + col * S::KSTRIDE + 16 * k + 8 * half);
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kop),
                                                            __builtin_bit_cast(bf16x8, qop[k]), s, 0, 0, 0);
            }
            // mask + online softmax; element e is key tile*32 + 8(e/4) + 4half + e%4
            float x[16];
            float mx = kNegInff;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int j = tile * kBN + 8 * (e >> 2) + 4 * half + (e & 3);
                x[e] = j <= limit ? s[e] * c : kNegInff;
                mx = fmaxf(mx, x[e]);
            }
            mx = fmaxf(mx, shfl_xor(mx, 32));
            const float mn = fmaxf(m, mx);
            const float alpha = fast_exp2(m - mn);
            float sum = 0.f;
            float p[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                p[e] = fast_exp2(x[e] - mn);
                sum += p[e];
            }
            l = l * alpha + sum;
            m = mn;
#pragma unroll
            for (int db = 0; db < DB; ++db) acc[db] *= alpha;
            // P^T operands for the two 16-key steps
            u32x4 pop[2];
#pragma unroll
            for (int t = 0; t < 2; ++t)
                pop[t] = u32x4{pack_bf16x2(p[8 * t + 0], p[8 * t + 1]), pack_bf16x2(p[8 * t + 2], p[8 * t + 3]),
                               pack_bf16x2(p[8 * t + 4], p[8 * t + 5]), pack_bf16x2(p[8 * t + 6], p[8 * t + 7])};
            // O^T += V^T . P^T; V^T operand: dim row 32db + col, keys 16t + 4half .. and 16t + 8 + 4half ..
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const uint16_t *vrow = vt + (32 * db + col) * S::VSTRIDE;
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const u32x2 lo = *reinterpret_cast<const u32x2 *>(vrow + 16 * t + 4 * half);
                    const u32x2 hi = *reinterpret_cast<const u32x2 *>(vrow + 16 * t + 8 + 4 * half);
                    const u32x4 vop = {lo[0], lo[1], hi[0], hi[1]};
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vop),
                                                                      __builtin_bit_cast(bf16x8, pop[t]), acc[db], 0,
                                                                      0, 0);
                }
            }
        }
        if (more) {
            store_tile<D>(nxt, regs);
            __syncthreads();
        }
    }

    // normalise and write: acc[db][e] is O^T[dim 32db + 8(e/4) + 4half + e%4][row]
    const float lt = l + shfl_xor(l, 32);
    if (!row_ok) return;
    const float inv = 1.f / lt;
    uint16_t *orow = (uint16_t *)a.out + ((int64_t)(q0 + i_row) * a.hq + h) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            const u32x2 v = {pack_bf16x2(acc[db][4 * e4] * inv, acc[db][4 * e4 + 1] * inv),
                             pack_bf16x2(acc[db][4 * e4 + 2] * inv, acc[db][4 * e4 + 3] * inv)};
            *reinterpret_cast<u32x2 *>(orow + 32 * db + 8 * e4 + 4 * half) = v;
        }
    if (half == 0 && a.lse) a.lse[(int64_t)(q0 + i_row) * a.hq + h] = (m + log2f(lt)) * kLn2f;
}

template <int D>
hipError_t launch_d(const PrefillArgs &a, hipStream_t stream) {
    const int n_qtiles = (a.max_q + kBM - 1) / kBM;
    const int64_t grid = (int64_t)a.batch * n_qtiles * a.hq;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&prefill_kernel<D>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, Smem<D>::BYTES);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL(prefill_kernel<D>, dim3((unsigned)grid), dim3(kThreads), Smem<D>::BYTES, stream, a,
                       n_qtiles);
    return hipGetLastError();
}

}  // namespace

size_t prefill_workspace(const PoolGeom &, int, int, int, int, int) { return 0; }

hipError_t launch_prefill(const PoolGeom &g, const PrefillArgs &a, hipStream_t stream) {
    if (a.max_q <= 0 || a.batch <= 0) return hipSuccess;
    switch (g.head_dim) {
        case 64: return launch_d<64>(a, stream);
        case 128: return launch_d<128>(a, stream);
        case 256: return launch_d<256>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace pkv
